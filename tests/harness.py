"""Test harness: run the HIP path and the oracle on the same seeded inputs and compare.

Inputs come from ``synth`` (shared by both sides); the oracle never sees anything the HIP
path produced.  Tolerances (the layer's stated bar for the BF16 output): max |y - y_ref| <=
2e-2 * max |y_ref| and mean relative error sum|y - y_ref| / sum|y_ref| <= 5e-3.  Dispatch
metadata must match bit for bit.

The E4M3 intermediate is checked element by element against a bound derived from the
arithmetic (see ``intermediate_bound``): the oracle's L1 block sums are exact, while the
matrix core returns each 128-long block sum within EPS_MFMA of the sum of its products'
magnitudes (asserted on the hardware by tests/test_gpu_mfma_error.py), and the two sides then
round the value to the nearest E4M3 code of their own group scale.
"""
from __future__ import annotations

import numpy as np
import torch

import dispatch_fp8_grouped_topk_amd as mm
import oracle
import synth

Y_MAX_REL = 2e-2
Y_MEAN_REL = 5e-3
CODE_MISMATCH_FRAC = 5e-3
# Error of one hardware 128-K block sum relative to the sum of its products' magnitudes
# (16x16x128 scaled F8F6F4 MFMA of gfx950; the bound tests/test_gpu_mfma_error.py asserts).
EPS_MFMA = 2.0 ** -11
SILU_SLOPE_MAX = 1.1       # max |d silu(g) / dg| = 1.0998 (at g = 2.3994)


def problem_of(spec: synth.Spec, flags: int = 0) -> mm.Problem:
    flags |= mm.FLAG_CLAMP_INPUTS if spec.clamp_inputs else 0
    flags |= mm.FLAG_INTER_SF64 if spec.inter_sf64 else 0
    return mm.Problem.make(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, spec.swiglu_clamp, flags)


def oracle_problem(spec: synth.Spec) -> oracle.Problem:
    return oracle.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, spec.swiglu_clamp,
                          spec.clamp_inputs, spec.inter_sf64)


def to_device(P: dict, device="cuda") -> dict:
    return {k: v.to(device).contiguous() for k, v in P.items()}


def run_gpu(spec: synth.Spec, D: dict, flags: int = 0, workspace=None, fill=None):
    """Run the HIP path on device inputs D; returns (y bf16 bits as int16 tensor, views, workspace)."""
    prob = problem_of(spec, flags)
    need = mm.mega_moe_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    if fill is not None:
        workspace.fill_(fill)
    y = torch.empty(spec.T, spec.H, dtype=torch.bfloat16, device="cuda")
    l1_sf, l2_sf = D["l1_sf"], D["l2_sf"]
    if flags & mm.FLAG_WEIGHT_SF_KMAJOR:          # the one-time weight-scale transform, then its layout
        l1_sf, l2_sf = mm.mega_moe_transform_weight_scales(prob, l1_sf, l2_sf)
    l1_w, l2_w = D["l1_w"], D["l2_w"]
    if flags & mm.FLAG_WEIGHT_E2M1_PAIRED:        # the one-time E2M1 weight transform, then its layout
        l1_w, l2_w = mm.mega_moe_transform_weights(prob, l1_w, l2_w)
    mm.mega_moe_forward(prob, D["x"], D["x_sf"], D["topk_idx"], D["topk_w"], l1_w, l1_sf,
                        l2_w, l2_sf, y, workspace)
    torch.cuda.synchronize()
    views = mm.mega_moe_workspace_views(prob, workspace) if spec.T > 0 else None
    return y.view(torch.int16), views, workspace


class LazyExperts:
    """Host copy of one expert's weights on demand (oracle input from a device tensor)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return self.t[e].cpu().numpy()


def run_oracle(spec: synth.Spec, P: dict, tokens=None) -> dict:
    """The oracle forward on the same inputs, with the L1 magnitude sums the intermediate
    tolerance is derived from."""
    host = {}
    for k, v in P.items():
        if k in ("l1_w", "l1_sf", "l2_w", "l2_sf") and v.is_cuda:
            host[k] = LazyExperts(v)
        else:
            host[k] = v.cpu().numpy()
    return oracle.forward(oracle_problem(spec), tokens=tokens, magnitudes=True, **host)


def y_errors(y_bits: np.ndarray, ref_bits: np.ndarray):
    y = oracle.bf16_bits_to_f32(y_bits.astype(np.uint16)).astype(np.float64)
    r = oracle.bf16_bits_to_f32(ref_bits.astype(np.uint16)).astype(np.float64)
    max_err = np.abs(y - r).max() if y.size else 0.0
    max_ref = np.abs(r).max() if r.size else 0.0
    mean_rel = np.abs(y - r).sum() / max(np.abs(r).sum(), 1e-300)
    return max_err, max_ref, mean_rel


def assert_y_close(y_bits: np.ndarray, ref_bits: np.ndarray, what=""):
    max_err, max_ref, mean_rel = y_errors(y_bits, ref_bits)
    assert max_err <= Y_MAX_REL * max_ref, f"{what}: max err {max_err} > {Y_MAX_REL} * {max_ref}"
    assert mean_rel <= Y_MEAN_REL, f"{what}: mean relative error {mean_rel}"
    return max_err / max(max_ref, 1e-300), mean_rel


def assert_dispatch_exact(spec: synth.Spec, idx: np.ndarray, views: dict):
    d = oracle.route(idx, spec.E)
    n = int(d["offset"][-1])
    assert np.array_equal(views["expert_count"].cpu().numpy(), d["count"])
    assert np.array_equal(views["expert_offset"].cpu().numpy(), d["offset"])
    assert np.array_equal(views["pool_src"].cpu().numpy()[:n], d["src"])
    assert np.array_equal(views["pair_pos"].cpu().numpy(), d["pos"])
    assert int(views["num_invalid"].cpu().numpy()[0]) == d["num_invalid"]
    return d


_E4M3 = oracle.e4m3_decode_table()


def e4m3_spacing(code_values: np.ndarray) -> np.ndarray:
    """Distance to the next E4M3 code above |c|: 2^(e-3) in binade e, 2^-9 for subnormals."""
    mag = np.maximum(np.abs(code_values), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(mag)) - 3)


def value_error_bound(spec, ref: dict, p: int) -> np.ndarray:
    """Largest |v_gpu - v_ref| the arithmetic allows for pool row p's pre-quantisation values.

    Gate and up are sums over H/128 K blocks; each hardware block sum is within EPS_MFMA of the
    magnitude sum of its products, and float32 accumulation of the blocks adds at most one
    rounding per block, so |dg| <= eps * A_g with eps = EPS_MFMA + (H/128 + 2) 2^-23 and A_g the
    oracle's magnitude sum (likewise for up).  SiLU is Lipschitz with constant 1.1 and clamping is
    1-Lipschitz, so s = silu(g) u moves by at most 1.1 (|u| + du) dg + (|silu(g)| + 1.1 dg) du;
    its float32 evaluation (hardware exp and reciprocal) adds 2^-19 |s|, the top-k weight and the
    scale multiply another 2^-20 |v|.
    """
    I = spec.I
    acc, mag = ref["l1_acc"][p], ref["l1_abs"][p]
    g, u = acc[:I], acc[I:]
    eps = EPS_MFMA + (spec.H // 128 + 2) * 2.0 ** -23
    dg, du = eps * mag[:I], eps * mag[I:]
    c = spec.swiglu_clamp
    if c > 0 and spec.clamp_inputs:
        g, u = np.clip(g, -c, c), np.clip(u, -c, c)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    ds = SILU_SLOPE_MAX * (np.abs(u) + du) * dg + (np.abs(silu) + SILU_SLOPE_MAX * dg) * du
    v = ref["v"][p]
    return abs(ref["w"][p]) * (ds + np.abs(silu * u) * 2.0 ** -19) + np.abs(v) * 2.0 ** -20


def assert_intermediate_close(spec, views, ref: dict, rows=None, max_code_frac=CODE_MISMATCH_FRAC):
    """Compare the E4M3 intermediate and its scales, element by element, for the pool rows the
    oracle computed (it must have been run with magnitudes=True).

    With x = v / sf rounded to the nearest code c on each side, |c sf - v| <= spacing(c) sf / 2,
    so the dequantised values may differ by half a code spacing on each side (each at its own
    scale) plus the value error bound.  Scales: the float scale amax/448 moves by at most the
    largest value error of its group / 448; a UE8M0 code by at most one.  Returns the fraction of
    codes that differ, which must also stay within max_code_frac: an empirical check beside the
    derived bound (the hardware's typical block-sum error is about a tenth of its worst case, so
    on real data few values lie close enough to a rounding boundary to flip; an error of the
    worst-case size everywhere would flip a fifth of the codes while staying inside the bound).
    """
    pool_rows = sorted(ref["inter_q"].keys()) if rows is None else rows
    if not pool_rows:
        return 0.0
    G = spec.inter_group
    got_q = views["inter_q"][pool_rows].cpu().numpy()
    exp_q = np.stack([ref["inter_q"][p] for p in pool_rows])
    got_s = views["inter_sf"][pool_rows].cpu().numpy()
    exp_s = np.stack([ref["inter_sf"][p] for p in pool_rows])
    if spec.recipe == 0:
        sg, se = got_s.astype(np.float64), exp_s.astype(np.float64)
    else:
        sg = np.ldexp(1.0, got_s.astype(np.int64) - 127)
        se = np.ldexp(1.0, exp_s.astype(np.int64) - 127)
    dv = np.stack([value_error_bound(spec, ref, p) for p in pool_rows])
    n, I = got_q.shape
    gv, ev = _E4M3[got_q], _E4M3[exp_q]
    sg_e, se_e = np.repeat(sg, G, axis=1), np.repeat(se, G, axis=1)
    got_v, exp_v = gv * sg_e, ev * se_e
    allowed = (e4m3_spacing(gv) * sg_e + e4m3_spacing(ev) * se_e) / 2 + dv * (1 + 2.0 ** -4)
    err = np.abs(got_v - exp_v)
    bad = err > allowed
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(
            f"{int(bad.sum())} of {bad.size} intermediate values outside the derived bound; first: pool row "
            f"{pool_rows[i]} channel {j}: gpu {got_v[i, j]!r} (code {got_q[i, j]}) ref {exp_v[i, j]!r} "
            f"(code {exp_q[i, j]}), |diff| {err[i, j]:.3e} > {allowed[i, j]:.3e}")
    frac = float((gv != ev).mean())
    assert frac <= max_code_frac, f"{frac:.4%} of intermediate codes differ"
    dv_group = dv.reshape(n, I // G, G).max(axis=2)
    if spec.recipe == 0:
        ds_ok = np.abs(sg - se) <= dv_group / 448.0 * (1 + 2.0 ** -4) + se * 2.0 ** -22
        assert ds_ok.all(), f"{int((~ds_ok).sum())} float scales outside the derived bound"
    else:
        assert np.abs(got_s.astype(np.int64) - exp_s.astype(np.int64)).max() <= 1
    return frac
