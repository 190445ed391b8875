"""Test harness: run the HIP path and the oracle on the same seeded inputs and compare.

Inputs come from ``synth`` (shared by both sides); the oracle never sees anything the HIP
path produced.  Tolerances (the layer's stated bar for the BF16 output): max |y - y_ref| <=
2e-2 * max |y_ref| and mean relative error sum|y - y_ref| / sum|y_ref| <= 5e-3.  Dispatch
metadata must match bit for bit.  Intermediate E4M3 codes may differ by one code step where
the SwiGLU value sits near a rounding boundary: the oracle's block sums are exact, while the
gfx950 FP8 MFMA returns a 128-long block sum with an absolute error of up to ~2.2e-4 of the
sum of the magnitudes of its products (measured on random E4M3 codes), which moves values by a
few 1e-5 of the group's amax.  At most 0.5% of codes may differ, and a differing code's value
(in units of its group scale, where amax maps to 448) may be off by at most one E4M3 spacing
plus 0.25 units (5.6e-4 of amax).
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


def problem_of(spec: synth.Spec, flags: int = 0) -> mm.Problem:
    flags |= mm.FLAG_CLAMP_INPUTS if spec.clamp_inputs else 0
    return mm.Problem.make(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, spec.swiglu_clamp, flags)


def oracle_problem(spec: synth.Spec) -> oracle.Problem:
    return oracle.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, spec.swiglu_clamp,
                          spec.clamp_inputs)


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
    mm.mega_moe_forward(prob, D["x"], D["x_sf"], D["topk_idx"], D["topk_w"], D["l1_w"], l1_sf,
                        D["l2_w"], l2_sf, y, workspace)
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
    host = {}
    for k, v in P.items():
        if k in ("l1_w", "l1_sf", "l2_w", "l2_sf") and v.is_cuda:
            host[k] = LazyExperts(v)
        else:
            host[k] = v.cpu().numpy()
    return oracle.forward(oracle_problem(spec), tokens=tokens, **host)


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


def assert_intermediate_close(spec, views, ref: dict, rows=None):
    """Compare the E4M3 intermediate and its scales for the pool rows the oracle computed."""
    pool_rows = sorted(ref["inter_q"].keys()) if rows is None else rows
    if not pool_rows:
        return 0.0
    got_q = views["inter_q"][pool_rows].cpu().numpy()
    exp_q = np.stack([ref["inter_q"][p] for p in pool_rows])
    gv, ev = _E4M3[got_q], _E4M3[exp_q]
    diff = np.abs(gv - ev)
    frac = float((diff != 0).mean())
    # E4M3 spacing at the reference value: 2^(e-3) for normal codes, 2^-9 for subnormals
    mag = np.maximum(np.abs(ev), 2.0 ** -6)
    spacing = 2.0 ** (np.floor(np.log2(mag)) - 3)
    bad = diff > spacing + 0.25
    assert not bad.any(), f"{int(bad.sum())} intermediate codes off by more than one step + 0.25"
    assert frac <= CODE_MISMATCH_FRAC, f"{frac:.4%} of intermediate codes differ"
    got_s = views["inter_sf"][pool_rows].cpu().numpy()
    exp_s = np.stack([ref["inter_sf"][p] for p in pool_rows])
    if spec.recipe == 0:
        np.testing.assert_allclose(got_s, exp_s, rtol=1e-3, atol=0)
    else:
        assert np.abs(got_s.astype(np.int64) - exp_s.astype(np.int64)).max() <= 1
    return frac
