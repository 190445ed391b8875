"""Pins for the oracle's arithmetic (CPU only).

* brute force: a per-token, per-element re-derivation with exact rational GEMM
  sums and a nearest-value FP8 search must reproduce the oracle bit for bit;
* a library special case: with E=1, k=1 the L1 GEMM is a dense matmul
  (torch.matmul in float64 on dequantised operands);
* SwiGLU against torch.nn.functional.silu;
* re-quantisation invariants and error bounds;
* layer invariants: power-of-two top-k weight scaling, one-hot weights, k=1,
  token permutation and expert relabelling.
"""
import math
import os
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(P):
    return {k: v.numpy() for k, v in P.items()}


def _prob(spec):
    return oracle.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, spec.swiglu_clamp,
                          spec.clamp_inputs, spec.inter_sf64)


# ----------------------------------------------------------------------------- brute force
def _e2m1_table():
    tab = {}
    with open(os.path.join(GOLDEN, "e2m1_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                n, v = line.split()
                tab[int(n)] = float(v)
    return tab


_FP8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
_FP4 = _e2m1_table()


def _nearest_fp8(r):
    """Brute-force nearest finite E4M3 code to r, exact ties to the even code."""
    best, bestd = None, None
    for c in range(256):
        v = _FP8[c]
        if math.isnan(v) or (math.copysign(1.0, v) != math.copysign(1.0, r)):
            continue
        d = abs(Fraction(v) - Fraction(float(r)))
        if best is None or d < bestd or (d == bestd and (c & 1) == 0 and (best & 1) == 1):
            best, bestd = c, d
    return best


def _row_vals_w(spec, w_row):
    if spec.recipe != 1:                            # E4M3 weight bytes (recipes 0 and 2)
        return [_FP8[b] for b in w_row]
    out = []
    for b in w_row:
        out.append(_FP4[int(b) & 0xF])
        out.append(_FP4[int(b) >> 4])
    return out


def _scale_x(spec, sf_row, kb):
    return Fraction(float(sf_row[kb])) if spec.recipe == 0 else Fraction(2) ** (int(sf_row[kb]) - 127)


def _scale_w(spec, sf_e, n, kb):
    if spec.recipe == 0:
        return Fraction(float(sf_e[n // 128][kb]))
    return Fraction(2) ** (int(sf_e[n][kb]) - 127)


def brute_force(spec, P):
    """Per-token loops; GEMMs in exact rationals, rounded once to float64."""
    T, H, I, E, k = spec.T, spec.H, spec.I, spec.E, spec.k
    G = spec.group
    x, x_sf, idx, tw = P["x"], P["x_sf"], P["topk_idx"], P["topk_w"]
    y = np.zeros((T, H), dtype=np.uint16)
    accs = {}
    for t in range(T):
        xa = [_FP8[b] for b in x[t]]
        total = np.float32(0.0)
        tot = np.zeros(H, dtype=np.float32)
        for j in range(k):
            e = int(idx[t, j])
            if e < 0 or e >= E:
                continue
            # L1
            acc = []
            for n in range(2 * I):
                wv = _row_vals_w(spec, P["l1_w"][e][n])
                s = Fraction(0)
                for kb in range(H // G):
                    blk = sum(Fraction(xa[h]) * Fraction(wv[h]) for h in range(kb * G, (kb + 1) * G))
                    s += blk * _scale_x(spec, x_sf[t], kb) * _scale_w(spec, P["l1_sf"][e], n, kb)
                acc.append(float(s))
            accs[(t, j)] = acc
            v32 = []
            for i in range(I):
                g, u = acc[i], acc[I + i]
                c = spec.swiglu_clamp
                if c > 0 and spec.clamp_inputs:          # activation clamp on gate and up
                    g, u = min(max(g, -c), c), min(max(u, -c), c)
                sv = g / (1.0 + math.exp(-g)) * u
                if c > 0 and not spec.clamp_inputs:      # clamp on silu(g) * u
                    sv = min(max(sv, -c), c)
                v32.append(np.float32(sv * float(np.float32(tw[t, j]))))
            # re-quantisation, group by group (Gq channels: the input block, or 64)
            Gq = 64 if spec.inter_sf64 else G
            deq = []
            for gi in range(I // Gq):
                grp = v32[gi * Gq:(gi + 1) * Gq]
                amax = max(abs(v) for v in grp)
                if spec.recipe == 0:
                    sf = np.float32(amax) / np.float32(448.0)
                    codes = [0] * Gq if sf == 0 else \
                        [_nearest_fp8(min(max(float(np.float32(v) / sf), -448.0), 448.0)) for v in grp]
                    gscale = Fraction(float(sf))
                else:
                    r = np.float32(amax) / np.float32(448.0)
                    c = 0
                    while c < 254 and Fraction(2) ** (c - 127) < Fraction(float(r)):
                        c += 1
                    codes = [0] * Gq if amax == 0 else \
                        [_nearest_fp8(min(max(float(v) * 2.0 ** (127 - c), -448.0), 448.0)) for v in grp]
                    gscale = Fraction(2) ** (c - 127)
                deq.append((codes, gscale))
            # L2: each Gq-channel group with its own scale and the weight scale of its K block
            for n in range(H):
                wv = _row_vals_w(spec, P["l2_w"][e][n])
                s = Fraction(0)
                for gi, (codes, gscale) in enumerate(deq):
                    blk = sum(Fraction(_FP8[codes[i]]) * Fraction(wv[gi * Gq + i]) for i in range(Gq))
                    s += blk * gscale * _scale_w(spec, P["l2_sf"][e], n, gi * Gq // G)
                o32 = np.float32(float(s))
                slot = torch.tensor([float(o32)], dtype=torch.float32).to(torch.bfloat16).float().item()
                tot[n] = np.float32(tot[n] + np.float32(slot))
        y[t] = torch.from_numpy(tot).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return y, accs


BRUTE_SPECS = {
    "fp8": synth.Spec(3, 256, 128, 3, 2, seed=11, weight_set=11),
    "fp8_clamp": synth.Spec(3, 256, 128, 3, 2, seed=12, weight_set=12, swiglu_clamp=0.01),
    "mxfp4": synth.Spec(3, 256, 128, 3, 2, recipe=1, seed=13, weight_set=13),
    "mxfp4_shared": synth.Spec(2, 128, 64, 3, 2, recipe=1, routing="uniform_shared", seed=14, weight_set=14),
    "fp8_clamp_inputs": synth.Spec(3, 256, 128, 3, 2, seed=15, weight_set=15, swiglu_clamp=0.2, clamp_inputs=True),
    "mxfp4_clamp_inputs": synth.Spec(3, 256, 128, 3, 2, recipe=1, seed=16, weight_set=16, swiglu_clamp=0.2,
                                     clamp_inputs=True),
    "mxfp8": synth.Spec(3, 256, 128, 3, 2, recipe=2, seed=18, weight_set=18),
    "mxfp8_shared_clamp": synth.Spec(2, 128, 64, 3, 2, recipe=2, routing="uniform_shared", seed=19,
                                     weight_set=19, swiglu_clamp=0.01),
    # per-64 float intermediate scales (design page section 5.4): I = 256 gives two 128-K blocks,
    # four 64-channel groups per row
    "fp8_sf64": synth.Spec(3, 256, 256, 3, 2, inter_sf64=True, seed=30, weight_set=30),
    "fp8_sf64_clamp": synth.Spec(3, 256, 128, 3, 2, inter_sf64=True, swiglu_clamp=0.01, seed=31, weight_set=31),
}


@pytest.mark.parametrize("name", list(BRUTE_SPECS))
def test_oracle_equals_brute_force(name):
    spec = BRUTE_SPECS[name]
    P = _np(synth.make_problem(spec))
    P["topk_idx"][1, 1] = -1                        # one masked slot
    ref, accs = brute_force(spec, P)
    r = oracle.forward(_prob(spec), **P)
    assert np.array_equal(r["y"], ref)
    # the exact rational L1 accumulators agree with the oracle's float64 block sums
    d = r["dispatch"]
    for (t, j), acc in accs.items():
        p = d["pos"][t * spec.k + j]
        e = int(P["topk_idx"][t, j])
        rows = oracle.expert_rows(_prob(spec), e, np.array([t]), P["topk_w"][t, j:j + 1],
                                  P["x"], P["x_sf"], P["l1_w"], P["l1_sf"], P["l2_w"], P["l2_sf"])
        # float64 rounding of the per-block scale products and the cross-block sum only
        np.testing.assert_allclose(rows["l1_acc"][0], np.array(acc), rtol=1e-14,
                                   atol=1e-15 * np.abs(np.array(acc)).max())
        assert p >= 0


# ----------------------------------------------------------------------------- library special cases
@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_l1_dense_special_case_matches_matmul(recipe):
    spec = synth.Spec(7, 512, 256, 1, 1, recipe=recipe, seed=21, weight_set=21)
    P = _np(synth.make_problem(spec))
    prob = _prob(spec)
    r = oracle.expert_rows(prob, 0, np.arange(7), np.ones(7, np.float32), P["x"], P["x_sf"],
                           P["l1_w"], P["l1_sf"], P["l2_w"], P["l2_sf"])
    x = torch.from_numpy(P["x"]).view(torch.float8_e4m3fn).double()
    if recipe == 0:
        xs = torch.from_numpy(P["x_sf"]).double().repeat_interleave(128, dim=1)
        w = torch.from_numpy(P["l1_w"][0]).view(torch.float8_e4m3fn).double()
        ws = torch.from_numpy(P["l1_sf"][0]).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    else:
        xs = torch.exp2(torch.from_numpy(P["x_sf"]).double() - 127).repeat_interleave(32, dim=1)
        lut = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], dtype=torch.float64)
        pk = torch.from_numpy(P["l1_w"][0]).long()
        w = torch.stack([lut[pk & 15], lut[pk >> 4]], dim=-1).reshape(pk.shape[0], -1)
        ws = torch.exp2(torch.from_numpy(P["l1_sf"][0]).double() - 127).repeat_interleave(32, dim=1)
    if recipe == 2:
        w = torch.from_numpy(P["l1_w"][0]).view(torch.float8_e4m3fn).double()
    ref = torch.matmul(x * xs, (w * ws).T).numpy()
    np.testing.assert_allclose(r["l1_acc"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(3)
    acc = rng.standard_normal((9, 2 * 64)) * 4
    acc[0, 0] = -800.0                                  # exp overflow branch
    w = rng.uniform(0, 1, 9).astype(np.float32)
    prob = oracle.Problem(9, 128, 64, 1, 1)
    got = oracle.swiglu_weighted(prob, acc, w)
    a = torch.from_numpy(acc)
    ref = (torch.nn.functional.silu(a[:, :64]) * a[:, 64:] * torch.from_numpy(w).double()[:, None]).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_clamp_applies_before_topk_weight():
    prob = oracle.Problem(1, 128, 2, 1, 1, swiglu_clamp=10.0)
    acc = np.array([[50.0, -50.0, 50.0, 50.0]])       # s = [~2500, ~-0]
    got = oracle.swiglu_weighted(prob, acc, np.array([0.5], np.float32))
    assert got[0, 0] == 5.0                             # clamp(2500) = 10, then * 0.5


def test_input_clamp_applies_to_gate_and_up():
    # design page section 10.1 step 3: gate and up clamped to [-c, c] before SiLU.  gate (50, -50)
    # and up (50, 50) with c = 10 become (10, -10) and (10, 10):
    #   silu(10) * 10 * 0.5  = 10 / (1 + e^-10) * 5 = 50 / 1.0000453999297625 = 49.99773010656487
    #   silu(-10) * 10 * 0.5 = -10 / (1 + e^10) * 5 = -50 / 22027.465794806718 = -0.0022698934351217193
    prob = oracle.Problem(1, 128, 2, 1, 1, swiglu_clamp=10.0, clamp_inputs=True)
    acc = np.array([[50.0, -50.0, 50.0, 50.0]])
    got = oracle.swiglu_weighted(prob, acc, np.array([0.5], np.float32))
    np.testing.assert_allclose(got[0], [49.99773010656487, -0.0022698934351217193], rtol=1e-13)
    # the product is not clamped (49.998 > 10), unlike the output clamp (first row: 5.0)
    assert got[0, 0] > 10.0


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_input_clamp_above_every_accumulator_changes_nothing(recipe):
    spec = synth.Spec(6, 512, 256, 5, 2, recipe=recipe, seed=17, weight_set=17)
    P = _np(synth.make_problem(spec))
    base = oracle.forward(_prob(spec), **P)
    wide = oracle.forward(oracle.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, 1e30, True), **P)
    assert np.array_equal(base["y"], wide["y"])
    # a clamp that binds changes the output
    tight = oracle.forward(oracle.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe, 0.05, True), **P)
    assert not np.array_equal(base["y"], tight["y"])


# ----------------------------------------------------------------------------- re-quantisation
@pytest.mark.parametrize("recipe,sf64", [(0, False), (1, False), (2, False), (0, True)],
                         ids=["fp8", "mxfp4", "mxfp8", "fp8_sf64"])
def test_requant_invariants(recipe, sf64):
    rng = np.random.default_rng(4)
    prob = oracle.Problem(1, 128, 256, 1, 1, recipe=recipe, inter_sf64=sf64)
    v = rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-4, 3, (64, 1))
    v[3] = 0.0
    v[5, 64:128] = 0.0                           # one zero 64-group inside a nonzero 128-group
    q, sf, vd = oracle.requant(prob, v)
    G = prob.inter_group
    assert sf.shape == (64, 256 // G)
    tab = oracle.e4m3_decode_table()
    qv = tab[q].reshape(64, 256 // G, G)
    v32 = v.astype(np.float32).astype(np.float64).reshape(64, 256 // G, G)
    nz = np.abs(v32).max(axis=2) > 0
    mx = np.abs(qv).max(axis=2)
    assert np.all(qv[~nz] == 0)
    if recipe == 0:
        assert np.all(mx[nz] == 448.0)                  # the amax element maps to +-448 exactly
        scale = sf.astype(np.float64)
    else:
        assert np.all((mx[nz] >= 224.0) & (mx[nz] <= 448.0))
        scale = np.ldexp(1.0, sf.astype(np.int64) - 127)
    # round-to-nearest bound of a 3-bit mantissa, plus the subnormal step 2^-9 * scale
    err = np.abs(vd.reshape(64, 256 // G, G) - v32)
    bound = np.maximum(np.abs(v32) * 2.0 ** -4, 2.0 ** -10 * scale[:, :, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


# ----------------------------------------------------------------------------- layer invariants
def _run(spec, P):
    return oracle.forward(_prob(spec), **P)


@pytest.mark.parametrize("spec", [synth.CONFIGS[0],
                                  synth.Spec(8, 512, 256, 8, 2, swiglu_clamp=0.05, seed=31, weight_set=31),
                                  synth.Spec(6, 512, 256, 5, 3, recipe=1, routing="uniform_shared",
                                             seed=32, weight_set=32)],
                         ids=["fp8", "fp8_clamp", "mxfp4"])
def test_power_of_two_weight_scaling_is_exact(spec):
    P = _np(synth.make_problem(spec))
    base = _run(spec, P)
    for m in (-3, 2):
        Q = dict(P)
        Q["topk_w"] = (P["topk_w"] * np.float32(2.0 ** m)).astype(np.float32)
        got = _run(spec, Q)
        yb = oracle.bf16_bits_to_f32(base["y"]).astype(np.float64) * 2.0 ** m
        assert np.array_equal(oracle.bf16_bits_to_f32(got["y"]).astype(np.float64), yb)


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_one_hot_weights_select_one_expert(recipe):
    spec = synth.Spec(8, 512, 256, 8, 3, recipe=recipe, seed=41, weight_set=41)
    P = _np(synth.make_problem(spec))
    P["topk_w"] = np.zeros_like(P["topk_w"])
    P["topk_w"][:, 1] = 1.0
    r = _run(spec, P)
    for t in range(spec.T):
        assert np.array_equal(r["y"][t], r["slot"][t * spec.k + 1])
        for j in (0, 2):
            assert not np.any(oracle.bf16_bits_to_f32(r["slot"][t * spec.k + j]))


def test_sf64_reduces_to_sf128_when_second_halves_vanish():
    """Per-64 intermediate scales equal the per-128 result bit for bit when the second 64
    channels of every 128-channel group are zero: the first half's per-64 scale is then the
    group's per-128 scale, the second half is all zero codes with scale 0, and the two-half L2 sum
    reduces to the one-block sum.  With the halves present the two recipes differ."""
    spec = synth.Spec(6, 256, 256, 3, 2, seed=32, weight_set=32)
    P = _np(synth.make_problem(spec))
    base = oracle.forward(_prob(spec), **P)
    half = replace(spec, inter_sf64=True)
    assert not np.array_equal(oracle.forward(_prob(half), **P)["y"], base["y"])
    I = spec.I
    for g in range(I // 128):            # up rows of channels 64..127 of each group: zero codes
        P["l1_w"][:, I + 128 * g + 64:I + 128 * (g + 1), :] = 0
    base = oracle.forward(_prob(spec), **P)
    r64 = oracle.forward(_prob(half), **P)
    assert np.array_equal(r64["y"], base["y"])
    for p, sf in r64["inter_sf"].items():
        assert np.array_equal(sf[1::2], np.zeros(I // 128, dtype=np.float32))
        assert np.array_equal(sf[0::2], base["inter_sf"][p])
        # equal values (a vanished half is +0 under its zero scale, -0 or +0 under the shared one)
        tab = oracle.e4m3_decode_table()
        assert np.array_equal(tab[r64["inter_q"][p]], tab[base["inter_q"][p]])


def test_k1_output_is_the_slot():
    spec = synth.Spec(9, 512, 256, 4, 1, seed=51, weight_set=51)
    P = _np(synth.make_problem(spec))
    r = _run(spec, P)
    for t in range(spec.T):
        assert np.array_equal(r["y"][t], r["slot"][t])


def test_token_permutation_and_expert_relabel_equivariance():
    spec = synth.CONFIGS[0]
    P = _np(synth.make_problem(spec))
    base = _run(spec, P)["y"]
    rng = np.random.default_rng(6)
    perm = rng.permutation(spec.T)
    Q = dict(P)
    for key in ("x", "x_sf", "topk_idx", "topk_w"):
        Q[key] = P[key][perm]
    assert np.array_equal(_run(spec, Q)["y"], base[perm])
    relabel = rng.permutation(spec.E)                 # expert e becomes relabel[e]
    R = dict(P)
    R["topk_idx"] = relabel[P["topk_idx"]].astype(np.int32)
    inv = np.argsort(relabel)
    for key in ("l1_w", "l1_sf", "l2_w", "l2_sf"):
        R[key] = P[key][inv]
    assert np.array_equal(_run(spec, R)["y"], base)


def test_masked_and_invalid_slots_contribute_nothing():
    spec = synth.CONFIGS[0]
    P = _np(synth.make_problem(spec))
    Q = dict(P)
    Q["topk_idx"] = P["topk_idx"].copy()
    Q["topk_idx"][:, 1] = -1
    R = dict(P)
    R["topk_idx"] = P["topk_idx"].copy()
    R["topk_idx"][:, 1] = spec.E + 3
    K1 = dict(P)
    K1["topk_idx"] = P["topk_idx"][:, :1].copy()
    K1["topk_w"] = P["topk_w"][:, :1].copy()
    s1 = synth.Spec(spec.T, spec.H, spec.I, spec.E, 1)
    ref = oracle.forward(_prob(s1), **K1)["y"]
    assert np.array_equal(_run(spec, Q)["y"], ref)
    rr = _run(spec, R)
    assert np.array_equal(rr["y"], ref)
    assert rr["dispatch"]["num_invalid"] == spec.T


def test_empty_batch():
    spec = synth.Spec(0, 512, 256, 8, 2)
    P = _np(synth.make_problem(spec))
    r = _run(spec, P)
    assert r["y"].shape == (0, 512)
    assert r["dispatch"]["count"].sum() == 0
