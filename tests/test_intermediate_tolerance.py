"""The derived intermediate-code tolerance of the GPU parity tests, checked on the CPU.

The harness accepts a GPU intermediate when every dequantised value lies within half a code
spacing (on each side) plus a value-error bound derived from the matrix core's block-sum error
(EPS_MFMA of the products' magnitude sum).  Here the oracle's own L1 sums are perturbed by up to
that error, re-quantised with the oracle's rule, and the result must pass; a perturbation 64
times larger (a planted mistake in the arithmetic) must fail.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import EPS_MFMA, assert_intermediate_close, oracle_problem


def _requant_views(spec, ref, scale_eps, seed):
    """Views as the GPU would leave them if its L1 sums were off by scale_eps * magnitude sum."""
    prob = oracle_problem(spec)
    rng = np.random.default_rng(seed)
    rows = sorted(ref["inter_q"])
    acc = np.stack([ref["l1_acc"][p] for p in rows])
    mag = np.stack([ref["l1_abs"][p] for p in rows])
    w = np.array([ref["w"][p] for p in rows], dtype=np.float32)
    pert = acc + scale_eps * mag * rng.uniform(-1, 1, size=acc.shape)
    v = oracle.moe.swiglu_weighted(prob, pert, w)
    q, sf, _ = oracle.moe.requant(prob, v)
    n = max(rows) + 1
    inter_q = torch.zeros(n, spec.I, dtype=torch.uint8)
    inter_q[rows] = torch.from_numpy(q)
    sf_t = torch.from_numpy(np.ascontiguousarray(sf))
    inter_sf = torch.zeros((n,) + tuple(sf_t.shape[1:]), dtype=sf_t.dtype)
    inter_sf[rows] = sf_t
    return dict(inter_q=inter_q, inter_sf=inter_sf)


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_bound_accepts_hardware_error_and_rejects_planted_error(recipe):
    spec = synth.Spec(48, 512, 256, 6, 3, recipe=recipe, swiglu_clamp=0.0, seed=140 + recipe,
                      weight_set=140 + recipe)
    P = synth.make_problem(spec)
    ref = oracle.forward(oracle_problem(spec), magnitudes=True, **{k: v.numpy() for k, v in P.items()})
    # an L1 error of up to EPS_MFMA of the magnitudes, everywhere, stays inside the derived
    # element bound (the empirical cap on the fraction of flipped codes is not meant for it) ...
    for seed in range(3):
        assert_intermediate_close(spec, _requant_views(spec, ref, EPS_MFMA, seed), ref, max_code_frac=1.0)
    # ... exact sums flip no code ...
    assert assert_intermediate_close(spec, _requant_views(spec, ref, 0.0, 0), ref) == 0.0
    # ... and 64 x the bound is caught by the element bound itself
    with pytest.raises(AssertionError, match="outside the derived bound"):
        assert_intermediate_close(spec, _requant_views(spec, ref, 64 * EPS_MFMA, 9), ref, max_code_frac=1.0)


def test_magnitude_sum_bounds_the_sum():
    """l1_abs >= |l1_acc| everywhere, with equality where every operand is non-negative."""
    spec = synth.Spec(16, 256, 128, 2, 1, seed=150, weight_set=150)
    P = {k: v.numpy() for k, v in synth.make_problem(spec).items()}
    ref = oracle.forward(oracle_problem(spec), magnitudes=True, **P)
    for p in ref["l1_acc"]:
        assert (ref["l1_abs"][p] >= np.abs(ref["l1_acc"][p]) * (1 - 1e-12)).all()
    P["x"] = P["x"] & 0x7F                      # clear every sign bit of x and w1
    P["l1_w"] = P["l1_w"] & 0x7F
    ref = oracle.forward(oracle_problem(spec), magnitudes=True, **P)
    for p in ref["l1_acc"]:
        np.testing.assert_allclose(ref["l1_abs"][p], ref["l1_acc"][p], rtol=1e-12, atol=0)
