"""The benchmark's algorithmic byte counts, against what the inputs and the oracle hold.

The roofline fraction bench.py reports is achieved / peak with achieved = the algorithmic bytes
(or flops) of the dominant kernel per launch / its duration, so the counts are checked here
against independent sources: the sizes of the tensors the input generator allocates (weights,
activations and their scales) and the intermediate the oracle produces for the same rows.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bench
import oracle
import synth

SPECS = {f"cfg{c}": synth.CONFIGS[c] for c in (1, 2, 3, 4)}
SPECS.update({f"cfg{c}_recipe2": dataclasses.replace(synth.CONFIGS[c], recipe=2) for c in (1, 3)})


def _nbytes(shape, dtype):
    return int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()


@pytest.mark.parametrize("name", list(SPECS))
def test_weight_bytes_per_expert_are_the_generated_tensors(name):
    spec = SPECS[name]
    shapes = synth.weight_shapes(spec)
    per_expert = {k: _nbytes(s[1:], dt) for k, (s, dt) in shapes.items()}
    l1, l2 = bench.weight_bytes_per_expert(spec)
    assert l1 == per_expert["l1_w"] + per_expert["l1_sf"]
    assert l2 == per_expert["l2_w"] + per_expert["l2_sf"]


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_activation_and_intermediate_bytes_are_the_tensors(recipe):
    spec = synth.Spec(6, 512, 256, 4, 2, recipe=recipe, seed=51, weight_set=51)
    P = synth.make_problem(spec)
    pairs = spec.T * spec.k
    ab = bench.algorithmic_bytes(spec, touched=0, P=pairs)
    xs = P["x"].numel() * P["x"].element_size() + P["x_sf"].numel() * P["x_sf"].element_size()
    # one pool row's intermediate codes and scales as the oracle re-quantises them
    prob = oracle.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, spec.recipe)
    q, sf, _ = oracle.requant(prob, np.ones((1, spec.I)))
    inter = pairs * (q.nbytes + sf.nbytes)
    # L1 reads x, x_sf and the pool's top-k weights (f32) and writes the intermediate
    assert ab["l1_gemm_swiglu"] == xs + pairs * 4 + inter
    # L2 reads the intermediate and writes one BF16 row per pair
    assert ab["l2_gemm"] == inter + pairs * spec.H * 2

