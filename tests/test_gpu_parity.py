"""Parity of the HIP path (through the C ABI) against the CPU oracle, on an MI355X.

Small problems are compared in full (every output element, every dispatch field, every
intermediate code); the benchmark-size workloads are compared on sampled tokens, with the
dispatch metadata still checked in full.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from harness import (assert_dispatch_exact, assert_intermediate_close, assert_y_close, problem_of, run_gpu,
                     run_oracle, to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _custom(spec, idx=None, w=None):
    P = synth.make_problem(spec)
    if idx is not None:
        P["topk_idx"] = torch.as_tensor(idx, dtype=torch.int32).contiguous()
    if w is not None:
        P["topk_w"] = torch.as_tensor(w, dtype=torch.float32).contiguous()
    return P


def _full_check(spec, P, flags=0):
    _say(f"spec={spec} flags={flags}")
    D = to_device(P)
    y, views, _ = run_gpu(spec, D, flags)
    ref = run_oracle(spec, P)
    assert_dispatch_exact(spec, P["topk_idx"].numpy(), views)
    assert_intermediate_close(spec, views, ref)
    return assert_y_close(y.cpu().numpy(), ref["y"], str(spec))


SMALL = {
    "tiny_c0": synth.CONFIGS[0],
    "ragged": synth.Spec(37, 640, 384, 12, 3, seed=101, weight_set=101),
    "multi_tile": synth.Spec(300, 512, 256, 4, 2, seed=102, weight_set=102),
    "clamp": synth.Spec(64, 512, 256, 8, 4, routing="biased", swiglu_clamp=0.05, seed=103, weight_set=103),
    "zipf": synth.Spec(512, 512, 384, 32, 4, routing="zipf", seed=104, weight_set=104),
    "T1": synth.Spec(1, 512, 256, 8, 2, seed=105, weight_set=105),
    "E1_k1": synth.Spec(70, 384, 256, 1, 1, seed=106, weight_set=106),
    "mxfp4": synth.Spec(40, 512, 256, 9, 5, recipe=1, routing="uniform_shared", seed=107, weight_set=107),
    "mxfp4_multi_tile": synth.Spec(200, 512, 256, 3, 2, recipe=1, seed=108, weight_set=108),
    "mxfp4_clamp": synth.Spec(48, 640, 384, 6, 3, recipe=1, swiglu_clamp=0.05, seed=109, weight_set=109),
    # the activation clamp on gate and up (flag MEGA_MOE_FLAG_CLAMP_INPUTS)
    "clamp_inputs": synth.Spec(64, 512, 256, 8, 4, routing="biased", swiglu_clamp=0.3, clamp_inputs=True,
                               seed=122, weight_set=122),
    "mxfp4_clamp_inputs": synth.Spec(48, 640, 384, 6, 3, recipe=1, swiglu_clamp=0.3, clamp_inputs=True,
                                     seed=123, weight_set=123),
    # E4M3 weights with per-32 UE8M0 scales (recipe 2): shared expert, multi-tile experts, every
    # column-group class under Zipf routing, and both clamp readings
    "mxfp8": synth.Spec(40, 512, 256, 9, 5, recipe=2, routing="uniform_shared", seed=130, weight_set=130),
    "mxfp8_multi_tile": synth.Spec(300, 512, 384, 4, 2, recipe=2, seed=131, weight_set=131),
    "mxfp8_zipf_clamp_inputs": synth.Spec(512, 640, 384, 32, 4, recipe=2, routing="zipf", swiglu_clamp=0.3,
                                          clamp_inputs=True, seed=132, weight_set=132),
    "mxfp8_clamp": synth.Spec(64, 512, 256, 8, 4, recipe=2, routing="biased", swiglu_clamp=0.05, seed=133,
                              weight_set=133),
    # more than 16384 pairs: dispatch runs 1024 pairs per workgroup; skewed so that experts
    # fill every large-M column-group class
    "wide_dispatch": synth.Spec(2100, 512, 256, 64, 8, routing="zipf", seed=115, weight_set=115),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_problem_full_parity(name):
    spec = SMALL[name]
    _full_check(spec, synth.make_problem(spec))


@pytest.mark.parametrize("flags", [0, 1, 2], ids=["auto", "small_only", "large_only"])
@pytest.mark.parametrize("name", ["ragged", "clamp", "mxfp4_clamp", "zipf", "mxfp8_clamp"])
def test_precise_silu(name, flags):
    """MEGA_MOE_FLAG_PRECISE_SILU (expf and IEEE division): the same bar against the oracle."""
    import dispatch_fp8_grouped_topk_amd as mm
    spec = SMALL[name]
    _full_check(spec, synth.make_problem(spec), flags | mm.FLAG_PRECISE_SILU)


@pytest.mark.parametrize("flags", [1, 2], ids=["small_only", "large_only"])
@pytest.mark.parametrize("name", ["ragged", "multi_tile", "zipf", "mxfp4", "mxfp4_multi_tile", "clamp_inputs",
                                  "mxfp4_clamp_inputs", "mxfp8", "mxfp8_multi_tile", "mxfp8_zipf_clamp_inputs"])
def test_forced_tile_class(name, flags):
    spec = SMALL[name]
    _full_check(spec, synth.make_problem(spec), flags)


@pytest.mark.parametrize("flags", [0, 16], ids=["rowmajor_sf", "kmajor_sf"])
def test_mxfp4_every_tile_size(flags):
    """MXFP4 experts of 1 to 10 row groups of 16 (the four-wave L2 kernel's tile sizes) beside a
    601-row expert (three tiles of the eight-wave kernel), compared in full, with the weight scales
    in either layout."""
    counts = [1, 17, 33, 49, 65, 81, 97, 113, 129, 150, 160, 601]
    T, k = sum(counts) // 2, 2
    ids = np.repeat(np.arange(len(counts)), counts)           # sorted; no expert holds T pairs
    idx = np.stack([ids[:T], ids[T:]], axis=1)                 # so each token's two differ
    idx = idx[np.random.default_rng(117).permutation(T)].astype(np.int32)
    assert (idx[:, 0] != idx[:, 1]).all()
    spec = synth.Spec(T, 512, 256, len(counts), k, recipe=1, seed=117, weight_set=117)
    _full_check(spec, _custom(spec, idx=idx), flags)


# ------------------------------------------------------------------------------ K-major weight scales
@pytest.mark.parametrize("flags", [0, 1, 2], ids=["auto", "small_only", "large_only"])
@pytest.mark.parametrize("name", ["mxfp4", "mxfp4_multi_tile", "mxfp4_clamp_inputs", "mxfp8", "mxfp8_multi_tile",
                                  "mxfp8_zipf_clamp_inputs"])
def test_weight_sf_kmajor(name, flags):
    """Weight scales transformed once (mega_moe_transform_weight_scales) and read K-major
    (MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR): the same bar against the oracle, which reads the originals."""
    import dispatch_fp8_grouped_topk_amd as mm
    spec = SMALL[name]
    _full_check(spec, synth.make_problem(spec), flags | mm.FLAG_WEIGHT_SF_KMAJOR)


@pytest.mark.parametrize("recipe", [1, 2])
def test_weight_sf_transform_is_a_transpose(recipe):
    """The transform writes [E, K/128, rows, 4] with the codes of [E, rows, K/32], bit for bit
    (K blocks 5 and 34: one and two 32-word tiles of the transform)."""
    import dispatch_fp8_grouped_topk_amd as mm
    for H, I, E in ((640, 384, 5), (4352, 128, 2)):
        spec = synth.Spec(8, H, I, E, 2, recipe=recipe, seed=135, weight_set=135)
        _say(f"transform {spec}")
        D = to_device(synth.make_problem(spec))
        k1, k2 = mm.mega_moe_transform_weight_scales(problem_of(spec), D["l1_sf"], D["l2_sf"])
        torch.cuda.synchronize()
        e1 = D["l1_sf"].view(E, 2 * I, H // 128, 4).permute(0, 2, 1, 3).contiguous()
        e2 = D["l2_sf"].view(E, H, I // 128, 4).permute(0, 2, 1, 3).contiguous()
        assert torch.equal(k1, e1) and torch.equal(k2, e2)


LIMITS = {
    # the largest expert count and top-k the library takes (LDS arrays of the route kernels)
    "max_experts_topk": synth.Spec(16, 128, 128, 8192, 64, seed=126, weight_set=126),
    # the largest hidden size: 128 K blocks in L1, the whole LDS weight-scale staging
    "max_hidden": synth.Spec(24, 16384, 128, 3, 2, seed=127, weight_set=127),
    "max_hidden_mxfp4": synth.Spec(24, 16384, 128, 3, 2, recipe=1, seed=128, weight_set=128),
    "max_hidden_mxfp8": synth.Spec(24, 16384, 128, 3, 2, recipe=2, seed=134, weight_set=134),
    # the largest intermediate size: 128 L1 slabs, 128 K blocks in L2
    "max_intermediate": synth.Spec(24, 128, 16384, 3, 2, seed=129, weight_set=129),
}


@pytest.mark.parametrize("name", list(LIMITS))
def test_size_limits_full_parity(name):
    spec = LIMITS[name]
    _full_check(spec, synth.make_problem(spec))


def test_all_tokens_on_one_expert():
    spec = synth.Spec(150, 512, 256, 8, 1, seed=110, weight_set=110)
    _full_check(spec, _custom(spec, idx=np.full((150, 1), 5)))


def test_masked_and_invalid_ids():
    spec = synth.Spec(33, 512, 256, 6, 3, seed=111, weight_set=111)
    P = synth.make_problem(spec)
    idx = P["topk_idx"].numpy().copy()
    rng = np.random.default_rng(0)
    idx[rng.random(idx.shape) < 0.2] = -1
    idx[rng.random(idx.shape) < 0.1] = 6 + 3
    _full_check(spec, _custom(spec, idx=idx))


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_cumulative_expert_recv_stats(recipe):
    """mega_moe_forward_stats adds each expert's received rows (masked and invalid slots
    excluded) to the caller's array, call after call, and leaves y unchanged."""
    import dispatch_fp8_grouped_topk_amd as mm
    import oracle
    from harness import problem_of
    spec = synth.Spec(40, 512, 256, 7, 3, recipe=recipe, seed=124 + recipe, weight_set=124 + recipe)
    P = synth.make_problem(spec)
    idx = P["topk_idx"].numpy().copy()
    rng = np.random.default_rng(1)
    idx[rng.random(idx.shape) < 0.2] = -1
    idx[rng.random(idx.shape) < 0.1] = 7 + 2
    D = to_device(_custom(spec, idx=idx))
    prob = problem_of(spec)
    ws = torch.empty(mm.mega_moe_workspace_size(prob), dtype=torch.uint8, device="cuda")
    args = (prob, D["x"], D["x_sf"], D["topk_idx"], D["topk_w"], D["l1_w"], D["l1_sf"], D["l2_w"], D["l2_sf"])
    y0 = torch.empty(spec.T, spec.H, dtype=torch.bfloat16, device="cuda")
    mm.mega_moe_forward(*args, y0, ws)
    stats = torch.full((spec.E,), 5, dtype=torch.int32, device="cuda")
    y = torch.empty_like(y0)
    for _ in range(2):
        mm.mega_moe_forward(*args, y, ws, recv_stats=stats)
    torch.cuda.synchronize()
    count = oracle.route(idx, spec.E)["count"]
    assert np.array_equal(stats.cpu().numpy(), 5 + 2 * np.asarray(count, dtype=np.int64))
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16))


def test_empty_experts_and_skew():
    spec = synth.Spec(90, 512, 256, 16, 2, seed=112, weight_set=112)
    rng = np.random.default_rng(1)
    idx = np.stack([rng.choice([0, 3, 15], 90), rng.choice([1, 4], 90)], axis=1)
    _full_check(spec, _custom(spec, idx=idx))


def test_zero_tokens_is_a_noop():
    spec = synth.Spec(0, 512, 256, 8, 2)
    D = to_device(synth.make_problem(spec))
    y, views, _ = run_gpu(spec, D)
    assert y.shape == (0, 512)


def test_repeatable_and_stale_workspace():
    spec = SMALL["zipf"]
    _say(f"repeatability {spec}")
    D = to_device(synth.make_problem(spec))
    y1, _, ws = run_gpu(spec, D)
    y2, _, _ = run_gpu(spec, D, workspace=ws)
    y3, _, _ = run_gpu(spec, D, workspace=ws, fill=0xFF)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


@pytest.mark.parametrize("recipe", [0, 1, 2])
def test_power_of_two_topk_weight_scaling_is_bitwise(recipe):
    spec = synth.Spec(64, 512, 256, 8, 3, recipe=recipe, seed=113, weight_set=113)
    _say(f"pow2 scaling {spec}")
    D = to_device(synth.make_problem(spec))
    y1, _, _ = run_gpu(spec, D)
    D2 = dict(D)
    D2["topk_w"] = D["topk_w"] * 0.25
    y2, _, _ = run_gpu(spec, D2)
    assert torch.equal(y1.view(torch.bfloat16).float() * 0.25, y2.view(torch.bfloat16).float())


def test_one_hot_weights_equal_selected_slot():
    spec = synth.Spec(40, 512, 256, 8, 3, seed=114, weight_set=114)
    P = synth.make_problem(spec)
    w = torch.zeros(40, 3)
    w[:, 2] = 1.0
    P["topk_w"] = w
    D = to_device(P)
    y, views, _ = run_gpu(spec, D)
    slot = views["slot"].view(40, 3, 512)[:, 2]
    assert torch.equal(y, slot)


# ------------------------------------------------------------------------------ benchmark sizes
_DEV_CACHE = {}


def _device_problem(cfg, recipe=None):
    """Benchmark-size inputs generated on the GPU (weights shared between configs 1 and 3);
    ``recipe`` replaces the workload's weight recipe."""
    spec = synth.CONFIGS[cfg]
    if recipe is not None:
        spec = replace(spec, recipe=recipe, name=f"{spec.name} recipe {recipe}")
    key = (spec.weight_set, spec.H, spec.I, spec.E, spec.recipe)
    if key not in _DEV_CACHE:
        _DEV_CACHE.clear()
        torch.cuda.empty_cache()
        _DEV_CACHE[key] = synth.make_weights(spec, "cuda")
    P = dict(_DEV_CACHE[key])
    idx, w = synth.make_routing(spec)
    x, x_sf = synth.make_activations(spec, "cuda")
    P.update(x=x, x_sf=x_sf, topk_idx=idx.cuda(), topk_w=w.cuda())
    return spec, P


def _sample_tokens(spec, idx, n=3):
    counts = np.bincount(idx[idx >= 0].reshape(-1), minlength=spec.E)
    hot = int(np.argmax(counts))
    last_hot = int(np.nonzero((idx == hot).any(axis=1))[0][-1])     # deepest row of the hottest pool
    toks = [0, spec.T - 1, last_hot][:n]
    return sorted(set(toks))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_benchmark_config_sampled_parity(cfg):
    spec, P = _device_problem(cfg)
    _say(f"config {cfg}: {spec.name}")
    y, views, _ = run_gpu(spec, P)
    idx = P["topk_idx"].cpu().numpy()
    assert_dispatch_exact(spec, idx, views)
    toks = _sample_tokens(spec, idx)
    ref = run_oracle(spec, P, tokens=toks)
    assert_intermediate_close(spec, views, ref)
    rel, mean_rel = assert_y_close(y.cpu().numpy()[toks], ref["y"], spec.name)
    _say(f"config {cfg}: tokens {toks} max-rel {rel:.3e} mean-rel {mean_rel:.3e}")


@pytest.mark.parametrize("cfg", [1, 3])
def test_mxfp8_benchmark_size_sampled_parity(cfg):
    """The decode and prefill shapes and routing with E4M3 weights and per-32 UE8M0 scales."""
    spec, P = _device_problem(cfg, recipe=2)
    _say(f"config {cfg} recipe 2: {spec.name}")
    y, views, _ = run_gpu(spec, P)
    idx = P["topk_idx"].cpu().numpy()
    assert_dispatch_exact(spec, idx, views)
    toks = _sample_tokens(spec, idx)
    ref = run_oracle(spec, P, tokens=toks)
    assert_intermediate_close(spec, views, ref)
    rel, mean_rel = assert_y_close(y.cpu().numpy()[toks], ref["y"], spec.name)
    _say(f"config {cfg} recipe 2: tokens {toks} max-rel {rel:.3e} mean-rel {mean_rel:.3e}")


@pytest.mark.parametrize("cfg,recipe", [(4, None), (3, 2)], ids=["mxfp4_c4", "mxfp8_prefill"])
def test_weight_sf_kmajor_benchmark_size_sampled_parity(cfg, recipe):
    """The benchmark shapes of the per-32 recipes with K-major weight scales."""
    import dispatch_fp8_grouped_topk_amd as mm
    spec, P = _device_problem(cfg, recipe=recipe)
    _say(f"config {cfg} K-major scales: {spec.name}")
    y, views, _ = run_gpu(spec, P, mm.FLAG_WEIGHT_SF_KMAJOR)
    idx = P["topk_idx"].cpu().numpy()
    assert_dispatch_exact(spec, idx, views)
    toks = _sample_tokens(spec, idx)
    ref = run_oracle(spec, P, tokens=toks)
    assert_intermediate_close(spec, views, ref)
    rel, mean_rel = assert_y_close(y.cpu().numpy()[toks], ref["y"], spec.name)
    _say(f"config {cfg} K-major: tokens {toks} max-rel {rel:.3e} mean-rel {mean_rel:.3e}")
