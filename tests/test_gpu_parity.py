"""Parity of the HIP path (through the C ABI) against the CPU oracle, on an MI355X.

Small problems are compared in full (every output element, every dispatch field, every
intermediate code).  At the benchmark sizes the decode and mid workloads are compared in full;
the prefill and MXFP4 workloads on a stratified sample of tokens (every tile of the hottest
experts, every column-group class), with the dispatch metadata always checked in full.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
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
    # about five rows per expert: four rounds of one-column-group L1 items and two of L2 items (the
    # decode regime at a small size; FP8 and E4M3-weight per-32 recipes)
    "decode_like": synth.Spec(160, 512, 512, 256, 8, seed=139, weight_set=139),
    "decode_like_mxfp8": synth.Spec(160, 512, 512, 256, 8, recipe=2, seed=140, weight_set=140),
    "mxfp4": synth.Spec(40, 512, 256, 9, 5, recipe=1, routing="uniform_shared", seed=107, weight_set=107),
    "mxfp4_multi_tile": synth.Spec(200, 512, 256, 3, 2, recipe=1, seed=108, weight_set=108),
    "mxfp4_clamp": synth.Spec(48, 640, 384, 6, 3, recipe=1, swiglu_clamp=0.05, seed=109, weight_set=109),
    # MXFP4 with I = 768: three wide L1 slabs (256 channels each) under Zipf routing, so experts of
    # every column-group class up to 5 run wide and the hotter ones in the narrow items
    "mxfp4_wide3": synth.Spec(400, 512, 768, 16, 4, recipe=1, routing="zipf", seed=137, weight_set=137),
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
    # 16800 pairs over 66 dispatch workgroups of 256 pairs; skewed so that experts fill every
    # large-M column-group class
    "wide_dispatch": synth.Spec(2100, 512, 256, 64, 8, routing="zipf", seed=115, weight_set=115),
    # per-64 float intermediate scales (flag MEGA_MOE_FLAG_INTER_SF64): ragged sizes, every
    # column-group class under Zipf routing, the output clamp, two 64-groups per L1 slab
    "sf64": synth.Spec(37, 640, 384, 12, 3, inter_sf64=True, seed=150, weight_set=150),
    "sf64_zipf": synth.Spec(512, 512, 384, 32, 4, routing="zipf", inter_sf64=True, seed=151, weight_set=151),
    "sf64_clamp": synth.Spec(64, 512, 256, 8, 4, routing="biased", swiglu_clamp=0.05, inter_sf64=True, seed=152,
                             weight_set=152),
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
                                  "mxfp4_clamp_inputs", "mxfp8", "mxfp8_multi_tile", "mxfp8_zipf_clamp_inputs",
                                  "sf64", "sf64_zipf", "sf64_clamp"])
def test_forced_tile_class(name, flags):
    spec = SMALL[name]
    _full_check(spec, synth.make_problem(spec), flags)


@pytest.mark.parametrize("flags", [0, 16, 16 | 128], ids=["rowmajor_sf", "kmajor_sf", "kmajor_sf_paired_w"])
def test_mxfp4_every_tile_size(flags):
    """MXFP4 experts of 1 to 10 row groups of 16 (the four-wave L2 kernel's tile sizes, and the
    L1 kernel's wide items up to 5 groups per wave) beside a 601-row expert (three tiles of the
    eight-wave kernel), compared in full, with the weight scales in either layout and the weights
    row-major or in row pairs."""
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


# ------------------------------------------------------------------------------ E2M1 row-pair weights
@pytest.mark.parametrize("flags", [0, 1, 2], ids=["auto", "small_only", "large_only"])
@pytest.mark.parametrize("name", ["mxfp4", "mxfp4_multi_tile", "mxfp4_clamp_inputs", "mxfp4_wide3"])
def test_weight_e2m1_paired(name, flags):
    """E2M1 weights transformed once (mega_moe_transform_weights) and read in row pairs
    (MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED), in every tile class: the same bar against the oracle,
    which reads the row-major originals."""
    import dispatch_fp8_grouped_topk_amd as mm
    spec = SMALL[name]
    _full_check(spec, synth.make_problem(spec), flags | mm.FLAG_WEIGHT_E2M1_PAIRED)


def test_e2m1_pair_transform_is_the_documented_permutation():
    """Row pair q of a [rows, K/2] expert becomes [K/128][2][64] bytes at q * K: K block kb of row
    2q, then of row 2q + 1 (one and many K blocks; L1 and L2 weights)."""
    import dispatch_fp8_grouped_topk_amd as mm
    for H, I, E in ((640, 384, 5), (128, 4352, 2)):
        spec = synth.Spec(8, H, I, E, 2, recipe=1, seed=136, weight_set=136)
        _say(f"pair transform {spec}")
        D = to_device(synth.make_problem(spec))
        p1, p2 = mm.mega_moe_transform_weights(problem_of(spec), D["l1_w"], D["l2_w"])
        torch.cuda.synchronize()
        e1 = D["l1_w"].view(E, I, 2, H // 128, 64).permute(0, 1, 3, 2, 4).reshape(E, 2 * I, H // 2)
        e2 = D["l2_w"].view(E, H // 2, 2, I // 128, 64).permute(0, 1, 3, 2, 4).reshape(E, H, I // 2)
        assert torch.equal(p1, e1) and torch.equal(p2, e2)


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


def test_dispatch_many_blocks():
    """80,000 pairs in 313 dispatch blocks (a block range of 78-79 blocks per part of the scan's
    first phase, a ragged last block), every token against the oracle."""
    spec = synth.Spec(20000, 128, 128, 64, 4, seed=138, weight_set=138)
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


def _device_problem(cfg, recipe=None, sf64=False):
    """Benchmark-size inputs generated on the GPU (weights shared between configs 1 and 3);
    ``recipe`` replaces the workload's weight recipe, ``sf64`` selects per-64 intermediate scales."""
    spec = synth.CONFIGS[cfg]
    if recipe is not None:
        spec = replace(spec, recipe=recipe, name=f"{spec.name} recipe {recipe}")
    if sf64:
        spec = replace(spec, inter_sf64=True, name=f"{spec.name} per-64 intermediate scales")
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


def _tile_starts(c):
    """Row ranges of the large-M tiles of an expert with c rows: ceil(c / 256) tiles over its
    16-row groups, dealt out in pairs, an odd last group going to the first tile with the smaller
    pair count (the split the route kernel writes into the tile list)."""
    n = (c + 255) // 256
    g = (c + 15) // 16
    pairs = g // 2
    q, r = divmod(pairs, n)
    st = [16 * (2 * (i * q + min(i, r)) + (1 if (g & 1) and i > r else 0)) for i in range(n)]
    return list(zip(st, st[1:] + [c]))


def _stratified_tokens(spec, idx):
    """Tokens whose pool rows cover: the first and last row of every large-M tile of the 8 hottest
    experts (every tile of a multi-tile expert there, the odd-group tile included), the first and
    last row of every tile of two experts of each column-group class 1..8 present (so every
    instantiation of the GEMM kernels, and the four-wave MXFP4 L2 kernel's tile sizes, are
    checked), the shared expert's tiles where there is one, and the first and last token."""
    d = oracle.route(idx, spec.E)
    count, offset, src = d["count"], d["offset"], d["src"]
    pick = set()

    def take_expert(e):
        for m0, m1 in _tile_starts(int(count[e])):
            for m in (m0, m1 - 1):
                pick.add(int(src[offset[e] + m]) // spec.k)

    order = np.argsort(-count, kind="stable")
    for e in order[:8]:
        if count[e] > 0:
            take_expert(int(e))
    by_class = {}
    for e in range(spec.E):
        c = int(count[e])
        if c == 0:
            continue
        m0, m1 = _tile_starts(c)[0]
        ng = ((m1 - m0 + 15) // 16 + 1) // 2
        by_class.setdefault(ng, []).append(e)
    for ng, es in sorted(by_class.items()):
        for e in es[:2]:
            take_expert(e)
    if spec.routing == "uniform_shared":
        take_expert(spec.E - 1)
    pick |= {0, spec.T - 1}
    classes = sorted(by_class)
    return sorted(pick), classes


def _assert_every_item_written(spec, y, views, n_rows):
    """With the workspace filled with 0xFF bytes before the forward (E4M3 NaN codes, BF16 NaNs),
    every intermediate code of the n_rows pool rows and every output must have been written by
    the GEMM items: an item left out of the persistent kernels' rounds leaves NaN codes in its
    slab of the intermediate (L1) or NaN slot rows that reach y through the combine (L2)."""
    assert torch.isfinite(y.view(torch.bfloat16)).all(), f"{spec.name}: non-finite outputs"
    q = views["inter_q"][:n_rows]
    assert not ((q & 0x7F) == 0x7F).any(), f"{spec.name}: intermediate codes left unwritten"


def _parity_at_size(cfg, recipe=None, flags=0, full=False, sf64=False):
    spec, P = _device_problem(cfg, recipe=recipe, sf64=sf64)
    _say(f"config {cfg} recipe {spec.recipe} flags {flags}: {spec.name}")
    y, views, _ = run_gpu(spec, P, flags, fill=0xFF)
    idx = P["topk_idx"].cpu().numpy()
    d = assert_dispatch_exact(spec, idx, views)
    _assert_every_item_written(spec, y, views, int(d["offset"][-1]))
    if full:
        toks, classes = list(range(spec.T)), None
    else:
        toks, classes = _stratified_tokens(spec, idx)
    ref = run_oracle(spec, P, tokens=None if full else toks)
    frac = assert_intermediate_close(spec, views, ref)
    yg = y.cpu().numpy() if full else y.cpu().numpy()[toks]
    rel, mean_rel = assert_y_close(yg, ref["y"], spec.name)
    pairs = len(ref["inter_q"])
    _say(f"config {cfg}: {len(toks)} of {spec.T} tokens, {pairs} of {int(d['offset'][-1])} pool rows compared"
         + (f" (column-group classes {classes})" if classes else "")
         + f"; codes differing {frac:.3e}; y max-rel {rel:.3e} mean-rel {mean_rel:.3e}")


@pytest.mark.parametrize("cfg", [1, 2])
def test_benchmark_config_full_parity(cfg):
    """Decode and mid workloads at their full sizes: every token, every pool row."""
    _parity_at_size(cfg, full=True)


def test_mxfp8_decode_full_parity():
    """The decode workload with E4M3 weights and per-32 UE8M0 scales, every token."""
    import dispatch_fp8_grouped_topk_amd as mm
    _parity_at_size(1, recipe=2, flags=mm.FLAG_WEIGHT_SF_KMAJOR, full=True)


@pytest.mark.parametrize("cfg", [3, 4])
def test_benchmark_config_stratified_parity(cfg):
    """Prefill and MXFP4 workloads at their full sizes on a stratified sample of tokens (every
    tile of the hottest experts, every column-group class), dispatch in full; MXFP4 with the
    weight layouts the benchmark uses (K-major scales, row-pair E2M1 weights)."""
    import dispatch_fp8_grouped_topk_amd as mm
    _parity_at_size(cfg, flags=mm.FLAG_WEIGHT_SF_KMAJOR | mm.FLAG_WEIGHT_E2M1_PAIRED if cfg == 4 else 0)


def test_mxfp4_paired_weights_bitwise_at_benchmark_size():
    """The MXFP4 workload: row-pair E2M1 weights give the same y, bit for bit, as row-major ones
    (every token)."""
    import dispatch_fp8_grouped_topk_amd as mm
    spec, P = _device_problem(4)
    y0, _, ws = run_gpu(spec, P, mm.FLAG_WEIGHT_SF_KMAJOR)
    y1, _, _ = run_gpu(spec, P, mm.FLAG_WEIGHT_SF_KMAJOR | mm.FLAG_WEIGHT_E2M1_PAIRED, workspace=ws)
    assert torch.equal(y0, y1)


def test_mxfp4_rowmajor_sf_stratified_parity():
    """The MXFP4 workload with the weight scales in their row-major input layout."""
    _parity_at_size(4)


def test_mxfp8_prefill_stratified_parity():
    """The prefill shape and routing with E4M3 weights and per-32 UE8M0 scales."""
    import dispatch_fp8_grouped_topk_amd as mm
    _parity_at_size(3, recipe=2, flags=mm.FLAG_WEIGHT_SF_KMAJOR)


def test_sf64_decode_full_parity():
    """The decode workload with per-64 float intermediate scales, every token."""
    _parity_at_size(1, full=True, sf64=True)


def test_sf64_prefill_stratified_parity():
    """The prefill workload with per-64 float intermediate scales, stratified tokens."""
    _parity_at_size(3, sf64=True)
