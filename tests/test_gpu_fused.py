"""The fused forward (MEGA_MOE_FLAG_FUSED: dispatch, both GEMMs and the combine in one cooperative
launch) on an MI355X, through the C ABI.

It runs the same device code as the split forward, so every result must be bit for bit equal to
the split forward's: y, the dispatch metadata, the intermediate and its scales.  Launches follow
each other with different inputs and sizes (its grid barriers count across launches), and the
decode workload is also compared in full with the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_topk_amd as mm
import synth
from harness import (assert_dispatch_exact, assert_intermediate_close, assert_y_close, problem_of, run_gpu,
                     run_oracle, to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-fused] {msg}", flush=True)
    sys.stdout.flush()


def _same_as_split(spec, D, flags=0):
    y0, v0, _ = run_gpu(spec, D, flags)
    y1, v1, ws = run_gpu(spec, D, flags | mm.FLAG_FUSED, fill=0xA5)
    assert torch.equal(y1, y0), "fused y differs from the split forward"
    P = spec.T * spec.k
    n = int(v0["expert_offset"][-1])
    for name in ("expert_count", "expert_offset", "pair_pos", "num_invalid"):
        assert torch.equal(v1[name], v0[name]), name
    assert torch.equal(v1["pool_src"][:n], v0["pool_src"][:n])
    assert torch.equal(v1["inter_q"][:n], v0["inter_q"][:n])
    assert torch.equal(v1["inter_sf"][:n], v0["inter_sf"][:n])
    return y1, v1


CASES = {
    "fp8_ragged": synth.Spec(37, 640, 384, 12, 3, seed=201, weight_set=201),
    "fp8_zipf_multi_tile": synth.Spec(900, 512, 384, 16, 4, routing="zipf", seed=202, weight_set=202),
    "fp8_clamp": synth.Spec(64, 512, 256, 8, 4, routing="biased", swiglu_clamp=0.05, seed=203, weight_set=203),
    "fp8_sf64": synth.Spec(300, 512, 256, 6, 2, inter_sf64=True, seed=204, weight_set=204),
    "mxfp4_shared": synth.Spec(200, 512, 256, 9, 5, recipe=1, routing="uniform_shared", seed=205, weight_set=205),
    "mxfp8_zipf": synth.Spec(512, 640, 384, 32, 4, recipe=2, routing="zipf", seed=206, weight_set=206),
    "T1": synth.Spec(1, 512, 256, 8, 2, seed=207, weight_set=207),
    "E1_k1": synth.Spec(70, 384, 256, 1, 1, seed=208, weight_set=208),
    "wide_dispatch": synth.Spec(2100, 512, 256, 64, 8, routing="zipf", seed=209, weight_set=209),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_split(name):
    spec = CASES[name]
    _say(f"{name}: {spec}")
    _same_as_split(spec, to_device(synth.make_problem(spec)))


def test_fused_masked_and_invalid_ids():
    spec = synth.Spec(33, 512, 256, 6, 3, seed=210, weight_set=210)
    P = synth.make_problem(spec)
    idx = P["topk_idx"].numpy().copy()
    rng = np.random.default_rng(3)
    idx[rng.random(idx.shape) < 0.2] = -1
    idx[rng.random(idx.shape) < 0.1] = 6 + 3
    P["topk_idx"] = torch.as_tensor(idx, dtype=torch.int32)
    _same_as_split(spec, to_device(P))


def test_fused_launches_back_to_back():
    """Several fused launches in a row with different sizes and inputs, no synchronisation in
    between, each equal to its split forward."""
    specs = [synth.Spec(T, 512, 256, 8, 2, seed=220 + T, weight_set=220) for T in (64, 5, 300, 64, 1)]
    outs = []
    for spec in specs:
        D = to_device(synth.make_problem(spec))
        prob = problem_of(spec, mm.FLAG_FUSED)
        ws = torch.empty(mm.mega_moe_workspace_size(prob), dtype=torch.uint8, device="cuda")
        y = torch.empty(spec.T, spec.H, dtype=torch.bfloat16, device="cuda")
        mm.mega_moe_forward(prob, D["x"], D["x_sf"], D["topk_idx"], D["topk_w"], D["l1_w"], D["l1_sf"],
                            D["l2_w"], D["l2_sf"], y, ws)
        outs.append((spec, D, y, ws))
    torch.cuda.synchronize()
    for spec, D, y, ws in outs:
        y0, _, _ = run_gpu(spec, D)
        assert torch.equal(y.view(torch.int16), y0)


def test_fused_decode_full_parity():
    """The decode workload through the fused forward: equal to the split forward and, every token,
    within the bar against the oracle."""
    spec = synth.CONFIGS[1]
    _say(f"decode: {spec.name}")
    P = synth.make_weights(spec, "cuda")
    idx, w = synth.make_routing(spec)
    x, x_sf = synth.make_activations(spec, "cuda")
    P.update(x=x, x_sf=x_sf, topk_idx=idx.cuda(), topk_w=w.cuda())
    y, views = _same_as_split(spec, P)
    assert_dispatch_exact(spec, idx.numpy(), views)
    ref = run_oracle(spec, P)
    assert_intermediate_close(spec, views, ref)
    rel, mean_rel = assert_y_close(y.cpu().numpy(), ref["y"], spec.name)
    _say(f"decode fused: y max-rel {rel:.3e} mean-rel {mean_rel:.3e}")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_fused_equals_split_at_benchmark_sizes(cfg):
    """Mid, prefill and MXFP4 workloads: the fused forward equals the split forward bit for bit."""
    spec = synth.CONFIGS[cfg]
    _say(f"config {cfg}: {spec.name}")
    P = synth.make_weights(spec, "cuda")
    idx, w = synth.make_routing(spec)
    x, x_sf = synth.make_activations(spec, "cuda")
    P.update(x=x, x_sf=x_sf, topk_idx=idx.cuda(), topk_w=w.cuda())
    flags = mm.FLAG_WEIGHT_SF_KMAJOR if spec.recipe != 0 else 0
    if spec.recipe == 1:
        flags |= mm.FLAG_WEIGHT_E2M1_PAIRED
    _same_as_split(spec, P, flags)


def test_fused_equals_split_paired_weights():
    """MXFP4 with row-pair weights (wide L1 items, each counting for two slabs of its tile)."""
    spec = CASES["mxfp4_shared"]
    _same_as_split(spec, to_device(synth.make_problem(spec)), mm.FLAG_WEIGHT_E2M1_PAIRED)
