"""mega_moe_forward_noalloc (the library's static per-GPU scratch instead of a workspace) against
mega_moe_forward on the same inputs, through the C ABI on an MI355X.

Two calls in a row on the same GPU, the second with a smaller input, so the second runs on the
scratch the first left behind; each must give y bit for bit equal to the workspace entry point's
(same kernels), and that y must meet the layer's bar against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_topk_amd as mm
import synth
from harness import assert_y_close, problem_of, run_oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(spec, weights):
    idx, w = synth.make_routing(spec)
    x, x_sf = synth.make_activations(spec, "cuda")
    P = dict(weights)
    P.update(x=x, x_sf=x_sf, topk_idx=idx.cuda(), topk_w=w.cuda())
    return P


def _both(spec, P):
    prob = problem_of(spec)
    args = (P["x"], P["x_sf"], P["topk_idx"], P["topk_w"], P["l1_w"], P["l1_sf"], P["l2_w"], P["l2_sf"])
    y_ref = torch.empty(spec.T, spec.H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mm.mega_moe_workspace_size(prob), dtype=torch.uint8, device="cuda")
    mm.mega_moe_forward(prob, *args, y_ref, ws)
    y = torch.full((spec.T, spec.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    mm.mega_moe_forward_noalloc(prob, *args, y)
    torch.cuda.synchronize()
    return y.view(torch.int16), y_ref.view(torch.int16)


@pytest.mark.parametrize("shape", ["decode", "small"])
def test_noalloc_matches_workspace_forward_twice(shape):
    if shape == "decode":
        big = synth.CONFIGS[1]                          # T = 128: 16.3 MiB of the 32 MiB scratch
        small = synth.Spec(40, big.H, big.I, big.E, big.k, seed=2101, weight_set=big.weight_set)
    else:
        big = synth.Spec(96, 640, 384, 12, 3, seed=2102, weight_set=2102)
        small = synth.Spec(9, 640, 384, 12, 3, seed=2103, weight_set=2102)
    weights = synth.make_weights(big, "cuda")
    for spec in (big, small):
        _say(f"{shape}: T={spec.T} H={spec.H} I={spec.I} E={spec.E} k={spec.k}")
        P = _inputs(spec, weights)
        y, y_ref = _both(spec, P)
        assert torch.equal(y, y_ref), "noalloc forward differs from the workspace forward"
        toks = [0, spec.T - 1]
        ref = run_oracle(spec, P, tokens=toks)
        assert_y_close(y.cpu().numpy()[toks], ref["y"], spec.name or str(spec))


def test_noalloc_rejects_problems_beyond_the_scratch():
    """A problem needing more than the scratch is refused before anything is enqueued."""
    spec = synth.Spec(4096, 7168, 2048, 1, 8)         # 0.5 GiB of workspace
    prob = problem_of(spec)
    assert mm.mega_moe_workspace_size(prob) > mm.NOALLOC_SCRATCH_BYTES
    t = {k: torch.zeros(s, dtype=dt, device="cuda") for k, (s, dt) in synth.weight_shapes(spec).items()}
    x = torch.zeros(spec.T, spec.H, dtype=torch.uint8, device="cuda")
    x_sf = torch.ones(spec.T, spec.H // 128, device="cuda")
    idx = torch.zeros(spec.T, spec.k, dtype=torch.int32, device="cuda")
    w = torch.zeros(spec.T, spec.k, device="cuda")
    y = torch.empty(spec.T, spec.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mm.MegaMoEError) as ei:
        mm.mega_moe_forward_noalloc(prob, x, x_sf, idx, w, t["l1_w"], t["l1_sf"], t["l2_w"], t["l2_sf"], y)
    assert ei.value.status == mm.ERR_SCRATCH_TOO_SMALL
