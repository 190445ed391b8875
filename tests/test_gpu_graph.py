"""The layer forward captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The forward only enqueues kernels on the caller's stream (no allocation, no memset, no
synchronisation), so it can be captured once and replayed.  Each replay must reproduce the eager
forward bit for bit (the kernels are deterministic), also after eager forwards of other inputs
have run on the same workspace between replays (every call re-initialises what it uses).
"""
from dataclasses import replace

import pytest
import torch

import dispatch_fp8_grouped_topk_amd as mm
import synth
from harness import problem_of, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp8": synth.CONFIGS[0],
    "zipf_fp8_multi_tile": synth.Spec(512, 512, 384, 32, 4, routing="zipf", seed=120, weight_set=120),
    "mxfp4_shared": synth.Spec(160, 512, 256, 9, 5, recipe=1, routing="uniform_shared", seed=121,
                               weight_set=121),
    "mxfp8_zipf": synth.Spec(512, 512, 384, 32, 4, recipe=2, routing="zipf", seed=124, weight_set=124),
    "mxfp4_shared_kmajor_sf": synth.Spec(160, 512, 256, 9, 5, recipe=1, routing="uniform_shared", seed=125,
                                         weight_set=125),
}
# cases whose weight scales go through the one-time K-major transform first
KMAJOR = {"mxfp4_shared_kmajor_sf"}


def _forward(prob, D, y, ws):
    mm.mega_moe_forward(prob, D["x"], D["x_sf"], D["topk_idx"], D["topk_w"], D["l1_w"], D["l1_sf"],
                        D["l2_w"], D["l2_sf"], y, ws)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    spec = CASES[name]
    print(f"[gpu-graph] {name}: {spec}", flush=True)
    D = to_device(synth.make_problem(spec))
    D_other = to_device(synth.make_problem(replace(spec, seed=spec.seed + 7)))
    prob = problem_of(spec, mm.FLAG_WEIGHT_SF_KMAJOR if name in KMAJOR else 0)
    if name in KMAJOR:
        for P in (D, D_other):
            P["l1_sf"], P["l2_sf"] = mm.mega_moe_transform_weight_scales(prob, P["l1_sf"], P["l2_sf"])
        torch.cuda.synchronize()
    ws = torch.empty(mm.mega_moe_workspace_size(prob), dtype=torch.uint8, device="cuda")
    y_eager = torch.empty(spec.T, spec.H, dtype=torch.bfloat16, device="cuda")
    _forward(prob, D, y_eager, ws)
    torch.cuda.synchronize()

    y_graph = torch.empty_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up outside the capture
        _forward(prob, D, y_graph, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _forward(prob, D, y_graph, ws)
    torch.cuda.synchronize()

    y_other = torch.empty_like(y_eager)
    for rep in range(3):
        y_graph.fill_(0)                          # eager work between replays
        _forward(prob, D_other, y_other, ws)      # leaves other contents in the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep} differs"
    assert not torch.equal(y_other.view(torch.int16), y_eager.view(torch.int16))
