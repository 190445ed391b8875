"""Seeded synthetic inputs for the MegaMoE expert layer.

This module is shared by the oracle side and the GPU side of every test and
of the benchmark, and it holds none of the layer's own arithmetic: it draws
random routing, activations and weights and stores them in the layer's input
formats using torch's library casts (``torch.float8_e4m3fn``) and plain
nearest-value rounding for E2M1.  Quantising the *inputs* is not a step of the
layer; the layer consumes the codes and scales produced here.

Workloads (sizes and distributions of the five benchmark shapes):

====  ======  =====  =====  =====  ===  ===========================================
cfg   T       H      I      E      k    routing / recipe
====  ======  =====  =====  =====  ===  ===========================================
0     8       512    256    8      2    uniform without replacement, FP8 / float-128
1     128     7168   2048   256    8    uniform, FP8 / float-128   (decode)
2     1024    4096   1536   128    8    N(0,1)+bias N(0,.5) top-8, clamp 10
3     8192    7168   2048   256    8    Zipf(1.1) popularity        (prefill)
4     4096    7168   2048   256+1  8+1  uniform + shared expert, MXFP4 weights
====  ======  =====  =====  =====  ===  ===========================================

Seeds: routing and activations use ``1000 + cfg``; weights are drawn per
expert from a generator seeded by (weight set, tensor, expert), so a large
weight set streams expert by expert.  Configs 1 and 3 share weight set 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

FP8_MAX = 448.0
FP4_MAX = 6.0

RECIPE_FP8 = 0
RECIPE_MXFP4 = 1
RECIPE_MXFP8 = 2       # E4M3 weights with a UE8M0 scale per (row, 32 K); activations as MXFP4's


@dataclass(frozen=True)
class Spec:
    T: int
    H: int
    I: int
    E: int                 # experts including appended shared experts
    k: int                 # top-k columns including the shared-expert column
    recipe: int = RECIPE_FP8
    routing: str = "uniform"   # uniform | biased | zipf | uniform_shared
    swiglu_clamp: float = 0.0
    clamp_inputs: bool = False     # the clamp applies to gate and up before SiLU
    inter_sf64: bool = False       # FP8 recipe: intermediate scales per 64 channels instead of 128
    seed: int = 1000
    weight_set: int = 0
    w_std: float = 0.02
    name: str = ""

    @property
    def group(self) -> int:
        return 128 if self.recipe == RECIPE_FP8 else 32

    @property
    def inter_group(self) -> int:
        """Channels per scale of the re-quantised intermediate."""
        return 64 if self.inter_sf64 else self.group

    @property
    def pairs(self) -> int:
        return self.T * self.k


CONFIGS = [
    Spec(8, 512, 256, 8, 2, seed=1000, weight_set=0, name="tiny T8 H512 I256 E8 top2"),
    Spec(128, 7168, 2048, 256, 8, seed=1001, weight_set=1,
         name="decode T128 H7168 I2048 E256 top8 uniform"),
    Spec(1024, 4096, 1536, 128, 8, routing="biased", swiglu_clamp=10.0, seed=1002, weight_set=2,
         name="mid T1024 H4096 I1536 E128 top8 biased clamp10"),
    Spec(8192, 7168, 2048, 256, 8, routing="zipf", seed=1003, weight_set=1,
         name="prefill T8192 H7168 I2048 E256 top8 zipf1.1"),
    Spec(4096, 7168, 2048, 257, 9, recipe=RECIPE_MXFP4, routing="uniform_shared", seed=1004,
         weight_set=4, name="mxfp4 T4096 H7168 I2048 E256+1shared top8+1"),
]


# ----------------------------------------------------------------------------- routing
def make_routing(spec: Spec):
    """topk_idx int32 [T, k] and topk_w float32 [T, k] on the CPU."""
    g = torch.Generator().manual_seed(spec.seed)
    T, E, k = spec.T, spec.E, spec.k
    if T == 0:
        return torch.zeros(0, k, dtype=torch.int32), torch.zeros(0, k, dtype=torch.float32)
    if spec.routing == "uniform":
        idx = torch.argsort(torch.rand(T, E, generator=g), dim=1)[:, :k]
        w = torch.softmax(torch.randn(T, k, generator=g), dim=1)
    elif spec.routing == "biased":
        bias = torch.randn(E, generator=g) * 0.5
        score = torch.randn(T, E, generator=g) + bias
        top = torch.topk(score, k, dim=1)
        idx = top.indices
        w = torch.softmax(top.values, dim=1)
    elif spec.routing == "zipf":
        perm = torch.randperm(E, generator=g)
        ranks = torch.empty(E)
        ranks[perm] = torch.arange(1, E + 1, dtype=torch.float32)
        logp = -1.1 * torch.log(ranks)
        u = torch.rand(T, E, generator=g).clamp_min(1e-20)
        gumbel = -torch.log(-torch.log(u))
        idx = torch.topk(logp[None, :] + gumbel, k, dim=1).indices
        w = torch.softmax(torch.randn(T, k, generator=g), dim=1)
    elif spec.routing == "uniform_shared":
        er = E - 1
        idx = torch.argsort(torch.rand(T, er, generator=g), dim=1)[:, :k - 1]
        w = torch.softmax(torch.randn(T, k - 1, generator=g), dim=1)
        idx = torch.cat([idx, torch.full((T, 1), er, dtype=idx.dtype)], dim=1)
        w = torch.cat([w, torch.ones(T, 1)], dim=1)
    else:
        raise ValueError(spec.routing)
    return idx.to(torch.int32).contiguous(), w.to(torch.float32).contiguous()


# ----------------------------------------------------------------------------- input quantisers
def _fp8_codes(v: torch.Tensor) -> torch.Tensor:
    return v.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def _pow2_code(amax: torch.Tensor, fmt_max: float) -> torch.Tensor:
    """UE8M0 code of a power-of-two scale that keeps amax/scale within fmt_max."""
    r = (amax / fmt_max).clamp_min(2.0 ** -126)
    m, e = torch.frexp(r)
    e = torch.where(m == 0.5, e - 1, e)
    return (e + 127).clamp(0, 254).to(torch.uint8)


def _fp4_codes(v: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code (ties to even mantissa), saturating at 6; returns uint8 codes 0..15."""
    mag = v.abs().clamp(max=FP4_MAX)
    bounds = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], device=v.device, dtype=v.dtype)
    code = torch.bucketize(mag, bounds, right=False)          # ties -> lower value
    up_ties = (mag == 0.75) | (mag == 1.75) | (mag == 3.5)    # upper neighbour has the even mantissa
    code = code + up_ties.to(code.dtype)
    code = code | (torch.signbit(v).to(code.dtype) << 3)
    return code.to(torch.uint8)


def _pack_fp4(codes: torch.Tensor) -> torch.Tensor:
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).contiguous()


def quant_act(xf: torch.Tensor, recipe: int):
    """Activations [T, H] float32 -> (codes u8 [T, H], scales)."""
    T, H = xf.shape
    if recipe == RECIPE_FP8:
        g = xf.view(T, H // 128, 128)
        amax = g.abs().amax(dim=2)
        sf = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        return _fp8_codes(g / sf[..., None]).view(T, H).contiguous(), sf.contiguous()
    g = xf.view(T, H // 32, 32)
    code = _pow2_code(g.abs().amax(dim=2), FP8_MAX)
    scale = torch.exp2(code.float() - 127)
    return _fp8_codes(g / scale[..., None]).view(T, H).contiguous(), code.contiguous()


def quant_weight(wf: torch.Tensor, recipe: int):
    """One expert's weight [N, K] float32 -> (codes, scales) in the layer's weight format."""
    N, K = wf.shape
    if recipe == RECIPE_FP8:
        g = wf.view(N // 128, 128, K // 128, 128)
        amax = g.abs().amax(dim=(1, 3))
        sf = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        codes = _fp8_codes(g / sf[:, None, :, None]).view(N, K)
        return codes, sf
    g = wf.view(N, K // 32, 32)
    if recipe == RECIPE_MXFP8:
        code = _pow2_code(g.abs().amax(dim=2), FP8_MAX)
        scale = torch.exp2(code.float() - 127)
        return _fp8_codes(g / scale[..., None]).view(N, K).contiguous(), code
    code = _pow2_code(g.abs().amax(dim=2), FP4_MAX)
    scale = torch.exp2(code.float() - 127)
    codes = _fp4_codes(g / scale[..., None]).view(N, K)
    return _pack_fp4(codes), code


# ----------------------------------------------------------------------------- full problem
def _weight_seed(spec: Spec, tensor_id: int, e: int) -> int:
    return ((2000 + spec.weight_set) * 16 + tensor_id) * 1_000_003 + e


def weight_shapes(spec: Spec):
    H, I, E = spec.H, spec.I, spec.E
    if spec.recipe == RECIPE_FP8:
        return dict(l1_w=((E, 2 * I, H), torch.uint8), l1_sf=((E, 2 * I // 128, H // 128), torch.float32),
                    l2_w=((E, H, I), torch.uint8), l2_sf=((E, H // 128, I // 128), torch.float32))
    if spec.recipe == RECIPE_MXFP8:
        return dict(l1_w=((E, 2 * I, H), torch.uint8), l1_sf=((E, 2 * I, H // 32), torch.uint8),
                    l2_w=((E, H, I), torch.uint8), l2_sf=((E, H, I // 32), torch.uint8))
    return dict(l1_w=((E, 2 * I, H // 2), torch.uint8), l1_sf=((E, 2 * I, H // 32), torch.uint8),
                l2_w=((E, H, I // 2), torch.uint8), l2_sf=((E, H, I // 32), torch.uint8))


def make_weights(spec: Spec, device="cpu", experts=None):
    """Per-expert seeded weights in the layer's format (allocated on ``device``)."""
    shapes = weight_shapes(spec)
    out = {k: torch.zeros(s, dtype=dt, device=device) for k, (s, dt) in shapes.items()}
    ex = range(spec.E) if experts is None else experts
    dev = torch.device(device)
    for e in ex:
        for tid, (wname, sname, n, kk) in enumerate((("l1_w", "l1_sf", 2 * spec.I, spec.H),
                                                     ("l2_w", "l2_sf", spec.H, spec.I))):
            g = torch.Generator(device=dev).manual_seed(_weight_seed(spec, tid, e))
            wf = torch.randn(n, kk, generator=g, device=dev, dtype=torch.float32) * spec.w_std
            codes, sf = quant_weight(wf, spec.recipe)
            out[wname][e].copy_(codes)
            out[sname][e].copy_(sf)
            del wf
    return out


def make_activations(spec: Spec, device="cpu"):
    g = torch.Generator(device=torch.device(device)).manual_seed(spec.seed + 7)
    xf = torch.randn(spec.T, spec.H, generator=g, device=device, dtype=torch.float32)
    return quant_act(xf, spec.recipe)


def make_problem(spec: Spec, device="cpu"):
    """All inputs of one forward call: dict of tensors on ``device`` (routing built on the CPU)."""
    idx, w = make_routing(spec)
    x, x_sf = make_activations(spec, device)
    out = dict(x=x, x_sf=x_sf, topk_idx=idx.to(device), topk_w=w.to(device))
    out.update(make_weights(spec, device))
    return out


def small_spec(**kw) -> Spec:
    """A parity-test problem derived from config 0 with the given fields replaced."""
    return replace(CONFIGS[0], **kw)
