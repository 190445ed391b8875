"""Plain CPU oracle of the MegaMoE expert-layer forward on one device.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code,
table or constant generator with the HIP kernels.

What it computes, step by step, with where the pages define each step:

1. Routing / dispatch.  Every (token t, top-k slot j) pair whose expert id
   e = topk_idx[t, j] is in [0, E) becomes one row of expert e's pool.  Rows
   of one expert are kept in row-major (t, j) order.  The research report
   (section 3.1 "dispatch", and the SM100 dispatch workgroup description) and
   the design page (section 9.2, "Dispatch Pull Path": source metadata
   {rank, token, topk}) define the count, the pool and the metadata; the
   stable order is the plain reading of "token-topk gather" (the pages' own
   order comes from racing atomics).  Ids < 0 are masked slots; ids >= E are
   dropped and counted.
2. L1 block-scaled GEMM (design page section 5.3, "Scale Factor
   Application", and section 15.2 for the weight-scale layout):
   acc[p, n] = sum over K blocks kb of sfa[t, kb] * sfb[e, n/128, kb] *
   (sum over k in kb of a[t, k] * b[e, n, k]).  The FP8 x MXFP4 recipe uses
   32-wide K blocks with power-of-two scales on both operands (PR #411); the
   FP8 x FP8 per-32 recipe does the same with E4M3 weights, the SM100 scale
   format (UE8M0 per 32 K for activations, weights and the intermediate: the
   research report, section 8.4 on scale-factor formats; the design page,
   section 2, scale-factor row of the architecture-gap table).
3. SwiGLU epilogue (design page section 10.1 "Register-Based Flow"):
   s = silu(gate) * up with gate = acc[:, :I], up = acc[:, I:]; optionally
   clamped (s to [-c, c], or, as in step 3 of that section, gate and up to
   [-c, c] before SiLU); multiplied by the row's top-k weight before the
   re-quantisation.
4. Re-quantisation per group of G output channels: amax, float scale
   amax/448 and an E4M3 cast of value/scale (design section 10.1 steps 4-5,
   G = 128), or a power-of-two UE8M0 scale per 32 channels for the two per-32
   recipes.
5. L2 block-scaled GEMM over the intermediate (same form as step 2), each
   row's FP32 result cast to BF16 (design page section 11.1).
6. Combine (design page section 11.2, "Combine Reduce"): per token, the BF16
   rows of its active top-k slots are summed in float32 in ascending slot
   order and cast to BF16.

Precision: GEMM block sums are formed in float64, where every FP8 x FP8 (and
FP8 x FP4) product and every 128-long block sum is exact; the scales are applied
in float64.  The quantisation decisions the pages make in float (the SwiGLU
value, its amax, amax/448, value/scale, the BF16 casts, the combine sum) are
taken in float32, as the pages state.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import codecs as C

RECIPE_FP8_B128 = 0      # E4M3 everywhere, float scales per 128 (x: per token row; w: 128x128)
RECIPE_MXFP4W_B32 = 1    # E4M3 activations, E2M1 weights, UE8M0 scales per 32 along K
RECIPE_MXFP8_B32 = 2     # E4M3 activations and weights, UE8M0 scales per 32 along K


@dataclass(frozen=True)
class Problem:
    T: int
    H: int
    I: int
    E: int
    k: int
    recipe: int = RECIPE_FP8_B128
    swiglu_clamp: float = 0.0
    clamp_inputs: bool = False     # clamp gate and up before SiLU instead of silu(gate) * up
    inter_sf64: bool = False       # FP8 recipe: intermediate re-quantised with a float scale per 64

    @property
    def group(self) -> int:
        """K block of the input scales (activations and weights)."""
        return 128 if self.recipe == RECIPE_FP8_B128 else 32

    @property
    def inter_group(self) -> int:
        """Channels per scale of the re-quantised intermediate: the input block, or 64 for the
        SM90 design's per-64 float scales (design page section 5.4, the L1 epilogue writing one
        float scale per 64 output columns, and section 10.1 step 6, the per-64 scale layout)."""
        return 64 if self.inter_sf64 else self.group


# --------------------------------------------------------------------------- dispatch
def route(topk_idx: np.ndarray, num_experts: int) -> dict:
    """Stable per-expert pools.

    Returns count[E], offset[E+1], src[n_valid] (pool row -> pair t*k+j),
    pos[T*k] (pair -> pool row, -1 when masked or invalid) and num_invalid.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    pools = [[] for _ in range(num_experts)]
    num_invalid = 0
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            if e >= num_experts:
                num_invalid += 1
                continue
            pools[e].append(t * k + j)
    count = np.array([len(p) for p in pools], dtype=np.int64)
    offset = np.zeros(num_experts + 1, dtype=np.int64)
    offset[1:] = np.cumsum(count)
    src = np.array([pair for p in pools for pair in p], dtype=np.int64)
    pos = np.full(T * k, -1, dtype=np.int64)
    pos[src] = np.arange(src.size)
    return dict(count=count, offset=offset, src=src, pos=pos, num_invalid=num_invalid)


# --------------------------------------------------------------------------- dequantisation
def _act_values(prob: Problem, x_rows: np.ndarray) -> np.ndarray:
    return C.e4m3_decode(x_rows)


def _act_scales(prob: Problem, sf_rows: np.ndarray) -> np.ndarray:
    if prob.recipe == RECIPE_FP8_B128:
        return np.asarray(sf_rows, dtype=np.float32).astype(np.float64)
    return C.ue8m0_decode(sf_rows)


def _weight_values(prob: Problem, w: np.ndarray) -> np.ndarray:
    if prob.recipe == RECIPE_MXFP4W_B32:
        return C.e2m1_unpack_decode(w)
    return C.e4m3_decode(w)


def _weight_scales_rows(prob: Problem, sf: np.ndarray, n_rows: int) -> np.ndarray:
    """Per-(row, K block) weight scale, float64 [n_rows, K/G]."""
    if prob.recipe == RECIPE_FP8_B128:
        blk = np.asarray(sf, dtype=np.float32).astype(np.float64)      # [rows/128, K/128]
        return np.repeat(blk, 128, axis=0)[:n_rows]
    return C.ue8m0_decode(sf)                                            # [rows, K/32]


def block_scaled_gemm(prob: Problem, a_vals, a_scale, b_vals, b_scale, group: int = 0) -> np.ndarray:
    """sum_kb a_scale[m,kb] * b_scale[n,kb] * sum_{k in kb} a[m,k] * b[n,k]  (float64).

    a_vals [M, K], a_scale [M, K/G], b_vals [N, K], b_scale [N, K/G]; G = K block (group, or the
    recipe's input block when 0).
    """
    G = group or prob.group
    M, K = a_vals.shape
    N = b_vals.shape[0]
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // G):
        blk = a_vals[:, kb * G:(kb + 1) * G] @ b_vals[:, kb * G:(kb + 1) * G].T
        out += blk * a_scale[:, kb:kb + 1] * b_scale[None, :, kb]
    return out


# --------------------------------------------------------------------------- epilogue
def swiglu_weighted(prob: Problem, acc: np.ndarray, w_rows: np.ndarray) -> np.ndarray:
    """s = silu(gate) * up times the top-k weight (float64).  With a clamp c > 0, s is clamped
    to [-c, c]; with clamp_inputs, gate and up are clamped to [-c, c] before SiLU instead (the
    design page's activation clamp, section 10.1 step 3)."""
    I = prob.I
    gate = acc[:, :I]
    up = acc[:, I:2 * I]
    c = prob.swiglu_clamp
    clamp = c > 0 and np.isfinite(c)
    if clamp and prob.clamp_inputs:
        gate = np.clip(gate, -c, c)
        up = np.clip(up, -c, c)
    with np.errstate(over="ignore"):
        s = gate / (1.0 + np.exp(-gate)) * up          # exp overflow -> silu(gate) = -0
    if clamp and not prob.clamp_inputs:
        s = np.clip(s, -c, c)
    return s * np.asarray(w_rows, dtype=np.float32).astype(np.float64)[:, None]


def requant(prob: Problem, v: np.ndarray):
    """Group-wise FP8 re-quantisation of the SwiGLU output.

    Returns (codes u8 [n, I], scales [n, I/G] (float32, or UE8M0 u8), dequantised float64).
    """
    n, I = v.shape
    G = prob.inter_group
    v32 = v.astype(np.float32).reshape(n, I // G, G)
    amax = np.max(np.abs(v32), axis=2)                                     # float32, exact
    if prob.recipe == RECIPE_FP8_B128:
        sf = (amax / np.float32(C.E4M3_MAX)).astype(np.float32)            # float32 division
        safe = np.where(sf > 0, sf, np.float32(1.0)).astype(np.float32)
        r = (v32 / safe[:, :, None]).astype(np.float32)                    # float32 division
        r = np.clip(r, -C.E4M3_MAX, C.E4M3_MAX)
        q = C.e4m3_encode_rne(r)
        q = np.where((sf > 0)[:, :, None], q, np.uint8(0)).astype(np.uint8)
        vd = C.e4m3_decode(q) * sf.astype(np.float64)[:, :, None]
        return q.reshape(n, I), sf, vd.reshape(n, I)
    code = C.ue8m0_code_for_amax(amax, C.E4M3_MAX)                         # u8 [n, I/32]
    scale = np.ldexp(1.0, code.astype(np.int64) - 127)
    r = v32.astype(np.float64) / scale[:, :, None]                         # exact power-of-two scaling
    r = np.clip(r, -C.E4M3_MAX, C.E4M3_MAX)
    q = C.e4m3_encode_rne(r)
    q = np.where((amax > 0)[:, :, None], q, np.uint8(0)).astype(np.uint8)
    vd = C.e4m3_decode(q) * scale[:, :, None]
    return q.reshape(n, I), code, vd.reshape(n, I)


# --------------------------------------------------------------------------- forward
def expert_rows(prob: Problem, e: int, t_rows: np.ndarray, w_rows: np.ndarray,
                x, x_sf, l1_w, l1_sf, l2_w, l2_sf, magnitudes: bool = False) -> dict:
    """Everything one expert does to a set of its pool rows (token ids t_rows).

    magnitudes: also return l1_abs, the same block-scaled sum over the magnitudes of every
    product, sum_kb |sa| |sb| sum_k |a| |b| (what bounds the rounding error of any summation
    order of the L1 products; the tests derive their intermediate-code tolerance from it)."""
    a = _act_values(prob, x[t_rows])
    sa = _act_scales(prob, x_sf[t_rows])
    w1 = _weight_values(prob, l1_w[e])
    s1 = _weight_scales_rows(prob, l1_sf[e], 2 * prob.I)
    acc = block_scaled_gemm(prob, a, sa, w1, s1)                           # [n, 2I]
    l1_abs = (block_scaled_gemm(prob, np.abs(a), np.abs(sa), np.abs(w1), np.abs(s1))
              if magnitudes else None)
    v = swiglu_weighted(prob, acc, w_rows)
    q, qsf, vd = requant(prob, v)
    w2 = _weight_values(prob, l2_w[e])
    s2 = _weight_scales_rows(prob, l2_sf[e], prob.H)
    if prob.recipe == RECIPE_FP8_B128:
        sq = qsf.astype(np.float64)
    else:
        sq = np.ldexp(1.0, qsf.astype(np.int64) - 127)
    # per-64 intermediate scales: each 128-K block of w2 is summed as two 64-K halves, each with
    # its own activation scale and the block's weight scale (design page section 5.4)
    Gi = prob.inter_group
    s2 = np.repeat(s2, prob.group // Gi, axis=1) if Gi < prob.group else s2
    o = block_scaled_gemm(prob, C.e4m3_decode(q), sq, w2, s2, group=Gi)    # [n, H]
    slot = C.bf16_bits_rne(o.astype(np.float32))
    return dict(l1_acc=acc, l1_abs=l1_abs, v=v, inter_q=q, inter_sf=qsf, o=o, slot=slot)


def forward(prob: Problem, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf,
            tokens=None, magnitudes: bool = False) -> dict:
    """The layer forward.  ``tokens`` (optional) restricts the work to those tokens.

    Returns y (BF16 bits, [len(tokens) or T, H]), the dispatch result, and per
    pool row (only rows of the selected tokens) the intermediate codes/scales
    and the BF16 slot rows.  With ``magnitudes``, also per pool row the L1
    result (l1_acc), its magnitude sum (l1_abs, see expert_rows), the
    pre-quantisation value v (float64) and the row's top-k weight.
    """
    T, k = prob.T, prob.k
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, dtype=np.float32)
    d = route(idx, prob.E)
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    want = np.zeros(T, dtype=bool)
    want[sel] = True
    slot = {}            # pair -> BF16 bits [H]
    inter_q, inter_sf = {}, {}
    extra = dict(l1_acc={}, l1_abs={}, v={}, w={}) if magnitudes else {}
    for e in range(prob.E):
        rows = d["src"][d["offset"][e]:d["offset"][e + 1]]
        rows = rows[want[rows // k]]
        if rows.size == 0:
            continue
        t_rows = rows // k
        w_rows = w.reshape(-1)[rows]
        r = expert_rows(prob, e, t_rows, w_rows, x, x_sf, l1_w, l1_sf, l2_w, l2_sf, magnitudes)
        for i, pair in enumerate(rows):
            p = int(d["pos"][pair])
            slot[int(pair)] = r["slot"][i]
            inter_q[p] = r["inter_q"][i]
            inter_sf[p] = r["inter_sf"][i]
            if magnitudes:
                extra["l1_acc"][p] = r["l1_acc"][i]
                extra["l1_abs"][p] = r["l1_abs"][i]
                extra["v"][p] = r["v"][i]
                extra["w"][p] = float(w_rows[i])
    y = np.zeros((sel.size, prob.H), dtype=np.uint16)
    for i, t in enumerate(sel):
        acc = np.zeros(prob.H, dtype=np.float32)
        for j in range(k):
            pair = int(t) * k + j
            if pair in slot:
                acc = (acc + C.bf16_bits_to_f32(slot[pair])).astype(np.float32)
        y[i] = C.bf16_bits_rne(acc)
    return dict(y=y, tokens=sel, dispatch=d, slot=slot, inter_q=inter_q, inter_sf=inter_sf, **extra)


def flops(prob: Problem, n_pairs: int) -> float:
    """Algorithmic FLOPs of the two GEMMs: 2*H*2I (L1) + 2*I*H (L2) per routed pair."""
    return 6.0 * prob.H * prob.I * n_pairs
