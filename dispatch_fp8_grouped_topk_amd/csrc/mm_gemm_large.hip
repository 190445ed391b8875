// Large-M grouped GEMM kernels (device code in mm_large_dev.h) and the four-wave MXFP4 L2
// kernel.
#include "mm_large_dev.h"

namespace mm {

namespace {

// The persistent kernels over the large-M items (see large_items).  H64: the FP8 L2 GEMM with
// per-64 intermediate scales (a kernel of its own, so the default kernels' code and register
// allocation do not carry its two-MFMA blocks).
template <int R, bool L1, bool H64 = false>
__global__ __launch_bounds__(kThreads) void k_large(Args a) {
  __shared__ __attribute__((aligned(1024))) Lds L;
  NoHooks hooks;
  large_items<R, L1, H64, true>(a, L, hooks);
}

// ------------------------------------------------------------------------------ four-wave kernel
// MXFP4 L2 tiles of at most 160 pool rows (experts whose first tile has at most kQuadMaxNG
// column groups per wave in the eight-wave kernel).  There, a K step of such a tile does a
// quarter to a half of a full tile's MFMA work behind the same barrier, LDS read burst and load
// issue, and both waves of each SIMD move through those phases in lockstep.  Here a workgroup is
// four waves (one per SIMD) with at most 80 KB of LDS, so two workgroups share each CU and their
// K steps, separated by independent barriers, overlap each other's stalls.  Wave w owns the
// weight rows of group w (64 rows of w2 in four MFMA row tiles, as wave w of the eight-wave
// kernel) and every 16-token column group of the tile, so a K step of a 128-row tile gives each
// wave the MFMA work of a full tile's wave.  Same slab items, operand layout, swizzles, UE8M0
// scale handling and BF16 epilogue as the eight-wave kernel.  Only two 128-K stages fit in
// 80 KB, so a step's loads have one step to land: enough for L2's 16-step loop over the
// intermediate, not for L1's 56-step weight stream from HBM, which stays in the eight-wave
// kernel with its four-stage ring (measured: L1 1.33 -> 1.71 ms, L2 0.77 -> 0.71 ms).
constexpr int kQThreads = 256;
constexpr int kQGroups = 2 * kQuadMaxNG;             // most 16-row column groups of a tile
constexpr int kQTok = 16 * kQGroups;                 // most rows of a tile (160)
constexpr int kQRingBudget = 80 * 1024 - 2 * 4 * kQTok - 1024;

// Ring of 128-K stages: 256 E2M1 weight rows (64 bytes each), the tile's 16 NC token rows (128
// bytes each) and 512 scale words (words [0, 256): the activation scale word of tile row r at
// r; words [256, 512): the weight scale word of weight row r at 256 + r), as deep as fits.
template <int NC>
struct QRing {
  static constexpr int kWBytes = kWRows * 64;
  static constexpr int kXRows = 16 * NC;
  static constexpr int kStageBytes = kWBytes + kXRows * 128 + 2048;
  static constexpr int kFit = kQRingBudget / kStageBytes;
  static constexpr int kStages = kFit > 4 ? 4 : kFit;
  static_assert(kStages >= 2, "two stages must fit");
};

struct QLds {
  uint8_t ring[kQRingBudget];
  int rowsrc[kQTok];                          // pool row of each tile row
  int aux[kQTok];                             // slot row (pair) of each tile row
};
static_assert(sizeof(QLds) <= 80 * 1024, "two workgroups per CU");


template <int NC>
__device__ __forceinline__ StageRef qstage_ref(uint8_t* ring, int slot) {
  uint8_t* b = ring + slot * QRing<NC>::kStageBytes;
  return StageRef{b, b + QRing<NC>::kWBytes,
                  reinterpret_cast<uint32_t*>(b + QRing<NC>::kWBytes + QRing<NC>::kXRows * 128)};
}

// One wave's share of a stage: four 1 KB loads of weight rows 64 w + 16 j + lane / 4, ceil(NC / 2)
// loads of 8-row token blocks w + 4 j (past the tile's 2 NC blocks, the last block again: the
// same bytes to the same place), the activation scale words of tile rows 64 w + lane and the
// weight scale words of weight rows 64 w + lane.
template <int NC>
constexpr int kQTokenLoads = (2 * NC + 3) / 4;
template <int NC>
constexpr int kQStageLoads = 4 + kQTokenLoads<NC> + 2;

struct QSrc {
  rsrc_t wr, xr, ar, sr;                      // weights, token rows, activation / weight scale words
  uint32_t wo[4];
  uint32_t xo[(2 * kQGroups + 3) / 4];
  uint32_t ao, so;
  uint32_t akb, skb;                          // bytes per K block of the two scale sources
  uint32_t wend;                              // bytes of the weight buffer (wr's size)
  int wkb;                                    // bytes per K block of a weight row (pair)
};

template <int NC>
__device__ __forceinline__ int qtoken_block(int w, int j) {
  const int b = w + 4 * j;
  return b < 2 * NC ? b : 2 * NC - 1;
}

// Load j of block kb; past the last block (kb >= KB) the weight loads read zeros through a lane
// offset at the buffer's end (no memory access) and the other loads fetch a copy of block KB - 1.
template <int NC>
__device__ __forceinline__ void qissue_load(const StageRef& F, const QSrc& s, int kb_, int KB, int w, int j) {
  constexpr int NT = kQTokenLoads<NC>;
  const int kb = min(kb_, KB - 1);
  if (j < 4) {
    const bool past = kb_ >= KB;
    lds_load16(s.wr, past ? s.wend : s.wo[j], past ? 0 : kb * s.wkb, F.w + (64 * w + 16 * j) * 64);
  } else if (j < 4 + NT) {
    lds_load16(s.xr, s.xo[j - 4], kb * 128, F.x + qtoken_block<NC>(w, j - 4) * 8 * 128);
  } else if (j == 4 + NT) {
    lds_load4(s.ar, s.ao, (int)((uint32_t)kb * s.akb), F.scl + 64 * w);
  } else {
    lds_load4(s.sr, s.so, (int)((uint32_t)kb * s.skb), F.scl + 256 + 64 * w);
  }
}

template <int NC>
__device__ __forceinline__ constexpr int qstage_split(int i) {
  constexpr int C = kQStageLoads<NC>, G = NC < kSpreadGroups ? NC : kSpreadGroups;
  return i >= G ? C : (C * i + G - 1) / G;
}

// K loop: acc[rt][i] += weight tile rt x column group i.  arow0: the lane's LDS row of weight
// tile 0.  As in the eight-wave kernel, every step issues one stage (past the end zeros for the
// weights and a copy of block KB - 1 for the rest, into a retired slot), so NS - 2 stages of
// loads stay in flight behind block kb.
template <int NC>
__device__ __forceinline__ void q_loop(QLds& L, const QSrc& src, int arow0, int KB, v4f acc[4][NC], int w,
                                       int lane) {
  constexpr int NS = QRing<NC>::kStages;
  const int lr = lane & 15, lg = lane >> 4;
  const int sw7 = (lr >> 1) & 7;
  const int wlo = arow0 * 64 + 16 * (lg ^ ((lr >> 2) & 3));
  const int xlo = lr * 128 + 16 * (lg ^ sw7);
  const int xhi = lr * 128 + 16 * ((lg | 4) ^ sw7);
  int swrow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) swrow[rt] = scl_w(arow0 + a_tile_rows<false>(rt));
#pragma unroll
  for (int b = 0; b < NS - 1; ++b) {
#pragma unroll
    for (int j = 0; j < kQStageLoads<NC>; ++j) qissue_load<NC>(qstage_ref<NC>(L.ring, b), src, b, KB, w, j);
  }
  int cur = 0;                               // ring slot of block kb
  for (int kb = 0; kb < KB; ++kb) {
    wait_vmcnt<(NS - 2) * kQStageLoads<NC>>();
    pipeline_barrier();                      // block kb landed for all four waves; kb-1 retired
    const int ahead = kb + NS - 1;
    const StageRef F = qstage_ref<NC>(L.ring, cur == 0 ? NS - 1 : cur - 1);
    auto fetch_part = [&](int i) {
#pragma unroll
      for (int j = qstage_split<NC>(i); j < qstage_split<NC>(i + 1); ++j) qissue_load<NC>(F, src, ahead, KB, w, j);
    };
    const StageRef S = qstage_ref<NC>(L.ring, cur);
    cur = cur + 1 == NS ? 0 : cur + 1;
    const uint8_t* xl = S.x + xlo;
    const uint8_t* xh = S.x + xhi;
    v8i B = lds_fp8_operand(xl, xh, 0);
    v8i A[4];
    int swv[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      A[rt] = lds_fp4_operand_lo(S.w + wlo, a_tile_rows<false>(rt) * 64);
      swv[rt] = (S.scl[swrow[rt]] >> (8 * lg)) & 0xFF;
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      v8i Bn;
      if (i + 1 < NC) Bn = lds_fp8_operand(xl, xh, 2048 * (i + 1));
      const int sx = (S.scl[16 * i + lr] >> (8 * lg)) & 0xFF;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][i] = mfma_fp4w_fp8(A[rt], B, acc[rt][i], swv[rt], sx);
      __builtin_amdgcn_sched_barrier(0);
      fetch_part(i);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < NC) B = Bn;
    }
  }
  wait_vmcnt<0>();
}

// Per-lane global offsets of one wave's loads; grow(r) maps a tile's weight row (0..255) to the
// w2 row within the expert, wrow_bytes / wsrow_bytes are the E2M1 row and scale row strides.
template <int NC, class F>
__device__ __forceinline__ void q_offsets(QSrc& s, const int* rowsrc, uint32_t xrow_bytes, F grow,
                                          uint32_t wrow_bytes, uint32_t wsrow_bytes, int off, int cnt, int w,
                                          int lane, bool paired) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 64 * w + 16 * j + (lane >> 2);
    const int g = grow(r);
    const uint32_t piece = 16u * (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
    s.wo[j] = paired ? (uint32_t)(g >> 1) * 2u * wrow_bytes + 64u * (uint32_t)(g & 1) + piece
                     : (uint32_t)g * wrow_bytes + piece;   // row-pair layout: see weight_offsets
  }
#pragma unroll
  for (int j = 0; j < kQTokenLoads<NC>; ++j) {
    const int r = 8 * qtoken_block<NC>(w, j) + (lane >> 3);
    s.xo[j] = (uint32_t)rowsrc[r] * xrow_bytes + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  const int r = 64 * w + lane;
  s.ao = 4u * (uint32_t)(off + (r < cnt ? r : cnt - 1));
  s.so = (uint32_t)grow(r) * wsrow_bytes;
}

template <int NC>
__device__ __forceinline__ void q_tile(const Args& a, int e, int off, int cnt, int slab, QLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, KB = I / 128;
  QSrc src;
  src.wr = make_rsrc(a.l2_w + (size_t)e * H * (I / 2), (size_t)H * (I / 2));
  src.xr = make_rsrc(a.inter_q, (size_t)a.P * I);
  src.ar = make_rsrc(a.inter_sf, (size_t)KB * a.P * 4);
  src.akb = 4u * (uint32_t)a.P;
  src.sr = make_rsrc(static_cast<const uint8_t*>(a.l2_sf) + (size_t)e * H * (I / 32), (size_t)H * (I / 32));
  src.wend = (uint32_t)((size_t)H * (I / 2));
  src.skb = a.wsf_kmajor ? 4u * (uint32_t)H : 4u;   // K-major weight scales: one K block's rows adjacent
  // output-column permutation of the eight-wave kernel (16 consecutive columns per lane)
  const auto grow = [&](int r) {
    const int m = r & 15, rt = (r >> 4) & 3;
    const int g = kWRows * slab + (r & ~63) + 16 * (m >> 2) + 4 * rt + (m & 3);
    return g < H ? g : g - 128;
  };
  q_offsets<NC>(src, L.rowsrc, I, grow, I / 2, a.wsf_kmajor ? 4 : I / 32, off, cnt, w, lane, a.w_paired != 0);
  src.wkb = a.w_paired ? 128 : 64;
  v4f acc[4][NC];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[rt][i] = v4f{0.f, 0.f, 0.f, 0.f};
  q_loop<NC>(L, src, 64 * w + lr, KB, acc, w, lane);

  // BF16 rows into the pair-ordered slot buffer; acc[rt][i][j] is output column
  // nbase + 16 lg + 4 rt + j of tile row 16 i + lr
  const int nbase = kWRows * slab + 64 * w;
  if (nbase >= H) return;                             // wave-uniform: H is a multiple of 128
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int col = 16 * i + lr;
    if (col >= cnt) continue;
    uint16_t* dst = a.slot + (size_t)L.aux[col] * H + nbase + 16 * lg;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4f o0 = acc[2 * h][i], o1 = acc[2 * h + 1][i];
      uint4 pk;
      pk.x = bf16_rne(o0[0]) | (bf16_rne(o0[1]) << 16);
      pk.y = bf16_rne(o0[2]) | (bf16_rne(o0[3]) << 16);
      pk.z = bf16_rne(o1[0]) | (bf16_rne(o1[1]) << 16);
      pk.w = bf16_rne(o1[2]) | (bf16_rne(o1[3]) << 16);
      *reinterpret_cast<uint4*>(dst + 8 * h) = pk;
    }
  }
}

// Persistent L2 item loop over the tiles [hdr[kHdrTilesQuad], hdr[kHdrTilesLarge]) of the large-M
// list, numbered in bands of kBand tiles as in k_large; workgroup slot `mine` (XCD-major) takes
// items r * G + mine.
__global__ __launch_bounds__(kQThreads, 2) void k_quad_l2(Args a) {
  __shared__ __attribute__((aligned(1024))) QLds L;
  const int t0 = a.hdr[kHdrTilesQuad];
  const int n_tiles = a.hdr[kHdrTilesLarge] - t0;
  const int n_slabs = (a.H + kWRows - 1) / kWRows;
  const int n_items = n_tiles * n_slabs;
  const int G = gridDim.x, per = G >> 3;
  const int mine = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int tid = threadIdx.x;
  for (int q = mine; q < n_items; q += G) {
    const ItemPos ip = band_pos(q, n_slabs, n_tiles, 0);
    const int2 td = a.tiles_l[t0 + ip.tile];
      const int e = tile_expert(td.x), cnt = tile_rows(td.x), off = td.y;
    lds_barrier();                               // the previous item is done with the LDS
    if (tid < kQTok) {
      const int pr = off + (tid < cnt ? tid : cnt - 1);
      L.rowsrc[tid] = pr;
      L.aux[tid] = a.pool_src[pr];
    }
    lds_barrier();
    switch ((cnt + 15) / 16) {
#define MM_QCASE(n) \
  case n: q_tile<n>(a, e, off, cnt, ip.slab, L); break;
      MM_QCASE(1) MM_QCASE(2) MM_QCASE(3) MM_QCASE(4) MM_QCASE(5)
      MM_QCASE(6) MM_QCASE(7) MM_QCASE(8) MM_QCASE(9) MM_QCASE(10)
#undef MM_QCASE
      default: break;                           // not a four-wave tile (cannot happen)
    }
  }
}

template <bool L1>
hipError_t launch_large(const Args& a, hipStream_t s) {
  if (a.max_tiles_l == 0 || a.tile_mode == 1) return hipSuccess;
  if (a.recipe == 0 && a.inter64 && !L1)
    hipLaunchKernelGGL((k_large<0, false, true>), dim3(a.large_grid), dim3(kThreads), 0, s, a);
  else if (a.recipe == 0) hipLaunchKernelGGL((k_large<0, L1>), dim3(a.large_grid), dim3(kThreads), 0, s, a);
  else if (a.recipe == 1) hipLaunchKernelGGL((k_large<1, L1>), dim3(a.large_grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_large<2, L1>), dim3(a.large_grid), dim3(kThreads), 0, s, a);
  if constexpr (!L1)
    if (a.recipe == 1 && a.quad) hipLaunchKernelGGL(k_quad_l2, dim3(a.quad_grid), dim3(kQThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_l1_large(const Args& a, hipStream_t s) { return launch_large<true>(a, s); }
hipError_t launch_l2_large(const Args& a, hipStream_t s) { return launch_large<false>(a, s); }

}  // namespace mm
