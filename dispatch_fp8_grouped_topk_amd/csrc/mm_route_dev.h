// Device code of dispatch (per-expert histogram, prefix scan, stable scatter + tile lists) and
// combine, shared by their stand-alone kernels (mm_route.hip) and the fused single-launch
// forward (mm_fused.hip).
//
// Dispatch follows the MegaMoE dispatch role (research report "MegaMoE on SM100/SM90",
// section 3.1; design page "MegaMoE SM90 Implementation Design", section 9.2): count the
// rows each expert receives, lay the experts' pools out back to back and record, per pool
// row, its source {token, top-k slot}.  The pages fill pools with racing atomics; here a
// pool keeps row-major (token, slot) order so the result is unique and repeatable: a pair's
// rank is (pairs of the same expert in earlier dispatch blocks) + (earlier pairs of the same
// expert inside its block), both computed from positions, never from atomic return order.
//
// Combine follows the design page's combine reduce (section 11.2): for each token, sum its
// active top-k BF16 rows in float32 in ascending slot order and store BF16.
//
// The workgroup-wide functions are written for NT threads (a multiple of 256): every thread
// of the workgroup calls them (they hold workgroup barriers), and threads past the work they
// cover take part in the barriers only.
#pragma once

#include "mm_common.h"

namespace mm {

// ---------------------------------------------------------------------------------- count
// Dispatch block b (256 consecutive pairs): LDS histogram of expert ids (written out as the
// block's row of blk[NB][E]) and each pair's rank among same-expert pairs of the block.
// LDS: hist[E], ids[256], inv_w[4].  Ends with a barrier, so the LDS can be reused at once.
template <int NT>
__device__ __forceinline__ void route_count_block(const Args& a, int b, int* hist, int* ids, int* inv_w) {
  const int tid = threadIdx.x;
  const bool act = tid < kRouteBlock;
  const int pair = b * kRouteBlock + tid;
  for (int i = tid; i < a.E; i += NT) hist[i] = 0;
  const int e = act && pair < a.P ? a.topk_idx[pair] : -1;
  const bool valid = e >= 0 && e < a.E;
  const bool invalid = act && pair < a.P && e >= a.E;
  if (act) ids[tid] = valid ? e : -1;
  __syncthreads();
  int rank = 0;
  if (valid) {
    for (int t = 0; t < tid; ++t) rank += (ids[t] == e);
    atomicAdd(&hist[e], 1);
  }
  const unsigned long long inv = __ballot(invalid);
  if (act && (tid & 63) == 0) inv_w[tid >> 6] = __popcll(inv);
  __syncthreads();
  for (int i = tid; i < a.E; i += NT) a.blk[(size_t)b * a.E + i] = hist[i];
  if (act && pair < a.P) a.pair_pos[pair] = valid ? rank : -1;
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kRouteBlock / 64; ++w) s += inv_w[w];
    a.blk_inv[b] = s;
  }
  __syncthreads();
}

// Inclusive scans of N ints per thread at once over an NT-thread workgroup (one round of
// barriers for all N); totals of each written to total[0..N).  sh must hold 32 * N ints.
template <int N, int NT>
__device__ __forceinline__ void block_scan_n(int v[N], int* sh, int total[N]) {
  static_assert(NT % 64 == 0 && NT <= 1024, "up to 16 waves");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int o = __shfl_up(v[n], d, 64);
      if (lane >= d) v[n] += o;
    }
  }
  if (lane == 63)
#pragma unroll
    for (int n = 0; n < N; ++n) sh[n * 32 + w] = v[n];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      int x = lane < NW ? sh[n * 32 + lane] : 0;
      for (int d = 1; d < 16; d <<= 1) {
        const int o = __shfl_up(x, d, 64);
        if (lane >= d) x += o;
      }
      if (lane < 16) sh[n * 32 + 16 + lane] = x;
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    v[n] += w > 0 ? sh[n * 32 + 16 + w - 1] : 0;
    total[n] = sh[n * 32 + 16 + NW - 1];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------- scan
// LDS of route_scan: s_count[kMaxExperts], part[NT / 256][256], sh[32 (kMaxNGClasses + 2)],
// s_class_base[kMaxNGClasses + 1].
struct ScanLds {
  int* s_count;
  int* part;
  int* sh;
  int* s_class_base;
};

// One workgroup: per-expert totals and per-block bases (in place in blk), expert offsets, the
// invalid-id total and the tile lists of both GEMM tile classes.
template <int NT>
__device__ __forceinline__ void route_scan(const Args& a, const ScanLds& S) {
  constexpr int NQ = NT / 256;                 // parts of the block range per expert
  int* s_count = S.s_count;
  int* sh = S.sh;
  int* s_class_base = S.s_class_base;
  const int tid = threadIdx.x;
  const int E = a.E, NB = a.NB;

  // 1. totals and block bases; threads (el, q): expert e0+el, part q of the blocks
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int el = tid & 255, q = tid >> 8;
    const int e = e0 + el;
    const int b_lo = (q * NB) / NQ, b_hi = ((q + 1) * NB) / NQ;
    int s = 0;
    if (e < E) {
#pragma unroll 8
      for (int b = b_lo; b < b_hi; ++b) s += a.blk[(size_t)b * E + e];
    }
    S.part[q * 256 + el] = s;
    __syncthreads();
    if (e < E) {
      int run = 0;
      for (int qq = 0; qq < q; ++qq) run += S.part[qq * 256 + el];
#pragma unroll 8
      for (int b = b_lo; b < b_hi; ++b) {
        const int c = a.blk[(size_t)b * E + e];
        a.blk[(size_t)b * E + e] = run;
        run += c;
      }
      if (q == NQ - 1) s_count[e] = run;
    }
    __syncthreads();
  }

  // 2. offsets (exclusive scan of counts) and the tile lists.  Large-M tiles are ordered by the
  // column-group count of their expert's first tile, largest first (the GEMM kernels deal them
  // out round-robin, so the costliest items start first and the cheapest fill the tail), and by
  // expert inside a class, so an expert's tiles stay adjacent.
  auto large_of = [&](int c) {
    if (a.tile_mode == 1) return false;
    if (a.tile_mode == 2) return c > 0;
    return c > 0 && c >= a.large_min_rows;
  };
  int carry = 0, carry_s = 0, carry_l = 0;
  if (E <= NT) {
    // one expert per thread: one scan of the counts, small tiles and large tiles per class gives
    // the offsets, the tile positions and, from the class totals, the class bases
    const int e = tid;
    const int c = e < E ? s_count[e] : 0;
    const bool large = large_of(c);
    const int nts = large ? 0 : (c + kSmallRows - 1) / kSmallRows;
    const int ntl = large ? large_tiles(c) : 0;
    const int cls = ntl ? large_first_ng(c) : 0;
    int v[kMaxNGClasses + 2], tv[kMaxNGClasses + 2];
    v[0] = c;
    v[1] = nts;
#pragma unroll
    for (int g = 0; g < kMaxNGClasses; ++g) v[2 + g] = cls == g + 1 ? ntl : 0;
    block_scan_n<kMaxNGClasses + 2, NT>(v, sh, tv);
    // class g starts after all classes above g
    int bl = 0, run = 0, base_quad = 0, base_wide = 0;
#pragma unroll
    for (int g = kMaxNGClasses; g >= 1; --g) {
      if (g == cls) bl = run + v[1 + g] - ntl;
      if (g == kQuadMaxNG) base_quad = run;
      if (g == kWideMaxNG) base_wide = run;
      run += tv[1 + g];
    }
    if (e < E) {
      a.count[e] = c;
      if (a.recv_stats) a.recv_stats[e] += c;
      a.offset[e] = v[0] - c;
      const int bs = v[1] - nts;
      for (int i = 0; i < nts; ++i) a.tiles_s[bs + i] = make_int2(e, i * kSmallRows);
      for (int i = 0; i < ntl; ++i) {
        const int m0 = large_tile_start(c, i);
        const int m1 = i + 1 < ntl ? large_tile_start(c, i + 1) : c;
        a.tiles_l[bl + i] = make_int2(e | ((m1 - m0) << 16) | (ntl == 1 ? kTileSingle : 0), v[0] - c + m0);
      }
    }
    if (tid == 0) {
      a.hdr[kHdrTilesQuad] = base_quad;        // tiles of the classes above kQuadMaxNG
      a.hdr[kHdrTilesWide] = base_wide;        // tiles of the classes above kWideMaxNG
    }
    carry = tv[0];
    carry_s = tv[1];
    carry_l = run;
  } else {                                     // experts in several passes of NT
    if (tid == 0)
      for (int g = 0; g <= kMaxNGClasses; ++g) s_class_base[g] = 0;
    __syncthreads();
    for (int e0 = 0; e0 < E; e0 += NT) {         // tiles per class
      const int e = e0 + tid;
      const int c = e < E ? s_count[e] : 0;
      const int ntl = large_of(c) ? large_tiles(c) : 0;
      const int cls = ntl ? large_first_ng(c) : 0;
      int v[kMaxNGClasses], tot[kMaxNGClasses];
#pragma unroll
      for (int g = 0; g < kMaxNGClasses; ++g) v[g] = cls == g + 1 ? ntl : 0;
      block_scan_n<kMaxNGClasses, NT>(v, sh, tot);
      if (tid == 0)
        for (int g = 1; g <= kMaxNGClasses; ++g) s_class_base[g] += tot[g - 1];
    }
    __syncthreads();
    if (tid == 0) {                              // class g starts after all classes above g
      int run = 0;
      for (int g = kMaxNGClasses; g >= 1; --g) {
        const int n = s_class_base[g];
        s_class_base[g] = run;
        run += n;
      }
      s_class_base[0] = run;                     // total large tiles
      a.hdr[kHdrTilesQuad] = s_class_base[kQuadMaxNG];   // tiles of the classes above kQuadMaxNG
      a.hdr[kHdrTilesWide] = s_class_base[kWideMaxNG];   // tiles of the classes above kWideMaxNG
    }
    __syncthreads();
    for (int e0 = 0; e0 < E; e0 += NT) {
      const int e = e0 + tid;
      const int c = e < E ? s_count[e] : 0;
      const bool large = large_of(c);
      const int nts = large ? 0 : (c + kSmallRows - 1) / kSmallRows;
      const int ntl = large ? large_tiles(c) : 0;
      const int cls = ntl ? large_first_ng(c) : 0;
      int v[kMaxNGClasses + 2], tv[kMaxNGClasses + 2];
      v[0] = c;
      v[1] = nts;
#pragma unroll
      for (int g = 0; g < kMaxNGClasses; ++g) v[2 + g] = cls == g + 1 ? ntl : 0;
      block_scan_n<kMaxNGClasses + 2, NT>(v, sh, tv);
      const int inc = v[0], tot = tv[0], inc_s = v[1], tot_s = tv[1];
      int bl = 0;
      if (cls > 0) bl = s_class_base[cls] + v[1 + cls] - ntl;
      __syncthreads();
      if (tid == 0)
        for (int g = 1; g <= kMaxNGClasses; ++g) s_class_base[g] += tv[1 + g];
      __syncthreads();
      if (e < E) {
        a.count[e] = c;
        if (a.recv_stats) a.recv_stats[e] += c;
        a.offset[e] = carry + inc - c;
        const int bs = carry_s + inc_s - nts;
        for (int i = 0; i < nts; ++i) a.tiles_s[bs + i] = make_int2(e, i * kSmallRows);
        for (int i = 0; i < ntl; ++i) {
          const int m0 = large_tile_start(c, i);
          const int m1 = i + 1 < ntl ? large_tile_start(c, i + 1) : c;
          a.tiles_l[bl + i] = make_int2(e | ((m1 - m0) << 16) | (ntl == 1 ? kTileSingle : 0), carry + inc - c + m0);
        }
      }
      carry += tot;
      carry_s += tot_s;
    }
    carry_l = s_class_base[0];
  }
  // ids >= E over all dispatch blocks: every thread sums a strided share of the per-block counts
  // (independent loads in flight), then one workgroup reduction
  int inv = 0;
  for (int b = tid; b < NB; b += NT) inv += a.blk_inv[b];
  int iv[1] = {inv}, itot[1];
  block_scan_n<1, NT>(iv, sh, itot);
  if (tid == 0) {
    a.offset[E] = carry;
    a.hdr[kHdrTilesSmall] = carry_s;
    a.hdr[kHdrTilesLarge] = carry_l;
    a.hdr[kHdrInvalid] = itot[0];
  }
}

// ---------------------------------------------------------------------------------- scatter
// Pair `pair` (of dispatch block pair / 256) to its pool row: pair_pos, pool_src, w_pool.
// Returns the pool row, or -1 for a masked or invalid slot.
__device__ __forceinline__ int route_scatter_pair(const Args& a, int pair) {
  const int r = a.pair_pos[pair];
  if (r < 0) return -1;
  const int e = a.topk_idx[pair];
  const int pos = a.offset[e] + a.blk[(size_t)(pair / kRouteBlock) * a.E + e] + r;
  a.pair_pos[pair] = pos;
  a.pool_src[pos] = pair;
  a.w_pool[pos] = a.topk_w[pair];
  return pos;
}

// ------------------------------------------------------------------------ pool-order scales
// x_sf_pool[kb][r] = the x_sf word of K block kb of pool row r's token (an f32 scale, or the
// four UE8M0 codes of the block), K-major, so that the large-M L1 kernel reads one K block's
// scales of a tile's rows from one contiguous kilobyte instead of one scattered word per row.
// One call copies K blocks kb0 .. kb0 + 7 of pool row r, whose token is t.
__device__ __forceinline__ void pool_scales_row_of(const Args& a, int r, int t, int kb0) {
  const int KB = a.H / 128;
  const uint32_t* src = static_cast<const uint32_t*>(a.x_sf) + (size_t)t * KB + kb0;
  uint32_t* dst = static_cast<uint32_t*>(a.x_sf_pool) + (size_t)kb0 * a.P + r;
  uint32_t v[8];
  if ((KB & 3) == 0) {                         // rows of whole 16-byte chunks
    const uint4 lo = *reinterpret_cast<const uint4*>(src);
    const uint4 hi = kb0 + 4 < KB ? *reinterpret_cast<const uint4*>(src + 4) : lo;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = kb0 + j < KB ? src[j] : 0u;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (kb0 + j < KB) dst[(size_t)j * a.P] = v[j];
}

// The same for pool row r < offset[E], its token read from pool_src.
__device__ __forceinline__ void pool_scales_row(const Args& a, int r, int kb0) {
  pool_scales_row_of(a, r, a.pool_src[r] / a.k, kb0);
}

// ---------------------------------------------------------------------------------- combine
// Chunk idx of the output: 8 columns of one token (idx = token * H / 8 + column / 8).  The slot
// rows of the token are fetched 8 top-k slots at a time (their pair_pos words first, then every
// active row's 16 bytes), so each thread keeps several loads in flight; the sum is still taken
// in ascending slot order.  Slot rows are read and y written with the non-temporal policy.
__device__ __forceinline__ void combine_chunk(const Args& a, long idx) {
  const int cpt = a.H / 8;                     // 8-column chunks per token
  const int t = (int)(idx / cpt);
  const int n0 = (int)(idx - (long)t * cpt) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < a.k; j0 += 8) {
    int pp[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) pp[jj] = j0 + jj < a.k ? a.pair_pos[(size_t)t * a.k + j0 + jj] : -1;
    v4i v[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      v[jj] = v4i{0, 0, 0, 0};
      if (pp[jj] >= 0)                         // masked or invalid slots contribute nothing
        v[jj] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(a.slot + ((size_t)t * a.k + j0 + jj) * a.H + n0));
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (pp[jj] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = (uint32_t)v[jj][i];
        acc[2 * i] += __uint_as_float(w << 16);
        acc[2 * i + 1] += __uint_as_float(w & 0xFFFF0000u);
      }
    }
  }
  v4i o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (int)(bf16_rne(acc[2 * i]) | (bf16_rne(acc[2 * i + 1]) << 16));
  __builtin_nontemporal_store(o, reinterpret_cast<v4i*>(a.y + (size_t)t * a.H + n0));   // read-once rows, write-once y
}

}  // namespace mm
