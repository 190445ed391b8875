// Dispatch (per-expert histogram, prefix scan, stable scatter + tile lists) and combine.
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
#include "mm_common.h"

namespace mm {

// ---------------------------------------------------------------------------------- count
// One workgroup per 256 consecutive pairs: LDS histogram of expert ids (written out as the
// block's row of blk[NB][E]) and each pair's rank among same-expert pairs of the block.
__global__ __launch_bounds__(kRouteBlock) void k_route_count(Args a) {
  extern __shared__ int hist[];             // [E]
  __shared__ int ids[kRouteBlock];
  __shared__ int inv_w[kRouteBlock / 64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int pair = b * kRouteBlock + tid;
  for (int i = tid; i < a.E; i += kRouteBlock) hist[i] = 0;
  int e = pair < a.P ? a.topk_idx[pair] : -1;
  const bool valid = e >= 0 && e < a.E;
  const bool invalid = pair < a.P && e >= a.E;
  ids[tid] = valid ? e : -1;
  __syncthreads();
  int rank = 0;
  if (valid) {
    for (int t = 0; t < tid; ++t) rank += (ids[t] == e);
    atomicAdd(&hist[e], 1);
  }
  unsigned long long inv = __ballot(invalid);
  if ((tid & 63) == 0) inv_w[tid >> 6] = __popcll(inv);
  __syncthreads();
  for (int i = tid; i < a.E; i += kRouteBlock) a.blk[(size_t)b * a.E + i] = hist[i];
  if (pair < a.P) a.pair_pos[pair] = valid ? rank : -1;
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kRouteBlock / 64; ++w) s += inv_w[w];
    a.blk_inv[b] = s;
  }
}

// Inclusive scans of N ints per thread at once over a 1024-thread workgroup (one round of
// barriers for all N); totals of each written to total[0..N).  sh must hold 32 * N ints.
template <int N>
__device__ void block_scan_1024_n(int v[N], int* sh, int total[N]) {
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
      int x = lane < 16 ? sh[n * 32 + lane] : 0;
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
    total[n] = sh[n * 32 + 31];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------- scan
// One workgroup of 1024 threads: per-expert totals and per-block bases (in place in blk),
// expert offsets, the invalid-id total and the tile lists of both GEMM tile classes.
__global__ __launch_bounds__(1024) void k_route_scan(Args a) {
  __shared__ int s_count[kMaxExperts];
  __shared__ int part[4][256];
  __shared__ int sh[32 * (kMaxNGClasses + 2)];
  const int tid = threadIdx.x;
  const int E = a.E, NB = a.NB;

  // 1. totals and block bases; threads (el, q): expert e0+el, quarter q of the blocks
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int el = tid & 255, q = tid >> 8;
    const int e = e0 + el;
    const int b_lo = (q * NB) >> 2, b_hi = ((q + 1) * NB) >> 2;
    int s = 0;
    if (e < E) {
#pragma unroll 8
      for (int b = b_lo; b < b_hi; ++b) s += a.blk[(size_t)b * E + e];
    }
    part[q][el] = s;
    __syncthreads();
    if (e < E) {
      int run = 0;
      for (int qq = 0; qq < q; ++qq) run += part[qq][el];
#pragma unroll 8
      for (int b = b_lo; b < b_hi; ++b) {
        const int c = a.blk[(size_t)b * E + e];
        a.blk[(size_t)b * E + e] = run;
        run += c;
      }
      if (q == 3) s_count[e] = run;
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
  __shared__ int s_class_base[kMaxNGClasses + 1];
  if (tid == 0)
    for (int g = 0; g <= kMaxNGClasses; ++g) s_class_base[g] = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 1024) {       // tiles per class
    const int e = e0 + tid;
    const int c = e < E ? s_count[e] : 0;
    const int ntl = large_of(c) ? large_tiles(c) : 0;
    const int cls = ntl ? large_first_ng(c) : 0;
    int v[kMaxNGClasses], tot[kMaxNGClasses];
#pragma unroll
    for (int g = 0; g < kMaxNGClasses; ++g) v[g] = cls == g + 1 ? ntl : 0;
    block_scan_1024_n<kMaxNGClasses>(v, sh, tot);
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
  }
  __syncthreads();
  int carry = 0, carry_s = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
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
    block_scan_1024_n<kMaxNGClasses + 2>(v, sh, tv);
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
  const int carry_l = s_class_base[0];
  // ids >= E over all dispatch blocks: every thread sums a strided share of the per-block counts
  // (independent loads in flight), then one workgroup reduction
  int inv = 0;
  for (int b = tid; b < NB; b += 1024) inv += a.blk_inv[b];
  int iv[1] = {inv}, itot[1];
  block_scan_1024_n<1>(iv, sh, itot);
  if (tid == 0) {
    a.offset[E] = carry;
    a.hdr[kHdrTilesSmall] = carry_s;
    a.hdr[kHdrTilesLarge] = carry_l;
    a.hdr[kHdrInvalid] = itot[0];
  }
}

// ---------------------------------------------------------------------------------- scatter
__global__ __launch_bounds__(kRouteBlock) void k_route_scatter(Args a) {
  const int b = blockIdx.x;
  const int pair = b * kRouteBlock + threadIdx.x;
  if (pair >= a.P) return;
  const int r = a.pair_pos[pair];
  if (r < 0) return;
  const int e = a.topk_idx[pair];
  const int pos = a.offset[e] + a.blk[(size_t)b * a.E + e] + r;
  a.pair_pos[pair] = pos;
  a.pool_src[pos] = pair;
  a.w_pool[pos] = a.topk_w[pair];
}

// ------------------------------------------------------------------------ pool-order scales
// x_sf_pool[kb][r] = the x_sf word of K block kb of pool row r's token (an f32 scale, or the
// four UE8M0 codes of the block), K-major, so that the large-M L1 kernel reads one K block's
// scales of a tile's rows from one contiguous kilobyte instead of one scattered word per row.
// grid (ceil(P / 256), ceil(KB / 8)); a thread copies 8 K blocks of one pool row.
__global__ __launch_bounds__(256) void k_pool_scales(Args a) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.offset[a.E]) return;
  const int KB = a.H / 128, kb0 = blockIdx.y * 8;
  const int t = a.pool_src[r] / a.k;
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

hipError_t launch_route(const Args& a, hipStream_t s) {
  if (a.P == 0) return hipSuccess;
  hipLaunchKernelGGL(k_route_count, dim3(a.NB), dim3(kRouteBlock), (size_t)a.E * sizeof(int), s, a);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(k_route_scatter, dim3(a.NB), dim3(kRouteBlock), 0, s, a);
  if (a.max_tiles_l > 0 && a.tile_mode != 1)
    hipLaunchKernelGGL(k_pool_scales, dim3((a.P + 255) / 256, (a.H / 128 + 7) / 8), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------- combine
// One thread per (token, 8 output columns), grid-stride over all of them.  The slot rows of a
// token are fetched 8 top-k slots at a time (their pair_pos words first, then every active
// row's 16 bytes), so each thread keeps several loads in flight; the sum is still taken in
// ascending slot order.
__global__ __launch_bounds__(256) void k_combine(Args a) {
  const int cpt = a.H / 8;                       // 8-column chunks per token
  const long total = (long)a.T * cpt;
  for (long idx = (long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long)gridDim.x * 256) {
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
}

hipError_t launch_combine(const Args& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const long total = (long)a.T * (a.H / 8);
  long blocks = (total + 255) / 256;
  blocks = blocks < 8192 ? blocks : 8192;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Weight-scale transform for the per-32 recipes, run once when the weights are loaded (the
// counterpart of the pages' model-load weight transform, design page section 15, which also
// re-lays the UE8M0 scale factors out for the kernels' loads): the caller's [E][rows][K/32] codes
// become [E][K/128][rows] words of four codes, so the GEMMs fetch one K block's scales of 64
// consecutive rows as 256 contiguous bytes.  A 64-row x 32-word tile per workgroup goes through
// LDS, so both the reads and the writes are coalesced.
__global__ __launch_bounds__(256) void k_sf_kmajor(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                   int rows, int KB, int row_tiles, int kb_tiles) {
  __shared__ uint32_t tile[64][33];
  const int b = blockIdx.x;
  const int e = b / (row_tiles * kb_tiles), rem = b - e * row_tiles * kb_tiles;
  const int r0 = 64 * (rem / kb_tiles), k0 = 32 * (rem % kb_tiles);
  const size_t base = (size_t)e * rows * KB;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;      // 32 x 8
  for (int r = ty; r < 64; r += 8)
    if (r0 + r < rows && k0 + tx < KB) tile[r][tx] = in[base + (size_t)(r0 + r) * KB + k0 + tx];
  __syncthreads();
  const int ox = threadIdx.x & 63, oy = threadIdx.x >> 6;      // 64 x 4
  for (int k = oy; k < 32; k += 4)
    if (r0 + ox < rows && k0 + k < KB) out[base + (size_t)(k0 + k) * rows + r0 + ox] = tile[ox][k];
}

hipError_t launch_sf_kmajor(const uint32_t* in, uint32_t* out, int E, int rows, int KB, hipStream_t s) {
  const int row_tiles = (rows + 63) / 64, kb_tiles = (KB + 31) / 32;
  const long blocks = (long)E * row_tiles * kb_tiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sf_kmajor, dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, KB, row_tiles, kb_tiles);
  return hipGetLastError();
}

}  // namespace mm
