// Dispatch (per-expert histogram, prefix scan, stable scatter + tile lists), combine and the
// per-32 recipes' weight-scale transform.
#include "mm_route_dev.h"

namespace mm {

// Stand-alone kernels of dispatch and combine over the device code in mm_route_dev.h.

// ---------------------------------------------------------------------------------- count
// One workgroup per 256 consecutive pairs.
__global__ __launch_bounds__(kRouteBlock) void k_route_count(Args a) {
  extern __shared__ int hist[];             // [E]
  __shared__ int ids[kRouteBlock];
  __shared__ int inv_w[kRouteBlock / 64];
  route_count_block<kRouteBlock>(a, blockIdx.x, hist, ids, inv_w);
}

// ---------------------------------------------------------------------------------- scan
// One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void k_route_scan(Args a) {
  __shared__ int s_count[kMaxExperts];
  __shared__ int part[4 * 256];
  __shared__ int sh[32 * (kMaxNGClasses + 2)];
  __shared__ int s_class_base[kMaxNGClasses + 1];
  route_scan<1024>(a, ScanLds{s_count, part, sh, s_class_base});
}

// ---------------------------------------------------------------------------------- scatter
__global__ __launch_bounds__(kRouteBlock) void k_route_scatter(Args a) {
  const int pair = blockIdx.x * kRouteBlock + threadIdx.x;
  if (pair < a.P) route_scatter_pair(a, pair);
}

// ------------------------------------------------------------------------ pool-order scales
// grid (ceil(P / 256), ceil(KB / 8)); a thread copies 8 K blocks of one pool row.
__global__ __launch_bounds__(256) void k_pool_scales(Args a) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < a.offset[a.E]) pool_scales_row(a, r, blockIdx.y * 8);
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
// One thread per (token, 8 output columns), grid-stride over all of them.
__global__ __launch_bounds__(256) void k_combine(Args a) {
  const long total = (long)a.T * (a.H / 8);
  for (long idx = (long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long)gridDim.x * 256)
    combine_chunk(a, idx);
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

// The row-pair layout of E2M1 weights (MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED): row pair q (rows 2q, 2q+1
// of the row-major [pairs * 2][KB * 64] bytes) becomes [KB][2][64] bytes at q * KB * 128, so each
// 128-K block of the two rows is one 128-byte line.  One thread per 16-byte piece: reads of a
// wave cover whole 64-byte row blocks, writes whole 128-byte lines.
__global__ __launch_bounds__(256) void k_e2m1_pairs(const uint4* __restrict__ in, uint4* __restrict__ out,
                                                     size_t pairs, int KB) {
  const size_t n = pairs * (size_t)KB * 8;                    // 16-byte pieces
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t q = i / ((size_t)KB * 8);
    const int r = (int)(i - q * (size_t)KB * 8);              // piece within the pair's output
    const int kb = r >> 3, h = (r >> 2) & 1, c = r & 3;
    out[i] = in[((2 * q + h) * (size_t)KB + kb) * 4 + c];
  }
}

hipError_t launch_e2m1_pairs(const uint8_t* in, uint8_t* out, size_t pairs, int KB, hipStream_t s) {
  const size_t n = pairs * (size_t)KB * 8;
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(k_e2m1_pairs, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const uint4*>(in),
                     reinterpret_cast<uint4*>(out), pairs, KB);
  return hipGetLastError();
}

hipError_t launch_sf_kmajor(const uint32_t* in, uint32_t* out, int E, int rows, int KB, hipStream_t s) {
  const int row_tiles = (rows + 63) / 64, kb_tiles = (KB + 31) / 32;
  const long blocks = (long)E * row_tiles * kb_tiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sf_kmajor, dim3((unsigned)blocks), dim3(256), 0, s, in, out, rows, KB, row_tiles, kb_tiles);
  return hipGetLastError();
}

}  // namespace mm
