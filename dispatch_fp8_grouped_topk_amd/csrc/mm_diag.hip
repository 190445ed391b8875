// Diagnostic: 16 x 16 block dot products computed with exactly the MFMA instruction, operand
// layout and scale encoding the grouped GEMMs use for one 128-K block, so that tests can measure
// how far the matrix core's block sum lies from the exact sum of its products (the tolerance of
// the intermediate codes is derived from that bound).
#include "mm_common.h"

namespace mm {
namespace {

// One wave per tile: D[m][n] = sum_k A[m][k] B[n][k] over a 128-long K block, A 16 rows
// (E4M3 bytes, or E2M1 nibbles packed two per byte with the low nibble the even K index),
// B 16 rows of E4M3 bytes.  fmt 0: unit scales (the float-scale recipe's MFMA, promoted
// outside); fmt 1: E2M1 x E4M3 with UE8M0 scales per (row, 32 K); fmt 2: E4M3 x E4M3 with UE8M0
// scales per (row, 32 K).
__global__ __launch_bounds__(64) void k_diag_mfma(int fmt, const uint8_t* __restrict__ a,
                                                  const uint8_t* __restrict__ b,
                                                  const uint8_t* __restrict__ sa,
                                                  const uint8_t* __restrict__ sb, float* __restrict__ out) {
  const int tile = blockIdx.x, lane = threadIdx.x, row = lane & 15, lg = lane >> 4;
  const int a_row_bytes = fmt == 1 ? 64 : 128;
  const uint8_t* ar = a + ((size_t)tile * 16 + row) * a_row_bytes;
  const uint8_t* br = b + ((size_t)tile * 16 + row) * 128;
  const v8i B = load_fp8_operand(br, lg);
  v4f d = {0.f, 0.f, 0.f, 0.f};
  if (fmt == 0) {
    d = mfma_fp8(load_fp8_operand(ar, lg), B);
  } else {
    // the scale of (row m, 32-K group g) is read from lane m + 16 g
    const int s_a = sa[((size_t)tile * 16 + row) * 4 + lg];
    const int s_b = sb[((size_t)tile * 16 + row) * 4 + lg];
    if (fmt == 1) d = mfma_fp4w_fp8(load_fp4_operand(ar, lg), B, d, s_a, s_b);
    else d = mfma_fp8_scaled(load_fp8_operand(ar, lg), B, d, s_a, s_b);
  }
  // lane l holds column n = l % 16 and rows m = 4 (l / 16) .. + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) out[(size_t)tile * 256 + (4 * lg + i) * 16 + row] = d[i];
}

}  // namespace

hipError_t launch_diag_mfma(int fmt, const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                            float* out, int n_tiles, hipStream_t s) {
  if (n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_diag_mfma, dim3(n_tiles), dim3(64), 0, s, fmt, a, b, sa, sb, out);
  return hipGetLastError();
}

}  // namespace mm
