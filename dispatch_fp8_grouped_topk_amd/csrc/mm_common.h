// Internal definitions shared by the HIP translation units of libmegamoe.
// gfx950 (CDNA4) only: 64-wide wavefronts, FP8/FP4 MFMA with E8M0 block scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_policy.h"

namespace mm {

// ------------------------------------------------------------------------------------------
// Limits and tile geometry
constexpr int kMaxExperts = 8192;     // LDS arrays of the scan kernel hold one int per expert
constexpr int kMaxTopk = 64;
constexpr int kRouteBlock = 256;      // pairs per dispatch workgroup
constexpr int kSmallRows = 64;        // pool rows per small-M tile (4 MFMA column groups of 16)
// Auto mode: experts with at least this many rows use the large-M class.  Measured on MI355X,
// the persistent large-M kernel (three-deep operand ring for small tiles) is at least as fast
// as the small-M kernels down to single-row experts, so it takes every expert.
constexpr int kLargeMinRows = 1;
constexpr int kL1SlabCh = 128;        // intermediate channels per L1 workgroup (gate+up = 256 rows)
constexpr int kL2SlabRows = 256;      // output columns (w2 rows) per L2 workgroup
constexpr int kMaxNGClasses = 8;      // large-M tiles: 1..8 column groups of 16 per wave
constexpr int kMaxKBlocks = 128;      // H/128 and I/128 limit (LDS scale staging)

// Large-M tile-list entry, .x: expert (bits 0-15), rows (bits 16-24), bit 30 set when the tile is
// its expert's only one (each weight line is then read by exactly one item per slab); .y: the
// tile's first pool row.
constexpr int kTileSingle = 1 << 30;
__host__ __device__ inline int tile_expert(int x) { return x & 0xFFFF; }
__host__ __device__ inline int tile_rows(int x) { return (x >> 16) & 0x1FF; }
__host__ __device__ inline bool tile_single(int x) { return (x & kTileSingle) != 0; }

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Workspace header words.
// kHdrTilesQuad: the first large-M tile (in list order) whose expert's first tile has at most
// kQuadMaxNG column groups per wave; with the MXFP4 recipe, the L2 GEMM of the tiles from there
// on runs in the four-wave kernel, two workgroups per CU.
// kHdrFusedFault: set by the fused forward when one of its bounded waits ran out (its results are
// then invalid).
enum { kHdrInvalid = 0, kHdrTilesSmall = 1, kHdrTilesLarge = 2, kHdrTilesQuad = 3, kHdrFusedFault = 4, kHdrTilesWide = 5,
       kHdrWords = 64 };
constexpr int kQuadMaxNG = 5;
// kHdrTilesWide: the first large-M tile whose expert's first tile has at most kWideMaxNG column
// groups per wave; with the MXFP4 recipe the L1 GEMM runs the tiles from there as wide items.
constexpr int kWideMaxNG = 5;

struct Args {
  // inputs
  const uint8_t* x;
  const void* x_sf;
  const int32_t* topk_idx;
  const float* topk_w;
  const uint8_t* l1_w;
  const void* l1_sf;
  const uint8_t* l2_w;
  const void* l2_sf;
  uint16_t* y;
  int32_t* recv_stats;  // [E] cumulative per-expert received rows (NULL: none)
  // workspace regions
  int32_t* hdr;
  int32_t* count;       // [E]
  int32_t* offset;      // [E+1]
  int32_t* blk;         // [NB][E] per-dispatch-block counts, then bases
  int32_t* blk_inv;     // [NB]
  int32_t* pair_pos;    // [P]
  int32_t* pool_src;    // [P]
  float* w_pool;        // [P]
  int2* tiles_s;        // small-M tile list {expert, first pool row}
  int2* tiles_l;        // large-M tile list {expert | rows << 16 | kTileSingle, first pool row}
  void* x_sf_pool;      // [H/128][P] words: the x_sf word of each K block of each pool row
  uint8_t* inter_q;     // [P, I]
  void* inter_sf;       // [I/128][P] words: f32 | 4 x UE8M0 (K-major, like x_sf_pool)
  uint16_t* slot;       // [P, H] bf16, row = pair
  int32_t* tile_done;   // fused forward: [max_tiles_l] L1 slabs stored per large-M tile, then the
                        // number of L1 items stored
  // sizes
  int T, H, I, E, k, P, NB;
  int recipe;
  float clamp;          // <= 0: none
  int clamp_inputs;     // 1: clamp gate and up before SiLU instead of silu(g)*u
  int precise_silu;     // 1: SiLU with expf and an IEEE division (else hardware exp / rcp)
  int tile_mode;        // 0 auto, 1 small only, 2 large only
  int large_min_rows;   // auto mode: experts with at least this many rows use the large class
  int max_tiles_s, max_tiles_l;
  int large_grid;       // workgroups of the persistent large-M kernels (multiple of 8)
  int quad;             // 1: MXFP4 L2 tiles of at most 160 rows go to the four-wave kernel
  int quad_grid;        // its workgroups (two per CU, multiple of 8)
  int w_paired;         // MXFP4: E2M1 weights in the row-pair layout (one 128-byte line per K block of two rows)
  int wsf_kmajor;       // per-32 recipes: weight scales as [E][K/128][rows] words (4 UE8M0 codes
                        // of one 128-K block of one row), else [E][rows][K/32] bytes
  int inter64;          // FP8 recipe: the intermediate has a float scale per 64 channels, inter_sf
                        // [I/64][P]; L2 sums each 128-K block as two 64-K halves
};

// ------------------------------------------------------------------------------------------
// Numeric helpers (device)

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Four floats -> four OCP E4M3FN bytes (element 0 in the low byte), round to nearest even.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// silu(g) = g / (1 + exp(-g)) with the hardware exp and reciprocal instructions (float32 to a
// few ulp); where exp(-g) overflows (g below about -88) the result is -0, as in the exact form.
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// silu(g) * u with the problem's clamp c > 0: on g and u before SiLU (inputs) or on the product;
// kPrecise: SiLU with the device library's expf and an IEEE division.  The caller picks the
// instantiation with one wave-uniform branch around its whole epilogue, so the default path
// carries no trace of the precise one.
template <bool kPrecise>
__device__ __forceinline__ float swiglu_f32(float g, float u, float c, bool clamp_in, bool clamp_out) {
  if (clamp_in) {
    g = fminf(fmaxf(g, -c), c);
    u = fminf(fmaxf(u, -c), c);
  }
  float s = (kPrecise ? g / (1.0f + expf(-g)) : silu_f32(g)) * u;
  if (clamp_out) s = fminf(fmaxf(s, -c), c);
  return s;
}

// E4M3 codes of four values divided by sf = amax / 448 (amax > 0): multiplied by m = 448 / amax,
// one IEEE division per group instead of one per value (the product is within about one ulp of
// the quotient before the E4M3 rounding), or divided by sf where m overflows (amax < ~2^-119).
__device__ __forceinline__ uint32_t e4m3_scaled4(float a, float b, float c, float d, float m, float sf) {
  if (__builtin_isfinite(m)) return pack_fp8x4(clamp448(a * m), clamp448(b * m), clamp448(c * m), clamp448(d * m));
  return pack_fp8x4(clamp448(a / sf), clamp448(b / sf), clamp448(c / sf), clamp448(d / sf));
}

// UE8M0 code of the smallest power of two 2^E with amax / 2^E <= 448:
// r = amax / 448 (IEEE division), E = ceil(log2 r) read off r's exponent and mantissa bits,
// code = clamp(E + 127, 0, 254); amax == 0 -> 0.
__device__ __forceinline__ uint32_t ue8m0_for_amax(float amax) {
  float r = amax / 448.0f;
  uint32_t u = __float_as_uint(r);
  uint32_t ex = (u >> 23) & 0xFFu;
  uint32_t man = u & 0x7FFFFFu;
  if (ex == 0) return 0u;                     // r subnormal or zero: E <= -127
  uint32_t code = man ? ex + 1 : ex;          // code = E + 127
  return code > 254u ? 254u : code;
}

// 16x16x128 FP8 x FP8 MFMA with unit block scales: D = A * B (C = 0).
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 E2M1 (A) x E4M3 (B) MFMA with per-32-K E8M0 scales, accumulating into c.
__device__ __forceinline__ v4f mfma_fp4w_fp8(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}

// E4M3 (A) x E4M3 (B) with E8M0 scales, accumulating into c.
__device__ __forceinline__ v4f mfma_fp8_scaled(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// The per-32 UE8M0 recipes' MFMA: E2M1 weights (recipe 1) or E4M3 weights (recipe 2) as A,
// E4M3 activations as B, both with their E8M0 scales, accumulating into c.  (The float-scale
// recipe 0 instantiates it in a branch it never takes.)
template <int R>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  if constexpr (R == 1) return mfma_fp4w_fp8(a, b, c, sa, sb);
  else return mfma_fp8_scaled(a, b, c, sa, sb);
}

// MFMA 16x16x128 operand layout on gfx950 (measured):
//  * FP8: lane l carries row (l % 16); its bytes 0..15 are K [16*(l/16), +16) and its
//    bytes 16..31 are K [64 + 16*(l/16), +16) of the 128-wide K block.
//  * FP4: lane l carries row (l % 16), K [32*(l/16), +32) as 16 bytes, low nibble first.
//  * E8M0 scales: the scale of (row m, 32-wide K group g) is read from lane m + 16*g.
//  * D (16x16 f32): lane l holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ v8i load_fp8_operand(const uint8_t* row_kblock, int lg) {
  v4i lo = *reinterpret_cast<const v4i*>(row_kblock + 16 * lg);
  v4i hi = *reinterpret_cast<const v4i*>(row_kblock + 64 + 16 * lg);
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// One 64-K half of an FP8 operand, the other half zeroed: by the layout above, a lane's bytes
// 0..15 lie in K [0, 64) of the block and its bytes 16..31 in K [64, 128), so an MFMA with
// half H of one operand sums exactly the products of that half of the block.
template <int H>
__device__ __forceinline__ v8i fp8_half(const v8i& b) {
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = H == 0 ? b[i] : 0;
    r[4 + i] = H == 1 ? b[4 + i] : 0;
  }
  return r;
}

__device__ __forceinline__ v8i load_fp4_operand(const uint8_t* row_kblock_packed, int lg) {
  v4i lo = *reinterpret_cast<const v4i*>(row_kblock_packed + 16 * lg);
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// XCD-aware workgroup order: the hardware deals workgroup ids round-robin over the 8 XCDs;
// this returns a logical id such that each XCD walks one contiguous range of logical ids.
__device__ __forceinline__ int xcd_logical_id(int hw_id, int grid) {
  int per = grid >> 3;                 // grid is a multiple of 8
  return (hw_id & 7) * per + (hw_id >> 3);
}

// Whether the route kernel can put any expert in the small-M class (known on the host, so the
// small-M launches are skipped when it cannot).
inline bool small_class_used(const Args& a) {
  if (a.max_tiles_s == 0 || a.tile_mode == 2) return false;
  return a.tile_mode == 1 || a.large_min_rows > 1;
}

}  // namespace mm

// Host launchers (one per translation unit).
namespace mm {
hipError_t launch_route(const Args& a, hipStream_t s);
hipError_t launch_l1_small(const Args& a, hipStream_t s);
hipError_t launch_l2_small(const Args& a, hipStream_t s);
hipError_t launch_l1_large(const Args& a, hipStream_t s);
hipError_t launch_l2_large(const Args& a, hipStream_t s);
hipError_t launch_combine(const Args& a, hipStream_t s);
// the whole forward in one cooperative launch (large-M tiles only)
hipError_t launch_fused(const Args& a, hipStream_t s);
// out[e][kb][r] = in[e][r][kb] over E experts of `rows` rows and KB words per row (32-bit words)
hipError_t launch_sf_kmajor(const uint32_t* in, uint32_t* out, int E, int rows, int KB, hipStream_t s);
hipError_t launch_e2m1_pairs(const uint8_t* in, uint8_t* out, size_t pairs, int KB, hipStream_t s);
// n_tiles 16 x 16 block dot products with the GEMMs' MFMA (fmt as in mega_moe_diag_mfma_block_sums)
hipError_t launch_diag_mfma(int fmt, const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                            float* out, int n_tiles, hipStream_t s);
}  // namespace mm
