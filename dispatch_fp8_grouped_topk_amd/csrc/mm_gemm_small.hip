// Small-M grouped GEMMs: experts holding few pool rows (decode), where the layer is bound by
// streaming expert weights from HBM.
//
// Orientation: the expert's weight rows are the MFMA M side and the tile's pool rows (up to
// 64 tokens, four 16-wide column groups) are the N side, so every weight byte is loaded once
// per tile straight into registers and used against all of the tile's tokens.  This is the
// MI355X counterpart of the pages' small-M answers (the SM90 swap-AB buckets of PR #411 and
// the BLOCK_M=32 single-warpgroup mode of the design page, section 7): keep the MFMA fed from
// the weight stream and never pad the token side beyond 16.
//
// L1 (design page sections 5.3 and 10.1): a workgroup owns one expert, up to 64 pool rows and
// one 128-channel slab of the intermediate, i.e. gate rows [128s, 128s+128) and up rows
// [I+128s, I+128s+128) of w1; the whole re-quantisation group (128 channels for the float
// recipe, 32 for the UE8M0 recipes) therefore lives inside the workgroup and the SwiGLU, top-k
// weight, amax, scale and E4M3 cast are fused after the K loop.
//
// L2 (design page section 11.1): a workgroup owns one expert, up to 64 pool rows and 256
// output columns (w2 rows); its BF16 results go straight to the pair-ordered slot rows.
//
// FP8 recipe: each 16x16x128 MFMA spans exactly one 128-wide scale block, so its result is
// promoted into the float32 accumulator with that block's activation x weight scale (the
// design page's software scale application, one FMA per accumulator element per block).
// Per-32 recipes: E2M1 (MXFP4) or E4M3 (MXFP8) weights and E4M3 activations go through the
// block-scaled MFMA with their per-32 UE8M0 scales; no promotion is needed.
#include "mm_common.h"

namespace mm {

namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kLdsScaleBytes = 32768;         // activation scales of the tile's 64 rows

template <int R>
struct OpLoad;

// FP8 weight rows: K block kb of a row starts at byte 128*kb.
template <>
struct OpLoad<0> {
  static __device__ __forceinline__ v8i w(const uint8_t* row, int kb, int lg, bool) {
    return load_fp8_operand(row + 128 * kb, lg);
  }
};
// E4M3 weight rows with per-32 UE8M0 scales: laid out as the FP8 recipe's.
template <>
struct OpLoad<2> : OpLoad<0> {};
// E2M1 weight rows: K block kb starts at byte 64*kb, or 128*kb in the row-pair layout (the row's
// offset within the expert from w_row_offset).
template <>
struct OpLoad<1> {
  static __device__ __forceinline__ v8i w(const uint8_t* row, int kb, int lg, bool paired) {
    return load_fp4_operand(row + (paired ? 128 : 64) * kb, lg);
  }
};

// Byte offset of weight row `row` within its expert: row-major, or (E2M1 only) the row-pair
// layout (MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED: rows 2q, 2q + 1 share 128-byte lines, K block by K block).
template <int R>
__device__ __forceinline__ size_t w_row_offset(const Args& a, int row, size_t wstride) {
  if (R == 1 && a.w_paired) return (size_t)(row >> 1) * 2 * wstride + 64 * (row & 1);
  return (size_t)row * wstride;
}

// ------------------------------------------------------------------------------------ L1
template <int R, int NSUB>
__device__ __forceinline__ void l1_tile(const Args& a, int e, int m0, int cnt, int slab,
                                        uint8_t* s_scale, float* s_red, int* s_tok) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int H = a.H, I = a.I;
  const int KB = H / 128;
  const int off = a.offset[e] + m0;

  if (tid < 64) s_tok[tid] = a.pool_src[off + (tid < cnt ? tid : cnt - 1)] / a.k;
  __syncthreads();
  if (R == 0) {
    float* sfa = reinterpret_cast<float*>(s_scale);           // [64][KB]
    const float* xsf = static_cast<const float*>(a.x_sf);
    for (int i = tid; i < 64 * KB; i += kThreads) sfa[i] = xsf[(size_t)s_tok[i / KB] * KB + i % KB];
  } else {
    const int G = H / 32;                                      // scale groups per row
    const uint32_t* xsf = static_cast<const uint32_t*>(a.x_sf);
    uint32_t* sfx = reinterpret_cast<uint32_t*>(s_scale);    // [64][G] bytes, copied as words
    for (int i = tid; i < 64 * (G / 4); i += kThreads)
      sfx[i] = xsf[(size_t)s_tok[i / (G / 4)] * (G / 4) + i % (G / 4)];
  }
  __syncthreads();

  // operand rows
  const size_t wstride = R == 1 ? (size_t)H / 2 : (size_t)H;
  const uint8_t* wrow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = (rt < 2 ? 0 : I) + 128 * slab + 32 * w + 16 * (rt & 1) + lr;
    wrow[rt] = a.l1_w + (size_t)e * 2 * I * wstride + w_row_offset<R>(a, row, wstride);
  }
  const uint8_t* xrow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) xrow[s] = a.x + (size_t)s_tok[16 * s + lr] * H;

  v4f acc[4][NSUB];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[rt][s] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i A[4], B[NSUB];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) A[rt] = OpLoad<R>::w(wrow[rt], 0, lg, a.w_paired != 0);
#pragma unroll
  for (int s = 0; s < NSUB; ++s) B[s] = load_fp8_operand(xrow[s], lg);

  if (R == 0) {
    const float* sfw = static_cast<const float*>(a.l1_sf) + (size_t)e * (2 * I / 128) * KB;
    const float* sfg = sfw + (size_t)slab * KB;
    const float* sfu = sfw + (size_t)(I / 128 + slab) * KB;
    const float* sfa = reinterpret_cast<const float*>(s_scale);
    for (int kb = 0; kb < KB; ++kb) {
      v8i An[4], Bn[NSUB];
      const int kn = kb + 1 < KB ? kb + 1 : kb;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) An[rt] = OpLoad<R>::w(wrow[rt], kn, lg, a.w_paired != 0);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) Bn[s] = load_fp8_operand(xrow[s] + 128 * kn, lg);
      const float sg = sfg[kb], su = sfu[kb];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const float sa = sfa[(16 * s + lr) * KB + kb];
        const float cg = sa * sg, cu = sa * su;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const v4f p = mfma_fp8(A[rt], B[s]);
          acc[rt][s] += p * (rt < 2 ? cg : cu);
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) A[rt] = An[rt];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) B[s] = Bn[s];
    }
  } else {
    const int G = H / 32;
    // a row's codes of K block kb: row * rs + kb * ks (row-major or K-major weight scales)
    const size_t rs = a.wsf_kmajor ? 4 : G, ks = a.wsf_kmajor ? (size_t)8 * I : 4;
    const uint8_t* sfw[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = (rt < 2 ? 0 : I) + 128 * slab + 32 * w + 16 * (rt & 1) + lr;
      sfw[rt] = static_cast<const uint8_t*>(a.l1_sf) + (size_t)e * 2 * I * G + row * rs + lg;
    }
    const uint8_t* sfx = s_scale;
    for (int kb = 0; kb < KB; ++kb) {
      v8i An[4], Bn[NSUB];
      const int kn = kb + 1 < KB ? kb + 1 : kb;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) An[rt] = OpLoad<R>::w(wrow[rt], kn, lg, a.w_paired != 0);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) Bn[s] = load_fp8_operand(xrow[s] + 128 * kn, lg);
      int sw[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sw[rt] = sfw[rt][ks * kb];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int sx = sfx[(16 * s + lr) * G + 4 * kb + lg];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt][s] = mfma_mx<R>(A[rt], B[s], acc[rt][s], sw[rt], sx);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) A[rt] = An[rt];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) B[s] = Bn[s];
    }
  }

  // ---------------- epilogue: SwiGLU, clamp, top-k weight, group amax, scale, E4M3 cast
  // acc[i][s][r] (gate) and acc[2+i][s][r] (up) are channel 32w + 16i + 4lg + r of the slab
  // for pool row 16s + lr of the tile.
  const bool clamp_in = a.clamp > 0.f && a.clamp_inputs, clamp_out = a.clamp > 0.f && !a.clamp_inputs;
  float v[NSUB][2][4];
  // one instantiation of the SwiGLU pass per SiLU form, chosen by one wave-uniform branch
  auto swiglu_pass = [&](auto precise) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int col = 16 * s + lr;
      const float wt = col < cnt ? a.w_pool[off + col] : 0.f;
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[i][s][r], u = acc[2 + i][s][r];
          const float sv = swiglu_f32<decltype(precise)::value>(g, u, a.clamp, clamp_in, clamp_out);
          const float x = sv * wt;
          v[s][i][r] = x;
          am = fmaxf(am, fabsf(x));
        }
      am = fmaxf(am, __shfl_xor(am, 16, 64));
      am = fmaxf(am, __shfl_xor(am, 32, 64));
      if (R == 0) {
        if (lg == 0) s_red[w * 64 + col] = am;
      } else {
        // per-32 recipes: the 32-channel group is this wave's two gate tiles
        const uint32_t code = ue8m0_for_amax(am);
        const int ex = 127 - (int)code;
        const bool valid = col < cnt;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint32_t q = 0;
          if (am > 0.f)
            q = pack_fp8x4(clamp448(ldexpf(v[s][i][0], ex)), clamp448(ldexpf(v[s][i][1], ex)),
                           clamp448(ldexpf(v[s][i][2], ex)), clamp448(ldexpf(v[s][i][3], ex)));
          if (valid)
            *reinterpret_cast<uint32_t*>(a.inter_q + (size_t)(off + col) * I + 128 * slab + 32 * w + 16 * i + 4 * lg) = q;
        }
        if (valid && lg == 0)
          static_cast<uint8_t*>(a.inter_sf)[((size_t)slab * a.P + off + col) * 4 + w] = (uint8_t)code;
      }
    }
  };
  if (a.precise_silu) swiglu_pass(BoolC<true>{});
  else swiglu_pass(BoolC<false>{});
  if (R == 0) {
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int col = 16 * s + lr;
      // per-128 scales: the group is the slab (all four waves' channels); per-64: waves 2h, 2h+1
      const int h = w >> 1;
      const float amax = a.inter64 ? fmaxf(s_red[2 * h * 64 + col], s_red[(2 * h + 1) * 64 + col])
                                   : fmaxf(fmaxf(s_red[col], s_red[64 + col]), fmaxf(s_red[128 + col], s_red[192 + col]));
      const float sf = amax / 448.0f, m = 448.0f / amax;
      const bool valid = col < cnt;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t q = 0;
        if (sf > 0.f) q = e4m3_scaled4(v[s][i][0], v[s][i][1], v[s][i][2], v[s][i][3], m, sf);
        if (valid)
          *reinterpret_cast<uint32_t*>(a.inter_q + (size_t)(off + col) * I + 128 * slab + 32 * w + 16 * i + 4 * lg) = q;
      }
      if (valid && lg == 0 && (a.inter64 ? (w & 1) == 0 : w == 0))
        static_cast<float*>(a.inter_sf)[(size_t)(a.inter64 ? 2 * slab + h : slab) * a.P + off + col] = sf;
    }
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void k_l1_small(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_scale[kLdsScaleBytes];
  __shared__ float s_red[4 * 64];
  __shared__ int s_tok[64];
  const int q = xcd_logical_id(blockIdx.x, gridDim.x);
  const int n_slabs = a.I / kL1SlabCh;
  const int slab = q / a.max_tiles_s;
  const int tile = q - slab * a.max_tiles_s;
  if (slab >= n_slabs || tile >= a.hdr[kHdrTilesSmall]) return;
  const int2 td = a.tiles_s[tile];
  const int e = td.x, m0 = td.y;
  const int rem = a.count[e] - m0;
  const int cnt = rem < kSmallRows ? rem : kSmallRows;
  const int nsub = (cnt + 15) >> 4;
  if (nsub == 1) l1_tile<R, 1>(a, e, m0, cnt, slab, s_scale, s_red, s_tok);
  else if (nsub == 2) l1_tile<R, 2>(a, e, m0, cnt, slab, s_scale, s_red, s_tok);
  else l1_tile<R, 4>(a, e, m0, cnt, slab, s_scale, s_red, s_tok);
}

// ------------------------------------------------------------------------------------ L2
template <int R, int NSUB>
__device__ __forceinline__ void l2_tile(const Args& a, int e, int m0, int cnt, int slab,
                                        uint8_t* s_scale, int* s_src) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int H = a.H, I = a.I;
  const int KB = I / 128;
  const int off = a.offset[e] + m0;

  if (tid < 64) s_src[tid] = a.pool_src[off + (tid < cnt ? tid : cnt - 1)];
  // float scales per 128 (KS = KB per row) or per 64 (KS = 2 KB: the two halves of each block)
  const int KS = a.inter64 ? 2 * KB : KB;
  if (R == 0) {
    float* sfa = reinterpret_cast<float*>(s_scale);           // [64][KS]
    const float* isf = static_cast<const float*>(a.inter_sf);
    for (int i = tid; i < 64 * KS; i += kThreads) {
      const int row = i / KS;
      sfa[i] = isf[(size_t)(i % KS) * a.P + off + (row < cnt ? row : cnt - 1)];
    }
  } else {
    const int G4 = I / 128;                                    // words of 4 UE8M0 codes per row
    const uint32_t* isf = static_cast<const uint32_t*>(a.inter_sf);
    uint32_t* sfx = reinterpret_cast<uint32_t*>(s_scale);
    for (int i = tid; i < 64 * G4; i += kThreads) {
      const int row = i / G4;
      sfx[i] = isf[(size_t)(i % G4) * a.P + off + (row < cnt ? row : cnt - 1)];
    }
  }
  __syncthreads();

  const int nbase = kL2SlabRows * slab + 64 * w;               // this wave's first output column
  if (nbase >= H) return;                                      // H is a multiple of 128: whole wave out

  const size_t wstride = R == 1 ? (size_t)I / 2 : (size_t)I;
  const uint8_t* wrow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) wrow[rt] = a.l2_w + (size_t)e * H * wstride + w_row_offset<R>(a, nbase + 16 * rt + lr, wstride);
  const uint8_t* qrow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int row = 16 * s + lr;
    qrow[s] = a.inter_q + (size_t)(off + (row < cnt ? row : cnt - 1)) * I;
  }

  v4f acc[4][NSUB];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[rt][s] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i A[4], B[NSUB];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) A[rt] = OpLoad<R>::w(wrow[rt], 0, lg, a.w_paired != 0);
#pragma unroll
  for (int s = 0; s < NSUB; ++s) B[s] = load_fp8_operand(qrow[s], lg);

  if (R == 0) {
    // weight scale block row nbase/128 is shared by the wave's 64 rows
    const float* sfw = static_cast<const float*>(a.l2_sf) + ((size_t)e * (H / 128) + nbase / 128) * KB;
    const float* sfa = reinterpret_cast<const float*>(s_scale);
    for (int kb = 0; kb < KB; ++kb) {
      v8i An[4], Bn[NSUB];
      const int kn = kb + 1 < KB ? kb + 1 : kb;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) An[rt] = OpLoad<R>::w(wrow[rt], kn, lg, a.w_paired != 0);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) Bn[s] = load_fp8_operand(qrow[s] + 128 * kn, lg);
      const float sb = sfw[kb];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (a.inter64) {                    // one MFMA per 64-K half, each with its own scale
          const float c0 = sfa[(16 * s + lr) * KS + 2 * kb] * sb, c1 = sfa[(16 * s + lr) * KS + 2 * kb + 1] * sb;
          const v8i B0 = fp8_half<0>(B[s]), B1 = fp8_half<1>(B[s]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const v4f p0 = mfma_fp8(A[rt], B0), p1 = mfma_fp8(A[rt], B1);
            acc[rt][s] += p0 * c0;
            acc[rt][s] += p1 * c1;
          }
        } else {
          const float c = sfa[(16 * s + lr) * KB + kb] * sb;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const v4f p = mfma_fp8(A[rt], B[s]);
            acc[rt][s] += p * c;
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) A[rt] = An[rt];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) B[s] = Bn[s];
    }
  } else {
    const int G = I / 32;
    const size_t rs = a.wsf_kmajor ? 4 : G, ks = a.wsf_kmajor ? (size_t)4 * H : 4;
    const uint8_t* sfw[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      sfw[rt] = static_cast<const uint8_t*>(a.l2_sf) + (size_t)e * H * G + (nbase + 16 * rt + lr) * rs + lg;
    const uint8_t* sfx = s_scale;
    for (int kb = 0; kb < KB; ++kb) {
      v8i An[4], Bn[NSUB];
      const int kn = kb + 1 < KB ? kb + 1 : kb;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) An[rt] = OpLoad<R>::w(wrow[rt], kn, lg, a.w_paired != 0);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) Bn[s] = load_fp8_operand(qrow[s] + 128 * kn, lg);
      int sw[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sw[rt] = sfw[rt][ks * kb];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int sx = sfx[(16 * s + lr) * G + 4 * kb + lg];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt][s] = mfma_mx<R>(A[rt], B[s], acc[rt][s], sw[rt], sx);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) A[rt] = An[rt];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) B[s] = Bn[s];
    }
  }

  // ---------------- epilogue: BF16 rows into the pair-ordered slot buffer
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int col = 16 * s + lr;
    if (col >= cnt) continue;
    uint16_t* dst = a.slot + (size_t)s_src[col] * H + nbase + 4 * lg;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const v4f o = acc[rt][s];
      uint2 pk;
      pk.x = bf16_rne(o[0]) | (bf16_rne(o[1]) << 16);
      pk.y = bf16_rne(o[2]) | (bf16_rne(o[3]) << 16);
      *reinterpret_cast<uint2*>(dst + 16 * rt) = pk;
    }
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void k_l2_small(Args a) {
  // per-64 intermediate scales: two floats per 128-K block of each of the 64 rows
  __shared__ __attribute__((aligned(16))) uint8_t s_scale[2 * kLdsScaleBytes];
  __shared__ int s_src[64];
  const int q = xcd_logical_id(blockIdx.x, gridDim.x);
  const int n_slabs = (a.H + kL2SlabRows - 1) / kL2SlabRows;
  const int slab = q / a.max_tiles_s;
  const int tile = q - slab * a.max_tiles_s;
  if (slab >= n_slabs || tile >= a.hdr[kHdrTilesSmall]) return;
  const int2 td = a.tiles_s[tile];
  const int e = td.x, m0 = td.y;
  const int rem = a.count[e] - m0;
  const int cnt = rem < kSmallRows ? rem : kSmallRows;
  const int nsub = (cnt + 15) >> 4;
  if (nsub == 1) l2_tile<R, 1>(a, e, m0, cnt, slab, s_scale, s_src);
  else if (nsub == 2) l2_tile<R, 2>(a, e, m0, cnt, slab, s_scale, s_src);
  else l2_tile<R, 4>(a, e, m0, cnt, slab, s_scale, s_src);
}

inline int round8(long v) { return (int)((v + 7) / 8 * 8); }

}  // namespace

hipError_t launch_l1_small(const Args& a, hipStream_t s) {
  if (!small_class_used(a)) return hipSuccess;
  const int grid = round8((long)a.max_tiles_s * (a.I / kL1SlabCh));
  if (a.recipe == 0) hipLaunchKernelGGL(k_l1_small<0>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.recipe == 1) hipLaunchKernelGGL(k_l1_small<1>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_l1_small<2>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_l2_small(const Args& a, hipStream_t s) {
  if (!small_class_used(a)) return hipSuccess;
  const int grid = round8((long)a.max_tiles_s * ((a.H + kL2SlabRows - 1) / kL2SlabRows));
  if (a.recipe == 0) hipLaunchKernelGGL(k_l2_small<0>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.recipe == 1) hipLaunchKernelGGL(k_l2_small<1>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_l2_small<2>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm
