// Large-M grouped GEMMs: experts holding more than 64 pool rows (mid-size and prefill
// batches), where one weight slab is reused by many token rows.
//
// Orientation as in the small-M kernels (weight rows = MFMA M side, tokens = N side) and the
// same workgroup decomposition (L1: one expert x one 128-channel slab, i.e. 256 w1 rows;
// L2: one expert x 256 output columns), with 128 pool rows per tile and four waves.  Each wave
// owns 64 weight rows (for L1 two 16-row gate tiles and the two matching up tiles, so SwiGLU
// stays lane-local) against all 128 tokens: 32 MFMAs per K block, 128 float32 accumulators.
//
// Operand paths are chosen by reuse.  A wave's weight rows are private to it, so they stream
// from memory straight into registers, one K block ahead, without touching LDS.  The token
// tile is needed by all four waves, so each K block of it is staged once in LDS with
// global_load_lds_dwordx4 (three K blocks in flight, 16-byte chunk c of row r stored at slot
// c ^ (r & 7) so the operand reads spread over the LDS banks), together with the per-row
// activation scales.  Per K block the LDS carries 16 KB in and 64 KB out, well inside its
// bandwidth at full MFMA rate.
//
// The epilogues are those of the small-M kernels: fused SwiGLU / clamp / top-k weight / group
// amax / scale / E4M3 cast after L1 (design page section 10.1), BF16 slot rows after L2
// (section 11.1).
#include "mm_common.h"

namespace mm {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTok = kLargeRows;              // 128 pool rows per tile
constexpr int kNS = kTok / 16;                // token column groups (all 8 per wave)
constexpr int kStages = 3;

struct Stage {
  uint8_t x[kTok * 128];                      // token rows of the K block (E4M3), swizzled
  uint32_t sx[kTok];                          // per-token scale word (f32 bits | 4 x UE8M0)
};

struct Lds {
  Stage st[kStages];
  int rowsrc[kTok];
  float red[4][kTok];                         // per wave (weight-row group): amax per token
  float wsc[2][kMaxKBlocks];                  // FP8 recipe: float weight scales of the K blocks
};

// per-wave LDS-direct load instructions per stage (vmcnt bookkeeping): 4 x 1 KB of token rows
// and one scale-word instruction
constexpr int kDmaPerStage = 5;

// LDS-direct loads: each active lane fetches `size` bytes from its global address into
// consecutive LDS bytes starting at the wave-uniform `lds` (lane i at lds + size*i).
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N and no wait on expcnt / lgkmcnt (gfx9 encoding)
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the K pipeline.  Unlike __syncthreads() it carries no memory fence,
// whose release semantics would wait for every outstanding LDS-direct load (vmcnt(0)) and so
// drain the prefetch queue at each K block.  Ordering is explicit instead: each wave waits for
// its own loads of the block about to be read (wait_vmcnt) before arriving, LDS-direct writes
// are complete in LDS once counted, and the empty asm statements stop the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v8i read_fp8_rows(const uint8_t* tile, int row, int lg) {
  const uint8_t* base = tile + row * 128;
  const int sw = row & 7;
  const v4i lo = *reinterpret_cast<const v4i*>(base + 16 * (lg ^ sw));
  const v4i hi = *reinterpret_cast<const v4i*>(base + 16 * ((lg | 4) ^ sw));
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Token-tile sources of one wave: rows 32w + 8j + lane/8 (j = 0..3), chunk (lane%8)^(lane/8),
// and the scale word of row 32w + lane (lanes < 32).
struct TokSrc {
  const uint8_t* x[4];
  const uint32_t* sx;
};

__device__ __forceinline__ void issue_tokens(Stage& S, const TokSrc& src, int kb, int w, int lane) {
  uint8_t* xd = S.x + w * 32 * 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) lds_load16(src.x[j] + (size_t)kb * 128, xd + j * 1024);
  if (lane < 32) lds_load4(src.sx + kb, &S.sx[32 * w]);
}

__device__ __forceinline__ TokSrc token_srcs(const uint8_t* base, size_t row_bytes, const uint32_t* sc,
                                             size_t sc_words, const int* rowsrc, int w, int lane) {
  TokSrc t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * w + 8 * j + (lane >> 3);
    t.x[j] = base + (size_t)rowsrc[row] * row_bytes + 16 * ((lane & 7) ^ (lane >> 3));
  }
  t.sx = sc + (size_t)rowsrc[32 * w + (lane & 31)] * sc_words;
  return t;
}

// Weight operand of one 16-row tile for K block kb (the lane's row pointer `row`).
template <int R>
__device__ __forceinline__ v8i load_w(const uint8_t* row, int kb, int lg) {
  if (R == 0) return load_fp8_operand(row + 128 * kb, lg);
  return load_fp4_operand(row + 64 * kb, lg);
}

// The K loop shared by L1 and L2: acc[rt][s] (+)= the wave's 4 weight tiles x the 8 token
// groups.  wrow[rt]: the lane's weight row for tile rt (E4M3 or E2M1 bytes).  FP8 recipe:
// L.wsc[wsel[rt]][kb] is tile rt's float weight scale for K block kb, and each MFMA (one
// 128-K scale block) is promoted into acc with (activation scale x weight scale).
// MXFP4 recipe: wsf[rt] points at the lane's UE8M0 scale bytes (row, 4kb + lane/16).
// One K block of the loop below: wait for / retire the pipeline stages, prefetch the next
// weight block into An (when there is one) and the token block kb+2 into LDS, then multiply.
template <int R>
__device__ __forceinline__ void k_step(Lds& L, const TokSrc& tsrc, const uint8_t* const wrow[4],
                                       const uint8_t* const wsf[4], const int wsel[4], int KB, int kb,
                                       const v8i A[4], const int sw[4], v8i An[4], int swn[4],
                                       v4f acc[4][kNS], int w, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  // outstanding: [tokens kb] [weights kb] [tokens kb+1]; keep the newest stage in flight
  if (kb + 1 < KB) wait_vmcnt<kDmaPerStage>();
  else wait_vmcnt<0>();
  pipeline_barrier();                    // token block kb landed for all waves; kb-1 retired
  if (kb + 1 < KB) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      An[rt] = load_w<R>(wrow[rt], kb + 1, lg);
      if (R == 1) swn[rt] = wsf[rt][4 * (kb + 1)];
    }
  }
  if (kb + 2 < KB) issue_tokens(L.st[(kb + 2) % kStages], tsrc, kb + 2, w, lane);
  const Stage& S = L.st[kb % kStages];
  float cw[4];
  if (R == 0) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) cw[rt] = L.wsc[wsel[rt]][kb];
  }
  // token group s+1 is read from LDS while group s is multiplied
  v8i B = read_fp8_rows(S.x, lr, lg);
  uint32_t sxw = S.sx[lr];
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    v8i Bn;
    uint32_t sxn = 0;
    if (s + 1 < kNS) {
      const int row = 16 * (s + 1) + lr;
      Bn = read_fp8_rows(S.x, row, lg);
      sxn = S.sx[row];
    }
    if (R == 0) {
      const float sa = __uint_as_float(sxw);
      v4f p[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) p[rt] = mfma_fp8(A[rt], B);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][s] += p[rt] * (sa * cw[rt]);
    } else {
      const int sx = (sxw >> (8 * lg)) & 0xFF;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][s] = mfma_fp4w_fp8(A[rt], B, acc[rt][s], sw[rt], sx);
    }
    if (s + 1 < kNS) {
      B = Bn;
      sxw = sxn;
    }
  }
}

// The K loop shared by L1 and L2: acc[rt][s] (+)= the wave's 4 weight tiles x the 8 token
// groups.  wrow[rt]: the lane's weight row for tile rt (E4M3 or E2M1 bytes).  FP8 recipe:
// L.wsc[wsel[rt]][kb] is tile rt's float weight scale for K block kb, and each MFMA (one
// 128-K scale block) is promoted into acc with (activation scale x weight scale).  MXFP4
// recipe: wsf[rt] points at the lane's UE8M0 scale bytes (row, 4kb + lane/16).  Two register
// sets of weights alternate between even and odd K blocks, so the prefetch of block kb+1 is
// only waited for when block kb+1 starts.
template <int R>
__device__ __forceinline__ void k_loop(Lds& L, const TokSrc& tsrc, const uint8_t* const wrow[4],
                                       const uint8_t* const wsf[4], const int wsel[4], int KB,
                                       v4f acc[4][kNS], int w, int lane) {
  const int lg = lane >> 4;
  v8i A0[4], A1[4];
  int s0[4] = {0, 0, 0, 0}, s1[4] = {0, 0, 0, 0};
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    A0[rt] = load_w<R>(wrow[rt], 0, lg);
    if (R == 1) s0[rt] = wsf[rt][0];
  }
  issue_tokens(L.st[0], tsrc, 0, w, lane);
  if (KB > 1) issue_tokens(L.st[1], tsrc, 1, w, lane);
  for (int kb = 0; kb < KB; kb += 2) {
    k_step<R>(L, tsrc, wrow, wsf, wsel, KB, kb, A0, s0, A1, s1, acc, w, lane);
    if (kb + 1 < KB) k_step<R>(L, tsrc, wrow, wsf, wsel, KB, kb + 1, A1, s1, A0, s0, acc, w, lane);
  }
}

// ------------------------------------------------------------------------------------ L1
template <int R>
__device__ __forceinline__ void l1_large_tile(const Args& a, int e, int m0, int cnt, int slab, Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, KB = H / 128;
  const int off = a.offset[e] + m0;

  if (tid < kTok) L.rowsrc[tid] = a.pool_src[off + (tid < cnt ? tid : cnt - 1)] / a.k;
  if (R == 0) {
    // float scales of the gate block (row 0) and the up block (row 1) for every K block
    const float* sfw = static_cast<const float*>(a.l1_sf) + (size_t)e * (2 * I / 128) * KB;
    for (int i = tid; i < 2 * KB; i += kThreads)
      L.wsc[i / KB][i % KB] = sfw[(size_t)(i < KB ? slab : I / 128 + slab) * KB + i % KB];
  }
  __syncthreads();

  const TokSrc tsrc = token_srcs(a.x, H, static_cast<const uint32_t*>(a.x_sf), H / 128, L.rowsrc, w, lane);
  const size_t wstride = R == 0 ? (size_t)H : (size_t)H / 2;
  const uint8_t* wrow[4];
  const uint8_t* wsf[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = (rt < 2 ? 0 : I) + 128 * slab + 32 * w + 16 * (rt & 1) + lr;
    wrow[rt] = a.l1_w + ((size_t)e * 2 * I + row) * wstride;
    wsf[rt] = static_cast<const uint8_t*>(a.l1_sf) + ((size_t)e * 2 * I + row) * (H / 32) + lg;
  }
  const int wsel[4] = {0, 0, 1, 1};

  v4f acc[4][kNS];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int s = 0; s < kNS; ++s) acc[rt][s] = v4f{0.f, 0.f, 0.f, 0.f};
  k_loop<R>(L, tsrc, wrow, wsf, wsel, KB, acc, w, lane);

  // ---------------- epilogue: SwiGLU, clamp, top-k weight, group amax, scale, E4M3 cast
  // acc[i][s][r] (gate) and acc[2+i][s][r] (up) are channel 32w + 16i + 4lg + r of the slab
  // for tile row 16s + lr.
  const bool do_clamp = a.clamp > 0.f;
  float v[kNS][2][4];
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    const int col = 16 * s + lr;
    const float wt = col < cnt ? a.w_pool[off + col] : 0.f;
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = acc[i][s][r], u = acc[2 + i][s][r];
        float sv = g / (1.0f + expf(-g)) * u;
        if (do_clamp) sv = fminf(fmaxf(sv, -a.clamp), a.clamp);
        const float x = sv * wt;
        v[s][i][r] = x;
        am = fmaxf(am, fabsf(x));
      }
    am = fmaxf(am, __shfl_xor(am, 16, 64));
    am = fmaxf(am, __shfl_xor(am, 32, 64));
    if (R == 0) {
      if (lg == 0) L.red[w][col] = am;
    } else {
      // MXFP4 recipe: the 32-channel group is this wave's two gate tiles
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
        static_cast<uint8_t*>(a.inter_sf)[(size_t)(off + col) * (I / 32) + 4 * slab + w] = (uint8_t)code;
    }
  }
  if (R == 0) {
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      const int col = 16 * s + lr;
      const float amax = fmaxf(fmaxf(L.red[0][col], L.red[1][col]), fmaxf(L.red[2][col], L.red[3][col]));
      const float sf = amax / 448.0f;
      const bool valid = col < cnt;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t q = 0;
        if (sf > 0.f)
          q = pack_fp8x4(clamp448(v[s][i][0] / sf), clamp448(v[s][i][1] / sf),
                         clamp448(v[s][i][2] / sf), clamp448(v[s][i][3] / sf));
        if (valid)
          *reinterpret_cast<uint32_t*>(a.inter_q + (size_t)(off + col) * I + 128 * slab + 32 * w + 16 * i + 4 * lg) = q;
      }
      if (valid && w == 0 && lg == 0) static_cast<float*>(a.inter_sf)[(size_t)(off + col) * (I / 128) + slab] = sf;
    }
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void k_l1_large(Args a) {
  __shared__ __attribute__((aligned(1024))) Lds L;
  const int q = xcd_logical_id(blockIdx.x, gridDim.x);
  const int n_slabs = a.I / kL1SlabCh;
  const int slab = q / a.max_tiles_l;
  const int tile = q - slab * a.max_tiles_l;
  if (slab >= n_slabs || tile >= a.hdr[kHdrTilesLarge]) return;
  const int2 td = a.tiles_l[tile];
  const int rem = a.count[td.x] - td.y;
  l1_large_tile<R>(a, td.x, td.y, rem < kTok ? rem : kTok, slab, L);
}

// ------------------------------------------------------------------------------------ L2
template <int R>
__device__ __forceinline__ void l2_large_tile(const Args& a, int e, int m0, int cnt, int slab, Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, KB = I / 128;
  const int off = a.offset[e] + m0;

  if (tid < kTok) L.rowsrc[tid] = off + (tid < cnt ? tid : cnt - 1);   // pool row feeding token row
  if (R == 0) {
    // float scales of the slab's two 128-row blocks of w2 for every K block (a block past H,
    // when H is not a multiple of 256, repeats the last one; its waves drop their results)
    const float* sfw = static_cast<const float*>(a.l2_sf) + (size_t)e * (H / 128) * KB;
    for (int i = tid; i < 2 * KB; i += kThreads) {
      int blk = 2 * slab + i / KB;
      blk = blk < H / 128 ? blk : H / 128 - 1;
      L.wsc[i / KB][i % KB] = sfw[(size_t)blk * KB + i % KB];
    }
  }
  __syncthreads();

  // the wave's output columns nbase .. nbase+63 (w2 rows); a wave past H (when H is not a
  // multiple of 256) still stages its share of the token tile but computes from valid rows
  // and drops its results
  const int nbase = kL2SlabRows * slab + 64 * w;
  const bool active = nbase < H;                 // wave-uniform: H is a multiple of 128
  const int nrow0 = active ? nbase : H - 64;
  const TokSrc tsrc = token_srcs(a.inter_q, I, static_cast<const uint32_t*>(a.inter_sf), I / 128,
                                 L.rowsrc, w, lane);
  const size_t wstride = R == 0 ? (size_t)I : (size_t)I / 2;
  const uint8_t* wrow[4];
  const uint8_t* wsf[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const size_t row = (size_t)e * H + nrow0 + 16 * rt + lr;
    wrow[rt] = a.l2_w + row * wstride;
    wsf[rt] = static_cast<const uint8_t*>(a.l2_sf) + row * (I / 32) + lg;
  }
  const int wsel[4] = {w >> 1, w >> 1, w >> 1, w >> 1};

  v4f acc[4][kNS];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int s = 0; s < kNS; ++s) acc[rt][s] = v4f{0.f, 0.f, 0.f, 0.f};
  k_loop<R>(L, tsrc, wrow, wsf, wsel, KB, acc, w, lane);

  if (!active) return;
  // ---------------- epilogue: BF16 rows into the pair-ordered slot buffer
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    const int col = 16 * s + lr;
    if (col >= cnt) continue;
    uint16_t* dst = a.slot + (size_t)a.pool_src[off + col] * H + nbase + 4 * lg;
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
__global__ __launch_bounds__(kThreads) void k_l2_large(Args a) {
  __shared__ __attribute__((aligned(1024))) Lds L;
  const int q = xcd_logical_id(blockIdx.x, gridDim.x);
  const int n_slabs = (a.H + kL2SlabRows - 1) / kL2SlabRows;
  const int slab = q / a.max_tiles_l;
  const int tile = q - slab * a.max_tiles_l;
  if (slab >= n_slabs || tile >= a.hdr[kHdrTilesLarge]) return;
  const int2 td = a.tiles_l[tile];
  const int rem = a.count[td.x] - td.y;
  l2_large_tile<R>(a, td.x, td.y, rem < kTok ? rem : kTok, slab, L);
}

inline int round8(long v) { return (int)((v + 7) / 8 * 8); }

}  // namespace

hipError_t launch_l1_large(const Args& a, hipStream_t s) {
  if (a.max_tiles_l == 0 || a.tile_mode == 1) return hipSuccess;
  const int grid = round8((long)a.max_tiles_l * (a.I / kL1SlabCh));
  if (a.recipe == 0) hipLaunchKernelGGL(k_l1_large<0>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_l1_large<1>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_l2_large(const Args& a, hipStream_t s) {
  if (a.max_tiles_l == 0 || a.tile_mode == 1) return hipSuccess;
  const int grid = round8((long)a.max_tiles_l * ((a.H + kL2SlabRows - 1) / kL2SlabRows));
  if (a.recipe == 0) hipLaunchKernelGGL(k_l2_large<0>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_l2_large<1>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm
