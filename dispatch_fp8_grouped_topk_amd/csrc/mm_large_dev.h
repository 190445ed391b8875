// Device code of the large-M grouped GEMMs, shared by their stand-alone kernels
// (mm_gemm_large.hip) and the fused single-launch forward (mm_fused.hip).
//
// Large-M grouped GEMMs, the default for every expert (a tile of one to 256 pool rows).
//
// Orientation as in the small-M kernels (weight rows = MFMA M side, tokens = N side) and the
// same slab decomposition (L1: one expert x one 128-channel slab, i.e. 256 w1 rows, gate and up;
// L2: one expert x 256 output columns).  A tile holds up to 256 pool rows of one expert; the
// route kernel splits an expert's rows into equal tiles of at most 256 (rounded up to 16).
// E2M1 L1 tiles of at most 5 column groups per wave run as wide items: 256 channels, 512 w1 rows
// (template parameter WX = 2; see item_space).
//
// Workgroup: 8 waves, two per SIMD, so that one wave's LDS reads and promotion arithmetic
// overlap the other's MFMAs.  Wave w owns weight rows of group wm = w & 3 (64 rows: for L1 two
// 16-row gate tiles and the two matching up tiles, so SwiGLU stays lane-local) and the 16-token
// column groups g = 2i + (w >> 2) of the tile.  The kernels are instantiated per number of
// column groups per wave (1..8), so a ragged tile costs at most one padded group per wave.
//
// Both operands and their scales are staged through LDS with LDS-direct buffer loads (no
// VGPRs in flight), in rings of 128-K blocks as deep as LDS allows for the tile shape (see
// Ring: four blocks for one column group per wave, a three-deep weight ring beside a two-deep
// token ring for FP8 tiles of 5-7 groups, two for the largest FP8 tiles): while block kb is
// multiplied, the later blocks are in flight.  16-byte chunk c of an
// FP8 row r sits at slot c ^ ((r >> 1) & 7) (FP4 rows of 64 bytes: c ^ ((r >> 2) & 3)): an
// operand read serves 16 lanes (16 consecutive rows, one chunk each) per cycle of the 64 LDS
// banks, and this swizzle puts their chunks in 16 different 16-byte bank groups.  FP8 recipe:
// each MFMA covers exactly one 128-K scale
// block and is promoted into the float accumulators with (activation scale x weight scale)
// one column group later, off the MFMA's critical path.  Per-32 recipes (E2M1 or E4M3
// weights): the UE8M0 scales go to the MFMA, which accumulates directly; the E4M3-weight recipe
// stages its weights exactly as the FP8 recipe does and its scales as the MXFP4 recipe does.
//
// The grid is persistent: the workgroups walk the (tile, slab) items in rounds, half of each
// round from the costly end of the item list and half from the cheap end (see k_large), and
// the 32 workgroups resident on one XCD take consecutive items, i.e. the slabs of the same one
// or two token tiles, which then share those token rows in the XCD's L2.
//
// The epilogues are those of the small-M kernels: fused SwiGLU / clamp / top-k weight / group
// amax / scale / E4M3 cast after L1 (design page section 10.1), BF16 slot rows after L2
// (section 11.1).
#pragma once

#include "mm_common.h"

namespace mm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTok = kLargeRows;              // pool rows per tile (256)
constexpr int kWRows = 256;                   // weight rows per tile

// Ring geometry for recipe R and NG column groups per wave.  A stage of block kb has a weight
// part (the 256 WX weight rows: 128 bytes of E4M3 or 64 of E2M1 each) and a token part (the first
// 32 NG token rows, 128 bytes each, and 256 + 256 WX scale words: words [0, 256) are activation
// scale words in the order (wn, lr, i) of the readers (see tok_scale_row), words [256, ...) the
// UE8M0 scale words (4 x UE8M0) of weight rows 0, 1, ...).  The weight parts and the token parts sit in
// two rings.  Where three or four whole stages fit in the LDS left beside the per-tile arrays,
// both rings take that depth; where only two would, the weight ring (streamed from HBM, the
// loads with the longest latency) takes three and the token ring (rows shared by the slabs of
// a tile, mostly served by L2) two, if that fits.
// The last kilobyte of the workgroup's LDS holds the fused forward's own variables (Lds::extra;
// the ring geometries below are the same with or without it).
constexpr int kRingBudget = 160 * 1024 - 3 * 1024 - 1024;

template <int R, int NG, int WX = 1>
struct Ring {
  static constexpr int kWBytes = kWRows * WX * (R == 1 ? 64 : 128);
  static constexpr int kXRows = 32 * NG;
  static constexpr int kTBytes = kXRows * 128 + 1024 * (1 + WX);
  static constexpr int kFit = kRingBudget / (kWBytes + kTBytes);
  static constexpr bool kSplit = kFit < 3 && 3 * kWBytes + 2 * kTBytes <= kRingBudget;
  static constexpr int kWStages = kSplit ? 3 : (kFit > 4 ? 4 : kFit);
  static constexpr int kTStages = kSplit ? 2 : kWStages;
  static_assert(kTStages >= 2, "two stages must fit");
  static_assert(kWStages * kWBytes + kTStages * kTBytes <= kRingBudget, "ring budget");
};
constexpr int kRingBytes = kRingBudget;

struct StageRef {
  uint8_t* w;
  uint8_t* x;
  uint32_t* scl;
};

// Weight part of ring slot sw and token part of ring slot st.
template <int R, int NG, int WX = 1>
__device__ __forceinline__ StageRef stage_ref(uint8_t* ring, int sw, int st) {
  using G = Ring<R, NG, WX>;
  uint8_t* t = ring + G::kWStages * G::kWBytes + st * G::kTBytes;
  return StageRef{ring + sw * G::kWBytes, t, reinterpret_cast<uint32_t*>(t + G::kXRows * 128)};
}

struct Lds {
  // the K loop's operand ring; after the K loop the FP8 L1 epilogue keeps the amax of each
  // (row group, token) in its last 4 KB (red)
  uint8_t ring[kRingBytes];
  int rowsrc[kTok];                           // source row of each tile row (token or pool row)
  int aux[kTok];                              // L1: top-k weight (f32 bits) / L2: slot row, per tile row
  float wsc[2 * kMaxKBlocks];                 // FP8 recipe: weight-block scale of row block b, K block kb at b KB + kb
  int2 td_next;                               // tile-list entry of the workgroup's next item
  // the fused forward's own variables (unused by the stand-alone kernels).  They live inside this
  // one LDS object on purpose: with a second LDS variable in the kernel the compiler can no longer
  // tell the ring's LDS-direct loads from other LDS accesses and waits for every load in flight
  // before each K step's first operand read
  alignas(16) uint8_t extra[512];
};
static_assert(sizeof(Lds) <= 160 * 1024, "LDS budget of one workgroup");

__device__ __forceinline__ float (*epilogue_red(Lds& L))[kTok] {
  return reinterpret_cast<float(*)[kTok]>(L.ring + kRingBytes - 4 * kTok * sizeof(float));
}

// LDS-direct buffer loads: each active lane fetches `size` bytes at byte offset voff + soff of
// the buffer into consecutive LDS bytes starting at the wave-uniform `lds` (lane i at
// lds + size*i).  Offsets at or past the buffer's size read zeros instead of faulting.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
// The same with the non-temporal cache policy (gfx950 `nt`): for the weight stream, which each
// item reads once.  A plain streaming read of HBM measured 7.2 TB/s with `nt` against 6.3 TB/s
// without (256 workgroups of 256 threads, 8 x 16-byte loads in flight per thread).
constexpr int kCPolNT = 2;
__device__ __forceinline__ void lds_load16_nt(rsrc_t r, uint32_t voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0,
                                           kCPolNT);
}
__device__ __forceinline__ void lds_load4(rsrc_t r, uint32_t voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// Workgroup barrier for the K pipeline.  Unlike __syncthreads() it carries no memory fence;
// ordering is explicit instead: each wave waits for its own LDS-direct loads of the block about
// to be read (wait_vmcnt) before arriving, such writes are complete in LDS once counted, and
// the empty asm statements stop the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are complete, but its
// global stores may still be in flight (__syncthreads() would wait for those too; vmcnt counts
// stores).  The LDS-direct loads are waited for explicitly (wait_vmcnt) where they matter.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Activation scale word d (0..255; wave d/64, lane d%64 of the scale load) belongs to token row
// 16 (2i + wn) + lr with wn = d / 128, lr = (d / 8) % 16, i = d % 8, so that the reader (wn, lr)
// finds the words of its column groups i = 0..7 at 8 consecutive positions, tok_scale_pos.
__device__ __forceinline__ int tok_scale_row(int d) { return 16 * (2 * (d & 7) + (d >> 7)) + ((d >> 3) & 15); }
__device__ __forceinline__ int tok_scale_pos(int wn, int lr) { return 128 * wn + 8 * lr; }
__device__ __forceinline__ int scl_w(int row) { return 256 + row; }

// Global sources of one wave's share of a stage: buffer descriptors and per-lane 32-bit byte
// offsets (the operand tensors are below 4 GiB; the host routes larger problems to the small
// class); the K block enters as the scalar offset.  Every wave issues the same loads per stage,
// with no branch, so that a K step is one basic block and the scheduling fences below hold:
//   weights: FP8 rows 32w + 8j + lane/8 (j < 4); E2M1 rows 32w + 16j + lane/4 (j < 2);
//   tokens:  ceil(NG/2) blocks of 8 rows, rows 8 token_block(w, j) + lane/8;
//   scales:  one word per lane: waves 0-3 the activation scale word 64w + lane, from the
//            K-major pool-order scale array (one K block of the tile's rows is one contiguous
//            kilobyte: a gather of one word per row costs the address unit about a lane a
//            cycle), waves 4-7 the UE8M0 scale word of weight row 64(w-4) + lane (FP8: a
//            filler, the first word of the array, into words nobody reads).
struct Src {
  rsrc_t wr;                                  // the expert's weight rows
  rsrc_t xr;                                  // token rows (activations or the intermediate)
  rsrc_t cr;                                  // this wave's scale source
  uint32_t wo[4];
  uint32_t xo[4];
  uint32_t co;
  int wkb;                                    // bytes per K block of a weight row
  uint32_t wend;                              // bytes of the weight buffer (wr's size)
  uint32_t ckb;                               // bytes per K block of this wave's scale source
  // wide E2M1 items only: the second scale load (UE8M0 words of weight rows 256 + 64 (w % 4) + lane)
  rsrc_t cr2;
  uint32_t co2, ckb2;
};

template <int R, int WX = 1>
constexpr int kWeightLoads = R == 1 ? 2 * WX : 4;
template <int WX>
constexpr int kScaleLoads = WX;                // wide items: 512 weight-scale words need a second load
constexpr int kSpreadGroups = 3;              // column groups the stage loads are spread over
template <int NG>
constexpr int kTokenLoads = (NG + 1) / 2;
template <int R, int NG, int WX = 1>
constexpr int kStageLoads = kWeightLoads<R, WX> + kTokenLoads<NG> + kScaleLoads<WX>;

// 8-row token block of load j of wave w: blocks w + 8j cover the 4 NG blocks of the tile; for
// odd NG, waves 4-7 have no block left in their last load and fetch wave w-4's again (the same
// bytes to the same place).
template <int NG>
__device__ __forceinline__ int token_block(int w, int j) {
  const int b = w + 8 * j;
  return (NG & 1) && j == kTokenLoads<NG> - 1 && w >= 4 ? b - 4 : b;
}

// Load j of a wave's share of one K step's loads: the weight part of block bw into F.w and the
// token part (token blocks, then the scale word) of block bt into F.x / F.scl.  With one ring
// depth (bw == bt) the weights go first; with a deeper weight ring the token part goes first, so
// that waiting for a block's token part leaves exactly the next block's weight loads in flight.
// bw >= KB (the steps past the last block): the weight loads take a lane offset at the end of the
// buffer, so every lane is out of range and reads zeros into the retired slot without touching
// memory, and they still count as loads, which keeps the number in flight constant.
template <int R, int NG, bool NTW, int WX = 1>
__device__ __forceinline__ void issue_load(const StageRef& F, const Src& s, int bw, int bt, int w, int j, int KB) {
  constexpr int NW = kWeightLoads<R, WX>, NT = kTokenLoads<NG>, NSC = kScaleLoads<WX>;
  constexpr bool split = Ring<R, NG, WX>::kSplit;
  const bool is_w = split ? j >= NT + NSC : j < NW;
  const int jt = split ? j : j - NW;                 // index within the token part
  const int jw = split ? j - NT - NSC : j;           // index within the weight part
  if (is_w) {
    uint8_t* dst = R != 1 ? F.w + (32 * w + 8 * jw) * 128 : F.w + (32 * WX * w + 16 * jw) * 64;
    const bool past = bw >= KB;
    const uint32_t vo = past ? s.wend : s.wo[jw];
    const int so = past ? 0 : bw * s.wkb;
    if (NTW) lds_load16_nt(s.wr, vo, so, dst);
    else lds_load16(s.wr, vo, so, dst);
  } else if (jt < NT) {
    lds_load16(s.xr, s.xo[jt], bt * 128, F.x + token_block<NG>(w, jt) * 8 * 128);
  } else if (jt == NT) {
    lds_load4(s.cr, s.co, (int)((uint32_t)bt * s.ckb), F.scl + 64 * w);
  } else {
    lds_load4(s.cr2, s.co2, (int)((uint32_t)bt * s.ckb2), F.scl + 512 + 64 * (w & 3));
  }
}

// The stage loads of a K step go out behind the MFMAs of its column groups: after group i,
// loads [stage_split(i), stage_split(i + 1)).  Issued all at once, a wave stalls in the address
// unit until the queue has room for them; spread out, the queue drains between groups.
template <int R, int NG, int WX = 1>
__device__ __forceinline__ constexpr int stage_split(int i) {
  constexpr int C = kStageLoads<R, NG, WX>, G = NG < kSpreadGroups ? NG : kSpreadGroups;
  return i >= G ? C : (C * i + G - 1) / G;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N) without waiting on expcnt / lgkmcnt (gfx9 encoding)
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Loads a wave may still have in flight once its loads of block kb have landed: step j issues
// the token part of block j + NST - 1 and the weight part of block j + NSW - 1 (the prologue
// plays the steps before 0), so with one depth NS the later NS - 2 steps' loads, and with
// NSW = NST + 1 the weight part of block kb + 1 (issued after block kb's token part) and the
// later NST - 2 steps' loads.
template <int R, int NG, int WX = 1>
constexpr int kInFlight = Ring<R, NG, WX>::kSplit
                              ? kWeightLoads<R, WX> + (Ring<R, NG, WX>::kTStages - 2) * kStageLoads<R, NG, WX>
                              : (Ring<R, NG, WX>::kWStages - 2) * kStageLoads<R, NG, WX>;

// LDS operand addressing.  Every row a lane reads has the same residue mod 16 (lr), so the
// chunk swizzle is the same for all of them and a lane needs two base offsets per tile (the
// 16-byte chunks of K [16 lg, +16) and [64 + 16 lg, +16) of its first row); the other rows are
// constant offsets, folded into the ds_read immediates.  L1 weight tiles rt: rows
// 32 wm + 16 (rt & 1) (+ 128 for the up tiles rt >= 2); L2: rows 64 wm + 16 rt.
// Wide E2M1 L1 items (WX = 2, 512 weight rows): tiles rt < 4 are the gate rows 64 wm + 16 rt, the
// up tiles rt >= 4 the rows 256 further on.
template <bool L1, int WX = 1>
__device__ __forceinline__ constexpr int a_tile_rows(int rt) {
  return L1 ? (rt >= 2 * WX ? 128 * WX : 0) + 16 * (rt & (2 * WX - 1)) : 16 * rt;
}

__device__ __forceinline__ v8i lds_fp8_operand(const uint8_t* lo, const uint8_t* hi, int off) {
  const v4i a = *reinterpret_cast<const v4i*>(lo + off);
  const v4i b = *reinterpret_cast<const v4i*>(hi + off);
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// E2M1 operand of one lane (16 bytes): the MFMA reads only the low four registers of an FP4
// operand, so the upper four are left undefined instead of zeroed (16 VGPRs fewer per four tiles).
__device__ __forceinline__ v8i lds_fp4_operand_lo(const uint8_t* lo, int off) {
  const v4i a = *reinterpret_cast<const v4i*>(lo + off);
  return __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
}

__device__ __forceinline__ v8i lds_fp4_operand(const uint8_t* lo, int off) {
  const v4i a = *reinterpret_cast<const v4i*>(lo + off);
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// The K loop shared by L1 and L2 for a wave with NG column groups: acc[rt][i] (+)= weight tile
// rt x column group 2i + wn.  arow0: the lane's LDS row of weight tile 0; wsel[rt]: the FP8
// weight-scale row block (of L.wsc) of tile rt.  H64 (FP8 L2 with per-64 intermediate scales): each
// 128-K block is two MFMAs, one per 64-K half of the token operand (the other half zeroed), each
// promoted with its own activation scale (stage words [0, 256) and [256, 512)).
template <int R, int NG, bool L1, bool NTW, bool H64 = false, int WX = 1>
__device__ __forceinline__ void k_loop(Lds& L, const Src& src, int arow0, const int wsel[4], int KB,
                                       v4f acc[4 * WX][NG], int w, int wn, int lane) {
  static_assert(WX == 1 || (R == 1 && L1 && !H64), "wide items: E2M1 L1 only");
  constexpr int NSW = Ring<R, NG, WX>::kWStages, NST = Ring<R, NG, WX>::kTStages;
  constexpr int NA = 4 * WX;                 // weight tiles per wave
  const int lr = lane & 15, lg = lane >> 4;
  const int tsp = tok_scale_pos(wn, lr);
  // lane offsets inside a stage's weight and token tiles
  const int sw7 = (lr >> 1) & 7;
  const int wlo = R != 1 ? arow0 * 128 + 16 * (lg ^ sw7) : arow0 * 64 + 16 * (lg ^ ((lr >> 2) & 3));
  const int whi = arow0 * 128 + 16 * ((lg | 4) ^ sw7);
  const int xrow0 = 16 * wn + lr;
  const int xlo = xrow0 * 128 + 16 * (lg ^ sw7);
  const int xhi = xrow0 * 128 + 16 * ((lg | 4) ^ sw7);
  int swrow[NA];                           // per-32 recipes: scale word index of each weight tile's row
#pragma unroll
  for (int rt = 0; rt < NA; ++rt) swrow[rt] = scl_w(arow0 + a_tile_rows<L1, WX>(rt));
  // Prologue: the issue of steps -(NSW - 1) .. -1.  Every step issues its loads without a
  // branch; past the last block the weight loads read zeros (a lane offset at the buffer's end:
  // no memory access) and the token loads a copy of block KB - 1, into the slots of retired blocks
  // (never read), so the number of loads in flight behind block kb is always kInFlight.
  static_assert(NSW == NST || NSW == NST + 1, "ring depths");
#pragma unroll
  for (int j = -(NSW - 1); j < 0; ++j) {
    const int bt = j + NST - 1, bw = j + NSW - 1;
    const StageRef F = stage_ref<R, NG, WX>(L.ring, bw, bt < 0 ? 0 : bt);
#pragma unroll
    for (int l = 0; l < kStageLoads<R, NG, WX>; ++l) {
      const bool is_w = Ring<R, NG, WX>::kSplit ? l >= kTokenLoads<NG> + kScaleLoads<WX> : l < kWeightLoads<R, WX>;
      if (is_w || bt >= 0) issue_load<R, NG, NTW, WX>(F, src, bw, min(bt < 0 ? 0 : bt, KB - 1), w, l, KB);
    }
  }
  int wslot = 0, tslot = 0;                // weight / token ring slots of block kb
  // FP8: the last column group's promotion of block kb is done in step kb + 1, behind group 0's
  // MFMAs, so that a wave reaches the barrier as soon as its last MFMAs are issued instead of
  // after they have drained (same FMAs, same order: bit-identical sums)
  v4f pend[4];
  float pend_s[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    pend[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    pend_s[rt] = 0.f;
  }
  for (int kb = 0; kb < KB; ++kb) {
    wait_vmcnt<kInFlight<R, NG, WX>>();
    pipeline_barrier();                    // block kb landed for all waves; block kb-1 retired
    // the weight part of block kb + NSW - 1 and the token part of block kb + NST - 1 go to the
    // slots block kb-1 used.  Their loads are issued behind column group 0's MFMAs: issued
    // right after the barrier, every wave's loads queue in the address unit at once and hold
    // the waves back from their first MFMA.
    const int bw = kb + NSW - 1, bt = min(kb + NST - 1, KB - 1);
    const int fw = wslot == 0 ? NSW - 1 : wslot - 1, ft = tslot == 0 ? NST - 1 : tslot - 1;
    const StageRef F = stage_ref<R, NG, WX>(L.ring, fw, ft);
    // fetch_part(i) issues the loads due after column group i: all of them after group
    // 0.  (The call sites of the later groups issue nothing, but their scheduling fences shape
    // the group loop's schedule.)
    auto fetch_part = [&](int i) {
#pragma unroll
      for (int j = stage_split<R, NG, WX>(i); j < stage_split<R, NG, WX>(i + 1); ++j) issue_load<R, NG, NTW, WX>(F, src, bw, bt, w, j, KB);
    };
    const StageRef S = stage_ref<R, NG, WX>(L.ring, wslot, tslot);
    wslot = wslot + 1 == NSW ? 0 : wslot + 1;
    tslot = tslot + 1 == NST ? 0 : tslot + 1;
    const uint8_t* xl = S.x + xlo;
    const uint8_t* xh = S.x + xhi;
    // Column group 0's operands first and alone (10 LDS reads, so the waits before its MFMAs can
    // count them individually; LDS returns in order); the scales and group 1 follow.
    v8i B = lds_fp8_operand(xl, xh, 0);
    v8i A[NA];
#pragma unroll
    for (int rt = 0; rt < NA; ++rt) {
      if (R != 1) A[rt] = lds_fp8_operand(S.w + wlo, S.w + whi, a_tile_rows<L1>(rt) * 128);
      else if (WX == 2) A[rt] = lds_fp4_operand_lo(S.w + wlo, a_tile_rows<L1, WX>(rt) * 64);
      else A[rt] = lds_fp4_operand(S.w + wlo, a_tile_rows<L1>(rt) * 64);
    }
    uint32_t sw8[8];                       // activation scale words of column groups 0..NG-1
    auto read_token_scales = [&]() {
      const v4i lo = *reinterpret_cast<const v4i*>(S.scl + tsp);
      sw8[0] = lo[0]; sw8[1] = lo[1]; sw8[2] = lo[2]; sw8[3] = lo[3];
      if (NG > 4) {
        const v4i hi = *reinterpret_cast<const v4i*>(S.scl + tsp + 4);
        sw8[4] = hi[0]; sw8[5] = hi[1]; sw8[6] = hi[2]; sw8[7] = hi[3];
      }
    };
    if (R == 0 && H64) {
      float cw[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) cw[rt] = L.wsc[wsel[rt] * KB + kb];
      read_token_scales();                 // first-half scales
      uint32_t sh8[8];                     // second-half scales of column groups 0..NG-1
      {
        const v4i lo = *reinterpret_cast<const v4i*>(S.scl + 256 + tsp);
        sh8[0] = lo[0]; sh8[1] = lo[1]; sh8[2] = lo[2]; sh8[3] = lo[3];
        if (NG > 4) {
          const v4i hi = *reinterpret_cast<const v4i*>(S.scl + 256 + tsp + 4);
          sh8[4] = hi[0]; sh8[5] = hi[1]; sh8[6] = hi[2]; sh8[7] = hi[3];
        }
      }
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        v8i Bn;
        if (i + 1 < NG) Bn = lds_fp8_operand(xl, xh, 4096 * (i + 1));
        const v8i B0 = fp8_half<0>(B), B1 = fp8_half<1>(B);
        v4f q0[4], q1[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          q0[rt] = mfma_fp8(A[rt], B0);
          q1[rt] = mfma_fp8(A[rt], B1);
        }
        const float s0 = __uint_as_float(sw8[i]), s1 = __uint_as_float(sh8[i]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          acc[rt][i] += q0[rt] * (s0 * cw[rt]);
          acc[rt][i] += q1[rt] * (s1 * cw[rt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        fetch_part(i);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < NG) B = Bn;
      }
    } else if (R == 0) {
      const v8i B1 = NG > 1 ? lds_fp8_operand(xl, xh, 4096) : B;
      v4f p[2][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) p[0][rt] = mfma_fp8(A[rt], B);
      // issue order: group 0's operands and group 1's token tile, then group 0's MFMAs, each
      // waiting only for its own operands
      __builtin_amdgcn_sched_group_barrier(0x100, NG > 1 ? 12 : 10, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
      fetch_part(0);
      __builtin_amdgcn_sched_barrier(0);
      float cw[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) cw[rt] = L.wsc[wsel[rt] * KB + kb];
      read_token_scales();
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][NG - 1] += pend[rt] * pend_s[rt];
      __builtin_amdgcn_sched_barrier(0);
      B = B1;
#pragma unroll
      for (int i = 1; i < NG; ++i) {
        v8i Bn;
        if (i + 1 < NG) Bn = lds_fp8_operand(xl, xh, 4096 * (i + 1));
        const float sp = __uint_as_float(sw8[i - 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          p[i & 1][rt] = mfma_fp8(A[rt], B);
          acc[rt][i - 1] += p[(i - 1) & 1][rt] * (sp * cw[rt]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // the next group's LDS reads first
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then up to five VALU
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
        fetch_part(i);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < NG) B = Bn;
      }
      const float sp = __uint_as_float(sw8[NG - 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        pend[rt] = p[(NG - 1) & 1][rt];
        pend_s[rt] = sp * cw[rt];
      }
    } else {
      int swv[NA];
#pragma unroll
      for (int rt = 0; rt < NA; ++rt) swv[rt] = (S.scl[swrow[rt]] >> (8 * lg)) & 0xFF;
      read_token_scales();
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        v8i Bn;
        if (i + 1 < NG) Bn = lds_fp8_operand(xl, xh, 4096 * (i + 1));
        const int sx = (sw8[i] >> (8 * lg)) & 0xFF;
#pragma unroll
        for (int rt = 0; rt < NA; ++rt) acc[rt][i] = mfma_mx<R>(A[rt], B, acc[rt][i], swv[rt], sx);
        __builtin_amdgcn_sched_barrier(0);
        fetch_part(i);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < NG) B = Bn;
      }
    }
  }
  if (R == 0 && !H64) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt][NG - 1] += pend[rt] * pend_s[rt];
  }
  // the loads issued past the last block land in retired slots; let them land before the
  // item ends, so none can reach the LDS once the next item (or kernel) has laid it out anew
  wait_vmcnt<0>();
}

// Per-lane global offsets of one wave's share of the token rows (tile rows
// 8 token_block(w, j) + lane/8) and of its scale word.  sf_pool: the K-major activation scales
// ([KB][P] words; the tile's rows are pool rows off .. off + cnt - 1, padding rows repeat the
// last); w_sf: the expert's UE8M0 weight scales, grow(r) maps a tile row to the weight row within
// the expert, a row's scale word of K block kb sits at grow(r) * wsrow_bytes + kb * wskb (row-major
// scales: one row's words are consecutive; K-major: one K block's rows are, so a wave's 64 rows
// are 256 contiguous bytes instead of 64 cache lines).
// h64 (FP8 recipe, L2 with per-64 intermediate scales, [I/64][P] words): K block kb's two halves
// are scale rows 2 kb and 2 kb + 1; waves 0-3 fetch the first half's words and waves 4-7, which
// have no weight scales to fetch in this recipe, the second half's into words [256, 512).
template <int R, int NG, int WX = 1, class F>
__device__ __forceinline__ void token_offsets(Src& s, const int* rowsrc, uint32_t row_bytes, rsrc_t sf_pool,
                                              int P, int off, int cnt, rsrc_t w_sf, F grow,
                                              uint32_t wsrow_bytes, int wskb, int w, int lane, bool h64 = false) {
#pragma unroll
  for (int j = 0; j < kTokenLoads<NG>; ++j) {
    const int r = 8 * token_block<NG>(w, j) + (lane >> 3);
    s.xo[j] = (uint32_t)rowsrc[r] * row_bytes + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  const int d = 64 * (w & 3) + lane;
  const bool wscale = R != 0 && w >= 4;
  const bool half2 = R == 0 && h64;
  s.cr = wscale ? w_sf : sf_pool;
  s.ckb = wscale ? (uint32_t)wskb : 4u * (half2 ? 2u : 1u) * (uint32_t)P;
  if (w < 4 || half2) {
    const int r = tok_scale_row(d);
    s.co = 4u * (uint32_t)(off + (r < cnt ? r : cnt - 1)) + (w >= 4 ? 4u * (uint32_t)P : 0u);
  } else {
    s.co = R != 0 ? (uint32_t)grow(d) * wsrow_bytes : 0u;   // FP8: one word, read by every lane
  }
  if (WX == 2) {                              // wide items: the words of weight rows 256 .. 511
    s.cr2 = w_sf;
    s.ckb2 = (uint32_t)wskb;
    s.co2 = (uint32_t)grow(256 + d) * wsrow_bytes;
  }
}

// Per-lane global offsets of one wave's share of the weight rows; grow(r) maps a tile row to
// the weight row within the expert.  paired (E2M1): the row-pair layout, where K block kb of rows
// 2q, 2q + 1 is the 128 bytes at (q * KB + kb) * 128 (row 2q + 1's half second), so a K block is
// 128 bytes further on (Src::wkb) and the lanes of a row pair read one whole line.
template <int R, int WX = 1, class F>
__device__ __forceinline__ void weight_offsets(Src& s, F grow, uint32_t row_bytes, int w, int lane,
                                               bool paired = false) {
  if (R != 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * w + 8 * j + (lane >> 3);
      s.wo[j] = (uint32_t)grow(r) * row_bytes + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2 * WX; ++j) {
      const int r = 32 * WX * w + 16 * j + (lane >> 2);
      const int g = grow(r);
      const uint32_t piece = 16u * (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
      s.wo[j] = paired ? (uint32_t)(g >> 1) * 2u * row_bytes + 64u * (uint32_t)(g & 1) + piece
                       : (uint32_t)g * row_bytes + piece;
    }
    if (WX == 1) s.wo[2] = s.wo[3] = 0;
  }
}

// ------------------------------------------------------------------------------------ L1
// WX = 2: a wide E2M1 item, 256 channels of the intermediate (512 rows of w1) per slab.
template <int R, int NG, bool NTW, int WX = 1>
__device__ __forceinline__ void l1_large_tile(const Args& a, int e, int off, int cnt, int slab, Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 3, wn = w >> 2;
  const int H = a.H, I = a.I, KB = H / 128;

  Src src;
  const size_t wrow_bytes = R == 1 ? (size_t)H / 2 : (size_t)H;
  src.wkb = R == 1 && !a.w_paired ? 64 : 128;
  src.wr = make_rsrc(a.l1_w + (size_t)e * 2 * I * wrow_bytes, 2 * (size_t)I * wrow_bytes);
  src.wend = (uint32_t)(2 * (size_t)I * wrow_bytes);
  src.xr = make_rsrc(a.x, (size_t)a.T * H);
  const rsrc_t sf_pool = make_rsrc(a.x_sf_pool, (size_t)KB * a.P * 4);
  const rsrc_t w_sf = make_rsrc(static_cast<const uint8_t*>(a.l1_sf) + (R != 0 ? (size_t)e * 2 * I * (H / 32) : 0),
                                2 * (size_t)I * (H / 32));
  // Gate tile row 32 wm + 16 t + m (and the up tile row 128 further on) holds channel
  // 32 wm + 8 (m / 4) + 4 t + m % 4 of the slab: the lane holding rows 4 lg .. 4 lg + 3 of both
  // gate tiles then holds 8 consecutive channels of its token, stored as one 8-byte piece.  Wide
  // items: gate tile row 64 wm + 16 t + m (up: 256 further on) holds channel
  // 64 wm + 32 (t / 2) + 8 (m / 4) + 4 (t % 2) + m % 4, so tiles 2p, 2p + 1 of a wave are again
  // one 32-channel group.
  const auto grow = [&](int r) {
    if (WX == 1) {
      const int q = r & 127, m = q & 15;
      const int c = (q & ~31) + 8 * (m >> 2) + 4 * ((q >> 4) & 1) + (m & 3);
      return (r < 128 ? 0 : I) + 128 * slab + c;
    }
    const int q = r & 255, m = q & 15, t = (q >> 4) & 3;
    const int c = (q & ~63) + 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
    return (r < 256 ? 0 : I) + 256 * slab + c;
  };
  weight_offsets<R, WX>(src, grow, (uint32_t)wrow_bytes, w, lane, R == 1 && a.w_paired);
  token_offsets<R, NG, WX>(src, L.rowsrc, H, sf_pool, a.P, off, cnt, w_sf, grow, a.wsf_kmajor ? 4 : H / 32,
                           a.wsf_kmajor ? 8 * I : 4, w, lane);
  int wsel[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) wsel[rt] = rt < 2 ? 0 : 1;

  v4f acc[4 * WX][NG];
#pragma unroll
  for (int rt = 0; rt < 4 * WX; ++rt)
#pragma unroll
    for (int i = 0; i < NG; ++i) acc[rt][i] = v4f{0.f, 0.f, 0.f, 0.f};
  k_loop<R, NG, true, NTW, false, WX>(L, src, 32 * WX * wm + lr, wsel, KB, acc, w, wn, lane);

  // ---------------- epilogue: SwiGLU, clamp, top-k weight, group amax, scale, E4M3 cast
  // acc[2p + t][i][r] (gate) and acc[2 WX + 2p + t][i][r] (up), p < WX, are channel
  // 32 WX wm + 32 p + 8 lg + 4 t + r of the slab for tile row 16 (2i + wn) + lr.
  static_assert(R != 0 || WX == 1, "FP8 items are not wide");
  const bool clamp_in = a.clamp > 0.f && a.clamp_inputs, clamp_out = a.clamp > 0.f && !a.clamp_inputs;
  // FP8: the group amax is reduced across the four row groups through the end of the ring, which
  // other waves may still be reading (their last K block) or filling (copies past the end)
  float(*red)[kTok] = epilogue_red(L);
  if (R == 0) lds_barrier();
  float v[NG][2][4];
  // one instantiation of the SwiGLU pass per SiLU form, chosen by one wave-uniform branch
  auto swiglu_pass = [&](auto precise) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int col = 16 * (2 * i + wn) + lr;
      const float wt = col < cnt ? __int_as_float(L.aux[col]) : 0.f;
#pragma unroll
      for (int p = 0; p < WX; ++p) {
        float am = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = acc[2 * p + t][i][r], u = acc[2 * WX + 2 * p + t][i][r];
            const float sv = swiglu_f32<decltype(precise)::value>(g, u, a.clamp, clamp_in, clamp_out);
            const float x = sv * wt;
            v[i][t][r] = x;
            am = fmaxf(am, fabsf(x));
          }
        am = fmaxf(am, __shfl_xor(am, 16, 64));
        am = fmaxf(am, __shfl_xor(am, 32, 64));
        if (R == 0) {
          if (lg == 0) red[wm][col] = am;
        } else {
          // per-32 recipes: the 32-channel group from channel cb is this wave's gate tiles 2p, 2p + 1
          const int cb = 128 * WX * slab + 32 * WX * wm + 32 * p;
          const uint32_t code = ue8m0_for_amax(am);
          const int ex = 127 - (int)code;
          const bool valid = col < cnt;
          uint2 q = make_uint2(0u, 0u);
          if (am > 0.f) {
            q.x = pack_fp8x4(clamp448(ldexpf(v[i][0][0], ex)), clamp448(ldexpf(v[i][0][1], ex)),
                             clamp448(ldexpf(v[i][0][2], ex)), clamp448(ldexpf(v[i][0][3], ex)));
            q.y = pack_fp8x4(clamp448(ldexpf(v[i][1][0], ex)), clamp448(ldexpf(v[i][1][1], ex)),
                             clamp448(ldexpf(v[i][1][2], ex)), clamp448(ldexpf(v[i][1][3], ex)));
          }
          if (valid) *reinterpret_cast<uint2*>(a.inter_q + (size_t)(off + col) * I + cb + 8 * lg) = q;
          if (valid && lg == 0)
            static_cast<uint8_t*>(a.inter_sf)[((size_t)(cb >> 7) * a.P + off + col) * 4 + ((cb >> 5) & 3)] =
                (uint8_t)code;
        }
      }
    }
  };
  if (a.precise_silu) swiglu_pass(BoolC<true>{});
  else swiglu_pass(BoolC<false>{});
  if (R == 0) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int col = 16 * (2 * i + wn) + lr;
      // per-128 scales: the group is the slab (all four row groups); per-64: row groups 2h, 2h+1
      const int h = wm >> 1;
      const float amax = a.inter64 ? fmaxf(red[2 * h][col], red[2 * h + 1][col])
                                   : fmaxf(fmaxf(red[0][col], red[1][col]), fmaxf(red[2][col], red[3][col]));
      const float sf = amax / 448.0f, m = 448.0f / amax;
      const bool valid = col < cnt;
      uint2 q = make_uint2(0u, 0u);
      if (sf > 0.f) {
        q.x = e4m3_scaled4(v[i][0][0], v[i][0][1], v[i][0][2], v[i][0][3], m, sf);
        q.y = e4m3_scaled4(v[i][1][0], v[i][1][1], v[i][1][2], v[i][1][3], m, sf);
      }
      if (valid)
        *reinterpret_cast<uint2*>(a.inter_q + (size_t)(off + col) * I + 128 * slab + 32 * wm + 8 * lg) = q;
      if (valid && lg == 0 && (a.inter64 ? (wm & 1) == 0 : wm == 0))
        static_cast<float*>(a.inter_sf)[(size_t)(a.inter64 ? 2 * slab + h : slab) * a.P + off + col] = sf;
    }
  }
}

// ------------------------------------------------------------------------------------ L2
template <int R, int NG, bool NTW, bool H64>
__device__ __forceinline__ void l2_large_tile(const Args& a, int e, int off, int cnt, int slab, Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 3, wn = w >> 2;
  const int H = a.H, I = a.I, KB = I / 128;

  Src src;
  const size_t wrow_bytes = R == 1 ? (size_t)I / 2 : (size_t)I;
  src.wkb = R == 1 && !a.w_paired ? 64 : 128;
  src.wr = make_rsrc(a.l2_w + (size_t)e * H * wrow_bytes, (size_t)H * wrow_bytes);
  src.wend = (uint32_t)((size_t)H * wrow_bytes);
  src.xr = make_rsrc(a.inter_q, (size_t)a.P * I);
  const rsrc_t sf_pool = make_rsrc(a.inter_sf, (size_t)KB * (H64 ? 2 : 1) * a.P * 4);
  const rsrc_t w_sf = make_rsrc(static_cast<const uint8_t*>(a.l2_sf) + (R != 0 ? (size_t)e * H * (I / 32) : 0),
                                (size_t)H * (I / 32));
  // Tile row 64 wm + 16 rt + m holds output column 64 wm + 16 (m / 4) + 4 rt + m % 4 of the
  // slab: the lane holding rows 4 lg .. 4 lg + 3 of the four tiles then holds 16 consecutive
  // output columns of its token, stored as two 16-byte pieces.  Columns past H (H a multiple
  // of 128 but not of 256) repeat valid rows; their results drop.
  const auto grow = [&](int r) {
    const int m = r & 15, rt = (r >> 4) & 3;
    const int g = kWRows * slab + (r & ~63) + 16 * (m >> 2) + 4 * rt + (m & 3);
    return g < H ? g : g - 128;
  };
  weight_offsets<R>(src, grow, (uint32_t)wrow_bytes, w, lane, R == 1 && a.w_paired);
  token_offsets<R, NG>(src, L.rowsrc, I, sf_pool, a.P, off, cnt, w_sf, grow, a.wsf_kmajor ? 4 : I / 32,
                       a.wsf_kmajor ? 4 * H : 4, w, lane, H64);
  int wsel[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) wsel[rt] = wm >> 1;

  v4f acc[4][NG];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < NG; ++i) acc[rt][i] = v4f{0.f, 0.f, 0.f, 0.f};
  k_loop<R, NG, false, NTW, H64>(L, src, 64 * wm + lr, wsel, KB, acc, w, wn, lane);

  const int nbase = kWRows * slab + 64 * wm;
  if (nbase >= H) return;                        // wave-uniform: H is a multiple of 128
  // ---------------- epilogue: BF16 rows into the pair-ordered slot buffer
  // acc[rt][i][j] is output column nbase + 16 lg + 4 rt + j of tile row 16 (2i + wn) + lr
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int col = 16 * (2 * i + wn) + lr;
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

// ------------------------------------------------------------------------------------ kernels
// Item numbering: the tile list is cut into bands of kBand consecutive tiles (the last band may
// be shorter), and a band's items run slab-major: item (band b, slab s, j-th tile of the band).
// 32 consecutive items, which one XCD's workgroups take together, then cover 32 / kBand slabs
// of kBand tiles, so an expert's weight slab is fetched into that XCD's L2 once for up to
// kBand of its tiles, and each tile's rows once for 32 / kBand slabs.
constexpr int kBand = 4;

// The item list of one GEMM launch: tiles [0, n_norm) in items of one slab, then (wide E2M1 L1
// items) tiles [n_norm, n_tiles) in items of two slabs, each part numbered in bands as above.
struct ItemSpace {
  int n_slabs, n_tiles, n_norm;
  __device__ __forceinline__ int count() const { return n_norm * n_slabs + (n_tiles - n_norm) * (n_slabs >> 1); }
};
struct ItemPos {
  int tile, slab;                               // slab: of the item's own width
  bool wide;
};
__device__ __forceinline__ ItemPos band_pos(int q, int n_slabs, int n_tiles, int t0) {
  const int per_band = kBand * n_slabs;
  const int b = q / per_band, r = q - b * per_band;
  const int in_band = min(kBand, n_tiles - b * kBand);
  const int s = r / in_band;
  return ItemPos{t0 + b * kBand + (r - s * in_band), s, false};
}
__device__ __forceinline__ ItemPos item_pos(int q, const ItemSpace& sp) {
  const int qn = sp.n_norm * sp.n_slabs;
  if (q < qn) return band_pos(q, sp.n_slabs, sp.n_norm, 0);
  ItemPos p = band_pos(q - qn, sp.n_slabs >> 1, sp.n_tiles - sp.n_norm, sp.n_norm);
  p.wide = true;
  return p;
}

// Column groups per wave of a tile of `rows` pool rows (two waves share its 16-row groups).
__device__ __forceinline__ int tile_ng(int rows) { return ((rows + 15) / 16 + 1) / 2; }

// Per-item set-up shared by L1 and L2: tile rows, their sources, the FP8 weight-block scales.
// The item's tile-list entry is in L.td_next (fetched during the previous item); q_next is the
// workgroup's next item (-1: none), whose entry this item fetches in turn.
template <int R, bool L1, bool H64, class Hooks>
__device__ __forceinline__ void run_item(const Args& a, int q, int q_next, const ItemSpace& sp, Lds& L,
                                         Hooks& hooks) {
  const int tid = threadIdx.x;
  const ItemPos ip = item_pos(q, sp);
  const int slab = ip.slab;
  const int H = a.H, I = a.I;
  hooks.before(ip.tile);                        // the fused forward waits here for the tile's inputs

  // the previous item is done with the LDS (its LDS-direct loads were waited for at the end of
  // its K loop; its output stores need not have completed)
  lds_barrier();
  const int2 td = L.td_next;
  const int e = tile_expert(td.x), cnt = tile_rows(td.x), off = td.y;
  // Weight lines of an expert with one tile are read once: stream them non-temporally (L1; in L2
  // only for tiles of at most 32 rows, the pure weight streams: measured, the hint made the L2 of
  // larger single tiles up to 6% slower while it takes 3-9% off these).  E2M1 weights only in the
  // row-pair layout: row-major, a K block is half a line, whose other half the next K step reads.
  const bool nt = (R != 1 || a.w_paired) && tile_single(td.x) && (L1 || cnt <= 32);
  if (L1) {
    if (tid < kTok) {
      const int pr = off + (tid < cnt ? tid : cnt - 1);
      const int src_pair = a.pool_src[pr];
      L.rowsrc[tid] = src_pair / a.k;
      L.aux[tid] = __float_as_int(a.w_pool[pr]);
    }
    if (R == 0) {
      // float scales of the gate block (row 0) and the up block (row 1) for every K block
      const int KB = H / 128;
      const float* sfw = static_cast<const float*>(a.l1_sf) + (size_t)e * (2 * I / 128) * KB;
      for (int i = tid; i < 2 * KB; i += kThreads)
        L.wsc[i] = sfw[(size_t)(i < KB ? slab : I / 128 + slab) * KB + i % KB];
    }
  } else {
    // L2: the tile rows are pool rows (no load), and the slot rows (waves 0-3) and the FP8 weight
    // scales of the slab's two 128-row blocks of w2, clamped past H (waves 4-7), go to LDS by
    // LDS-direct loads: the K loop's first wait covers them, so the set-up waits on no load, nor
    // on the previous item's output stores ahead of them in the same counter
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // (a scalar branch per wave)
    if (wv < kTok / 64) {
      const int pr = off + (tid < cnt ? tid : cnt - 1);
      L.rowsrc[tid] = pr;
      lds_load4(make_rsrc(a.pool_src, (size_t)a.P * 4), 4u * (uint32_t)pr, 0, &L.aux[64 * wv]);
    } else if (R == 0) {
      const int KB = I / 128, i = tid - kTok;    // 2 KB <= 256 scales: one per lane of waves 4-7
      int blk = 2 * slab + i / KB;
      blk = blk < H / 128 ? blk : H / 128 - 1;
      const uint8_t* sfw = static_cast<const uint8_t*>(a.l2_sf) +
                           (size_t)__builtin_amdgcn_readfirstlane(e) * (H / 128) * KB * 4;   // uniform: no waterfall
      lds_load4(make_rsrc(sfw, (size_t)(H / 128) * KB * 4), i < 2 * KB ? 4u * (uint32_t)(blk * KB + i % KB) : ~0u,
                0, &L.wsc[64 * (wv - kTok / 64)]);
    }
  }
  lds_barrier();
  // every wave has read td: fetch the next item's entry straight into LDS (two lanes of wave 0);
  // it is older than all of this item's stage loads, so the K loop's first wait covers it
  if (q_next >= 0 && tid < 2)
    lds_load4(make_rsrc(a.tiles_l, (size_t)a.max_tiles_l * 8),
              (uint32_t)item_pos(q_next, sp).tile * 8u + 4u * tid, 0,
              &L.td_next);

  const int nw = tile_ng(cnt);                 // column groups per wave
  if (R == 1 && L1 && ip.wide) {                // wide E2M1 L1 items: tiles of at most kWideMaxNG groups per wave
    switch (nw) {
#define MM_WCASE(n)                                                    \
  case n:                                                              \
    if constexpr (R == 1 && L1) {                                      \
      if (nt) l1_large_tile<R, n, true, 2>(a, e, off, cnt, slab, L);   \
      else l1_large_tile<R, n, false, 2>(a, e, off, cnt, slab, L);     \
    }                                                                  \
    break;
      MM_WCASE(1) MM_WCASE(2) MM_WCASE(3) MM_WCASE(4)
      default: MM_WCASE(5)
#undef MM_WCASE
    }
    hooks.after(ip.tile);
    return;
  }
  switch (nw) {
#define MM_CASE(n)                                                                   \
  case n:                                                                            \
    if (nt) {                                                                        \
      if (L1) l1_large_tile<R, n, true>(a, e, off, cnt, slab, L);                    \
      else l2_large_tile<R, n, true, H64>(a, e, off, cnt, slab, L);                  \
    } else {                                                                         \
      if (L1) l1_large_tile<R, n, false>(a, e, off, cnt, slab, L);                   \
      else l2_large_tile<R, n, false, H64>(a, e, off, cnt, slab, L);                 \
    }                                                                                \
    break;
    MM_CASE(1) MM_CASE(2) MM_CASE(3) MM_CASE(4) MM_CASE(5) MM_CASE(6) MM_CASE(7)
    default: MM_CASE(8)
#undef MM_CASE
  }
  hooks.after(ip.tile);                         // the fused forward signals the tile's L1 slab done
}

// Hooks of the stand-alone kernels: nothing to wait for or signal (kernel boundaries order them).
struct NoHooks {
  __device__ __forceinline__ void before(int) {}
  __device__ __forceinline__ void after(int) {}
};


// Persistent item loop over the items numbered as above.  Round r gives XCD x
// (hardware workgroup id mod 8) the items r*G + x*(G/8) + j for its workgroups j.
// The items of this workgroup, round by round.  The item list runs from the costliest tiles (most
// column groups: MFMA-bound) to the cheapest (few tokens per weight byte: HBM-bound).  Each
// round, half the grid (four XCDs) takes the next items from the front of the list and the other
// half the next ones from the back, and the halves swap every round, so both kinds run side by
// side (the weight stream of the cheap items overlaps the MFMA work of the costly ones) and every
// workgroup alternates between them.  Slot `mine` is XCD-major, so each XCD still takes
// consecutive items.
// The last round is usually partial (T < G items).  With `balanced` set (balance_last_round),
// its items go to the T workgroups with the least work in the full rounds instead.
struct ItemRounds {
  int n_items, n_front, n_back, half, k0, rounds, mine;
  bool first_half;
  bool balanced = false;
  int last_item = -1;                           // balanced: this workgroup's item of the last round
  __device__ __forceinline__ ItemRounds(int n) : n_items(n) {
    const int G = gridDim.x, per = G >> 3;
    half = G >> 1;
    mine = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    n_front = (n_items + 1) >> 1;
    n_back = n_items - n_front;
    first_half = mine < half;
    k0 = first_half ? mine : mine - half;
    rounds = (n_front + half - 1) / half;
  }
  // item of slot m in round r of the unbalanced order, -1 if none
  __device__ __forceinline__ int slot_item(int m, int r) const {
    if (r >= rounds) return -1;
    const bool fh = m < half;
    const int k = r * half + (fh ? m : m - half);
    if (fh == ((r & 1) == 0)) return k < n_front ? k : -1;
    return k < n_back ? n_items - 1 - k : -1;
  }
  // item of round r, -1 if none (once a round has none, no later round has one)
  __device__ __forceinline__ int item(int r) const {
    if (balanced && r == rounds - 1) return last_item;
    return slot_item(mine, r);
  }
};

// Relative cost of an item with ng column groups per wave (wide: two slabs), fitted to per-item
// traces of the benchmark workloads: the weight stream sets a floor shared by all tiles, and
// each column group beyond the first adds MFMA and epilogue work, more in L1 (longer K, SwiGLU
// epilogue) than in L2.
__device__ __forceinline__ int item_cost(int ng, bool wide, bool l1) {
  const int c = 40 + (l1 ? 3 : 1) * max(0, 2 * ng - 3);
  return wide ? 2 * c : c;
}
constexpr int kBalanceMaxTiles = 32768;         // tiles whose costs fit the LDS scratch

// Balance the last, partial round (T < G items; rounds - 1 >= 1 full rounds before it).  Every
// workgroup computes the modelled work of every slot in the full rounds (item_cost of its items),
// ranks the slots by (work, slot), and the slot of rank j < T takes the j-th item of the last
// round.  Those items are the T consecutive items from (rounds - 1) * G / 2 on (the middle of the
// list, where front and back meet), so every item is still taken exactly once.  Called by every
// thread of the workgroup before its first item, with the ring as scratch; returns this
// workgroup's item of the last round (-1: none), or -2 to keep the rounds as they are (no partial
// round, too many tiles for the scratch, or every tile of the same cost: the tile list is ordered
// by column groups, so first and last tile agree).  Not inlined, so that its registers do not
// weigh on the item loop's allocation.
__device__ __noinline__ int balanced_last_item(const int2* tiles, int n_tiles, int n_norm, int n_slabs,
                                               int n_items, bool l1, uint8_t* ring) {
  const ItemSpace sp{n_slabs, n_tiles, n_norm};
  const ItemRounds rs(n_items);
  const int G = gridDim.x, r_last = rs.rounds - 1;
  const int T = n_items - r_last * G;
  if (r_last < 1 || T <= 0 || T >= G || G > kThreads || n_tiles > kBalanceMaxTiles) return -2;
  // (values read from memory or LDS pass through readfirstlane: the compiler then knows them to
  // be wave-uniform)
  const int x_first = __builtin_amdgcn_readfirstlane(tiles[0].x);
  const int x_last = __builtin_amdgcn_readfirstlane(tiles[n_tiles - 1].x);
  if (tile_ng(tile_rows(x_first)) == tile_ng(tile_rows(x_last)) && n_norm == n_tiles) return -2;
  uint8_t* cost = ring;                                            // per tile
  uint32_t* work = reinterpret_cast<uint32_t*>(ring + kBalanceMaxTiles);   // per slot
  int* per_wave = reinterpret_cast<int*>(work + kThreads);
  const int tid = threadIdx.x;
  for (int t = tid; t < n_tiles; t += kThreads) cost[t] = (uint8_t)item_cost(tile_ng(tile_rows(tiles[t].x)), false, l1);
  __syncthreads();
  if (tid < G) {
    uint32_t s = 0;
    for (int r = 0; r < r_last; ++r) {
      const ItemPos ip = item_pos(rs.slot_item(tid, r), sp);
      s += (uint32_t)cost[ip.tile] * (ip.wide ? 2u : 1u);
    }
    work[tid] = s;
  }
  __syncthreads();
  // rank of this slot: the slots before it in (work, slot) order, counted per wave (in the
  // scratch: no LDS variable of its own, the ring stays the kernel's only LDS object)
  const uint32_t my = work[rs.mine];
  const bool before = tid < G && (work[tid] < my || (work[tid] == my && tid < rs.mine));
  const unsigned long long bal = __ballot(before);
  if ((tid & 63) == 0) per_wave[tid >> 6] = __popcll(bal);
  __syncthreads();
  int rank = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) rank += per_wave[i];
  __syncthreads();                              // scratch reads done before the first item's loads
  rank = __builtin_amdgcn_readfirstlane(rank);
  return rank < T ? r_last * rs.half + rank : -1;
}

// Large-M tiles of the GEMM (with the four-wave kernel on, the MXFP4 L2 tiles from
// hdr[kHdrTilesQuad] on are left to it) and slabs per tile.
template <int R, bool L1>
__device__ __forceinline__ int large_tiles_of(const Args& a) {
  return R == 1 && !L1 && a.quad ? a.hdr[kHdrTilesQuad] : a.hdr[kHdrTilesLarge];
}
template <bool L1>
__device__ __forceinline__ int large_slabs_of(const Args& a) {
  return L1 ? a.I / kL1SlabCh : (a.H + kWRows - 1) / kWRows;
}

// The persistent item loop of one GEMM over this workgroup's items.
// The item list of the GEMM.  E2M1 L1 (I a multiple of 256): the tiles of experts whose first
// tile has at most kWideMaxNG column groups per wave (from hdr[kHdrTilesWide] on in the tile
// list, which is ordered by that count) run as wide items, 512 rows of w1 each: a K step then
// does twice the MFMA work behind the same barrier, operand reads of the token tile and scale
// words, and its fixed costs, while a wave's accumulators (8 tiles x at most 5 groups) still fit.
template <int R, bool L1>
__device__ __forceinline__ ItemSpace item_space(const Args& a) {
  const int n_tiles = large_tiles_of<R, L1>(a);
  const bool wide = R == 1 && L1 && (a.I % 256) == 0;
  return ItemSpace{large_slabs_of<L1>(a), n_tiles, wide ? min(a.hdr[kHdrTilesWide], n_tiles) : n_tiles};
}

// kBalance: balance the last round (the stand-alone kernels; the fused forward replays the plain
// rounds to count its L1 arrivals).
template <int R, bool L1, bool H64, bool kBalance = false, class Hooks>
__device__ __forceinline__ void large_items(const Args& a, Lds& L, Hooks& hooks) {
  const ItemSpace sp = item_space<R, L1>(a);
  ItemRounds rs(sp.count());
  if (kBalance) {
    const int last = balanced_last_item(a.tiles_l, sp.n_tiles, sp.n_norm, sp.n_slabs, sp.count(), L1, L.ring);
    if (last != -2) {
      rs.balanced = true;
      rs.last_item = last;
    }
  }
  int q = rs.item(0);
  if (q >= 0 && threadIdx.x == 0) L.td_next = a.tiles_l[item_pos(q, sp).tile];
  for (int r = 0; q >= 0; ++r) {
    const int q_next = rs.item(r + 1);
    run_item<R, L1, H64>(a, q, q_next, sp, L, hooks);
    q = q_next;
  }
}

}  // namespace
}  // namespace mm
