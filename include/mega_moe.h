/*
 * mega_moe.h -- C ABI of the MegaMoE expert layer for AMD Instinct MI355X (gfx950).
 *
 * One call computes, on one GPU, the forward of a mixture-of-experts FFN layer:
 *
 *   1. dispatch   every (token t, top-k slot j) pair with expert id e in [0, E)
 *                 joins expert e's pool; rows of a pool keep row-major (t, j) order.
 *                 (Research report "MegaMoE on SM100/SM90", section 3.1, dispatch
 *                 role; design page "MegaMoE SM90 Implementation Design",
 *                 section 9.2, source metadata {rank, token, topk}.)
 *   2. L1 GEMM    acc = sum_kb sx[t,kb] * sw1[e,n,kb] * sum_{k in kb} x[t,k] w1[e,n,k]
 *                 over n in [0, 2I)  (design page section 5.3, scale application;
 *                 section 15.2, weight-scale layout).
 *   3. SwiGLU     v = clamp(silu(acc[:, :I]) * acc[:, I:]) * topk_w[t, j]
 *                 then per group of G channels: float scale amax/448 (G = 128) or
 *                 UE8M0 scale (G = 32) and an E4M3 cast  (design page section 10.1).
 *   4. L2 GEMM    o = the same block-scaled product of the re-quantised
 *                 intermediate with w2, cast to BF16 per (token, slot) row
 *                 (design page section 11.1).
 *   5. combine    y[t] = bf16( sum_j f32(slot row (t, j)) ), ascending j, float32
 *                 accumulation (design page section 11.2).
 *
 * Recipes:
 *   MEGA_MOE_RECIPE_FP8_B128   x, w1, w2 and the intermediate are OCP E4M3FN bytes;
 *                              float32 scales: x per (token, 128 channels), weights
 *                              per 128x128 block, intermediate per (row, 128 channels).
 *                              (The SM90 FP8 path of the design page, section 1.1.)
 *   MEGA_MOE_RECIPE_MXFP4W_B32 x and the intermediate are E4M3FN with a UE8M0 scale per
 *                              32 channels; w1, w2 are E2M1 nibbles (two per byte, low
 *                              nibble = even K index) with a UE8M0 scale per (row, 32 K).
 *                              (PR #411 "SM90 FP8 x MXFP4 MegaMoE"; UE8M0 = 2^(code-127).)
 *   MEGA_MOE_RECIPE_MXFP8_B32  as MXFP4W_B32, but w1, w2 are E4M3FN bytes (one per K index) with a
 *                              UE8M0 scale per (row, 32 K): FP8 activations and weights with the
 *                              SM100 scale format, packed UE8M0 per 32 K for activations, weights
 *                              and the intermediate (research report "MegaMoE on SM100/SM90",
 *                              section 8.4, scale-factor formats; design page section 2, the
 *                              scale-factor row of the SM100/SM90 comparison).
 *
 * Layouts (all row-major, contiguous, device memory):
 *   x        u8  [T, H]                     x_sf  f32 [T, H/128]  | u8 [T, H/32]  (per-32 recipes)
 *   topk_idx i32 [T, k]                     topk_w f32 [T, k]
 *   l1_w     u8  [E, 2I, H]  | [E, 2I, H/2] rows 0..I-1 gate, I..2I-1 up   (MXFP8: [E, 2I, H])
 *   l1_sf    f32 [E, 2I/128, H/128]         | u8 [E, 2I, H/32]            (MXFP8: as MXFP4)
 *   l2_w     u8  [E, H, I]   | [E, H, I/2]                                 (MXFP8: [E, H, I])
 *   l2_sf    f32 [E, H/128, I/128]          | u8 [E, H, I/32]             (MXFP8: as MXFP4)
 *   y        bf16 (u16 bits) [T, H]
 * Every pointer must be 16-byte aligned.  Ids < 0 in topk_idx mark masked slots; ids
 * >= E are dropped (contribute nothing) and counted in the num_invalid view.
 *
 * Ownership: the caller allocates every buffer, including the workspace.  The library
 * allocates, frees and synchronises nothing; all work is enqueued on `stream` and the
 * call returns at once.  Inputs are read only; y is fully overwritten.  The workspace
 * needs no initialisation (each call re-initialises what it uses) and stays readable
 * through mega_moe_workspace_views() until the next call that uses it.  Concurrent
 * calls need distinct workspaces.
 *
 * Errors: the functions validate their arguments synchronously and return 0 or one of
 * the negative MEGA_MOE_ERR_* codes.  Nothing is enqueued when validation fails; after
 * MEGA_MOE_ERR_HIP (a failed launch) part of the sequence may have been enqueued and y is
 * undefined.  T * k must stay below 2^30.
 */
#ifndef MEGA_MOE_H
#define MEGA_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEGA_MOE_ABI_VERSION 1

typedef enum {
  MEGA_MOE_RECIPE_FP8_B128 = 0,
  MEGA_MOE_RECIPE_MXFP4W_B32 = 1,
  MEGA_MOE_RECIPE_MXFP8_B32 = 2
} mega_moe_recipe;

/* flags: bits 0-1 select the GEMM tile class (0 = library default, chosen per expert from
   its row count (currently the large-M class for every expert), 1 = small-M class only,
   2 = large-M class only); bit 2 is MEGA_MOE_FLAG_CLAMP_INPUTS, bit 3 MEGA_MOE_FLAG_PRECISE_SILU,
   bit 4 MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR, bit 5 MEGA_MOE_FLAG_INTER_SF64, bit 6 MEGA_MOE_FLAG_FUSED,
   bit 7 MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED; other bits must be 0. */
#define MEGA_MOE_FLAG_TILE_AUTO  0u
#define MEGA_MOE_FLAG_TILE_SMALL 1u
#define MEGA_MOE_FLAG_TILE_LARGE 2u
#define MEGA_MOE_FLAG_TILE_MASK  3u
/* flags bit 2: with swiglu_clamp = c > 0, clamp the gate and up halves of the L1 result to
 * [-c, c] before SiLU and leave silu(g)*u unclamped (the activation clamp of the design page
 * "MegaMoE SM90 Implementation Design", section 10.1, step 3).  Without it, c clamps
 * silu(g)*u, the reading of the mid-size workload's "SwiGLU output clamped".  Ignored when
 * there is no clamp. */
#define MEGA_MOE_FLAG_CLAMP_INPUTS 4u
/* flags bit 3: SiLU with the device library's expf and an IEEE division (the pages' fast_math =
 * false, design page section 10.1 step 3); by default the hardware exp and reciprocal
 * instructions (fast_math = true), float32 to a few ulp. */
#define MEGA_MOE_FLAG_PRECISE_SILU 8u
/* flags bit 4 (per-32 recipes only; INVALID_ARG with MEGA_MOE_RECIPE_FP8_B128): l1_sf and l2_sf
 * are in the K-major layout that mega_moe_transform_weight_scales() writes, [E][K/128][rows]
 * 32-bit words, each the four UE8M0 codes of one row's 128-K block (K = H, rows = 2I for l1_sf;
 * K = I, rows = H for l2_sf).  Same sizes as the row-major layout; the results are identical. */
#define MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR 16u
/* flags bit 7 (MEGA_MOE_RECIPE_MXFP4W_B32 only; INVALID_ARG with the other recipes): l1_w and
 * l2_w are in the row-pair layout that mega_moe_transform_weights() writes: for each pair of
 * weight rows (2q, 2q + 1) of an expert and each 128-K block kb, the 64 bytes of row 2q's block
 * followed by the 64 bytes of row 2q + 1's, so one K block of two rows is one 128-byte line
 * (offset (q * K/128 + kb) * 128 + (row % 2) * 64 within the expert).  Same sizes as the
 * row-major layout; the results are identical. */
#define MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED 128u
/* flags bit 5 (MEGA_MOE_RECIPE_FP8_B128 only; INVALID_ARG with the per-32 recipes): the SM90
 * design's per-64 intermediate scales.  The L1 epilogue re-quantises the SwiGLU output with one
 * float scale amax/448 per 64 channels instead of per 128, and the L2 GEMM sums each 128-K block
 * of w2 as two 64-K halves, each scaled by its own intermediate scale times the block's weight
 * scale (design page "MegaMoE SM90 Implementation Design", section 5.4, L2 per-64 dual-half
 * scale application; section 10.1 step 6, the per-64 scale layout).  The inter_sf view is then
 * [I/64, T*k] float32. */
#define MEGA_MOE_FLAG_INTER_SF64 32u
/* flags bit 6: the fused forward, the whole layer (dispatch, L1 GEMM + SwiGLU, L2 GEMM, combine)
 * in one persistent cooperative launch, one workgroup per compute unit (design page "MegaMoE SM90
 * Implementation Design", section 3.3, the fused kernel pipeline; section 14.3, cross-phase
 * synchronisation: the L2 GEMM of a pool tile starts as soon as every L1 slab of that tile is
 * stored, while other L1 work still runs).  Same results bit for bit as the split forward.  Every
 * expert runs in the large-M class: INVALID_ARG with MEGA_MOE_FLAG_TILE_SMALL or for a problem too
 * large for the large-M kernels' 32-bit offsets.  Fused forwards on one GPU must not overlap
 * (each needs every compute unit; cooperative launches are not run side by side).  The events of
 * mega_moe_forward_profiled are all recorded after the one launch except events[0]. */
#define MEGA_MOE_FLAG_FUSED 64u

enum {
  MEGA_MOE_OK = 0,
  MEGA_MOE_ERR_INVALID_ARG = -1,        /* a field out of range or not a multiple of 128 */
  MEGA_MOE_ERR_NULL_POINTER = -2,       /* a required pointer is NULL */
  MEGA_MOE_ERR_MISALIGNED = -3,         /* a pointer is not 16-byte aligned */
  MEGA_MOE_ERR_WORKSPACE_TOO_SMALL = -4,/* workspace_bytes < mega_moe_workspace_size() */
  MEGA_MOE_ERR_UNSUPPORTED_DEVICE = -5, /* the current device is not gfx950 */
  MEGA_MOE_ERR_HIP = -6,                /* a HIP runtime call or launch failed */
  MEGA_MOE_ERR_SCRATCH_TOO_SMALL = -7   /* mega_moe_forward_noalloc: the problem needs more workspace
                                           than the library's static scratch holds */
};

typedef struct {
  int64_t num_tokens;    /* T >= 0; T == 0 is a valid no-op */
  int32_t hidden;        /* H in (0, 16384], multiple of 128 */
  int32_t intermediate;  /* I in (0, 16384], multiple of 128 */
  int32_t num_experts;   /* E in [1, 8192]; an always-on shared expert is one more expert */
  int32_t topk;          /* k in [1, 64] columns of topk_idx / topk_w */
  int32_t recipe;        /* mega_moe_recipe */
  float swiglu_clamp;    /* 0 or +inf: no clamp; c > 0: silu(g)*u clamped to [-c, c]
                            before the top-k weight multiplies it (or, with
                            MEGA_MOE_FLAG_CLAMP_INPUTS, gate and up clamped before SiLU) */
  uint32_t flags;        /* MEGA_MOE_FLAG_* */
} mega_moe_problem;

/* Device pointers into a workspace after a forward call (for inspection and tests): the buffer
   views the pages' buffer query hands back for correctness checks of the dispatch state (research
   report "MegaMoE on SM100/SM90", section 6.4, the buffer-size query that lays out the workspace,
   pools and combine buffer and returns tensor views of them; development log of the SM90 port,
   first entry, the Phase 1 buffer query returning its views).  Every pointer lies inside the
   caller's workspace; nothing is allocated. */
typedef struct {
  const int32_t* expert_count;   /* [E]   rows per expert */
  const int32_t* expert_offset;  /* [E+1] exclusive prefix of expert_count */
  const int32_t* pool_src;       /* [T*k] pool row -> pair t*k+j (first offset[E] valid) */
  const int32_t* pair_pos;       /* [T*k] pair -> pool row, -1 when masked or invalid */
  const int32_t* num_invalid;    /* [1]   ids >= E seen in topk_idx */
  const uint8_t* inter_q;        /* [T*k, I] E4M3 intermediate per pool row */
  const void* inter_sf;          /* K-major: [I/128, T*k] f32 | [I/128, T*k, 4] u8 (the four
                                    per-32 codes of one 128 block); pool row r, block b at b*T*k+r;
                                    with MEGA_MOE_FLAG_INTER_SF64 [I/64, T*k] f32 */
  const uint16_t* slot;          /* [T*k, H] BF16 L2 output per pair (t*k+j order) */
} mega_moe_views;

/* Bytes of workspace a forward call of this problem needs: the separate sizing query of the
   pages' interface (research report "MegaMoE on SM100/SM90", section 6.4, key APIs: the buffer-size
   query; design page "MegaMoE SM90 Implementation Design", section 16.1, the SM90 entry's size
   query registered beside the forward).  The workspace holds the dispatch counts and offsets,
   the pool metadata, the GEMM tile lists, the pool-order activation scales, the E4M3 intermediate
   with its scales and the BF16 slot rows, each region 256-byte aligned.  A forward accepts any
   workspace of at least this many bytes (a >= check, not ==).
   Errors: NULL_POINTER (p or bytes_out), INVALID_ARG (a field out of range); *bytes_out is
   written only on success. */
int mega_moe_workspace_size(const mega_moe_problem* p, size_t* bytes_out);

/* The layer forward; see the top of this file for the arithmetic and the layouts.
   stream: a hipStream_t, NULL for the default stream. */
int mega_moe_forward(const mega_moe_problem* p,
                     const void* x, const void* x_sf,
                     const int32_t* topk_idx, const float* topk_w,
                     const void* l1_w, const void* l1_sf,
                     const void* l2_w, const void* l2_sf,
                     void* y, void* workspace, size_t workspace_bytes,
                     void* stream);

/* mega_moe_forward, additionally recording caller-created hipEvent_t handles on `stream` at
   the phase boundaries, for timing each kernel of the layer on the stream it runs on:
     events[0] before dispatch, [1] after dispatch (before L1), [2] after the L1 GEMM,
     [3] after the L2 GEMM, [4] after the combine.
   num_events in [0, MEGA_MOE_NUM_PHASE_EVENTS]; events beyond num_events are not recorded.
   The caller owns the events.  With T == 0 nothing is recorded. */
#define MEGA_MOE_NUM_PHASE_EVENTS 5
int mega_moe_forward_profiled(const mega_moe_problem* p,
                              const void* x, const void* x_sf,
                              const int32_t* topk_idx, const float* topk_w,
                              const void* l1_w, const void* l1_sf,
                              const void* l2_w, const void* l2_sf,
                              void* y, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int num_events);

/* mega_moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
   tight serving loops, harnesses that forbid allocation): no workspace argument; the call uses
   the library's own static device scratch of MEGA_MOE_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU,
   which each GPU the library runs on holds until the process ends.  Problems whose
   mega_moe_workspace_size exceeds it are rejected with MEGA_MOE_ERR_SCRATCH_TOO_SMALL before
   anything is enqueued (the decode shape T = 128, H = 7168, I = 2048, E = 256, k = 8 needs
   16.3 MiB; about 250 tokens fit at that shape).  The call allocates, frees and synchronises
   nothing.  Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
   different streams, or from several threads) race and must be ordered by the caller; the scratch
   keeps the last call's contents, and each call re-initialises everything it reads.  Same
   arguments, results and errors as mega_moe_forward otherwise (bit-identical y). */
#define MEGA_MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int mega_moe_forward_noalloc(const mega_moe_problem* p,
                             const void* x, const void* x_sf,
                             const int32_t* topk_idx, const float* topk_w,
                             const void* l1_w, const void* l1_sf,
                             const void* l2_w, const void* l2_sf,
                             void* y, void* stream);

/* mega_moe_forward that also adds each expert's received row count (its pool size: pairs
   routed to it, masked and invalid slots excluded) of this call to the caller's device array
   cumulative_expert_recv_stats[E] (int32), the per-expert receive statistics of the research
   report's and the design page's interface (`cumulative_local_expert_recv_stats`; design page
   section 10.2).  The array is never cleared by the library; NULL skips the update.  The add
   runs on `stream` after the dispatch counts are known; calls that share one array must be
   ordered on one stream (concurrent calls race on it). */
int mega_moe_forward_stats(const mega_moe_problem* p,
                           const void* x, const void* x_sf,
                           const int32_t* topk_idx, const float* topk_w,
                           const void* l1_w, const void* l1_sf,
                           const void* l2_w, const void* l2_sf,
                           void* y, void* workspace, size_t workspace_bytes,
                           int32_t* cumulative_expert_recv_stats, void* stream);

/* The per-32 recipes' weight-scale transform, run once when the weights are loaded (the pages'
   model-load weight transform re-lays the UE8M0 scale factors out for the kernels' loads: design
   page "MegaMoE SM90 Implementation Design", section 15; research report section 6.2).  Reads the
   row-major l1_sf [E, 2I, H/32] and l2_sf [E, H, I/32] codes and writes the same codes K-major
   into l1_sf_kmajor [E, H/128, 2I, 4] and l2_sf_kmajor [E, I/128, H, 4] (caller-allocated, same
   sizes, distinct from the inputs), for forward calls with MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR, whose
   GEMMs then fetch one K block's scales of 64 consecutive rows as 256 contiguous bytes instead of
   64 scattered words.  Enqueued on `stream` (a hipStream_t, NULL for the default stream).
   Errors: INVALID_ARG for the FP8_B128 recipe, an invalid problem or overlapping buffers;
   NULL_POINTER; MISALIGNED (16 bytes); UNSUPPORTED_DEVICE; HIP. */
int mega_moe_transform_weight_scales(const mega_moe_problem* p, const void* l1_sf, const void* l2_sf,
                                     void* l1_sf_kmajor, void* l2_sf_kmajor, void* stream);

/* The MXFP4 recipe's weight transform, run once when the weights are loaded (the same model-load
   weight re-layout: design page "MegaMoE SM90 Implementation Design", section 15; research report
   section 6.2).  Reads the row-major E2M1 weights l1_w [E, 2I, H/2] and l2_w [E, H, I/2] bytes and
   writes them in the row-pair layout of MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED into l1_w_paired and
   l2_w_paired (caller-allocated, same sizes, distinct from the inputs): a 128-K block of an E2M1
   row is half a 128-byte line, and in this layout the GEMMs fetch whole lines (and can stream the
   weights of single-tile experts past the caches).  Enqueued on `stream` (NULL: default stream).
   Errors: INVALID_ARG for a recipe other than MXFP4W_B32, an invalid problem or overlapping
   buffers; NULL_POINTER; MISALIGNED (16 bytes); UNSUPPORTED_DEVICE; HIP. */
int mega_moe_transform_weights(const mega_moe_problem* p, const void* l1_w, const void* l2_w,
                               void* l1_w_paired, void* l2_w_paired, void* stream);

/* Fill *out with device pointers into `workspace` for problem p (the layout of
   mega_moe_workspace_size; see mega_moe_views).  The views stay valid while the workspace does and
   hold the last forward's results until the next call that uses the workspace.
   Errors: NULL_POINTER (p, workspace or out), INVALID_ARG (a field out of range). */
int mega_moe_workspace_views(const mega_moe_problem* p, const void* workspace,
                             mega_moe_views* out);

/* Diagnostic: n_tiles independent 16 x 16 block dot products over one 128-long K block, computed
   with the same matrix-core instruction, operand layout and scale encoding the grouped GEMMs use,
   so that the error of the hardware block sum against the exact sum of its products can be
   measured (it bounds how far an intermediate value, and so its E4M3 code, may lie from the
   exactly summed one; design page "MegaMoE SM90 Implementation Design", section 20.3, tolerance,
   and the development log entry of 2026-06-18 01:10 on accumulator error and E4M3 code flips).
     out[t][m][n] = sum_{k<128} A[t][m][k] * B[t][n][k] * 2^(sa[t][m][k/32]-127) * 2^(sb[t][n][k/32]-127)
   fmt 0: A, B E4M3FN bytes [n_tiles][16][128], unit scales (scale arrays ignored, may be NULL);
   fmt 1: A E2M1 nibbles [n_tiles][16][64] (low nibble = even k), B E4M3FN [n_tiles][16][128],
          UE8M0 scales sa, sb [n_tiles][16][4];
   fmt 2: A, B E4M3FN [n_tiles][16][128] with UE8M0 scales sa, sb [n_tiles][16][4].
   out: float32 [n_tiles][16][16].  Device pointers, 16-byte aligned (scales: any alignment).
   Enqueued on `stream` (a hipStream_t, NULL for the default stream).  Errors: INVALID_ARG (fmt or
   n_tiles), NULL_POINTER, MISALIGNED, UNSUPPORTED_DEVICE, HIP. */
int mega_moe_diag_mfma_block_sums(int fmt, const void* a, const void* b, const void* a_scale,
                                  const void* b_scale, float* out, int n_tiles, void* stream);

/* Static text for a status code. */
const char* mega_moe_strerror(int status);

/* MEGA_MOE_ABI_VERSION of the loaded library. */
int mega_moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MEGA_MOE_H */
