// C ABI of libmegamoe: argument validation, workspace carving and the launch sequence.
// No allocation, no synchronisation: every kernel is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "mega_moe.h"
#include "mm_common.h"

#define MM_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

struct Layout {
  size_t hdr, count, offset, blk, blk_inv, pair_pos, pool_src, w_pool, tiles_s, tiles_l, x_sf_pool,
      inter_q, inter_sf, slot, tile_done, total;
  int P, NB, max_tiles_s, max_tiles_l;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int check_problem(const mega_moe_problem* p) {
  if (!p) return MEGA_MOE_ERR_NULL_POINTER;
  if (p->num_tokens < 0) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->hidden <= 0 || p->hidden % 128 || p->hidden > 16384) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->intermediate <= 0 || p->intermediate % 128 || p->intermediate > 16384) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->num_experts < 1 || p->num_experts > mm::kMaxExperts) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->topk < 1 || p->topk > mm::kMaxTopk) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->recipe != MEGA_MOE_RECIPE_FP8_B128 && p->recipe != MEGA_MOE_RECIPE_MXFP4W_B32 &&
      p->recipe != MEGA_MOE_RECIPE_MXFP8_B32)
    return MEGA_MOE_ERR_INVALID_ARG;
  if (std::isnan(p->swiglu_clamp) || p->swiglu_clamp < 0.f) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->flags & ~(MEGA_MOE_FLAG_TILE_MASK | MEGA_MOE_FLAG_CLAMP_INPUTS | MEGA_MOE_FLAG_PRECISE_SILU |
                   MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR | MEGA_MOE_FLAG_INTER_SF64 | MEGA_MOE_FLAG_FUSED |
                   MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED))
    return MEGA_MOE_ERR_INVALID_ARG;
  // the row-pair weight layout exists for the E2M1 weights only
  if ((p->flags & MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED) && p->recipe != MEGA_MOE_RECIPE_MXFP4W_B32)
    return MEGA_MOE_ERR_INVALID_ARG;
  // the fused forward runs the large-M GEMMs only
  if ((p->flags & MEGA_MOE_FLAG_FUSED) && (p->flags & MEGA_MOE_FLAG_TILE_MASK) == MEGA_MOE_FLAG_TILE_SMALL)
    return MEGA_MOE_ERR_INVALID_ARG;
  // per-64 float intermediate scales exist for the float-scale recipe only
  if ((p->flags & MEGA_MOE_FLAG_INTER_SF64) && p->recipe != MEGA_MOE_RECIPE_FP8_B128)
    return MEGA_MOE_ERR_INVALID_ARG;
  // the K-major weight-scale layout exists for the per-32 (UE8M0) recipes only
  if ((p->flags & MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR) && p->recipe == MEGA_MOE_RECIPE_FP8_B128)
    return MEGA_MOE_ERR_INVALID_ARG;
  if ((p->flags & MEGA_MOE_FLAG_TILE_MASK) == MEGA_MOE_FLAG_TILE_MASK) return MEGA_MOE_ERR_INVALID_ARG;
  if (p->num_tokens * (int64_t)p->topk > (int64_t)(INT_MAX / 2)) return MEGA_MOE_ERR_INVALID_ARG;
  return MEGA_MOE_OK;
}

Layout make_layout(const mega_moe_problem* p) {
  Layout L{};
  const size_t T = (size_t)p->num_tokens, H = p->hidden, I = p->intermediate, E = p->num_experts;
  const size_t P = T * (size_t)p->topk;
  L.P = (int)P;
  L.NB = (int)((P + mm::kRouteBlock - 1) / mm::kRouteBlock);
  const size_t ts = P ? std::min(P, (P + mm::kSmallRows - 1) / mm::kSmallRows + E) : 0;
  const size_t tl = P ? std::min(P, (P + mm::kLargeRows - 1) / mm::kLargeRows + E) : 0;
  L.max_tiles_s = (int)ts;
  L.max_tiles_l = (int)tl;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.hdr = take(mm::kHdrWords * 4);
  L.count = take(E * 4);
  L.offset = take((E + 1) * 4);
  L.blk = take((size_t)L.NB * E * 4);
  L.blk_inv = take((size_t)L.NB * 4);
  L.pair_pos = take(P * 4);
  L.pool_src = take(P * 4);
  L.w_pool = take(P * 4);
  L.tiles_s = take(ts * 8);
  L.tiles_l = take(tl * 8);
  L.x_sf_pool = take(P * (H / 128) * 4);
  L.inter_q = take(P * I);
  const size_t inter_groups = (p->flags & MEGA_MOE_FLAG_INTER_SF64) ? I / 64 : I / 128;
  L.inter_sf = take(p->recipe == MEGA_MOE_RECIPE_FP8_B128 ? P * inter_groups * 4 : P * (I / 32));
  L.slot = take(P * H * 2);
  L.tile_done = take((tl + 1) * 4);
  L.total = o;
  return L;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MEGA_MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MEGA_MOE_ERR_UNSUPPORTED_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MEGA_MOE_ERR_HIP;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MEGA_MOE_OK : MEGA_MOE_ERR_UNSUPPORTED_DEVICE;
}

// Per-device compute-unit count (0 = not yet queried).
std::atomic<int> g_num_cus[64];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = g_num_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_num_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

inline bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

}  // namespace

MM_EXPORT int mega_moe_abi_version(void) { return MEGA_MOE_ABI_VERSION; }

MM_EXPORT const char* mega_moe_strerror(int status) {
  switch (status) {
    case MEGA_MOE_OK: return "ok";
    case MEGA_MOE_ERR_INVALID_ARG: return "invalid argument (a problem field is out of range)";
    case MEGA_MOE_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MEGA_MOE_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case MEGA_MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mega_moe_workspace_size()";
    case MEGA_MOE_ERR_UNSUPPORTED_DEVICE: return "the current device is not gfx950 (MI355X)";
    case MEGA_MOE_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case MEGA_MOE_ERR_SCRATCH_TOO_SMALL:
      return "the problem needs more workspace than the static scratch of mega_moe_forward_noalloc (32 MiB)";
    default: return "unknown status";
  }
}

MM_EXPORT int mega_moe_workspace_size(const mega_moe_problem* p, size_t* bytes_out) {
  const int st = check_problem(p);
  if (st) return st;
  if (!bytes_out) return MEGA_MOE_ERR_NULL_POINTER;
  *bytes_out = make_layout(p).total;
  return MEGA_MOE_OK;
}

MM_EXPORT int mega_moe_workspace_views(const mega_moe_problem* p, const void* workspace,
                                       mega_moe_views* out) {
  const int st = check_problem(p);
  if (st) return st;
  if (!workspace || !out) return MEGA_MOE_ERR_NULL_POINTER;
  const Layout L = make_layout(p);
  const uint8_t* b = static_cast<const uint8_t*>(workspace);
  out->expert_count = reinterpret_cast<const int32_t*>(b + L.count);
  out->expert_offset = reinterpret_cast<const int32_t*>(b + L.offset);
  out->pool_src = reinterpret_cast<const int32_t*>(b + L.pool_src);
  out->pair_pos = reinterpret_cast<const int32_t*>(b + L.pair_pos);
  out->num_invalid = reinterpret_cast<const int32_t*>(b + L.hdr) + mm::kHdrInvalid;
  out->inter_q = b + L.inter_q;
  out->inter_sf = b + L.inter_sf;
  out->slot = reinterpret_cast<const uint16_t*>(b + L.slot);
  return MEGA_MOE_OK;
}

namespace {
int forward_impl(const mega_moe_problem* p, const void* x, const void* x_sf,
                 const int32_t* topk_idx, const float* topk_w, const void* l1_w,
                 const void* l1_sf, const void* l2_w, const void* l2_sf, void* y,
                 void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                 int num_events, int32_t* recv_stats) {
  int st = check_problem(p);
  if (st) return st;
  const Layout L = make_layout(p);
  if (p->num_tokens == 0) return MEGA_MOE_OK;
  const void* ptrs[] = {x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace};
  for (const void* q : ptrs)
    if (!q) return MEGA_MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (misaligned(q)) return MEGA_MOE_ERR_MISALIGNED;
  if (workspace_bytes < L.total) return MEGA_MOE_ERR_WORKSPACE_TOO_SMALL;
  st = check_device();
  if (st) return st;

  mm::Args a{};
  a.x = static_cast<const uint8_t*>(x);
  a.x_sf = x_sf;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.l1_w = static_cast<const uint8_t*>(l1_w);
  a.l1_sf = l1_sf;
  a.l2_w = static_cast<const uint8_t*>(l2_w);
  a.l2_sf = l2_sf;
  a.y = static_cast<uint16_t*>(y);
  a.recv_stats = recv_stats;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  a.hdr = reinterpret_cast<int32_t*>(w + L.hdr);
  a.count = reinterpret_cast<int32_t*>(w + L.count);
  a.offset = reinterpret_cast<int32_t*>(w + L.offset);
  a.blk = reinterpret_cast<int32_t*>(w + L.blk);
  a.blk_inv = reinterpret_cast<int32_t*>(w + L.blk_inv);
  a.pair_pos = reinterpret_cast<int32_t*>(w + L.pair_pos);
  a.pool_src = reinterpret_cast<int32_t*>(w + L.pool_src);
  a.w_pool = reinterpret_cast<float*>(w + L.w_pool);
  a.tiles_s = reinterpret_cast<int2*>(w + L.tiles_s);
  a.tiles_l = reinterpret_cast<int2*>(w + L.tiles_l);
  a.x_sf_pool = w + L.x_sf_pool;
  a.inter_q = w + L.inter_q;
  a.inter_sf = w + L.inter_sf;
  a.slot = reinterpret_cast<uint16_t*>(w + L.slot);
  a.tile_done = reinterpret_cast<int32_t*>(w + L.tile_done);
  a.T = (int)p->num_tokens;
  a.H = p->hidden;
  a.I = p->intermediate;
  a.E = p->num_experts;
  a.k = p->topk;
  a.P = L.P;
  a.NB = L.NB;
  a.recipe = p->recipe;
  a.clamp = std::isinf(p->swiglu_clamp) ? 0.f : p->swiglu_clamp;
  a.clamp_inputs = (p->flags & MEGA_MOE_FLAG_CLAMP_INPUTS) != 0;
  a.precise_silu = (p->flags & MEGA_MOE_FLAG_PRECISE_SILU) != 0;
  a.wsf_kmajor = (p->flags & MEGA_MOE_FLAG_WEIGHT_SF_KMAJOR) != 0;
  a.w_paired = (p->flags & MEGA_MOE_FLAG_WEIGHT_E2M1_PAIRED) != 0;
  a.inter64 = (p->flags & MEGA_MOE_FLAG_INTER_SF64) != 0;
  a.tile_mode = (int)(p->flags & MEGA_MOE_FLAG_TILE_MASK);
  a.large_min_rows = mm::kLargeMinRows;
  a.max_tiles_s = L.max_tiles_s;
  a.max_tiles_l = L.max_tiles_l;
  // the large-M kernels address activations, the intermediate and the pool-order scale words
  // through 32-bit buffer descriptors and offsets: larger problems go to the small-M kernels
  if (!mm::large_kernels_addressable(a.T, a.H, a.I, a.k)) a.tile_mode = 1;
  const int cus = device_cus();
  if (cus <= 0) return MEGA_MOE_ERR_HIP;
  a.large_grid = cus < 8 ? 8 : cus / 8 * 8;
  const bool fused = (p->flags & MEGA_MOE_FLAG_FUSED) != 0;
  // the fused forward needs every expert in the large-M class, which needs 32-bit offsets
  if (fused && a.tile_mode == 1) return MEGA_MOE_ERR_INVALID_ARG;
  a.quad = a.recipe == MEGA_MOE_RECIPE_MXFP4W_B32 && a.tile_mode == 0 && !fused;
  a.quad_grid = 2 * a.large_grid;

  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> bool {
    return i >= num_events || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };
  if (!mark(0)) return MEGA_MOE_ERR_HIP;
  if (fused) {   // one launch: every phase event after it
    if (mm::launch_fused(a, s) != hipSuccess) return MEGA_MOE_ERR_HIP;
    for (int i = 1; i < MEGA_MOE_NUM_PHASE_EVENTS; ++i)
      if (!mark(i)) return MEGA_MOE_ERR_HIP;
    return MEGA_MOE_OK;
  }
  if (mm::launch_route(a, s) != hipSuccess || !mark(1)) return MEGA_MOE_ERR_HIP;
  if (mm::launch_l1_small(a, s) != hipSuccess || mm::launch_l1_large(a, s) != hipSuccess || !mark(2))
    return MEGA_MOE_ERR_HIP;
  if (mm::launch_l2_small(a, s) != hipSuccess || mm::launch_l2_large(a, s) != hipSuccess || !mark(3))
    return MEGA_MOE_ERR_HIP;
  if (mm::launch_combine(a, s) != hipSuccess || !mark(4)) return MEGA_MOE_ERR_HIP;
  return MEGA_MOE_OK;
}
}  // namespace

MM_EXPORT int mega_moe_forward(const mega_moe_problem* p, const void* x, const void* x_sf,
                               const int32_t* topk_idx, const float* topk_w, const void* l1_w,
                               const void* l1_sf, const void* l2_w, const void* l2_sf, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(p, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace,
                      workspace_bytes, stream, nullptr, 0, nullptr);
}

// ----------------------------------------------------------------------------- no-alloc forward
// The workspace of mega_moe_forward_noalloc: a static device array, one copy per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to the kernels.
static __device__ __align__(256) uint8_t scratch[MEGA_MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up)

// The current device's scratch address, or null when the lookup fails.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

MM_EXPORT int mega_moe_forward_noalloc(const mega_moe_problem* p, const void* x, const void* x_sf,
                                       const int32_t* topk_idx, const float* topk_w, const void* l1_w,
                                       const void* l1_sf, const void* l2_w, const void* l2_sf, void* y,
                                       void* stream) {
  int st = check_problem(p);
  if (st) return st;
  if (p->num_tokens == 0) return MEGA_MOE_OK;
  if (make_layout(p).total > (size_t)MEGA_MOE_NOALLOC_SCRATCH_BYTES) return MEGA_MOE_ERR_SCRATCH_TOO_SMALL;
  st = check_device();
  if (st) return st;
  void* ws = device_scratch();
  if (!ws) return MEGA_MOE_ERR_HIP;
  return forward_impl(p, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, ws,
                      (size_t)MEGA_MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0, nullptr);
}

MM_EXPORT int mega_moe_forward_stats(const mega_moe_problem* p, const void* x, const void* x_sf,
                                     const int32_t* topk_idx, const float* topk_w, const void* l1_w,
                                     const void* l1_sf, const void* l2_w, const void* l2_sf, void* y,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t* cumulative_expert_recv_stats, void* stream) {
  if ((reinterpret_cast<uintptr_t>(cumulative_expert_recv_stats) & 3u) != 0) return MEGA_MOE_ERR_MISALIGNED;
  return forward_impl(p, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace,
                      workspace_bytes, stream, nullptr, 0, cumulative_expert_recv_stats);
}

MM_EXPORT int mega_moe_forward_profiled(const mega_moe_problem* p, const void* x, const void* x_sf,
                                        const int32_t* topk_idx, const float* topk_w,
                                        const void* l1_w, const void* l1_sf, const void* l2_w,
                                        const void* l2_sf, void* y, void* workspace,
                                        size_t workspace_bytes, void* stream, void* const* events,
                                        int num_events) {
  if (num_events < 0 || num_events > MEGA_MOE_NUM_PHASE_EVENTS || (num_events > 0 && !events))
    return MEGA_MOE_ERR_INVALID_ARG;
  for (int i = 0; i < num_events; ++i)
    if (!events[i]) return MEGA_MOE_ERR_NULL_POINTER;
  return forward_impl(p, x, x_sf, topk_idx, topk_w, l1_w, l1_sf, l2_w, l2_sf, y, workspace,
                      workspace_bytes, stream, events, num_events, nullptr);
}

MM_EXPORT int mega_moe_transform_weight_scales(const mega_moe_problem* p, const void* l1_sf, const void* l2_sf,
                                               void* l1_sf_kmajor, void* l2_sf_kmajor, void* stream) {
  int st = check_problem(p);
  if (st) return st;
  if (p->recipe == MEGA_MOE_RECIPE_FP8_B128) return MEGA_MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {l1_sf, l2_sf, l1_sf_kmajor, l2_sf_kmajor};
  for (const void* q : ptrs)
    if (!q) return MEGA_MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (misaligned(q)) return MEGA_MOE_ERR_MISALIGNED;
  const int H = p->hidden, I = p->intermediate, E = p->num_experts;
  // out of place only: neither output may overlap an input or the other output
  const auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
  };
  const size_t n1 = (size_t)E * 2 * I * (H / 32), n2 = (size_t)E * H * (I / 32);
  if (overlap(l1_sf_kmajor, n1, l1_sf, n1) || overlap(l1_sf_kmajor, n1, l2_sf, n2) ||
      overlap(l2_sf_kmajor, n2, l1_sf, n1) || overlap(l2_sf_kmajor, n2, l2_sf, n2) ||
      overlap(l1_sf_kmajor, n1, l2_sf_kmajor, n2))
    return MEGA_MOE_ERR_INVALID_ARG;
  st = check_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mm::launch_sf_kmajor(static_cast<const uint32_t*>(l1_sf), static_cast<uint32_t*>(l1_sf_kmajor), E, 2 * I,
                           H / 128, s) != hipSuccess ||
      mm::launch_sf_kmajor(static_cast<const uint32_t*>(l2_sf), static_cast<uint32_t*>(l2_sf_kmajor), E, H,
                           I / 128, s) != hipSuccess)
    return MEGA_MOE_ERR_HIP;
  return MEGA_MOE_OK;
}

MM_EXPORT int mega_moe_transform_weights(const mega_moe_problem* p, const void* l1_w, const void* l2_w,
                                         void* l1_w_paired, void* l2_w_paired, void* stream) {
  int st = check_problem(p);
  if (st) return st;
  if (p->recipe != MEGA_MOE_RECIPE_MXFP4W_B32) return MEGA_MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {l1_w, l2_w, l1_w_paired, l2_w_paired};
  for (const void* q : ptrs)
    if (!q) return MEGA_MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (misaligned(q)) return MEGA_MOE_ERR_MISALIGNED;
  const int H = p->hidden, I = p->intermediate, E = p->num_experts;
  const auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
  };
  const size_t n1 = (size_t)E * 2 * I * (H / 2), n2 = (size_t)E * H * (I / 2);
  if (overlap(l1_w_paired, n1, l1_w, n1) || overlap(l1_w_paired, n1, l2_w, n2) ||
      overlap(l2_w_paired, n2, l1_w, n1) || overlap(l2_w_paired, n2, l2_w, n2) ||
      overlap(l1_w_paired, n1, l2_w_paired, n2))
    return MEGA_MOE_ERR_INVALID_ARG;
  st = check_device();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mm::launch_e2m1_pairs(static_cast<const uint8_t*>(l1_w), static_cast<uint8_t*>(l1_w_paired),
                            (size_t)E * I, H / 128, s) != hipSuccess ||
      mm::launch_e2m1_pairs(static_cast<const uint8_t*>(l2_w), static_cast<uint8_t*>(l2_w_paired),
                            (size_t)E * H / 2, I / 128, s) != hipSuccess)
    return MEGA_MOE_ERR_HIP;
  return MEGA_MOE_OK;
}

MM_EXPORT int mega_moe_diag_mfma_block_sums(int fmt, const void* a, const void* b, const void* a_scale,
                                            const void* b_scale, float* out, int n_tiles, void* stream) {
  if (fmt < 0 || fmt > 2 || n_tiles < 0) return MEGA_MOE_ERR_INVALID_ARG;
  if (n_tiles == 0) return MEGA_MOE_OK;
  if (!a || !b || !out || (fmt != 0 && (!a_scale || !b_scale))) return MEGA_MOE_ERR_NULL_POINTER;
  if (misaligned(a) || misaligned(b) || misaligned(out)) return MEGA_MOE_ERR_MISALIGNED;
  const int st = check_device();
  if (st) return st;
  if (mm::launch_diag_mfma(fmt, static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b),
                           static_cast<const uint8_t*>(a_scale), static_cast<const uint8_t*>(b_scale), out,
                           n_tiles, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MEGA_MOE_ERR_HIP;
  return MEGA_MOE_OK;
}
