// The fused forward: dispatch -> L1 GEMM + SwiGLU -> L2 GEMM -> combine in one persistent,
// cooperatively launched kernel (design page "MegaMoE SM90 Implementation Design", section 3.3,
// the fused kernel pipeline; section 14.3, the cross-phase synchronisation: an arrival count
// releases the L1 work, a per-block arrival releases each L2 block, and a barrier precedes the
// combine; research report "MegaMoE on SM100/SM90", section 4.1, the single-kernel data flow).
//
// One workgroup per CU (the large-M GEMM workgroup: 8 waves, the whole LDS), all co-resident
// (cooperative launch).  The phases run the same device code as the stand-alone kernels, so the
// results are bit-identical to the split forward:
//   A. count: the dispatch blocks' histograms, spread over the workgroups;
//   B. scan: the last workgroup to finish A computes offsets and tile lists (the others wait);
//   C. scatter: pool order, source metadata, pool-order activation scales, one thread per pair;
//      then a grid barrier;
//   D. L1 items (as the stand-alone L1 kernel); a workgroup done with its L1 items publishes
//      their intermediate rows and adds one to each item's tile's arrival count;
//   E. L2 items (as the stand-alone L2 kernel, MXFP4 tiles included); an item first waits until
//      its tile's arrival count covers every L1 slab of the tile, so L2 work starts while the last
//      L1 items still run (the workgroups with no L1 item left in the last round take L2 items at
//      once), instead of after a kernel boundary;
//   F. a grid barrier, then the combine.
//
// Cross-workgroup order: a workgroup's writes are published by every wave waiting for its own
// stores to be acknowledged, a workgroup barrier, and one agent-scope release fence (the L2 write
// back) before an agent-scope atomic add; a waiter spins on the counter with agent-scope loads and
// follows with an agent-scope acquire fence (L1 and L2 invalidation) before it reads the data.
// Every wait is bounded: a wait that runs out of spins records a fault (workspace header word
// kHdrFusedFault and a sticky library flag that makes later fused launches exit at once) and
// carries on, so a broken invariant cannot hang the GPU; the results of such a launch are invalid.
#include "mm_large_dev.h"
#include "mm_route_dev.h"

namespace mm {

namespace {

// The grid barriers' counters: monotonic, in device memory owned by the library (zero when the
// module loads; one copy per GPU).  Every launch adds exactly G (its workgroup count, fixed per
// device) to words 0, 2 and 3 and exactly 1 to word 1, so at the start of a launch word 0 is a
// multiple of G and word 0 / G = word 1 = the number of earlier launches: each workgroup learns
// that launch index from its own add to word 0 and derives every target from it.  Fused launches
// on one GPU must not overlap (cooperative launches do not).
static __device__ unsigned long long g_sync[4];
static __device__ int g_fault;                  // sticky: a bounded wait ran out of spins

constexpr long kSpinLimit = 1L << 22;           // a few seconds: far beyond any legitimate wait

// Thread 0: wait until *w >= target, then acquire; false when the spins ran out.
__device__ __forceinline__ bool wait_at_least(const unsigned long long* w, unsigned long long target) {
  for (long i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}
__device__ __forceinline__ bool wait_at_least(const int* w, int target) {
  for (long i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Every wave's stores acknowledged, then (thread 0) the agent-scope release: the workgroup's
// writes so far are visible to any workgroup that acquires after observing the next add.
__device__ __forceinline__ void publish() {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

__device__ __forceinline__ void record_fault(int* hdr) {
  __hip_atomic_store(&g_fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&hdr[kHdrFusedFault], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier on counter w of launch `launch`: publish, add 1, wait for all G adds.
__device__ __forceinline__ void grid_barrier(int* hdr, int w, unsigned long long launch) {
  publish();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&g_sync[w], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!wait_at_least(&g_sync[w], (launch + 1) * gridDim.x)) record_fault(hdr);
  }
  __syncthreads();
}

// After a workgroup's last L1 item: publish its intermediate rows and scales once (one L2 write
// back for all its items), then add one to the arrival count done[tile] of each of its items'
// tiles, replaying its item rounds, and its item count to done[n], the count of all L1 items
// stored.  (Publishing after every item instead, so that a tile's arrival count grows item by
// item, costs a write back and a store round trip per item: measured slower at every workload.)
template <int R>
__device__ __forceinline__ void l1_arrive(const Args& a) {
  publish();
  if (threadIdx.x != 0) return;
  const ItemSpace sp = item_space<R, true>(a);
  const ItemRounds rs(sp.count());
  int items = 0;                                  // in slabs: a wide item counts for two
  for (int r = 0;; ++r) {
    const int q = rs.item(r);
    if (q < 0) break;
    const ItemPos ip = item_pos(q, sp);
    __hip_atomic_fetch_add(&a.tile_done[ip.tile], ip.wide ? 2 : 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    items += ip.wide ? 2 : 1;
  }
  __hip_atomic_fetch_add(&a.tile_done[a.max_tiles_l], items, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// L2 items: wait until every L1 slab of the tile has arrived, then acquire.  Once a workgroup has
// seen all L1 items arrive (and acquired), no later item of it needs to wait.
struct L2Wait {
  const int* done;
  int n;
  int* hdr;
  int* s_all;                                     // LDS flag: all L1 items seen
  int n_l1_slabs, n_l1_items;
  __device__ __forceinline__ void before(int tile) {
    if (*s_all) return;                           // uniform: written before a barrier
    __syncthreads();
    if (threadIdx.x == 0) {
      if (!wait_at_least(&done[tile], n_l1_slabs)) record_fault(hdr);
      if (__hip_atomic_load(&done[n], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_l1_items) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_all = 1;
      }
    }
    __syncthreads();
  }
  __device__ __forceinline__ void after(int) {}
};

// The arguments, read word by word from their LDS copy into scalar registers (every lane holds the
// same words).
__device__ __forceinline__ Args uniform_copy(const Args& s) {
  constexpr int N = sizeof(Args) / 4;
  uint32_t w[N];
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = __builtin_amdgcn_readfirstlane(reinterpret_cast<const uint32_t*>(&s)[i]);
  Args b;
  __builtin_memcpy(&b, w, sizeof(Args));
  return b;
}

// Registers: the phases after L1 read the arguments from an LDS copy, and the launch index from
// LDS, so no argument value is live across the L1 phase; otherwise the L1 K loop runs short of
// scalar registers and reloads spilled ones at every step.
template <int R, bool H64>
__global__ __launch_bounds__(kThreads) void k_fused(Args a) {
  __shared__ __attribute__((aligned(1024))) Lds L;
  // the fused kernel's own LDS variables, in the one LDS object (see Lds::extra)
  struct Extra {
    Args args;
    unsigned long long launch;
    int last, all;
  };
  static_assert(sizeof(Extra) <= sizeof(L.extra), "fused variables fit Lds::extra");
  Extra& X = *reinterpret_cast<Extra*>(L.extra);
  Args& s_args = X.args;
  unsigned long long& s_launch = X.launch;
  int& s_last = X.last;
  int& s_all = X.all;
  constexpr int NT = kThreads;
  const int tid = threadIdx.x, G = gridDim.x;
  if (__hip_atomic_load(&g_fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;   // uniform
  static_assert(sizeof(Args) % 4 == 0 && sizeof(Args) / 4 <= NT, "one word per thread");
  if (tid < (int)(sizeof(Args) / 4))
    reinterpret_cast<uint32_t*>(&s_args)[tid] = reinterpret_cast<const uint32_t*>(&a)[tid];

  // A. count (LDS: the ring as scratch); the arrival counts start from zero
  {
    int* hist = reinterpret_cast<int*>(L.ring);
    int* ids = hist + kMaxExperts;
    int* inv_w = ids + kRouteBlock;
    for (int b = blockIdx.x; b < a.NB; b += G) route_count_block<NT>(a, b, hist, ids, inv_w);
    for (int i = blockIdx.x * NT + tid; i <= a.max_tiles_l; i += G * NT) a.tile_done[i] = 0;
    if (blockIdx.x == 0 && tid == 0) a.hdr[kHdrFusedFault] = 0;
  }
  publish();
  if (tid == 0) {
    const unsigned long long old = __hip_atomic_fetch_add(&g_sync[0], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_launch = old / G;
    s_last = old % G == (unsigned long long)(G - 1);
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // every workgroup's counts
  }
  __syncthreads();
  const unsigned long long launch = s_launch;

  // B. scan by the last workgroup to arrive; the others wait for it
  if (s_last) {
    int* lds = reinterpret_cast<int*>(L.ring);
    route_scan<NT>(a, ScanLds{lds, lds + kMaxExperts, lds + kMaxExperts + (NT / 256) * 256,
                              lds + kMaxExperts + (NT / 256) * 256 + 32 * (kMaxNGClasses + 2)});
    publish();
    if (tid == 0) __hip_atomic_fetch_add(&g_sync[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (tid == 0) {
    if (!wait_at_least(&g_sync[1], launch + 1)) record_fault(a.hdr);
  }
  __syncthreads();

  // C. scatter: every pair to its pool row, with its row's activation scale words (K-major)
  for (int pair = blockIdx.x * NT + tid; pair < a.P; pair += G * NT) {
    const int pos = route_scatter_pair(a, pair);
    if (pos >= 0)
      for (int kb0 = 0; kb0 < a.H / 128; kb0 += 8) pool_scales_row_of(a, pos, pair / a.k, kb0);
  }
  grid_barrier(a.hdr, 2, launch);

  // D. L1 items, then their arrivals
  {
    NoHooks none;
    large_items<R, true, false>(a, L, none);
    l1_arrive<R>(a);
  }
  // E. L2 items (arguments from the LDS copy)
  {
    const Args b = uniform_copy(s_args);
    if (tid == 0) s_all = 0;
    __syncthreads();
    const int n_l1_slabs = b.I / kL1SlabCh;
    L2Wait wt{b.tile_done, b.max_tiles_l, b.hdr, &s_all, n_l1_slabs, b.hdr[kHdrTilesLarge] * n_l1_slabs};
    large_items<R, false, H64>(b, L, wt);
  }
  // F. combine after every L2 item (arguments from the LDS copy again)
  {
    const Args b = uniform_copy(s_args);
    grid_barrier(b.hdr, 3, s_launch);
    const long total = (long)b.T * (b.H / 8);
    for (long idx = (long)blockIdx.x * NT + tid; idx < total; idx += (long)G * NT) combine_chunk(b, idx);
  }
}

}  // namespace

hipError_t launch_fused(const Args& a, hipStream_t s) {
  void* args[] = {const_cast<Args*>(&a)};
  const void* fn = a.recipe == 0 ? (a.inter64 ? reinterpret_cast<const void*>(&k_fused<0, true>)
                                              : reinterpret_cast<const void*>(&k_fused<0, false>))
                 : a.recipe == 1 ? reinterpret_cast<const void*>(&k_fused<1, false>)
                                 : reinterpret_cast<const void*>(&k_fused<2, false>);
  return hipLaunchCooperativeKernel(fn, dim3(a.large_grid), dim3(kThreads), args, 0, s);
}

}  // namespace mm
