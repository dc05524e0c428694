// Resident block cache for offloaded decode: which of the blocks a layer
// needs are already on the GPU, and where the missing ones go.
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "Three speedups, three different baselines" (Table 4:
// offloaded decode at 128K peaks at batch 64, which needs most selected
// blocks to stay on the GPU between decode steps).  The pages do not
// describe the cache; the policy here is least-recently-used per (batch, KV
// head): listed blocks already held keep their slot, the missing ones take
// the unlisted slots in order of (last use, slot), empty slots first, and
// every listed slot is stamped with (lookup number, list position).
//
// One workgroup per (b, g): the slot table (tags, stamps) is read into LDS;
// every slot looks its block up in the sorted list (binary search); the
// missing entries are numbered by a block scan over the list; the unlisted
// slots are ranked by (stamp, slot) with one comparison per pair (S <= 1024
// slots, a few thousand LDS reads per thread at most); the k-th missing entry
// takes the slot of rank k.  The copies are listed compactly (list positions
// of the missing entries, in list order), so the copy kernel touches only
// the (b, g) that miss something: at steady state most have nothing to copy.
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

constexpr int kCacheMaxSlots = 1024;
constexpr int kCacheMaxList = 1024;

__global__ __launch_bounds__(kThreads) void cache_reset_kernel(int32_t* __restrict__ tags,
                                                             int64_t* __restrict__ stamps,
                                                             int64_t* __restrict__ clock, int64_t n_slots_total,
                                                             int n_bg) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n_slots_total) {
    tags[i] = -1;
    stamps[i] = -1;
  }
  if (i < n_bg) clock[i] = 0;
}

struct CachePlanSmem {
  int32_t list[kCacheMaxList];
  int32_t slot_of[kCacheMaxList];
  int32_t tag[kCacheMaxSlots];
  int64_t stamp[kCacheMaxSlots];
  int32_t victim[kCacheMaxSlots];
  uint8_t keep[kCacheMaxSlots];
  int scan_tmp[4];
};

__global__ __launch_bounds__(kThreads) void cache_plan_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt, int U,
                                                            int32_t* __restrict__ tags, int64_t* __restrict__ stamps,
                                                            int64_t* __restrict__ clock, int S,
                                                            int32_t* __restrict__ slot_out,
                                                            int32_t* __restrict__ fill_out,
                                                            int32_t* __restrict__ n_fill_out) {
  __shared__ CachePlanSmem sm;
  const int bg = blockIdx.x, tid = threadIdx.x;
  const int c = max(0, min(cnt[bg], U));
  const int32_t* lst = idx + (int64_t)bg * U;
  int32_t* tg = tags + (int64_t)bg * S;
  int64_t* st = stamps + (int64_t)bg * S;
  for (int u = tid; u < U; u += kThreads) {
    sm.list[u] = u < c ? lst[u] : INT32_MAX;
    sm.slot_of[u] = -1;
  }
  for (int s = tid; s < S; s += kThreads) {
    sm.tag[s] = tg[s];
    sm.stamp[s] = st[s];
    sm.keep[s] = 0;
  }
  __syncthreads();
  // listed blocks already held: each slot finds its block in the sorted list
  for (int s = tid; s < S; s += kThreads) {
    const int32_t t = sm.tag[s];
    if (t < 0) continue;
    int lo = 0, hi = c;   // first position with list[pos] >= t
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sm.list[mid] < t) lo = mid + 1;
      else hi = mid;
    }
    if (lo < c && sm.list[lo] == t) {
      sm.slot_of[lo] = s;
      sm.keep[s] = 1;
    }
  }
  __syncthreads();
  // number the missing entries in list order: each thread owns a run of
  // consecutive positions
  constexpr int PPT = kCacheMaxList / kThreads;
  const int u0 = tid * PPT;
  int mine = 0;
#pragma unroll
  for (int e = 0; e < PPT; ++e) mine += (u0 + e < c && sm.slot_of[u0 + e] < 0) ? 1 : 0;
  int n_miss;
  int rank = block_excl_scan(mine, sm.scan_tmp, n_miss);
  // rank the unlisted slots by (stamp, slot); the first n_miss are taken
  for (int s = tid; s < S; s += kThreads) {
    if (sm.keep[s]) continue;
    const int64_t ks = sm.stamp[s];
    int r = 0;
    for (int s2 = 0; s2 < S; ++s2) {
      const int64_t k2 = sm.stamp[s2];
      r += (!sm.keep[s2] && (k2 < ks || (k2 == ks && s2 < s))) ? 1 : 0;
    }
    if (r < n_miss) sm.victim[r] = s;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    const int u = u0 + e;
    if (u < c && sm.slot_of[u] < 0) {
      const int s = sm.victim[rank];
      sm.slot_of[u] = s;
      sm.tag[s] = sm.list[u];
      fill_out[(int64_t)bg * U + rank] = u;   // the rank-th copy: list position u
      ++rank;
    }
  }
  for (int k = n_miss + tid; k < U; k += kThreads) fill_out[(int64_t)bg * U + k] = -1;
  __syncthreads();
  const int64_t now = clock[bg] + 1;
  for (int u = tid; u < U; u += kThreads) {
    const int s = u < c ? sm.slot_of[u] : -1;
    slot_out[(int64_t)bg * U + u] = s;
    if (s >= 0) st[s] = now * U + u;
  }
  for (int s = tid; s < S; s += kThreads) tg[s] = sm.tag[s];
  if (tid == 0) {
    clock[bg] = now;
    if (n_fill_out) n_fill_out[bg] = n_miss;
  }
}

// Copy of the missing blocks into their slots: workgroup w takes the (b, g)
// w, w + grid, ...; for each, its n_fill blocks one after another (K and V,
// all 16-byte loads of a block issued before its stores, as in the ring
// prefetch).  A (b, g) with nothing to copy costs one load.
template <int CPT>
__global__ __launch_bounds__(kThreads) void cache_fill_kernel(const uint4* __restrict__ src_k,
                                                            const uint4* __restrict__ src_v, int64_t sb, int64_t sg,
                                                            int64_t st, int64_t src_len, int row16,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ slot,
                                                            const int32_t* __restrict__ fill,
                                                            const int32_t* __restrict__ n_fill,
                                                            uint4* __restrict__ cache_k, uint4* __restrict__ cache_v,
                                                            int H, int U, int S, int block, int n_bg) {
  // strides sb, sg, st in 16-byte units; row16 = 16-byte chunks per token
  const int per_item = block * row16;
  for (int bg = blockIdx.x; bg < n_bg; bg += gridDim.x) {
    const int nf = min(n_fill[bg], U);
    const int b = bg / H, g = bg % H;
    for (int k = 0; k < nf; ++k) {
      const int u = fill[(int64_t)bg * U + k];
      if (u < 0 || u >= U) continue;
      const int j = idx[(int64_t)bg * U + u];
      const int s = slot[(int64_t)bg * U + u];
      if (j < 0 || ((int64_t)j + 1) * block > src_len || s < 0 || s >= S) continue;   // stay inside both buffers
      const int64_t sbase = b * sb + g * sg + (int64_t)j * block * st;
      const int64_t dbase = ((int64_t)bg * S + s) * per_item;
      uint4 rk[CPT], rv[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int ch = threadIdx.x + i * kThreads;   // per_item == CPT * kThreads
        const int t = ch / row16, w = ch % row16;
        rk[i] = src_k[sbase + t * st + w];
        rv[i] = src_v[sbase + t * st + w];
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int ch = threadIdx.x + i * kThreads;
        cache_k[dbase + ch] = rk[i];
        cache_v[dbase + ch] = rv[i];
      }
    }
  }
}

hipError_t launch_cache_fill(const CacheFillArgs& a) {
  const int row16 = a.D * a.esize / 16;
  const int per_item = a.block * row16;
  const int n_bg = a.B * a.H;
  const int64_t sb = a.sb * a.esize / 16, sg = a.sg * a.esize / 16, st = a.st * a.esize / 16;
  const dim3 grid(a.n_workgroups < n_bg ? a.n_workgroups : n_bg);
#define BSKV_FILL(CPT)                                                                                           \
  hipLaunchKernelGGL(cache_fill_kernel<CPT>, grid, dim3(kThreads), 0, a.stream, (const uint4*)a.src_k,             \
                     (const uint4*)a.src_v, sb, sg, st, a.src_len, row16, a.idx, a.slot, a.fill, a.n_fill,         \
                     (uint4*)a.cache_k, (uint4*)a.cache_v, a.H, a.U, a.S, a.block, n_bg)
  // per_item = 64 rows x (head_dim x element size / 16) = 512, 1024 or 2048 chunks
  if (per_item == 2 * kThreads) BSKV_FILL(2);
  else if (per_item == 4 * kThreads) BSKV_FILL(4);
  else BSKV_FILL(8);
#undef BSKV_FILL
  return hipGetLastError();
}

hipError_t launch_cache_reset(int32_t* tags, int64_t* stamps, int64_t* clock, int n_bg, int S, hipStream_t stream) {
  const int64_t n = (int64_t)n_bg * S;
  const int64_t m = n > n_bg ? n : n_bg;
  hipLaunchKernelGGL(cache_reset_kernel, dim3((unsigned)((m + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     tags, stamps, clock, n, n_bg);
  return hipGetLastError();
}

hipError_t launch_cache_plan(const CachePlanArgs& a) {
  hipLaunchKernelGGL(cache_plan_kernel, dim3(a.n_bg), dim3(kThreads), 0, a.stream, a.idx, a.cnt, a.U, a.tags,
                     a.stamps, a.clock, a.S, a.slot, a.fill, a.n_fill);
  return hipGetLastError();
}

}  // namespace bskv
