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
// missing entries are numbered by a block scan over the list; the k-th
// missing entry takes the unlisted slot of rank k by (stamp, slot); with few
// misses the victims are found one workgroup minimum at a time, else every
// unlisted slot is ranked against every other (S <= 1024 slots, a few
// thousand LDS reads per thread at most).  The copies are listed compactly (list positions
// of the missing entries, in list order), so the copy kernel touches only
// the (b, g) that miss something: at steady state most have nothing to copy.
#include "bskv_device.hpp"
#include "bskv_launch.hpp"
#include "cache_fill.hpp"

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
  int64_t wmin[2][4];
  int scan_tmp[4];
};

// Up to this many missing blocks per (b, g) the victims are found one at a
// time (a workgroup minimum per victim) instead of ranking every unlisted
// slot against every other.
constexpr int kCacheArgminMiss = 16;

__device__ __forceinline__ int64_t wave_min_i64(int64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t o = __shfl_xor(v, off);
    v = o < v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void cache_plan_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt, int U,
                                                            int32_t* __restrict__ tags, int64_t* __restrict__ stamps,
                                                            int64_t* __restrict__ clock, int S,
                                                            int32_t* __restrict__ slot_out,
                                                            int32_t* __restrict__ fill_out,
                                                            int32_t* __restrict__ n_fill_out) {
  __shared__ CachePlanSmem sm;
  const int bg = blockIdx.x, tid = threadIdx.x;
  const int32_t* lst = idx + (int64_t)bg * U;
  int32_t* tg = tags + (int64_t)bg * S;
  int64_t* st = stamps + (int64_t)bg * S;
  // every load is issued before any is used (one round trip): the count,
  // the clock, the whole list (entries past the count are masked after),
  // the slot table
  const int c = max(0, min(cnt[bg], U));
  const int64_t now = clock[bg] + 1;
  for (int u = tid; u < U; u += kThreads) {
    const int32_t j = lst[u];
    sm.list[u] = u < c ? j : INT32_MAX;
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
  // the n_miss unlisted slots of least (stamp, slot) are taken, in that
  // order.  Few misses (the common case at steady state, none at all for
  // most (b, g)): one workgroup minimum of the key (stamp + 1) * 1024 + slot
  // per victim, the taken slot's key then set to the maximum.
  if (n_miss > 0 && n_miss <= kCacheArgminMiss) {
    constexpr int SPT = kCacheMaxSlots / kThreads;
    const int lane = tid & 63, wid = tid >> 6;
    int64_t key[SPT];
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      const int sl = tid + e * kThreads;
      key[e] = (sl < S && !sm.keep[sl]) ? ((sm.stamp[sl] + 1) << 10) + sl : INT64_MAX;
    }
    for (int r = 0; r < n_miss; ++r) {
      int64_t m = key[0];
#pragma unroll
      for (int e = 1; e < SPT; ++e) m = key[e] < m ? key[e] : m;
      m = wave_min_i64(m);
      if (lane == 0) sm.wmin[r & 1][wid] = m;
      __syncthreads();
      int64_t best = sm.wmin[r & 1][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) best = sm.wmin[r & 1][w] < best ? sm.wmin[r & 1][w] : best;
      const int vs = (int)(best & 1023);
      if (tid == 0) sm.victim[r] = vs;
#pragma unroll
      for (int e = 0; e < SPT; ++e)
        if (tid + e * kThreads == vs) key[e] = INT64_MAX;
    }
  }
  // more misses: rank every unlisted slot by (stamp, slot)
  for (int s = tid; s < S && n_miss > kCacheArgminMiss; s += kThreads) {
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

// Copy of the missing blocks into their slots, dealt out over the grid
// (cache_fill_wg).
template <int CPT>
__global__ __launch_bounds__(kThreads) void cache_fill_kernel(CacheFillParams f) {
  __shared__ CacheFillSmem sm;
  cache_fill_wg<CPT>(f, blockIdx.x, gridDim.x, sm);
}

CacheFillParams make_fill_params(const CacheFillArgs& a) {
  CacheFillParams f;
  f.src_k = (const uint4*)a.src_k; f.src_v = (const uint4*)a.src_v;
  f.sb = a.sb * a.esize / 16; f.sg = a.sg * a.esize / 16; f.st = a.st * a.esize / 16;
  f.src_len = a.src_len;
  f.row16 = a.D * a.esize / 16;
  f.idx = a.idx; f.slot = a.slot; f.fill = a.fill; f.n_fill = a.n_fill;
  f.cache_k = (uint4*)a.cache_k; f.cache_v = (uint4*)a.cache_v;
  f.H = a.H; f.U = a.U; f.S = a.S; f.block = a.block; f.n_bg = a.B * a.H;
  return f;
}

hipError_t launch_cache_fill(const CacheFillArgs& a) {
  const CacheFillParams f = make_fill_params(a);
  const dim3 grid(a.n_workgroups < f.n_bg ? a.n_workgroups : f.n_bg);
  // chunks per block = 64 rows x (head_dim x element size / 16) = 512, 1024 or 2048
  const int per_item = a.block * f.row16;
  if (per_item == 2 * kThreads) hipLaunchKernelGGL(cache_fill_kernel<2>, grid, dim3(kThreads), 0, a.stream, f);
  else if (per_item == 4 * kThreads) hipLaunchKernelGGL(cache_fill_kernel<4>, grid, dim3(kThreads), 0, a.stream, f);
  else hipLaunchKernelGGL(cache_fill_kernel<8>, grid, dim3(kThreads), 0, a.stream, f);
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
