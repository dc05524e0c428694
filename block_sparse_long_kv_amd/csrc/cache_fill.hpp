// Copy of a layer's missing blocks into its resident block cache by n_wg
// workgroups (shared by the standalone fill kernel and by the cached
// attention kernel that carries the next layer's fill in the same launch).
#pragma once
#include "bskv_device.hpp"

namespace bskv {

struct CacheFillParams {
  const uint4* src_k; const uint4* src_v;
  int64_t sb, sg, st;          // source strides in 16-byte units
  int64_t src_len;             // tokens in the source
  int row16;                   // 16-byte chunks per token
  const int32_t* idx; const int32_t* slot; const int32_t* fill; const int32_t* n_fill;
  uint4* cache_k; uint4* cache_v;
  int H, U, S, block, n_bg;
};

// One missing block (K and V) of unit bg: the k-th entry of its fill list,
// all 16-byte loads issued before the stores.  CPT: 16-byte chunks per
// thread and block (block * row16 == CPT * kThreads).
template <int CPT>
__device__ __forceinline__ void cache_fill_one(const CacheFillParams& f, int bg, int k) {
  const int u = f.fill[(int64_t)bg * f.U + k];
  if (u < 0 || u >= f.U) return;
  const int j = f.idx[(int64_t)bg * f.U + u];
  const int s = f.slot[(int64_t)bg * f.U + u];
  if (j < 0 || ((int64_t)j + 1) * f.block > f.src_len || s < 0 || s >= f.S) return;   // inside both buffers
  const int b = bg / f.H, g = bg % f.H;
  const int64_t sbase = b * f.sb + g * f.sg + (int64_t)j * f.block * f.st;
  const int64_t dbase = ((int64_t)bg * f.S + s) * (f.block * f.row16);
  uint4 rk[CPT], rv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = threadIdx.x + i * kThreads;
    const int t = ch / f.row16, w = ch % f.row16;
    rk[i] = f.src_k[sbase + t * f.st + w];
    rv[i] = f.src_v[sbase + t * f.st + w];
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = threadIdx.x + i * kThreads;
    f.cache_k[dbase + ch] = rk[i];
    f.cache_v[dbase + ch] = rv[i];
  }
}

// Up to kFillFlatUnits (b, g) units the copies are dealt out one block at a
// time over the whole layer: block i of the layer (the units' fill lists
// laid end to end, unit-major) goes to workgroup i mod n_wg, so every
// workgroup requests its blocks at once and no unit's blocks wait behind
// one another (host reads have microseconds of latency).  Each workgroup
// builds the prefix of the units' counts in LDS and finds a block's unit by
// binary search.  Above that, workgroup w takes the units w, w + n_wg, ...
// and copies each unit's blocks in turn.
constexpr int kFillFlatUnits = 4096;
struct CacheFillSmem {
  int pre[kFillFlatUnits];
  int scan_tmp[4];
};

template <int CPT>
__device__ __forceinline__ void cache_fill_wg(const CacheFillParams& f, int wg, int n_wg, CacheFillSmem& sm) {
  if (f.n_bg <= kFillFlatUnits) {
    constexpr int PER = kFillFlatUnits / kThreads;   // units per thread
    const int u0 = (int)threadIdx.x * PER;
    int c[PER], sum = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int bg = u0 + e;
      c[e] = bg < f.n_bg ? min(max(f.n_fill[bg], 0), f.U) : 0;
      sum += c[e];
    }
    int total;
    int run = block_excl_scan(sum, sm.scan_tmp, total);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      sm.pre[u0 + e] = run;
      run += c[e];
    }
    __syncthreads();
    for (int i = wg; i < total; i += n_wg) {
      // the unit holding block i: the last one whose prefix is <= i
      int lo = 0, hi = f.n_bg - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm.pre[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      cache_fill_one<CPT>(f, lo, i - sm.pre[lo]);
    }
    return;
  }
  for (int bg = wg; bg < f.n_bg; bg += n_wg) {
    const int nf = min(f.n_fill[bg], f.U);
    for (int k = 0; k < nf; ++k) cache_fill_one<CPT>(f, bg, k);
  }
}

}  // namespace bskv
