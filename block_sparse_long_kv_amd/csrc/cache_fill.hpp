// Copy of a layer's missing blocks into its resident block cache, run by
// one workgroup over the (b, g) units wg, wg + n_wg, ... (shared by the
// standalone fill kernel and by the cached attention kernel that carries
// the next layer's fill in the same launch).
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

// For each (b, g) of this workgroup: its n_fill blocks one after another (K
// and V, all 16-byte loads of a block issued before its stores).  A (b, g)
// with nothing to copy costs one load.  CPT: 16-byte chunks per thread and
// block (block * row16 == CPT * kThreads).
template <int CPT>
__device__ __forceinline__ void cache_fill_wg(const CacheFillParams& f, int wg, int n_wg) {
  const int per_item = f.block * f.row16;
  for (int bg = wg; bg < f.n_bg; bg += n_wg) {
    const int nf = min(f.n_fill[bg], f.U);
    const int b = bg / f.H, g = bg % f.H;
    for (int k = 0; k < nf; ++k) {
      const int u = f.fill[(int64_t)bg * f.U + k];
      if (u < 0 || u >= f.U) continue;
      const int j = f.idx[(int64_t)bg * f.U + u];
      const int s = f.slot[(int64_t)bg * f.U + u];
      if (j < 0 || ((int64_t)j + 1) * f.block > f.src_len || s < 0 || s >= f.S) continue;   // inside both buffers
      const int64_t sbase = b * f.sb + g * f.sg + (int64_t)j * f.block * f.st;
      const int64_t dbase = ((int64_t)bg * f.S + s) * per_item;
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
  }
}

}  // namespace bskv
