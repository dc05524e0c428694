// Lookahead prefetch: gather the selected K/V blocks of the next layer from
// a host-pinned pool (read by the GPU over the host link) into a device ring.
//
// Sources: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Alg. 2 (fetch of the next
// layer's block set from CPU pinned memory on a dedicated prefetch stream,
// waited on before that layer attends); Chinese SparDA overview
// (deepresearch2agi.pages.dev), section 系统实现 (the GPU reads host memory
// directly through unified addressing; the thread-block count follows the
// batch size).
//
// Design: a persistent grid of n_workgroups workgroups walks the
// (b, g, slot) items.  Each item is two contiguous runs (K and V) of
// block * head_dim elements; a workgroup issues all of its 16-byte loads of
// an item before storing, so every workgroup keeps ~32 KB of host reads in
// flight, and the caller chooses how many workgroups share the link.
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

template <int CPT>
__global__ __launch_bounds__(kThreads) void gather_kernel(const uint4* __restrict__ src_k,
                                                        const uint4* __restrict__ src_v, int64_t sb, int64_t sg,
                                                        int64_t st, int64_t src_len, int row16, const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ cnt, uint4* __restrict__ ring_k,
                                                        uint4* __restrict__ ring_v, int H, int U, int block,
                                                        int total) {
  // strides sb, sg, st are in 16-byte units; row16 = 16-byte chunks per token
  const int per_item = block * row16;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int bg = item / U, u = item % U;
    if (u >= cnt[bg]) continue;
    const int j = idx[(int64_t)bg * U + u];
    if (j < 0 || ((int64_t)j + 1) * block > src_len) continue;  // never read outside the source
    const int b = bg / H, g = bg % H;
    const int64_t sbase = b * sb + g * sg + (int64_t)j * block * st;
    const int64_t dbase = ((int64_t)bg * U + u) * per_item;
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
      ring_k[dbase + ch] = rk[i];
      ring_v[dbase + ch] = rv[i];
    }
  }
}

hipError_t launch_gather(const GatherArgs& a) {
  const int row16 = a.D * a.esize / 16;
  const int per_item = a.block * row16;
  const int total = a.B * a.H * a.U;
  const int64_t sb = a.sb * a.esize / 16, sg = a.sg * a.esize / 16, st = a.st * a.esize / 16;
  dim3 grid(a.n_workgroups);
#define BSKV_GATHER(CPT)                                                                                         \
  hipLaunchKernelGGL(gather_kernel<CPT>, grid, dim3(kThreads), 0, a.stream, (const uint4*)a.src_k,                 \
                     (const uint4*)a.src_v, sb, sg, st, a.src_len, row16, a.idx, a.cnt, (uint4*)a.ring_k, (uint4*)a.ring_v, a.H, \
                     a.U, a.block, total)
  // per_item = 64 rows x (head_dim x element size / 16) = 512, 1024 or 2048 chunks
  if (per_item == 2 * kThreads) BSKV_GATHER(2);
  else if (per_item == 4 * kThreads) BSKV_GATHER(4);
  else BSKV_GATHER(8);
#undef BSKV_GATHER
  return hipGetLastError();
}

}  // namespace bskv
