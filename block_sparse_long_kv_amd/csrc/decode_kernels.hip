// Per-operation decode kernels of the C ABI: block mean-pooling, the
// Forecast projection (split + ordered reduce), decode scoring + top-k
// (score slices, then one top-k workgroup per (b, g)), and decode attention
// (splits, then one merge workgroup per (b, g)).  Every merge runs in a
// second kernel, so no workgroup waits on or fences for another.
//
// Sources: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection" (Eqs. 3-5, Alg. 2), "One
// Forecast head per GQA group" (Sec. 4.1), "The problem InfLLM-V2 leaves on
// the table" (mean-pooled keys).
#include "bskv_launch.hpp"
#include "cache_fill.hpp"
#include "decode_ops.hpp"

namespace bskv {

// ------------------------------------------------------------------ meanpool
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void meanpool_kernel(const T* __restrict__ k, int64_t sb, int64_t sg,
                                                          int64_t st, int64_t kv_len, int H,
                                                          const int64_t* __restrict__ seq_len, int64_t j0,
                                                          int64_t j1, int newest_only, float* __restrict__ kc,
                                                          int64_t nb_cap) {
  __shared__ MeanpoolSmem<T, D> sm;
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t L = min(seq_len[b], kv_len);
  int64_t j;
  if (newest_only) {
    if (L <= 0 || (L % kBlk) != 0) return;
    j = L / kBlk - 1;
    if (j < j0 || j >= j1) return;
  } else {
    j = j0 + blockIdx.x;
    if (j >= j1 || (j + 1) * (int64_t)kBlk > L) return;
  }
  meanpool_wg<T, D>(k + b * sb + g * sg + j * kBlk * st, st, kc + ((int64_t)(b * H + g) * nb_cap + j) * D, sm);
}

template <typename T, int D>
static hipError_t launch_meanpool_t(const MeanpoolArgs& a) {
  const int64_t nx = a.newest_only ? 1 : (a.blk_end - a.blk_begin);
  if (nx <= 0) return hipSuccess;
  dim3 grid((unsigned)nx, (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((meanpool_kernel<T, D>), grid, dim3(kThreads), 0, a.stream, (const T*)a.k, a.sb, a.sg, a.st,
                     a.kv_len, a.H, a.seq_len, a.blk_begin, a.blk_end, a.newest_only, a.kc, a.nb_cap);
  return hipGetLastError();
}

hipError_t launch_meanpool(const MeanpoolArgs& a) {
  if (a.dtype == 0) return a.D == 64 ? launch_meanpool_t<float, 64>(a) : launch_meanpool_t<float, 128>(a);
  return a.D == 64 ? launch_meanpool_t<bf16_bits, 64>(a) : launch_meanpool_t<bf16_bits, 128>(a);
}

// ------------------------------------------------------------------ forecast projection
template <typename T>
__global__ __launch_bounds__(kThreads) void proj_partial_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                              int B, int hidden, int N, float* __restrict__ part) {
  if constexpr (std::is_same<T, bf16_bits>::value) {
    __shared__ ProjMfmaSmem sm;
    proj_partial_mfma_wg<kProjRows>(x, w, B, hidden, N, blockIdx.x, blockIdx.y, part, sm);
  } else {
    __shared__ ProjSmem sm;
    proj_partial_wg<T>(x, w, B, hidden, N, blockIdx.x, blockIdx.y, part, sm);
  }
}

__global__ __launch_bounds__(kThreads) void proj_reduce_kernel(const float* __restrict__ part, int n_splits, int B,
                                                             int N, float* __restrict__ f) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= B * N) return;
  f[i] = proj_reduce_one(part, n_splits, B, N, i / N, i % N);
}

// partials of the projection: one per kProjRows rows (fp32) or per
// kProjPartRows rows (bf16, whatever row span its workgroups take)
int proj_splits(int hidden, int dtype) { return hidden / (dtype == 0 ? kProjRows : kProjPartRows); }
int proj_tiles(int N, int dtype) { return N / (dtype == 0 ? 64 : 128); }

size_t proj_workspace_bytes(int B, int hidden, int N, int dtype) {
  return (size_t)proj_splits(hidden, dtype) * B * N * sizeof(float);
}

template <typename T>
void launch_proj_partial(const void* x, const void* w, int B, int hidden, int N, float* part, hipStream_t s) {
  dim3 grid(N / proj_tile_cols_host<T>(), hidden / kProjRows);
  hipLaunchKernelGGL((proj_partial_kernel<T>), grid, dim3(kThreads), 0, s, (const T*)x, (const T*)w, B, hidden, N,
                     part);
}
template void launch_proj_partial<float>(const void*, const void*, int, int, int, float*, hipStream_t);
template void launch_proj_partial<bf16_bits>(const void*, const void*, int, int, int, float*, hipStream_t);

hipError_t launch_proj(const ProjArgs& a) {
  float* part = (float*)a.ws;
  if (a.dtype == 0) launch_proj_partial<float>(a.x, a.w, a.B, a.hidden, a.N, part, a.stream);
  else launch_proj_partial<bf16_bits>(a.x, a.w, a.B, a.hidden, a.N, part, a.stream);
  const int n = a.B * a.N;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, a.stream, part,
                     proj_splits(a.hidden, a.dtype), a.B, a.N, a.f);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode score + top-k
template <int D>
__global__ __launch_bounds__(kThreads) void score_decode_kernel(const float* __restrict__ f,
                                                              const float* __restrict__ kc, int64_t nb_cap,
                                                              const int64_t* __restrict__ seq_len, int H, int n_init,
                                                              int n_local, int n_splits, float* __restrict__ sc,
                                                              float* __restrict__ dbg) {
  __shared__ __attribute__((aligned(16))) float fvec[D];
  const int bg = blockIdx.y, split = blockIdx.x;
  const DecodeCands dc = decode_cands(seq_len[bg / H], nb_cap, n_init, n_local);
  const int n = dc.c1 - dc.c0;
  const int per = (n + n_splits - 1) / n_splits;
  const int lo = dc.c0 + split * per, hi = min(dc.c1, lo + per);
  for (int i = threadIdx.x; i < D; i += kThreads) fvec[i] = f[(int64_t)bg * D + i];
  __syncthreads();
  float* row = sc + (int64_t)bg * nb_cap;
  score_slice_wg<D>(fvec, kc + (int64_t)bg * nb_cap * D, lo, hi, row);
  if (dbg) {
    __syncthreads();
    float* drow = dbg + (int64_t)bg * nb_cap;
    for (int j = lo + threadIdx.x; j < hi; j += kThreads) drow[j] = row[j];
    if (split == 0)
      for (int j = threadIdx.x; j <= min(dc.cur, (int)nb_cap - 1); j += kThreads)
        if (j < dc.c0 || j >= dc.c1) drow[j] = -INFINITY;
  }
}

__global__ __launch_bounds__(kThreads) void topk_decode_kernel(const float* __restrict__ sc, int64_t nb_cap,
                                                             const int64_t* __restrict__ seq_len, int H, int topk,
                                                             int n_init, int n_local, int U, int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ cnt) {
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  const int bg = blockIdx.x;
  const DecodeCands dc = decode_cands(seq_len[bg / H], nb_cap, n_init, n_local);
  topk_decode_wg(sc + (int64_t)bg * nb_cap, nb_cap, dc, topk, n_init, n_local, U, idx + (int64_t)bg * U, cnt + bg, keys, sh);
}

size_t score_decode_workspace_bytes(int B, int H, int64_t nb_cap) { return (size_t)B * H * nb_cap * sizeof(float); }

void launch_topk_decode(const float* sc, int64_t nb_cap, const int64_t* seq_len, int n_bg, int H, int topk,
                        int n_init, int n_local, int U, int32_t* idx, int32_t* cnt, hipStream_t s) {
  const int64_t cap = nb_cap < kMaxCandidates ? nb_cap : kMaxCandidates;
  hipLaunchKernelGGL(topk_decode_kernel, dim3(n_bg), dim3(kThreads), (size_t)cap * sizeof(uint32_t), s, sc, nb_cap,
                     seq_len, H, topk, n_init, n_local, U, idx, cnt);
}

hipError_t launch_score_topk_decode(const ScoreTopkArgs& a) {
  const int n_bg = a.B * a.H;
  const int ns = score_split_plan(n_bg, a.nb_cap);
  float* sc = (float*)a.ws;
  dim3 grid(ns, n_bg);
  if (a.D == 64)
    hipLaunchKernelGGL(score_decode_kernel<64>, grid, dim3(kThreads), 0, a.stream, (const float*)a.f, a.kc, a.nb_cap,
                       a.seq_len, a.H, a.n_init, a.n_local, ns, sc, a.scores);
  else
    hipLaunchKernelGGL(score_decode_kernel<128>, grid, dim3(kThreads), 0, a.stream, (const float*)a.f, a.kc, a.nb_cap,
                       a.seq_len, a.H, a.n_init, a.n_local, ns, sc, a.scores);
  launch_topk_decode(sc, a.nb_cap, a.seq_len, n_bg, a.H, a.topk, a.n_init, a.n_local, a.U, a.idx, a.cnt, a.stream);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode attention
// grid (units, splits): the workgroups of one split are consecutive, so
// the XCDs, dealt consecutive workgroups in turn, all get the same mix of
// long and short splits
template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads, 3) void attn_split_kernel(AttnDecodeParams p) {
  __shared__ typename AttnSmemSel<T, D, G>::type sm;
  attn_split_wg<T, D, G>(p, blockIdx.x, blockIdx.y, sm);
}

// The split kernel with another layer's cache fill in the same launch: the
// first n_fill workgroups copy that layer's missing blocks (host reads with
// long latency; dispatched first, they overlap the whole attention), the
// rest are the attention splits of this layer.
template <typename T, int D, int G, int CPT>
__global__ __launch_bounds__(kThreads, 3) void attn_split_fill_kernel(AttnDecodeParams p, CacheFillParams f,
                                                                     int n_fill) {
  __shared__ union {
    typename AttnSmemSel<T, D, G>::type attn;
    CacheFillSmem fill;
  } sm;
  const int bid = (int)blockIdx.x;
  if (bid < n_fill) {
    cache_fill_wg<CPT>(f, bid, n_fill, sm.fill);
    return;
  }
  const int a = bid - n_fill, n_bg = ((int)gridDim.x - n_fill) / p.n_splits;   // split-major, as above
  attn_split_wg<T, D, G>(p, a % n_bg, a / n_bg, sm.attn);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnDecodeParams p) {
  __shared__ CombineSmem<D, G> sm;
  attn_combine_wg<D, G>(p, blockIdx.x, sm);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int U) {
  int ns, bps;
  const int n_bg = B * Hkv, G = Hq / Hkv;
  attn_split_plan(n_bg, U, ns, bps);
  const size_t o = (size_t)n_bg * ns * G * D * sizeof(float);
  return ((o + 255) / 256) * 256 + (size_t)n_bg * ns * G * 2 * sizeof(float);
}

AttnDecodeParams make_attn_params(const AttnDecodeArgs& a, void* ws) {
  AttnDecodeParams p;
  int ns, bps;
  const int n_bg = a.B * a.Hkv, G = a.Hq / a.Hkv;
  // a cache fill in the same launch takes its workgroups first; the split
  // count never exceeds the workspace's (sized without a reserve)
  int reserve = 0;
  if (a.fill) reserve = a.fill->n_workgroups < n_bg ? a.fill->n_workgroups : n_bg;
  attn_split_plan(n_bg, a.U, ns, bps, reserve);
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.sb = a.sb; p.sg = a.sg; p.st = a.st; p.kv_len = a.kv_len; p.ring = a.ring; p.slot = a.slot;
  p.idx = a.idx; p.cnt = a.cnt; p.seq_len = a.seq_len;
  p.Hkv = a.Hkv; p.U = a.U;
  p.qscale = a.scale * 1.4426950408889634f;
  p.bps = bps; p.n_splits = ns;
  p.out = a.out;
  const size_t o = (size_t)n_bg * ns * G * a.D * sizeof(float);
  p.ws_o = (float*)ws;
  p.ws_ml = (float*)((char*)ws + ((o + 255) / 256) * 256);
  return p;
}

template <typename T, int D, int G>
static void launch_attn_t(const AttnDecodeParams& p, int n_bg, const CacheFillArgs* fill, hipStream_t s) {
  if (fill) {
    const CacheFillParams f = make_fill_params(*fill);
    const int n_fill = fill->n_workgroups < f.n_bg ? fill->n_workgroups : f.n_bg;
    const dim3 grid(n_fill + p.n_splits * n_bg);
    // chunks per block = 64 rows x (head_dim x element size / 16) = 512, 1024 or 2048
    const int per_item = fill->block * f.row16;
    if (per_item == 2 * kThreads)
      hipLaunchKernelGGL((attn_split_fill_kernel<T, D, G, 2>), grid, dim3(kThreads), 0, s, p, f, n_fill);
    else if (per_item == 4 * kThreads)
      hipLaunchKernelGGL((attn_split_fill_kernel<T, D, G, 4>), grid, dim3(kThreads), 0, s, p, f, n_fill);
    else
      hipLaunchKernelGGL((attn_split_fill_kernel<T, D, G, 8>), grid, dim3(kThreads), 0, s, p, f, n_fill);
  } else {
    hipLaunchKernelGGL((attn_split_kernel<T, D, G>), dim3(n_bg, p.n_splits), dim3(kThreads), 0, s, p);
  }
  hipLaunchKernelGGL((attn_combine_kernel<D, G>), dim3(n_bg), dim3(kThreads), 0, s, p);
}

template <typename T, int D>
static void launch_attn_g(const AttnDecodeParams& p, int G, int n_bg, const CacheFillArgs* fill, hipStream_t s) {
  switch (G) {
    case 1: launch_attn_t<T, D, 1>(p, n_bg, fill, s); break;
    case 2: launch_attn_t<T, D, 2>(p, n_bg, fill, s); break;
    case 4: launch_attn_t<T, D, 4>(p, n_bg, fill, s); break;
    default: launch_attn_t<T, D, 8>(p, n_bg, fill, s); break;
  }
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a) {
  const AttnDecodeParams p = make_attn_params(a, a.ws);
  const int n_bg = a.B * a.Hkv, G = a.Hq / a.Hkv;
  if (a.dtype == 0) {
    if (a.D == 64) launch_attn_g<float, 64>(p, G, n_bg, a.fill, a.stream);
    else launch_attn_g<float, 128>(p, G, n_bg, a.fill, a.stream);
  } else {
    if (a.D == 64) launch_attn_g<bf16_bits, 64>(p, G, n_bg, a.fill, a.stream);
    else launch_attn_g<bf16_bits, 128>(p, G, n_bg, a.fill, a.stream);
  }
  return hipGetLastError();
}

}  // namespace bskv
