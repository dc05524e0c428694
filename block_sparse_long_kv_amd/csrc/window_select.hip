// Overlapping key compression and the Forecast selection on it (decode).
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "One Forecast head per GQA group", closing paragraph:
// the evaluated models pool keys with a 32-token window at stride 16 (blocks
// of 64); "Training": the selector's window scores are max-pooled to block
// scores in a final step.  A block's score is the maximum of the scores of
// the complete windows that share at least one token with it (windows
// 4j-1 .. 4j+3 of block j on the 32/16 grid).
//
// Window mean-pool: one workgroup per (window, KV head, sequence), the
// window's rows summed by 16-byte column chunks and reduced across row
// lanes in LDS (the block mean-pool's workgroup with 32 or 64 rows).
// Decode selection: window scores F . K~w over the windows touching the
// candidate blocks, in slices (the block selector's score slices on window
// rows); then one workgroup per (b, g) max-pools them into block scores
// and runs the radix select + union of the block selector (on the 32/16
// grid up to 2048 candidates each thread loads its 8 blocks' 33 windows at
// once and keeps the keys in registers; otherwise the keys go through LDS).  Prefill selection: one workgroup per query block (below).
#include "decode_ops.hpp"
#include "bskv_launch.hpp"

namespace bskv {

template <typename T, int D, int W>
__global__ __launch_bounds__(kThreads) void window_meanpool_kernel(const T* __restrict__ k, int64_t sb, int64_t sg,
                                                                 int64_t st, int64_t kv_len, int H, int stride,
                                                                 const int64_t* __restrict__ seq_len, int64_t w0,
                                                                 int64_t w1, int newest_only, float* __restrict__ kcw,
                                                                 int64_t nw_cap) {
  __shared__ MeanpoolSmem<T, D> sm;
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t L = min(seq_len[b], kv_len);
  int64_t w;
  if (newest_only) {
    // the window the newest token completed, if any
    if (L < W || (L - W) % stride != 0) return;
    w = (L - W) / stride;
    if (w < w0 || w >= w1) return;
  } else {
    w = w0 + blockIdx.x;
    if (w >= w1 || w * stride + W > L) return;
  }
  meanpool_wg<T, D, W>(k + b * sb + g * sg + w * stride * st, st, kcw + ((int64_t)(b * H + g) * nw_cap + w) * D, sm);
}

template <typename T, int D>
static void launch_window_meanpool_t(const WindowMeanpoolArgs& a) {
  const int64_t nx = a.newest_only ? 1 : (a.w_end - a.w_begin);
  if (nx <= 0) return;
  const dim3 grid((unsigned)nx, (unsigned)a.H, (unsigned)a.B);
  if (a.window == 32)
    hipLaunchKernelGGL((window_meanpool_kernel<T, D, 32>), grid, dim3(kThreads), 0, a.stream, (const T*)a.k, a.sb,
                       a.sg, a.st, a.kv_len, a.H, a.stride, a.seq_len, a.w_begin, a.w_end, a.newest_only, a.kcw,
                       a.nw_cap);
  else
    hipLaunchKernelGGL((window_meanpool_kernel<T, D, 64>), grid, dim3(kThreads), 0, a.stream, (const T*)a.k, a.sb,
                       a.sg, a.st, a.kv_len, a.H, a.stride, a.seq_len, a.w_begin, a.w_end, a.newest_only, a.kcw,
                       a.nw_cap);
}

hipError_t launch_window_meanpool(const WindowMeanpoolArgs& a) {
  if (a.dtype == 0) {
    if (a.D == 64) launch_window_meanpool_t<float, 64>(a);
    else launch_window_meanpool_t<float, 128>(a);
  } else {
    if (a.D == 64) launch_window_meanpool_t<bf16_bits, 64>(a);
    else launch_window_meanpool_t<bf16_bits, 128>(a);
  }
  return hipGetLastError();
}

// windows of the grid (window, stride) sharing a token with block j
__device__ __forceinline__ int win_lo(int j, int window, int stride) {
  const int x = kBlk * j - window;
  return x < 0 ? 0 : x / stride + 1;
}
__device__ __forceinline__ int win_hi(int j, int stride) { return kBlk * (j + 1) / stride - 1; }
// complete windows of a sequence of L tokens: 0 .. n-1
__device__ __forceinline__ int64_t win_count(int64_t L, int window, int stride) {
  return L < window ? 0 : (L - window) / stride + 1;
}

template <int D>
__global__ __launch_bounds__(kThreads) void window_score_kernel(const float* __restrict__ f,
                                                              const float* __restrict__ kcw, int64_t nw_cap,
                                                              const int64_t* __restrict__ seq_len, int H, int n_init,
                                                              int n_local, int window, int stride, int64_t nb_cap,
                                                              int n_splits, float* __restrict__ sc) {
  __shared__ __attribute__((aligned(16))) float fvec[D];
  const int bg = blockIdx.y, split = blockIdx.x;
  const int64_t L = seq_len[bg / H];
  const DecodeCands dc = decode_cands(L, nb_cap, n_init, n_local);
  const int64_t nwc = min(win_count(L, window, stride), nw_cap);
  int wl = 0, wh = 0;   // windows [wl, wh) touching the candidates
  if (dc.c1 > dc.c0) {
    wl = win_lo(dc.c0, window, stride);
    wh = (int)min((int64_t)win_hi(dc.c1 - 1, stride) + 1, nwc);
    if (wh < wl) wh = wl;
  }
  const int n = wh - wl;
  const int per = (n + n_splits - 1) / n_splits;
  const int lo = wl + split * per, hi = min(wh, lo + per);
  for (int i = threadIdx.x; i < D; i += kThreads) fvec[i] = f[(int64_t)bg * D + i];
  __syncthreads();
  score_slice_wg<D>(fvec, kcw + (int64_t)bg * nw_cap * D, lo, hi, sc + (int64_t)bg * nw_cap);
}

__global__ __launch_bounds__(kThreads) void window_topk_kernel(const float* __restrict__ sc, int64_t nw_cap,
                                                             int64_t nb_cap, const int64_t* __restrict__ seq_len,
                                                             int H, int window, int stride, int topk, int n_init,
                                                             int n_local, int U, int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ cnt, float* __restrict__ bs_out) {
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  const int bg = blockIdx.x;
  const int64_t L = seq_len[bg / H];
  const DecodeCands dc = decode_cands(L, nb_cap, n_init, n_local);
  const int nwc = (int)min(win_count(L, window, stride), nw_cap);
  const int n = dc.c1 - dc.c0;
  const float* row = sc + (int64_t)bg * nw_cap;
  if (window == 32 && stride == 16 && n <= 8 * kThreads) {
    // thread t: candidates 8t .. 8t+7 (blocks j = c0 + 8t + e), whose windows
    // 4j-1 .. 4j+3 are the 33 consecutive windows from 4(c0 + 8t) - 1: all
    // loaded at once, each block's maximum and key from registers
    const int i0 = 8 * (int)threadIdx.x;
    const int w0 = 4 * (dc.c0 + i0) - 1;
    float ws[33];
#pragma unroll
    for (int t = 0; t < 33; ++t) {
      const int w = w0 + t;
      ws[t] = (i0 < n && w >= 0 && w < nwc) ? row[w] : -INFINITY;
    }
    uint32_t kin[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float m = ws[4 * e];
#pragma unroll
      for (int t = 1; t < 5; ++t) m = fmaxf(m, ws[4 * e + t]);   // max-pool of the block's windows
      kin[e] = orderable_key(m);
      if (bs_out && i0 + e < n) bs_out[(int64_t)bg * nb_cap + dc.c0 + i0 + e] = m;
    }
    topk_union_fast(dc.c0, dc.c0, dc.c1, topk, dc.cur, n_init, n_local, U, idx + (int64_t)bg * U, cnt + bg, sh, kin);
    return;
  }
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int j = dc.c0 + i;
    const int lo = win_lo(j, window, stride), hi = min(win_hi(j, stride), nwc - 1);
    float s = -INFINITY;
    for (int w = lo; w <= hi; ++w) s = fmaxf(s, row[w]);   // max-pool of the block's windows
    keys[i] = orderable_key(s);
    if (bs_out) bs_out[(int64_t)bg * nb_cap + j] = s;
  }
  __syncthreads();
  topk_union(keys, n, dc.c0, topk, dc.cur, n_init, n_local, U, idx + (int64_t)bg * U, cnt + bg, sh);
}

// Prefill: grid (n_qb, B*H), one workgroup per query block.  The block's
// Forecast vectors are summed; each candidate block's score is the maximum of
// the pooled Forecast's dot products with the windows that touch it and whose
// tokens all precede the query block (8 lanes per candidate, its windows in
// turn); then the block selector's top-k + union.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void window_prefill_kernel(const T* __restrict__ f, int Tq, int64_t q_start,
                                                                const float* __restrict__ kcw, int64_t nw_cap,
                                                                int64_t nb_cap, int window, int stride, int topk,
                                                                int n_init, int n_local, int U, int n_qb,
                                                                int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
  constexpr int LPR = 8;
  constexpr int F4 = D / 4 / LPR;
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  __shared__ PoolRowsSmem<T, D> ps;
  const int qi = blockIdx.x, bg = blockIdx.y;
  const int t0 = qi * kBlk, t1 = min(Tq, t0 + kBlk);
  pool_rows<T, D>(f + ((int64_t)bg * Tq + t0) * D, t1 - t0, ps);
  const int cur = (int)(q_start / kBlk) + qi;
  const int c0 = n_init, c1 = (int)min((int64_t)(cur - n_local + 1), nb_cap);
  const int n = max(0, c1 - c0);
  // windows that end at or before the query block's first token
  const int64_t first = (int64_t)cur * kBlk;
  const int nvis = first < window ? 0 : (int)min((first - window) / stride + 1, nw_cap);
  const int sub = threadIdx.x % LPR, row0 = threadIdx.x / LPR;
  float4 fv[F4];
#pragma unroll
  for (int i = 0; i < F4; ++i) fv[i] = *reinterpret_cast<const float4*>(ps.fpool + (i * LPR + sub) * 4);
  const float* kcw_bg = kcw + (int64_t)bg * nw_cap * D;
  for (int j = c0 + row0; j < c1; j += kThreads / LPR) {
    const int lo = win_lo(j, window, stride), hi = min(win_hi(j, stride), nvis - 1);
    float m = -INFINITY;
    for (int w = lo; w <= hi; ++w) {   // the 8 lanes of the candidate run the same windows
      const float* row = kcw_bg + (int64_t)w * D;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < F4; ++i) {
        const float4 k4 = *reinterpret_cast<const float4*>(row + (i * LPR + sub) * 4);
        acc += fv[i].x * k4.x;
        acc += fv[i].y * k4.y;
        acc += fv[i].z * k4.z;
        acc += fv[i].w * k4.w;
      }
      m = fmaxf(m, sum8(acc));
    }
    if (sub == 0) keys[j - c0] = orderable_key(m);
  }
  __syncthreads();
  topk_union(keys, n, c0, topk, cur, n_init, n_local, U, idx + ((int64_t)bg * n_qb + qi) * U,
             cnt + (int64_t)bg * n_qb + qi, sh);
}

size_t window_select_workspace_bytes(int B, int H, int n_q_tokens, int64_t nw_cap) {
  return n_q_tokens > 0 ? 0 : (size_t)B * H * nw_cap * sizeof(float);
}

hipError_t launch_window_select(const WindowSelectArgs& a) {
  const int n_bg = a.B * a.H;
  const int64_t cap = a.nb_cap < kMaxCandidates ? a.nb_cap : kMaxCandidates;
  if (a.n_q_tokens > 0) {
    const int n_qb = (a.n_q_tokens + kBlk - 1) / kBlk;
    const dim3 grid(n_qb, n_bg);
#define BSKV_WIN_PREFILL(T, DD)                                                                                   \
  hipLaunchKernelGGL((window_prefill_kernel<T, DD>), grid, dim3(kThreads), (size_t)cap * sizeof(uint32_t), a.stream, \
                     (const T*)a.f, a.n_q_tokens, a.q_start, a.kcw, a.nw_cap, a.nb_cap, a.window, a.stride, a.topk,  \
                     a.n_init, a.n_local, a.U, n_qb, a.idx, a.cnt)
    if (a.f_dtype == 0) {
      if (a.D == 64) BSKV_WIN_PREFILL(float, 64); else BSKV_WIN_PREFILL(float, 128);
    } else {
      if (a.D == 64) BSKV_WIN_PREFILL(bf16_bits, 64); else BSKV_WIN_PREFILL(bf16_bits, 128);
    }
#undef BSKV_WIN_PREFILL
    return hipGetLastError();
  }
  const int ns = score_split_plan(n_bg, a.nw_cap);
  float* sc = (float*)a.ws;
  const dim3 grid(ns, n_bg);
  const float* f = (const float*)a.f;
  if (a.D == 64)
    hipLaunchKernelGGL(window_score_kernel<64>, grid, dim3(kThreads), 0, a.stream, f, a.kcw, a.nw_cap, a.seq_len,
                       a.H, a.n_init, a.n_local, a.window, a.stride, a.nb_cap, ns, sc);
  else
    hipLaunchKernelGGL(window_score_kernel<128>, grid, dim3(kThreads), 0, a.stream, f, a.kcw, a.nw_cap, a.seq_len,
                       a.H, a.n_init, a.n_local, a.window, a.stride, a.nb_cap, ns, sc);
  hipLaunchKernelGGL(window_topk_kernel, dim3(n_bg), dim3(kThreads), (size_t)cap * sizeof(uint32_t), a.stream, sc,
                     a.nw_cap, a.nb_cap, a.seq_len, a.H, a.window, a.stride, a.topk, a.n_init, a.n_local, a.U, a.idx,
                     a.cnt, a.scores);
  return hipGetLastError();
}

}  // namespace bskv
