// Baseline multi-head block selector (decode), kept beside the Forecast
// selector so that the two can be compared on the same GPU.
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "One Forecast head per GQA group", the baseline
// selector listing of Sec. 3.1: every query head of a KV group scores every
// candidate block against the compressed keys, the per-head scores are
// summed into a shared score, a softmax of the shared score / sqrt(d) weights
// the candidates, and the top-k of those weights is taken; the block set is
// completed with the initial and local blocks as for the Forecast selector
// ("The problem InfLLM-V2 leaves on the table", block-set formula).
//
// Kernel 1 (score slices): workgroup (split, b*Hkv + g) holds the G query
// rows of the group (fp32) and streams its slice of compressed-key rows with
// 128-bit nontemporal loads, 8 lanes per row; each lane adds the products of
// all G heads over its part of the row, one 8-lane sum gives the shared score.
// Kernel 2 (softmax + top-k), one workgroup per (b, g): maximum and
// exponential sum over the candidates (block reductions), the weights as
// orderable keys, then the radix select + union of the Forecast selector;
// up to 8 * kThreads candidates the row is read once and stays in
// registers, above that the keys go through LDS.
#include "decode_ops.hpp"
#include "bskv_launch.hpp"

namespace bskv {

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void mh_score_kernel(const T* __restrict__ q, const float* __restrict__ kc,
                                                          int64_t nb_cap, const int64_t* __restrict__ seq_len, int H,
                                                          int n_init, int n_local, int n_splits,
                                                          float* __restrict__ sc) {
  constexpr int LPR = 8;                 // lanes per key row
  constexpr int F4 = D / 4 / LPR;        // float4 of a row per lane
  constexpr int RPP = kThreads / LPR;    // rows per pass
  constexpr int UNR = 4;                 // passes whose loads are in flight together
  __shared__ __attribute__((aligned(16))) float qs[G][D];
  const int bg = blockIdx.y, split = blockIdx.x;
  const int b = bg / H, g = bg % H;
  const DecodeCands dc = decode_cands(seq_len[b], nb_cap, n_init, n_local);
  const int n = dc.c1 - dc.c0;
  const int per = (n + n_splits - 1) / n_splits;
  const int lo = dc.c0 + split * per, hi = min(dc.c1, lo + per);
  for (int i = threadIdx.x; i < G * D; i += kThreads)
    qs[i / D][i % D] = to_f32<T>(q[((int64_t)b * H * G + (int64_t)g * G) * D + i]);
  __syncthreads();
  const int sub = threadIdx.x % LPR, row0 = threadIdx.x / LPR;
  float4 qv[G][F4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < F4; ++i) qv[h][i] = *reinterpret_cast<const float4*>(&qs[h][(i * LPR + sub) * 4]);
  const float* kc_bg = kc + (int64_t)bg * nb_cap * D;
  float* out = sc + (int64_t)bg * nb_cap;
  for (int base = lo; base < hi; base += RPP * UNR) {
    float4 kv[UNR][F4];
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int j = base + row0 + uu * RPP;
      if (j < hi) {
#pragma unroll
        for (int i = 0; i < F4; ++i) kv[uu][i] = ld16f_nt(kc_bg + (int64_t)j * D + (i * LPR + sub) * 4);
      }
    }
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int j = base + row0 + uu * RPP;
      float acc = 0.f;
      if (j < hi) {
#pragma unroll
        for (int h = 0; h < G; ++h)        // the G heads' score rows, summed
#pragma unroll
          for (int i = 0; i < F4; ++i)
            acc += qv[h][i].x * kv[uu][i].x + qv[h][i].y * kv[uu][i].y + qv[h][i].z * kv[uu][i].z +
                   qv[h][i].w * kv[uu][i].w;
      }
      acc = sum8(acc);   // the 8 lanes of the row (all active together)
      if (sub == 0 && j < hi) out[j] = acc;
    }
  }
}

// max (op 0) or sum (op 1) over the 256 threads of the block
template <int OP>
__device__ __forceinline__ float block_reduce(float v, float* tmp) {
  v = OP == 0 ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) tmp[wid] = v;
  __syncthreads();
  float r = tmp[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = OP == 0 ? fmaxf(r, tmp[w]) : r + tmp[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void mh_topk_kernel(const float* __restrict__ sc, int64_t nb_cap,
                                                         const int64_t* __restrict__ seq_len, int H, int topk,
                                                         int n_init, int n_local, int U, float scale_log2e,
                                                         int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                         float* __restrict__ w_out) {
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  __shared__ float red[kThreads / 64];
  const int bg = blockIdx.x;
  const DecodeCands dc = decode_cands(seq_len[bg / H], nb_cap, n_init, n_local);
  const int n = dc.c1 - dc.c0;
  const float* row = sc + (int64_t)bg * nb_cap + dc.c0;
  if (n <= 8 * kThreads) {
    // the row read once into registers (thread t: candidates 8t .. 8t+7),
    // the maximum, the sum and the weights from there
    float v[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * (int)threadIdx.x + e;
      v[e] = i < n ? row[i] : -INFINITY;
      mx = fmaxf(mx, v[e]);
    }
    mx = block_reduce<0>(mx, red);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += 8 * (int)threadIdx.x + e < n ? __builtin_amdgcn_exp2f((v[e] - mx) * scale_log2e) : 0.f;
    sum = block_reduce<1>(sum, red);
    const float inv = n > 0 ? 1.f / sum : 0.f;
    uint32_t kin[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * (int)threadIdx.x + e;
      const float w = __builtin_amdgcn_exp2f((v[e] - mx) * scale_log2e) * inv;   // softmax weight
      kin[e] = orderable_key(i < n ? w : 0.f);
      if (w_out && i < n) w_out[(int64_t)bg * nb_cap + dc.c0 + i] = w;
    }
    topk_union_fast(dc.c0, dc.c0, dc.c1, topk, dc.cur, n_init, n_local, U, idx + (int64_t)bg * U, cnt + bg, sh, kin);
    return;
  }
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kThreads) mx = fmaxf(mx, row[i]);
  mx = block_reduce<0>(mx, red);
  float sum = 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) sum += __builtin_amdgcn_exp2f((row[i] - mx) * scale_log2e);
  sum = block_reduce<1>(sum, red);
  const float inv = n > 0 ? 1.f / sum : 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const float w = __builtin_amdgcn_exp2f((row[i] - mx) * scale_log2e) * inv;   // softmax weight
    keys[i] = orderable_key(w);
    if (w_out) w_out[(int64_t)bg * nb_cap + dc.c0 + i] = w;
  }
  __syncthreads();
  topk_union(keys, n, dc.c0, topk, dc.cur, n_init, n_local, U, idx + (int64_t)bg * U, cnt + bg, sh);
}

template <typename T, int D>
static void launch_mh_score_t(const MultiheadSelectArgs& a, int ns, float* sc) {
  const dim3 grid(ns, a.B * a.H);
  const T* q = (const T*)a.q;
  switch (a.G) {
    case 1: hipLaunchKernelGGL((mh_score_kernel<T, D, 1>), grid, dim3(kThreads), 0, a.stream, q, a.kc, a.nb_cap,
                               a.seq_len, a.H, a.n_init, a.n_local, ns, sc); break;
    case 2: hipLaunchKernelGGL((mh_score_kernel<T, D, 2>), grid, dim3(kThreads), 0, a.stream, q, a.kc, a.nb_cap,
                               a.seq_len, a.H, a.n_init, a.n_local, ns, sc); break;
    case 4: hipLaunchKernelGGL((mh_score_kernel<T, D, 4>), grid, dim3(kThreads), 0, a.stream, q, a.kc, a.nb_cap,
                               a.seq_len, a.H, a.n_init, a.n_local, ns, sc); break;
    default: hipLaunchKernelGGL((mh_score_kernel<T, D, 8>), grid, dim3(kThreads), 0, a.stream, q, a.kc, a.nb_cap,
                                a.seq_len, a.H, a.n_init, a.n_local, ns, sc); break;
  }
}

size_t multihead_select_workspace_bytes(int B, int H, int64_t nb_cap) { return (size_t)B * H * nb_cap * sizeof(float); }

hipError_t launch_multihead_select(const MultiheadSelectArgs& a) {
  const int n_bg = a.B * a.H;
  const int ns = score_split_plan(n_bg, a.nb_cap);
  float* sc = (float*)a.ws;
  if (a.q_dtype == 0) {
    if (a.D == 64) launch_mh_score_t<float, 64>(a, ns, sc);
    else launch_mh_score_t<float, 128>(a, ns, sc);
  } else {
    if (a.D == 64) launch_mh_score_t<bf16_bits, 64>(a, ns, sc);
    else launch_mh_score_t<bf16_bits, 128>(a, ns, sc);
  }
  const int64_t cap = a.nb_cap < kMaxCandidates ? a.nb_cap : kMaxCandidates;
  hipLaunchKernelGGL(mh_topk_kernel, dim3(n_bg), dim3(kThreads), (size_t)cap * sizeof(uint32_t), a.stream, sc,
                     a.nb_cap, a.seq_len, a.H, a.topk, a.n_init, a.n_local, a.U, a.scale * 1.4426950408889634f,
                     a.idx, a.cnt, a.weights);
  return hipGetLastError();
}

}  // namespace bskv
