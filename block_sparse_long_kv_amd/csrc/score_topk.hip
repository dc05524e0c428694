// Forecast block scoring, causal top-k and union with the initial and local
// blocks, for decode and for prefill chunks.
//
// Sources: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection" (Eq. 4; Alg. 1 prefill and
// Alg. 2 decode selection), "One Forecast head per GQA group" (Sec. 4.1:
// one raw dot product per block, ranking only), "Training" (Eq. 7 comment:
// top-k after the causal mask, without the initial and local blocks),
// "The problem InfLLM-V2 leaves on the table" (block-set formula).
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

// Scores of rows [lo, hi) of kc against the fp32 vector fv (held as F4
// float4 per lane, 8 lanes per row).  Each 8-lane group handles one row per
// pass; 32 rows per pass for 256 threads.  Calls sink(j, score) from the
// group's lane 0.
template <int D, typename Sink>
__device__ __forceinline__ void score_rows(const float* __restrict__ kc_bg, const float4* fv, int lo, int hi,
                                           Sink sink) {
  constexpr int LPR = 8;
  constexpr int F4 = D / 4 / LPR;
  const int sub = threadIdx.x % LPR, row0 = threadIdx.x / LPR;
  for (int j = lo + row0; j < hi; j += kThreads / LPR) {
    const float* row = kc_bg + (int64_t)j * D;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const float4 k4 = *reinterpret_cast<const float4*>(row + (i * LPR + sub) * 4);
      acc += fv[i].x * k4.x;
      acc += fv[i].y * k4.y;
      acc += fv[i].z * k4.z;
      acc += fv[i].w * k4.w;
    }
    acc = sum8(acc);   // the 8 lanes of the row (all active together)
    if (sub == 0) sink(j, acc);
  }
}

template <int D>
__device__ __forceinline__ void load_fvec(const float* src, float4* fv) {
  constexpr int LPR = 8;
  constexpr int F4 = D / 4 / LPR;
  const int sub = threadIdx.x % LPR;
#pragma unroll
  for (int i = 0; i < F4; ++i) fv[i] = *reinterpret_cast<const float4*>(src + (i * LPR + sub) * 4);
}

// ---------------------------------------------------------------------------
// Prefill: grid (n_qb, B*H); one workgroup per query block.  It sums the
// block's Forecast vectors (fp32), scores every candidate compressed key
// into LDS and runs the top-k + union.
// ---------------------------------------------------------------------------
// POOLED: f already holds each query block's Forecast sum, fp32
// [B*H, n_qb, D] (as the widened projection writes it); Tq is unused.
template <typename T, int D, bool POOLED = false>
__global__ __launch_bounds__(kThreads) void score_topk_prefill_kernel(
    const T* __restrict__ f, int Tq, int64_t q_start, const float* __restrict__ kc, int64_t nb_cap, int H, int block,
    int topk, int n_init, int n_local, int U, int n_qb, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out) {
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  __shared__ PoolRowsSmem<T, D> ps;

  const int qi = blockIdx.x, bg = blockIdx.y;
  if constexpr (POOLED) {
    for (int t = threadIdx.x; t < D; t += kThreads) ps.fpool[t] = f[((int64_t)bg * n_qb + qi) * D + t];
    __syncthreads();
  } else {
    // pooled Forecast of the query block: sum of its tokens' vectors
    const int t0 = qi * block, t1 = min(Tq, t0 + block);
    pool_rows<T, D>(f + ((int64_t)bg * Tq + t0) * D, t1 - t0, ps);
  }
  const int cur = (int)(q_start / block) + qi;
  const int c0 = n_init, c1 = min(cur - n_local + 1, (int)nb_cap);
  const int n = max(0, c1 - c0);
  float4 fv[D / 32];
  load_fvec<D>(ps.fpool, fv);
  const float* kc_bg = kc + (int64_t)bg * nb_cap * D;
  score_rows<D>(kc_bg, fv, c0, c1, [&](int j, float s) { keys[j - c0] = orderable_key(s); });
  __syncthreads();
  topk_union(keys, n, c0, topk, cur, n_init, n_local, U, idx_out + ((int64_t)bg * n_qb + qi) * U,
             cnt_out + (int64_t)bg * n_qb + qi, sh);
}

size_t score_decode_workspace_bytes(int B, int H, int64_t nb_cap);
hipError_t launch_score_topk_decode(const ScoreTopkArgs& a);

size_t score_topk_workspace_bytes(int B, int H, int n_q_tokens, int64_t nb_cap, int D) {
  (void)D;
  return n_q_tokens > 0 ? 0 : score_decode_workspace_bytes(B, H, nb_cap);
}

hipError_t launch_score_topk_pooled(const float* f_pooled, int n_qb, int64_t q_start, const float* kc,
                                   int64_t nb_cap, int B, int H, int D, int topk, int n_init, int n_local,
                                   int32_t* idx, int32_t* cnt, hipStream_t stream) {
  const int64_t cand_cap = nb_cap < kMaxCandidates ? nb_cap : kMaxCandidates;
  const size_t lds = (size_t)cand_cap * sizeof(uint32_t);
  const dim3 grid(n_qb, B * H);
  const int U = topk + n_init + n_local;
  if (D == 64)
    hipLaunchKernelGGL((score_topk_prefill_kernel<float, 64, true>), grid, dim3(kThreads), lds, stream, f_pooled, 0,
                       q_start, kc, nb_cap, H, 64, topk, n_init, n_local, U, n_qb, idx, cnt);
  else
    hipLaunchKernelGGL((score_topk_prefill_kernel<float, 128, true>), grid, dim3(kThreads), lds, stream, f_pooled, 0,
                       q_start, kc, nb_cap, H, 64, topk, n_init, n_local, U, n_qb, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_score_topk(const ScoreTopkArgs& a) {
  const int n_bg = a.B * a.H;
  const int64_t cand_cap = a.nb_cap < kMaxCandidates ? a.nb_cap : kMaxCandidates;
  const size_t lds = (size_t)cand_cap * sizeof(uint32_t);
  if (a.n_q_tokens == 0) return launch_score_topk_decode(a);
  const int n_qb = (a.n_q_tokens + a.block - 1) / a.block;
  dim3 grid(n_qb, n_bg);
#define BSKV_PREFILL_LAUNCH(T, DD)                                                                           \
  hipLaunchKernelGGL((score_topk_prefill_kernel<T, DD>), grid, dim3(kThreads), lds, a.stream, (const T*)a.f, \
                     a.n_q_tokens, a.q_start, a.kc, a.nb_cap, a.H, a.block, a.topk, a.n_init, a.n_local, a.U, n_qb, \
                     a.idx, a.cnt)
  if (a.f_dtype == 0) {
    if (a.D == 64) BSKV_PREFILL_LAUNCH(float, 64); else BSKV_PREFILL_LAUNCH(float, 128);
  } else {
    if (a.D == 64) BSKV_PREFILL_LAUNCH(bf16_bits, 64); else BSKV_PREFILL_LAUNCH(bf16_bits, 128);
  }
#undef BSKV_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace bskv
