// Forecast block scoring, causal top-k and union with the initial and local
// blocks, for decode and for prefill chunks.
//
// Sources: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection" (Eq. 4; Alg. 1 prefill and
// Alg. 2 decode selection), "One Forecast head per GQA group" (Sec. 4.1:
// one raw dot product per block, ranking only), "Training" (Eq. 7 comment:
// top-k after the causal mask, without the initial and local blocks),
// "The problem InfLLM-V2 leaves on the table" (block-set formula).
#include <algorithm>

#include "decode_ops.hpp"
#include "bskv_launch.hpp"

namespace bskv {

// ---------------------------------------------------------------------------
// Prefill, in three launches:
//   1. (per-token Forecasts only) each query block's Forecast vectors are
//      summed into one fp32 row: fp [B*H, n_qb, D];
//   2. scores of every query block of the chunk against every causal
//      compressed key as one fp32 MFMA contraction per (b, g):
//      S^T = K~ Fp^T with v_mfma_f32_16x16x4_f32, a workgroup per 128 blocks
//      x 32 query blocks (each K~ row is read once per 32 query blocks,
//      instead of once per query block);
//   3. one top-k + union workgroup per query block over its candidates
//      (the decode selector's workgroup on the query block's score row).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pool_forecast_kernel(const T* __restrict__ f, int Tq, int n_qb,
                                                               float* __restrict__ fp) {
  __shared__ PoolRowsSmem<T, D> ps;
  const int qi = blockIdx.x, bg = blockIdx.y;
  const int t0 = qi * 64, t1 = min(Tq, t0 + 64);
  pool_rows<T, D>(f + ((int64_t)bg * Tq + t0) * D, t1 - t0, ps);
  for (int t = threadIdx.x; t < D; t += kThreads) fp[((int64_t)bg * n_qb + qi) * D + t] = ps.fpool[t];
}

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

// Scores S[qi][j] of query blocks qi0 .. qi0+31 against blocks j0 .. j0+127
// (wave w: blocks j0 + 32w .. +31).  fp32 MFMA 16x16x4: A = K~ rows (lane:
// block l16, dims 4lg..4lg+3 of each 16-dim slice), B = Fp^T (lane: query
// block l16, the same dims); each lane loads 16-byte pieces and feeds one
// component per MFMA.  Rows past nb_span or n_qb are zero and not stored.
template <int D>
__global__ __launch_bounds__(kThreads) void score_prefill_mfma_kernel(const float* __restrict__ fp,
                                                                    const float* __restrict__ kc, int64_t nb_cap,
                                                                    int nb_span, int n_qb, float* __restrict__ sc) {
  constexpr int S4 = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int bg = blockIdx.z, qi0 = blockIdx.y * 32, j0 = blockIdx.x * 128 + 32 * wid;
  const float* kc_bg = kc + (int64_t)bg * nb_cap * D;
  const float* fp_bg = fp + (int64_t)bg * n_qb * D;
  float4 a[2][S4], b[2][S4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int j = j0 + 16 * mt + l16;
#pragma unroll
    for (int s4 = 0; s4 < S4; ++s4)
      a[mt][s4] = j < nb_span ? *reinterpret_cast<const float4*>(kc_bg + (int64_t)j * D + 16 * s4 + 4 * lg)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = qi0 + 16 * nt + l16;
#pragma unroll
    for (int s4 = 0; s4 < S4; ++s4)
      b[nt][s4] = qi < n_qb ? *reinterpret_cast<const float4*>(fp_bg + (int64_t)qi * D + 16 * s4 + 4 * lg)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  f32x4v_t acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < S4; ++s4)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float av = c == 0 ? a[mt][s4].x : c == 1 ? a[mt][s4].y : c == 2 ? a[mt][s4].z : a[mt][s4].w;
          const float bv = c == 0 ? b[nt][s4].x : c == 1 ? b[nt][s4].y : c == 2 ? b[nt][s4].z : b[nt][s4].w;
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[mt][nt], 0, 0, 0);
        }
  // lane (l16, lg) of tile (mt, nt) holds S[query block qi0 + 16nt + l16][block j0 + 16mt + 4lg + i]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = qi0 + 16 * nt + l16;
    if (qi >= n_qb) continue;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = j0 + 16 * mt + 4 * lg;
      if (j >= nb_span) continue;
      float* dst = sc + ((int64_t)bg * n_qb + qi) * nb_cap + j;
      if (j + 4 <= nb_span) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]);
      } else {
        for (int i = 0; i < nb_span - j; ++i) dst[i] = acc[mt][nt][i];
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void topk_prefill_kernel(const float* __restrict__ sc, int64_t nb_cap,
                                                              int64_t q_start, int n_qb, int topk, int n_init,
                                                              int n_local, int U, int32_t* __restrict__ idx_out,
                                                              int32_t* __restrict__ cnt_out) {
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  const int qi = blockIdx.x, bg = blockIdx.y;
  const int64_t prob = (int64_t)bg * n_qb + qi;
  DecodeCands dc;
  dc.cur = (int)(q_start / 64) + qi;
  dc.c0 = n_init;
  dc.c1 = (int)min((int64_t)(dc.cur - n_local + 1), nb_cap);
  if (dc.c1 < dc.c0) dc.c1 = dc.c0;
  topk_decode_wg(sc + prob * nb_cap, nb_cap, dc, topk, n_init, n_local, U, idx_out + prob * U, cnt_out + prob, keys, sh);
}

// fp: [B*H, n_qb, D] fp32 summed Forecasts; sc: workspace [B*H, n_qb, nb_cap]
static hipError_t launch_prefill_select(const float* fp, int n_qb, int64_t q_start, const float* kc, int64_t nb_cap,
                                        int n_bg, int D, int topk, int n_init, int n_local, int32_t* idx,
                                        int32_t* cnt, float* sc, hipStream_t stream) {
  // blocks any query block of the chunk may score: below the last one's local window
  const int64_t cur_last = q_start / 64 + n_qb - 1;
  const int nb_span = (int)std::max<int64_t>(0, std::min<int64_t>(cur_last - n_local + 1, nb_cap));
  if (nb_span > 0) {
    const dim3 grid((nb_span + 127) / 128, (n_qb + 31) / 32, n_bg);
    if (D == 64)
      hipLaunchKernelGGL(score_prefill_mfma_kernel<64>, grid, dim3(kThreads), 0, stream, fp, kc, nb_cap, nb_span, n_qb,
                         sc);
    else
      hipLaunchKernelGGL(score_prefill_mfma_kernel<128>, grid, dim3(kThreads), 0, stream, fp, kc, nb_cap, nb_span,
                         n_qb, sc);
  }
  const int64_t cap = nb_cap < kMaxCandidates ? nb_cap : kMaxCandidates;
  hipLaunchKernelGGL(topk_prefill_kernel, dim3(n_qb, n_bg), dim3(kThreads), (size_t)cap * sizeof(uint32_t), stream, sc,
                     nb_cap, q_start, n_qb, topk, n_init, n_local, topk + n_init + n_local, idx, cnt);
  return hipGetLastError();
}

static size_t al256(size_t x) { return ((x + 255) / 256) * 256; }

size_t prefill_select_workspace_bytes(int n_bg, int n_qb, int64_t nb_cap, int D, bool pooled) {
  return al256((size_t)n_bg * n_qb * nb_cap * sizeof(float)) + (pooled ? 0 : (size_t)n_bg * n_qb * D * sizeof(float));
}

hipError_t launch_score_topk_pooled(const float* f_pooled, int n_qb, int64_t q_start, const float* kc,
                                   int64_t nb_cap, int B, int H, int D, int topk, int n_init, int n_local,
                                   int32_t* idx, int32_t* cnt, void* ws, hipStream_t stream) {
  return launch_prefill_select(f_pooled, n_qb, q_start, kc, nb_cap, B * H, D, topk, n_init, n_local, idx, cnt,
                               (float*)ws, stream);
}

size_t score_decode_workspace_bytes(int B, int H, int64_t nb_cap);
hipError_t launch_score_topk_decode(const ScoreTopkArgs& a);

size_t score_topk_workspace_bytes(int B, int H, int n_q_tokens, int64_t nb_cap, int D) {
  if (n_q_tokens > 0) return prefill_select_workspace_bytes(B * H, (n_q_tokens + 63) / 64, nb_cap, D, false);
  return score_decode_workspace_bytes(B, H, nb_cap);
}

hipError_t launch_score_topk(const ScoreTopkArgs& a) {
  if (a.n_q_tokens == 0) return launch_score_topk_decode(a);
  const int n_bg = a.B * a.H;
  const int n_qb = (a.n_q_tokens + a.block - 1) / a.block;
  char* ws = (char*)a.ws;
  float* sc = (float*)ws;
  float* fp = (float*)(ws + al256((size_t)n_bg * n_qb * a.nb_cap * sizeof(float)));
  const dim3 grid(n_qb, n_bg);
  if (a.f_dtype == 0) {
    if (a.D == 64) hipLaunchKernelGGL((pool_forecast_kernel<float, 64>), grid, dim3(kThreads), 0, a.stream,
                                      (const float*)a.f, a.n_q_tokens, n_qb, fp);
    else hipLaunchKernelGGL((pool_forecast_kernel<float, 128>), grid, dim3(kThreads), 0, a.stream,
                            (const float*)a.f, a.n_q_tokens, n_qb, fp);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((pool_forecast_kernel<bf16_bits, 64>), grid, dim3(kThreads), 0, a.stream,
                                      (const bf16_bits*)a.f, a.n_q_tokens, n_qb, fp);
    else hipLaunchKernelGGL((pool_forecast_kernel<bf16_bits, 128>), grid, dim3(kThreads), 0, a.stream,
                            (const bf16_bits*)a.f, a.n_q_tokens, n_qb, fp);
  }
  return launch_prefill_select(fp, n_qb, a.q_start, a.kc, a.nb_cap, n_bg, a.D, a.topk, a.n_init, a.n_local, a.idx,
                               a.cnt, sc, a.stream);
}

}  // namespace bskv
