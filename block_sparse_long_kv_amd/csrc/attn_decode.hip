// Block-sparse decode attention: one query token per (batch, query head)
// attends to the tokens of its KV head's selected blocks only.
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Eq. 5 and Alg. 2 (attention
// of the layer's own query over K/V of the selected blocks).
//
// Design (gfx950): grid (n_splits, B*Hkv).  A workgroup owns one KV head and
// a run of `bps` listed blocks, and serves all G query heads of that KV head,
// so every K/V byte is read from HBM once per step.  Per 64-token block:
//   QK  4 lanes per token, each 4 x 16-byte loads interleaved so a token's
//       4 lanes read 64 contiguous bytes per load; G dot products per lane,
//       2 xor-shuffles to finish them.
//   softmax  wave w keeps the running max / sum of heads w, w+4 (base-2
//       exponent: q is pre-scaled by scale*log2(e)).
//   PV  lane = (16-byte column chunk, token lane); G x VEC fp32 accumulators.
// The split's partial (o, m, l) goes to the workspace; the last workgroup of
// the KV head (agent-scope counter) merges the splits in split order, so the
// result does not depend on scheduling.
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

constexpr int kAttnBlock = 64;
constexpr int kMaxSplits = 64;

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t sb, int64_t sg, int64_t st,
    int64_t kv_len, int ring, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, const int64_t* __restrict__ seq_len,
    int Hkv, int U, float qscale, int bps, int n_splits, float* __restrict__ out, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, int* __restrict__ ws_count) {
  constexpr int BLK = kAttnBlock;
  constexpr int VEC = VecN<T>::N;
  constexpr int NKL = D / 4 / VEC;       // 16-byte K loads per lane
  constexpr int DCH = D / VEC;           // 16-byte column chunks of a row
  constexpr int TL = kThreads / DCH;     // token lanes in PV
  constexpr int TPL = BLK / TL;          // tokens per lane in PV
  constexpr int HW = (G + 3) / 4;        // heads per softmax wave
  __shared__ float qs[G][D];
  __shared__ float sraw[G][BLK];
  __shared__ float ps[G][BLK];
  __shared__ float alpha_s[G];
  __shared__ float red[4][G][D];
  __shared__ float wts[kMaxSplits][G];
  __shared__ float den_s[G];
  __shared__ int is_last;

  const int bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv, split = blockIdx.x;
  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c = min(cnt[bg], U);
  const int u0 = split * bps, u1 = min(c, u0 + bps);
  const int64_t L = seq_len[b];

  for (int i = tid; i < G * D; i += kThreads)
    qs[i / D][i % D] = to_f32<T>(q[((int64_t)b * Hq + g * G) * D + i]) * qscale;
  float m_run[HW], l_run[HW];
#pragma unroll
  for (int i = 0; i < HW; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  float acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  __syncthreads();

  const int tok = tid >> 2, part = tid & 3;
  const int dc = tid % DCH, tl = tid / DCH;
  const T* kbase = k + b * sb + g * sg;
  const T* vbase = v + b * sb + g * sg;

  for (int u = u0; u < u1; ++u) {
    const int j = idx[(int64_t)bg * U + u];
    const int64_t tb = (int64_t)(ring ? u : j) * BLK;
    // a block id outside the buffers is skipped (uniform over the workgroup)
    if (j < 0 || tb + BLK > kv_len) continue;
    const int64_t rem = L - (int64_t)j * BLK;
    const int nvalid = rem <= 0 ? 0 : (rem >= BLK ? BLK : (int)rem);
    uint4 kr[NKL], vr[TPL];
    const T* kp = kbase + (tb + tok) * st + part * VEC;
#pragma unroll
    for (int i = 0; i < NKL; ++i) kr[i] = ld16(kp + i * 4 * VEC);
#pragma unroll
    for (int i = 0; i < TPL; ++i) vr[i] = ld16(vbase + (tb + tl + i * TL) * st + dc * VEC);

    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      float kf[VEC];
      cvt16<T>(kr[i], kf);
      const int d0 = (i * 4 + part) * VEC;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[h] += kf[e] * qs[h][d0 + e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] += __shfl_xor(s[h], 1);
      s[h] += __shfl_xor(s[h], 2);
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
      if ((h & 3) == part) sraw[h][tok] = (tok < nvalid) ? s[h] : -INFINITY;
    __syncthreads();

#pragma unroll
    for (int i = 0; i < HW; ++i) {
      const int h = wid + 4 * i;
      if (h < G) {
        const float x = sraw[h][lane];
        const float mn = fmaxf(m_run[i], wave_max(x));
        float p, al;
        if (mn == -INFINITY) { p = 0.f; al = 1.f; }
        else { p = exp2f(x - mn); al = exp2f(m_run[i] - mn); }
        l_run[i] = l_run[i] * al + wave_sum(p);
        m_run[i] = mn;
        ps[h][lane] = p;
        if (lane == 0) alpha_s[h] = al;
      }
    }
    __syncthreads();

#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = alpha_s[h];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int t = tl + i * TL;
      if (t < nvalid) {
        float vf[VEC];
        cvt16<T>(vr[i], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = ps[h][t];
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] += p * vf[e];
        }
      }
    }
  }

  // sum the token lanes: first inside the wave, then across the 4 waves
#pragma unroll
  for (int o = DCH; o < 64; o <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
  if (lane < DCH) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) red[wid][h][dc * VEC + e] = acc[h][e];
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)bg * n_splits + split) * G;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    ws_o[(pbase + h) * D + d] = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
  }
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const int h = wid + 4 * i;
    if (h < G && lane == 0) {
      ws_ml[(pbase + h) * 2 + 0] = m_run[i];
      ws_ml[(pbase + h) * 2 + 1] = l_run[i];
    }
  }

  // the last workgroup of this KV head merges the splits in split order
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(&ws_count[bg], 1) == n_splits - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const int64_t sbase = (int64_t)bg * n_splits * G;
  if (tid < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, ws_ml[(sbase + sp * G + tid) * 2]);
    float den = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) {
      const float m = ws_ml[(sbase + sp * G + tid) * 2], l = ws_ml[(sbase + sp * G + tid) * 2 + 1];
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
      wts[sp][tid] = w;
      den += w * l;
    }
    den_s[tid] = den;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float num = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) num += wts[sp][h] * ws_o[(sbase + sp * G + h) * D + d];
    const float den = den_s[h];
    out[((int64_t)b * Hq + g * G + h) * D + d] = den > 0.f ? num / den : 0.f;
  }
  if (tid == 0) ws_count[bg] = 0;
}

// Split plan: about 1024 workgroups, every split the same number of listed
// blocks, at most kMaxSplits splits.
static void decode_split_plan(int n_bg, int U, int& n_splits, int& bps) {
  int ns = (1024 + n_bg - 1) / n_bg;
  if (ns > U) ns = U;
  if (ns > kMaxSplits) ns = kMaxSplits;
  if (ns < 1) ns = 1;
  bps = (U + ns - 1) / ns;
  n_splits = (U + bps - 1) / bps;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int U) {
  int ns, bps;
  const int n_bg = B * Hkv, G = Hq / Hkv;
  decode_split_plan(n_bg, U, ns, bps);
  auto al = [](size_t x) { return ((x + 255) / 256) * 256; };
  return al((size_t)n_bg * ns * G * D * sizeof(float)) + al((size_t)n_bg * ns * G * 2 * sizeof(float)) +
         al((size_t)n_bg * sizeof(int));
}

template <typename T, int D, int G>
static void launch_attn_decode_t(const AttnDecodeArgs& a, int ns, int bps, float* wo, float* wml, int* ctr) {
  const float qscale = a.scale * 1.4426950408889634f;
  dim3 grid(ns, a.B * a.Hkv);
  hipLaunchKernelGGL((attn_decode_kernel<T, D, G>), grid, dim3(kThreads), 0, a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, a.sb, a.sg, a.st, a.kv_len, a.ring, a.idx, a.cnt, a.seq_len, a.Hkv, a.U, qscale, bps, ns,
                     a.out, wo, wml, ctr);
}

template <typename T, int D>
static void launch_attn_decode_g(const AttnDecodeArgs& a, int G, int ns, int bps, float* wo, float* wml, int* ctr) {
  switch (G) {
    case 1: launch_attn_decode_t<T, D, 1>(a, ns, bps, wo, wml, ctr); break;
    case 2: launch_attn_decode_t<T, D, 2>(a, ns, bps, wo, wml, ctr); break;
    case 4: launch_attn_decode_t<T, D, 4>(a, ns, bps, wo, wml, ctr); break;
    default: launch_attn_decode_t<T, D, 8>(a, ns, bps, wo, wml, ctr); break;
  }
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a) {
  int ns, bps;
  const int n_bg = a.B * a.Hkv, G = a.Hq / a.Hkv;
  decode_split_plan(n_bg, a.U, ns, bps);
  auto al = [](size_t x) { return ((x + 255) / 256) * 256; };
  float* wo = (float*)a.ws;
  float* wml = (float*)((char*)wo + al((size_t)n_bg * ns * G * a.D * sizeof(float)));
  int* ctr = (int*)((char*)wml + al((size_t)n_bg * ns * G * 2 * sizeof(float)));
  if (a.dtype == 0) {
    if (a.D == 64) launch_attn_decode_g<float, 64>(a, G, ns, bps, wo, wml, ctr);
    else launch_attn_decode_g<float, 128>(a, G, ns, bps, wo, wml, ctr);
  } else {
    if (a.D == 64) launch_attn_decode_g<bf16_bits, 64>(a, G, ns, bps, wo, wml, ctr);
    else launch_attn_decode_g<bf16_bits, 128>(a, G, ns, bps, wo, wml, ctr);
  }
  return hipGetLastError();
}

}  // namespace bskv
