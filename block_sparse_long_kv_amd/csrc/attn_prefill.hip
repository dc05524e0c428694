// Block-sparse causal prefill attention on bf16 MFMA (fp32 accumulate).
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Eq. 5 and Alg. 1 (attention
// of the chunk's queries over the K/V of each query block's selected blocks).
//
// Design (gfx950, v_mfma_f32_16x16x32_bf16):
//   * One workgroup per (query block of 64 tokens, KV head): 2G wavefronts,
//     wave w serves query head g*G + w/2, rows (w%2)*32 .. +31, so the G
//     query heads of a KV head share every K/V block staged in LDS.
//   * Scores are computed transposed, S^T = K Q^T (keys on the MFMA M side):
//     the accumulator layout then gives each lane one query column, so the
//     online-softmax statistics and the probabilities stay in the lane that
//     owns them, and P^T feeds O^T = V^T P^T as the B operand directly.
//   * K and V are staged row-major in LDS with 16-byte writes (rows padded);
//     the V^T operand is read with gfx950's transposing LDS read
//     (ds_read_b64_tr_b16), two per operand.
//   * Two LDS stages and a register prefetch: while block u is computed from
//     LDS stage u%2, block u+1 (already in registers) is written to the other
//     stage and block u+2 is requested from memory; one barrier per block.
//   * Softmax VALU kept to the minimum (it is the other half of the work at
//     head_dim 128): raw v_exp_f32, the scale folded into one FMA, the causal
//     mask only on the diagonal block, a finite initial running max instead
//     of -inf guards, and the output rescaled only when some row max moved.
//   * Workgroups are ordered so that consecutive query blocks of one KV head
//     run on the same XCD: neighbouring query blocks share most of their
//     local-window blocks, which then hit in that XCD's L2.
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& r) { return __builtin_bit_cast(bf16x8_t, r); }

template <int D, int G>
__global__ __launch_bounds__(G * 128) void attn_prefill_kernel(
    const bf16_bits* __restrict__ q, const bf16_bits* __restrict__ k, const bf16_bits* __restrict__ v, int64_t sb,
    int64_t sg, int64_t st, int64_t kv_len, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    int64_t q_start, int Tq, int Hkv, int U, int n_qb, float qscale, bf16_bits* __restrict__ out) {
  constexpr int BLK = 64;
  constexpr int NT = G * 128;          // threads
  constexpr int KSTR = D + 8;          // LDS row of K: D bf16 + 16 bytes
  constexpr int VSTR = D + 16;         // LDS row of V: D bf16 + 32 bytes (transposing reads hit distinct banks)
  constexpr int RCH = D / 8;           // 16-byte chunks per token row
  constexpr int NCH = BLK * RCH;       // 16-byte chunks per block per tensor
  constexpr int CPT = (NCH + NT - 1) / NT;  // chunks per thread per tensor
  constexpr int KS = D / 32;           // k-steps of S^T
  constexpr int MD = D / 16;           // d tiles of O^T
  // two LDS stages: block u+1 is written while block u is read
  __shared__ __attribute__((aligned(16))) bf16_bits Ks[2][BLK * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_bits Vs[2][BLK * VSTR];

  const int n_tiles = gridDim.x;
  int lin = blockIdx.x;
  if ((n_tiles & 7) == 0) lin = (lin & 7) * (n_tiles >> 3) + (lin >> 3);
  const int qi = lin % n_qb, bg = lin / n_qb;
  const int b = bg / Hkv, g = bg % Hkv;
  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = g * G + (wid >> 1);
  const int row0 = (wid & 1) * 32;
  const int l16 = lane & 15, lg = lane >> 4;
  const int qb = (int)(q_start / BLK) + qi;
  const int tq0 = qi * BLK;

  // Q^T fragments (B operand of S^T): query rows row0 + 16*nq + l16
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int t = tq0 + row0 + 16 * nq + l16;
    const bf16_bits* qp = q + (((int64_t)b * Hq + h) * Tq + t) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (t < Tq) r = ld16(qp + 32 * ks);
      qf[nq][ks] = as_bf16x8(r);
    }
  }

  f32x4_t o[MD][2];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) o[md][nq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // running max (base-2, scaled) starts finite: a fully masked block then
  // gives p = 0 and alpha = 1 without special cases
  float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.f, 0.f};

  const int64_t prob = (int64_t)bg * n_qb + qi;
  const int c = min(cnt[prob], U);
  const int32_t* list = idx + prob * U;
  const bf16_bits* kb = k + b * sb + g * sg;
  const bf16_bits* vb = v + b * sb + g * sg;

  // a listed block is used only if it lies inside the K/V buffers
  auto valid = [&](int jj) { return jj >= 0 && ((int64_t)jj + 1) * BLK <= kv_len; };
  uint4 kreg[CPT], vreg[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) kreg[i] = vreg[i] = make_uint4(0, 0, 0, 0);
  auto gload = [&](int jj) {
    if (!valid(jj)) return;
    const bf16_bits* kq = kb + (int64_t)jj * BLK * st;
    const bf16_bits* vq = vb + (int64_t)jj * BLK * st;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * NT, r = ch / RCH, cc = ch % RCH;
      if (NCH % NT == 0 || ch < NCH) {
        kreg[i] = ld16(kq + (int64_t)r * st + cc * 8);
        vreg[i] = ld16(vq + (int64_t)r * st + cc * 8);
      }
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * NT, r = ch / RCH, cc = ch % RCH;
      if (NCH % NT != 0 && ch >= NCH) continue;
      *reinterpret_cast<uint4*>(&Ks[stage][r * KSTR + cc * 8]) = kreg[i];
      *reinterpret_cast<uint4*>(&Vs[stage][r * VSTR + cc * 8]) = vreg[i];
    }
  };
  if (c > 0) {
    gload(list[0]);
    lstore(0);
    if (c > 1) gload(list[1]);
  }
  __syncthreads();

  for (int u = 0; u < c; ++u) {
    const int j = list[u];
    const int stage = u & 1;
    // stage the next block into the other LDS buffer, then prefetch the one after
    if (u + 1 < c) {
      lstore(stage ^ 1);
      if (u + 2 < c) gload(list[u + 2]);
    }

    // S^T tiles: keys 16*mt .. (M), queries row0 + 16*nq .. (N)
    f32x4_t s[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) s[mt][nq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8_t a =
            as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[stage][(16 * mt + l16) * KSTR + 32 * ks + 8 * lg]));
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) s[mt][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nq][ks], s[mt][nq], 0, 0, 0);
      }
    }

    // causal mask: only the diagonal block (uniform over the workgroup);
    // a listed block outside the buffers is masked whole
    if (j >= qb || !valid(j)) {
      const bool ok = valid(j);
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        const int rq = row0 + 16 * nq + l16;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!ok || 16 * mt + 4 * lg + i > rq) s[mt][nq][i] = -INFINITY;
      }
    }

    // online softmax per query column (lane-local, 2 xor-shuffles per reduction)
    bf16x8_t pb[2][2];
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      float mx = s[0][nq][0];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][nq][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_run[nq], mx * qscale);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nq] - mn);
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nq][i], qscale, -mn));
          s[mt][nq][i] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      l_run[nq] = l_run[nq] * alpha + sum;
      m_run[nq] = mn;
      // rescale the output only when some row's max moved (rare after the first blocks)
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md][nq] *= alpha;
      }
      // P^T operand for key step s2: slots 0..3 <- tile 2*s2, slots 4..7 <- tile 2*s2+1
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8_t p8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p8[e] = (__bf16)s[2 * s2][nq][e];
          p8[4 + e] = (__bf16)s[2 * s2 + 1][nq][e];
        }
        pb[s2][nq] = p8;
      }
    }

    // O^T += V^T P^T.  The V^T operand (lane: d = 16*md + l16, keys 32*s2 + 4*lg + {0..3}
    // and 32*s2 + 16 + 4*lg + {0..3}) comes from row-major V with transposing LDS reads:
    // within each 16-lane group, lane 4r+c reads key row r, columns 4c..4c+3, and
    // ds_read_b64_tr_b16 hands lane i element i%4 of lane 4r+i/4 for r = 0..3.
    const int tr_row = 4 * lg + (l16 >> 2), tr_col = 4 * (l16 & 3);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const bf16_bits* v0 = &Vs[stage][(32 * s2 + tr_row) * VSTR + 16 * md + tr_col];
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)v0);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v0 + 16 * VSTR));
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) o[md][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[s2][nq], o[md][nq], 0, 0, 0);
      }
    }
    __syncthreads();   // stage^1 is complete for everyone; stage may be overwritten next
  }

  // epilogue: O[query][d] = O^T[d][query] / l
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int t = tq0 + row0 + 16 * nq + l16;
    if (t < Tq) {
      const float inv = l_run[nq] > 0.f ? 1.f / l_run[nq] : 0.f;
      bf16_bits* op = out + (((int64_t)b * Hq + h) * Tq + t) * D + 4 * lg;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const uint32_t w0 = (uint32_t)f32_to_bf16(o[md][nq][0] * inv) | ((uint32_t)f32_to_bf16(o[md][nq][1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(o[md][nq][2] * inv) | ((uint32_t)f32_to_bf16(o[md][nq][3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + 16 * md) = make_uint2(w0, w1);
      }
    }
  }
}

template <int D, int G>
static void launch_prefill_t(const AttnPrefillArgs& a) {
  const int n_qb = (a.Tq + 63) / 64;
  const int n_tiles = n_qb * a.B * a.Hkv;
  const float qscale = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_prefill_kernel<D, G>), dim3(n_tiles), dim3(G * 128), 0, a.stream, (const bf16_bits*)a.q,
                     (const bf16_bits*)a.k, (const bf16_bits*)a.v, a.sb, a.sg, a.st, a.kv_len, a.idx, a.cnt, a.q_start, a.Tq,
                     a.Hkv, a.U, n_qb, qscale, (bf16_bits*)a.out);
}

template <int D>
static void launch_prefill_d(const AttnPrefillArgs& a, int G) {
  switch (G) {
    case 1: launch_prefill_t<D, 1>(a); break;
    case 2: launch_prefill_t<D, 2>(a); break;
    case 4: launch_prefill_t<D, 4>(a); break;
    default: launch_prefill_t<D, 8>(a); break;
  }
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (a.D == 64) launch_prefill_d<64>(a, G);
  else launch_prefill_d<128>(a, G);
  return hipGetLastError();
}

}  // namespace bskv
