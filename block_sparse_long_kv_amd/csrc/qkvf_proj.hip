// The layer's projection widened by the Forecast head group:
// (Q, K, V, F) = X [W_Q | W_K | W_V | W_F].
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Eq. 3 (the existing linear
// projection, widened by one small head group, emits F_l next to Q, K, V)
// and Alg. 1 (prefill: F selects per 64-token query block, whose score is
// the sum over its tokens).  Columns of W: query heads, key heads, value
// heads, Forecast heads, head_dim columns each.
//
// Decode (one token per sequence): split-K partials on MFMA (the Forecast
// projection's kernel, over all columns), then one pass that adds the splits
// and scatters: Q (bf16), the new token's K and V (bf16, into the cache at
// position seq_len-1) and F (fp32).
//
// Prefill: a bf16 MFMA GEMM computing C^T = W^T X^T per 128 x 128 tile
// (columns x tokens of one sequence), hidden in steps of 64 staged through
// LDS in two buffers (the next step's global loads are issued before the
// current step's MFMAs).  W^T is read from its row-major tile with the
// transposing LDS read (as in the Forecast projection), X^T straight from
// the token rows.  Each wave owns 64 columns x 64 tokens -- one query block
// -- so the epilogue writes Q/K/V rows as bf16 and, for the Forecast
// columns, adds the wave's 64 tokens in registers and across the 16 lanes of
// each row group: only the per-query-block sum leaves the kernel.
#include "decode_ops.hpp"
#include "bskv_launch.hpp"

namespace bskv {

// ------------------------------------------------------------------ decode
__global__ __launch_bounds__(kThreads) void qkvf_scatter_kernel(const float* __restrict__ part, int n_splits, int B,
                                                              int Hq, int H, int D, bf16_bits* __restrict__ q,
                                                              bf16_bits* __restrict__ kc, bf16_bits* __restrict__ vc,
                                                              int64_t sb, int64_t sg, int64_t st, int64_t kv_len,
                                                              const int64_t* __restrict__ seq_len,
                                                              float* __restrict__ f) {
  const int N = (Hq + 3 * H) * D;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= B * N) return;
  const int b = i / N, n = i % N;
  const float y = proj_reduce_one(part, n_splits, B, N, b, n);
  const int head = n / D, e = n % D;
  if (head < Hq) {
    q[((int64_t)b * Hq + head) * D + e] = f32_to_bf16(y);
    return;
  }
  const int r = head - Hq;
  if (r < 2 * H) {
    const int64_t pos = seq_len[b] - 1;
    if (pos < 0 || pos >= kv_len) return;      // the new token's row must be inside the cache
    const int g = r % H;
    bf16_bits* dst = r < H ? kc : vc;
    dst[b * sb + g * sg + pos * st + e] = f32_to_bf16(y);
    return;
  }
  f[((int64_t)b * H + (r - 2 * H)) * D + e] = y;
}

size_t qkvf_decode_workspace_bytes(int B, int hidden, int N) {
  return (size_t)proj_splits(hidden) * B * N * sizeof(float);
}

hipError_t launch_qkvf_decode(const QkvfDecodeArgs& a) {
  const int N = (a.Hq + 3 * a.H) * a.D;
  float* part = (float*)a.ws;
  launch_proj_partial<bf16_bits>(a.x, a.w, a.B, a.hidden, N, part, a.stream);
  const int n = a.B * N;
  hipLaunchKernelGGL(qkvf_scatter_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, a.stream, part,
                     proj_splits(a.hidden), a.B, a.Hq, a.H, a.D, (bf16_bits*)a.q, (bf16_bits*)a.k, (bf16_bits*)a.v,
                     a.sb, a.sg, a.st, a.kv_len, a.seq_len, a.f);
  return hipGetLastError();
}

// ------------------------------------------------------------------ prefill
constexpr int kGemmBM = 128;              // tokens per tile
constexpr int kGemmBN = 128;              // output columns per tile
constexpr int kGemmBK = 64;               // hidden rows per stage
constexpr int kGemmWStr = kGemmBN + 16;   // W tile row: 288 bytes (conflict-free transposing reads)
constexpr int kGemmXStr = kGemmBK + 8;    // X tile row: 144 bytes

struct QkvfGemmSmem {
  bf16_bits w[2][kGemmBK * kGemmWStr];
  bf16_bits x[2][kGemmBM * kGemmXStr];
};

struct QkvfPrefillParams {
  const bf16_bits* x; const bf16_bits* w;
  int B, Tq, hidden, Hq, H, D, n_qb;
  int n_tiles_n, n_tiles_t, swizzle;   // column tiles, token tiles per sequence, XCD-aware order
  int64_t q_start;
  bf16_bits* q; bf16_bits* kc; bf16_bits* vc;
  int64_t sb, sg, st, kv_len;
  float* f_pooled;
};

__global__ __launch_bounds__(kThreads, 2) void qkvf_prefill_kernel(QkvfPrefillParams p) {
  __shared__ __attribute__((aligned(16))) QkvfGemmSmem sm;
  constexpr int CW = kGemmBK * kGemmBN / 8 / kThreads;   // 16-byte chunks of the W tile per thread (4)
  constexpr int CX = kGemmBM * kGemmBK / 8 / kThreads;   // of the X tile (4)
  const int N = (p.Hq + 3 * p.H) * p.D;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2).  With the swizzle, XCD x takes a contiguous run of the tile space
  // in 8 x 8 groups of (token tile, column tile): the ~64 workgroups one XCD
  // runs at a time share 8 token tiles and 8 column tiles, so each K-step's
  // operands are fetched into that L2 once and read by 8 workgroups.
  int tn, tm;
  {
    const int bid = blockIdx.x, n_m = p.n_tiles_t * p.B;
    if (p.swizzle) {
      const int per_xcd = (int)gridDim.x / 8;
      const int L = (bid % 8) * per_xcd + bid / 8;
      const int within = L % 64, group = L / 64;
      const int groups_m = n_m / 8;
      tm = (group % groups_m) * 8 + within % 8;
      tn = (group / groups_m) * 8 + within / 8;
    } else {
      tm = bid % n_m;
      tn = bid / n_m;
    }
  }
  const int b = tm / p.n_tiles_t;
  const int n0 = tn * kGemmBN, t0 = (tm % p.n_tiles_t) * kGemmBM;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wn = wid & 1, wm = wid >> 1;
  const bf16_bits* xb = p.x + (int64_t)b * p.Tq * p.hidden;

  uint4 rw[CW], rx[CX];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int c = tid + i * kThreads, r = c >> 4, cc = c & 15;
      rw[i] = ld16(p.w + (int64_t)(k0 + r) * N + n0 + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = tid + i * kThreads, r = c >> 3, cc = c & 7;
      const int t = t0 + r;
      rx[i] = t < p.Tq ? ld16(xb + (int64_t)t * p.hidden + k0 + cc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int c = tid + i * kThreads, r = c >> 4, cc = c & 15;
      *reinterpret_cast<uint4*>(&sm.w[buf][r * kGemmWStr + cc * 8]) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = tid + i * kThreads, r = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&sm.x[buf][r * kGemmXStr + cc * 8]) = rx[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int tr_row = 4 * lg + (l16 >> 2), tr_col = 4 * (l16 & 3);
  const int n_steps = p.hidden / kGemmBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < n_steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < n_steps) gload((s + 1) * kGemmBK);
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 32; ++ks) {
      bf16x8_t a[4], bx[4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        // A = W^T: lane (column l16, group lg) holds hidden rows 4lg..4lg+3 and 16+4lg..16+4lg+3
        const bf16_bits* v0 = &sm.w[buf][(32 * ks + tr_row) * kGemmWStr + 64 * wn + 16 * ni + tr_col];
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)v0);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v0 + 16 * kGemmWStr));
        a[ni] = __builtin_bit_cast(bf16x8_t, s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        // B = X^T: lane (token l16, group lg) holds the same hidden rows of its token
        const bf16_bits* xp = &sm.x[buf][(64 * wm + 16 * mi + l16) * kGemmXStr + 32 * ks + 4 * lg];
        const uint2 lo = *reinterpret_cast<const uint2*>(xp);
        const uint2 hi = *reinterpret_cast<const uint2*>(xp + 16);
        bx[mi] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ni], bx[mi], acc[ni][mi], 0, 0, 0);
    }
    if (s + 1 < n_steps) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // lane (l16, lg) of tile (ni, mi) holds C[token 64wm + 16mi + l16][column 64wn + 16ni + 4lg + i], i < 4
  const int seg_q = p.Hq * p.D, seg_k = seg_q + p.H * p.D, seg_v = seg_k + p.H * p.D;
  if (n0 < seg_v) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = n0 + 64 * wn + 16 * ni + 4 * lg;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int t = t0 + 64 * wm + 16 * mi + l16;
        if (t >= p.Tq) continue;
        const uint32_t w01 = (uint32_t)f32_to_bf16(acc[ni][mi][0]) | ((uint32_t)f32_to_bf16(acc[ni][mi][1]) << 16);
        const uint32_t w23 = (uint32_t)f32_to_bf16(acc[ni][mi][2]) | ((uint32_t)f32_to_bf16(acc[ni][mi][3]) << 16);
        bf16_bits* dst;
        if (n < seg_q) {
          dst = p.q + (((int64_t)b * p.Hq + n / p.D) * p.Tq + t) * p.D + n % p.D;
        } else {
          const int64_t pos = p.q_start + t;
          if (pos >= p.kv_len) continue;            // the row must be inside the cache
          const int r = n - seg_q, g = (r / p.D) % p.H;
          dst = (r < p.H * p.D ? p.kc : p.vc) + b * p.sb + g * p.sg + pos * p.st + r % p.D;
        }
        *reinterpret_cast<uint2*>(dst) = make_uint2(w01, w23);
      }
    }
  } else {
    // Forecast columns: the wave's 64 tokens are one query block
    const int qb = (t0 + 64 * wm) / kBlk;
    if (qb * kBlk >= p.Tq) return;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = 0.f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) v += acc[ni][mi][i];
        s[i] = sum16(v);                           // the 16 tokens of each lane row group
      }
      if (l16 == 0) {
        const int r = n0 + 64 * wn + 16 * ni + 4 * lg - seg_v, g = r / p.D;
        *reinterpret_cast<float4*>(p.f_pooled + (((int64_t)b * p.H + g) * p.n_qb + qb) * p.D + r % p.D) =
            make_float4(s[0], s[1], s[2], s[3]);
      }
    }
  }
}

hipError_t launch_qkvf_prefill(const QkvfPrefillArgs& a) {
  QkvfPrefillParams p;
  p.x = (const bf16_bits*)a.x; p.w = (const bf16_bits*)a.w;
  p.B = a.B; p.Tq = a.Tq; p.hidden = a.hidden; p.Hq = a.Hq; p.H = a.H; p.D = a.D;
  p.n_qb = (a.Tq + kBlk - 1) / kBlk;
  p.q_start = a.q_start;
  p.q = (bf16_bits*)a.q; p.kc = (bf16_bits*)a.k; p.vc = (bf16_bits*)a.v;
  p.sb = a.sb; p.sg = a.sg; p.st = a.st; p.kv_len = a.kv_len;
  p.f_pooled = a.f_pooled;
  const int N = (a.Hq + 3 * a.H) * a.D;
  p.n_tiles_n = N / kGemmBN;
  p.n_tiles_t = (a.Tq + kGemmBM - 1) / kGemmBM;
  const int n_m = p.n_tiles_t * a.B, total = n_m * p.n_tiles_n;
  p.swizzle = (n_m % 8 == 0 && p.n_tiles_n % 8 == 0) ? 1 : 0;   // then total is a multiple of 64
  hipLaunchKernelGGL(qkvf_prefill_kernel, dim3(total), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace bskv
