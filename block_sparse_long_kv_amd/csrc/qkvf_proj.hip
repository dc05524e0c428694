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
// Decode (one token per sequence): one GEMV kernel on MFMA whose waves split
// the hidden axis and meet in LDS, then write Q (bf16), the new token's K and
// V (bf16, into the cache at position seq_len-1) and F (fp32).
//
// Prefill: a bf16 MFMA GEMM computing C^T = W^T X^T per tile of columns x
// tokens of one sequence, hidden in steps of 64 staged through LDS in two
// buffers (the next step's global loads are issued before the current
// step's MFMAs).  The weight is taken as W^T [N, hidden] and X is
// [tokens, hidden], so both operands are hidden-major.  Each wave owns whole
// 64-token query blocks, so the epilogue writes Q/K/V rows as bf16 and, for
// the Forecast columns, adds each query block's tokens in registers and
// across the 16 lanes of each row group: only the per-query-block sum
// leaves the kernel.
#include "decode_ops.hpp"
#include "bskv_launch.hpp"

namespace bskv {

// ------------------------------------------------------------------ decode
// GEMV on W^T [N, hidden]: workgroup = 16 output columns; its waves split
// the hidden axis evenly and run their range in steps of 32 with
// v_mfma_f32_16x16x32_bf16: A = 16 rows of W^T (one 16-byte load per lane),
// B = the batch's x rows (up to 16 sequences per MFMA, several chunks for
// larger batches); the waves' partial sums meet in LDS and wave 0 scatters:
// Q (bf16), the new token's K and V into the cache (bf16) and F (fp32).
// XL: the batch's x rows are first staged in LDS (rows padded by 64 bytes),
// so the weight stream is the only global read in the loop (up to 8
// sequences at hidden 4096: 66 KB, two workgroups per CU).
constexpr int kQkvfMaxBatch = 64;

// NW waves split the hidden axis; NB batch chunks of 16; UN hidden steps of
// 32 per load batch (hidden / NW a multiple of 32 UN)
template <int NW, int NB, int UN, bool XL>
__global__ __launch_bounds__(NW * 64) void qkvf_decode_kernel(const bf16_bits* __restrict__ x,
                                                             const bf16_bits* __restrict__ w, int B, int hidden,
                                                             int Hq, int H, int D, bf16_bits* __restrict__ q,
                                                             bf16_bits* __restrict__ kc, bf16_bits* __restrict__ vc,
                                                             int64_t sb, int64_t sg, int64_t st, int64_t kv_len,
                                                             const int64_t* __restrict__ seq_len,
                                                             float* __restrict__ f) {
  __shared__ float red[NW][NB][64][4];
  extern __shared__ uint4 xs[];        // XL: the batch's x rows, padded by 64 bytes
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int kq = hidden / NW, k_begin = wid * kq;
  const int rowq = hidden / 8 + 4;     // 16-byte units per staged row
  if constexpr (XL) {
    for (int i = tid; i < B * (hidden / 8); i += NW * 64) {
      const int b = i / (hidden / 8), c = i % (hidden / 8);
      xs[b * rowq + c] = ld16(x + (int64_t)b * hidden + 8 * c);
    }
    __syncthreads();
  }
  const bf16_bits* wrow = w + (int64_t)(n0 + l16) * hidden + 8 * lg;
  f32x4_t acc[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = k_begin; k < k_begin + kq; k += 32 * UN) {
    uint4 a[UN];
#pragma unroll
    // plain loads: one instruction reads 64 of a row's 128-byte line, the
    // next the other half, which then comes from L2 (a nontemporal load
    // would fetch the line twice)
    for (int u = 0; u < UN; ++u) a[u] = ld16(wrow + k + 32 * u);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int b = 16 * c + l16;
      uint4 xb[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u)
        xb[u] = b < B ? (XL ? xs[b * rowq + (k + 32 * u) / 8 + lg] : ld16(x + (int64_t)b * hidden + k + 32 * u + 8 * lg))
                      : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < UN; ++u)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[u]),
                                                         __builtin_bit_cast(bf16x8_t, xb[u]), acc[c], 0, 0, 0);
    }
  }
  // lane (b = l16, lg) of chunk c holds column n0 + 4lg + i for sequence 16c + l16
#pragma unroll
  for (int c = 0; c < NB; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wid][c][lane][i] = acc[c][i];
  __syncthreads();
  if (wid != 0) return;
  const int64_t seg_q = (int64_t)Hq * D, seg_kv = (int64_t)H * D;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int b = 16 * c + l16;
    if (b >= B) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) y += red[v][c][lane][i];
      const int n = n0 + 4 * lg + i;
      if (n < seg_q) {
        q[(int64_t)b * seg_q + n] = f32_to_bf16(y);
      } else if (n < seg_q + 2 * seg_kv) {
        const int64_t pos = seq_len[b] - 1;
        if (pos < 0 || pos >= kv_len) continue;   // the new token's row must be inside the cache
        const int r = n - (int)seg_q, g = (r / D) % H;
        (r < seg_kv ? kc : vc)[b * sb + g * sg + pos * st + r % D] = f32_to_bf16(y);
      } else {
        f[(int64_t)b * seg_kv + (n - seg_q - 2 * seg_kv)] = y;
      }
    }
  }
}

hipError_t launch_qkvf_decode(const QkvfDecodeArgs& a) {
  const int N = (a.Hq + 3 * a.H) * a.D;
  const dim3 grid(N / 16);
#define BSKV_QKVF_DEC(NW, NB, UN, XL)                                                                             \
  hipLaunchKernelGGL((qkvf_decode_kernel<NW, NB, UN, XL>), grid, dim3(NW * 64),                                    \
                     XL ? (size_t)a.B * (a.hidden / 8 + 4) * 16 : 0, a.stream, (const bf16_bits*)a.x,              \
                     (const bf16_bits*)a.w, a.B, a.hidden, a.Hq, a.H, a.D, (bf16_bits*)a.q, (bf16_bits*)a.k,       \
                     (bf16_bits*)a.v, a.sb, a.sg, a.st, a.kv_len, a.seq_len, a.f)
  // hidden is a multiple of 1024.  Up to 16 sequences, hidden a multiple of
  // 4096: eight waves of 512 hidden columns each issue all their weight loads
  // at once; otherwise four waves in steps of 8 x 32 (a quarter of hidden is
  // a multiple of 256)
  if (a.B <= 8 && a.hidden == 4096) BSKV_QKVF_DEC(8, 1, 8, true);
  else if (a.B <= 16 && a.hidden % 4096 == 0) BSKV_QKVF_DEC(8, 1, 8, false);
  else if (a.B <= 16) BSKV_QKVF_DEC(4, 1, 8, false);
  else if (a.B <= 32) BSKV_QKVF_DEC(4, 2, 8, false);
  else BSKV_QKVF_DEC(4, 4, 8, false);
#undef BSKV_QKVF_DEC
  return hipGetLastError();
}

// ------------------------------------------------------------------ prefill
// W^T [N, hidden] row-major (one row per output column, as a linear layer
// stores its weight) and X [tokens, hidden]: both operands are hidden-major,
// so every MFMA operand fragment is one 16-byte LDS read.
constexpr int kGemmBK = 64;               // hidden columns per stage
struct QkvfPrefillParams {
  const bf16_bits* x; const bf16_bits* w;
  int B, Tq, hidden, Hq, H, D, n_qb;
  int n_tiles_n, n_tiles_t, swizzle;   // column tiles, token tiles per sequence, XCD-aware order
  int64_t q_start;
  bf16_bits* q; bf16_bits* kc; bf16_bits* vc;
  int64_t sb, sg, st, kv_len;
  float* f_pooled;
};

// Epilogue of one wave's WN x WM accumulator tile: Q rows to q, K and V
// rows into the caches at their positions, and the Forecast columns summed
// over each 64-token query block into f_pooled.
template <int MI, int NI, int WM, int WN>
__device__ __forceinline__ void qkvf_epilogue(const QkvfPrefillParams& p, const f32x4_t (&acc)[NI][MI], int b, int n0,
                                              int t0, int wm, int wn, int l16, int lg) {
  // lane (l16, lg) of tile (ni, mi) holds C[token WM wm + 16mi + l16][column WN wn + 16ni + 4lg + i], i < 4
  const int seg_q = p.Hq * p.D, seg_k = seg_q + p.H * p.D, seg_v = seg_k + p.H * p.D;
  if (n0 < seg_v) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = n0 + WN * wn + 16 * ni + 4 * lg;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int t = t0 + WM * wm + 16 * mi + l16;
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
    // Forecast columns: each run of four token tiles is one query block
#pragma unroll
    for (int qs = 0; qs < WM / 64; ++qs) {
      const int qb = (t0 + WM * wm + 64 * qs) / kBlk;
      if (qb * kBlk >= p.Tq) break;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        float sum[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = 0.f;
#pragma unroll
          for (int mi = 4 * qs; mi < 4 * qs + 4; ++mi) v += acc[ni][mi][i];
          sum[i] = sum16(v);                         // the 16 tokens of each lane row group
        }
        if (l16 == 0) {
          const int r = n0 + WN * wn + 16 * ni + 4 * lg - seg_v, g = r / p.D;
          *reinterpret_cast<float4*>(p.f_pooled + (((int64_t)b * p.H + g) * p.n_qb + qb) * p.D + r % p.D) =
              make_float4(sum[0], sum[1], sum[2], sum[3]);
        }
      }
    }
  }
}

// C^T = W^T X^T per BN x BM tile (columns x tokens of one sequence), NW
// waves of WN columns x WM tokens (WM a multiple of 64: whole query blocks).
// The operand tiles are copied straight from HBM into an NSTG-stage LDS ring
// (global_load_lds_dwordx4, 1024 contiguous LDS bytes per wave
// instruction): no registers hold tiles in transit, no LDS writes are
// issued, and a stage's copy is issued NSTG-1 K-steps before its use.
// LDS rows are the K-step's 64 hidden columns (128 bytes) with 16-byte
// chunks XOR-swizzled per row (chunk c of row r at c ^ ((r / 2) % 8)), so the
// 16 rows of a fragment read cover all banks.  Token rows past the chunk are
// copied from its last row and then zeroed in LDS, so they add nothing to
// the pooled Forecast.
template <int BM, int BN, int WM, int WN, int NSTG>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void qkvf_prefill_ring_kernel(QkvfPrefillParams p) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int RB = kGemmBK * 2;                 // bytes per LDS row
  constexpr int XT = BM * RB, WT = BN * RB;       // bytes of one stage's X and W^T tiles
  constexpr int PX = XT / 1024, PW = WT / 1024;   // 1024-byte copy pieces
  constexpr int PPW = (PX + PW) / NW;             // pieces per wave per stage
  static_assert(WM % 64 == 0 && WN % 16 == 0 && (PX + PW) % NW == 0 && NSTG >= 2, "tiling");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
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
  const int n0 = tn * BN, t0 = (tm % p.n_tiles_t) * BM;
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int wn = wid % (BN / WN), wm = wid / (BN / WN);
  const bf16_bits* xb = p.x + (int64_t)b * p.Tq * p.hidden;
  const bool tail = t0 + BM > p.Tq;
  const uint32_t lds0 = lds_u32(smem_raw);

  // this lane's chunk of each of the wave's pieces: row r, stored chunk q & 7
  auto issue = [&](int s) {
    const int k0 = s * kGemmBK;
    const uint32_t base = lds0 + (uint32_t)((s % NSTG) * (XT + WT));
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int piece = wid * PPW + i;
      const bool is_x = piece < PX;
      const int pc = is_x ? piece : piece - PX;
      const int q = pc * 64 + lane, r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
      const bf16_bits* src = is_x ? xb + (int64_t)min(t0 + r, p.Tq - 1) * p.hidden + k0 + 8 * c
                                  : p.w + (int64_t)(n0 + r) * p.hidden + k0 + 8 * c;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(base + (uint32_t)((is_x ? 0 : XT) + pc * 1024)));
    }
  };
  // token rows past the chunk: this lane's X chunks of stage s read zero
  auto zero_tail = [&](int s) {
    unsigned char* base = smem_raw + (s % NSTG) * (XT + WT);
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int piece = wid * PPW + i;
      if (piece < PX && t0 + ((piece * 64 + lane) >> 3) >= p.Tq)
        *reinterpret_cast<uint4*>(base + piece * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  };

  f32x4_t acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // fragment offsets: row 16 x + l16 of a tile, chunk 4 ks + lg, swizzle (l16 / 2)
  const int swz = l16 >> 1;
  const int off0 = l16 * RB + 16 * ((0 + lg) ^ swz), off1 = l16 * RB + 16 * ((4 + lg) ^ swz);

  const int n_steps = p.hidden / kGemmBK;
#pragma unroll
  for (int s = 0; s < NSTG - 1; ++s)
    if (s < n_steps) issue(s);
  for (int s = 0; s < n_steps; ++s) {
    if (s + NSTG - 2 < n_steps) wait_vm<(NSTG - 2) * PPW>();
    else wait_vm<0>();
    if (tail) zero_tail(s);
    __syncthreads();                  // stage s complete; stage s-1 read by every wave
    if (s + NSTG - 1 < n_steps) issue(s + NSTG - 1);
    const unsigned char* xs = smem_raw + (s % NSTG) * (XT + WT);
    const unsigned char* ws = xs + XT;
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 32; ++ks) {
      const int off = ks == 0 ? off0 : off1;
      bf16x8_t a[NI], bx[MI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        a[ni] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ws + (WN * wn + 16 * ni) * RB + off));
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        bx[mi] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(xs + (WM * wm + 16 * mi) * RB + off));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ni], bx[mi], acc[ni][mi], 0, 0, 0);
    }
  }
  qkvf_epilogue<MI, NI, WM, WN>(p, acc, b, n0, t0, wm, wn, l16, lg);
}

template <int BM, int BN, int WM, int WN, int NSTG>
static hipError_t launch_qkvf_prefill_ring_t(QkvfPrefillParams p, int N, hipStream_t stream) {
  p.n_tiles_n = N / BN;
  p.n_tiles_t = (p.Tq + BM - 1) / BM;
  const int n_m = p.n_tiles_t * p.B, total = n_m * p.n_tiles_n;
  p.swizzle = (n_m % 8 == 0 && p.n_tiles_n % 8 == 0) ? 1 : 0;
  const size_t lds = (size_t)NSTG * (BM + BN) * kGemmBK * 2;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((qkvf_prefill_ring_kernel<BM, BN, WM, WN, NSTG>), dim3(total), dim3(NT), lds, stream, p);
  return hipGetLastError();
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
  // Two-stage LDS ring.  Per 8192 x 4096 x 7168 chunk: 256 x 256 tiles (eight
  // waves, one workgroup per CU) 411 us = 1.17 PFLOP/s; 128 x 128 tiles (two
  // workgroups per CU) 424 us, and the same tiles staged through registers
  // 549 us; 256 x 128 with three stages 451 us; 128 x 128 with four stages
  // 592 us.  A 256-column tile must not straddle the Forecast columns.
  const int seg_v = (a.Hq + 2 * a.H) * a.D;
  if (N % 256 == 0 && seg_v % 256 == 0) return launch_qkvf_prefill_ring_t<256, 256, 128, 64, 2>(p, N, a.stream);
  return launch_qkvf_prefill_ring_t<128, 128, 64, 64, 2>(p, N, a.stream);
}

}  // namespace bskv
