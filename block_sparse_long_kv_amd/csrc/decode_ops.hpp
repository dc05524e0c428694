// Workgroup-level building blocks of the decode hot path.  Each function is
// the whole work of one workgroup for one work item, so the same code runs
// in the per-operation kernels of the C ABI and in the fused per-layer
// pipeline.  No function communicates with other workgroups: every
// cross-workgroup combination (projection splits, score slices, attention
// splits) is done by a workgroup of a LATER kernel, after the kernel
// boundary has made the partial results visible.  (An agent-scope fence per
// workgroup costs an L2 writeback on gfx950, which serialises per XCD.)
//
// Sources: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection" (Eq. 3 projection, Eq. 4
// selection, Eq. 5 attention, Alg. 2 decode step), "One Forecast head per
// GQA group" (Sec. 4.1 raw-score selector, one head per KV head), "The
// problem InfLLM-V2 leaves on the table" (mean-pooled keys, block set),
// "Training" (Eq. 7 comment: top-k after the causal mask, without the initial
// and local blocks).
#pragma once

#include <type_traits>

#include "bskv_device.hpp"

namespace bskv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kBlk = 64;            // tokens per KV block
constexpr int kMaxSplitsDecode = 32;   // attention splits per KV head

// ---------------------------------------------------------------------------
// Forecast projection, split over the hidden dimension.
//   part[split][b][n] = sum_{r in split} x[b, r] W[r, n]
// Workgroup (tile, split): TC = 16*VEC columns, kProjRows rows.  Thread =
// (row lane 0..15, 16-byte column chunk 0..15) holding its kProjRows/16 rows
// of W in registers (all loads issued first); the batch is processed in
// passes of kProjPass rows that reuse those registers; the 16 row lanes are
// added through LDS, one barrier pair per pass.
// ---------------------------------------------------------------------------
// 256 rows of W per split: at hidden 4096 that is 16 splits x 8 column tiles =
// 128 workgroups (bf16), which with the decode top-k's 64 workgroups in the
// fused layer's first kernel leaves every workgroup a CU of its own (B8 x
// 128K: first kernel 6.1-6.2 vs 7.1 us, step 1.417-1.423 vs 1.444-1.468 ms
// against 128 rows; 512 rows 1.48-1.50 ms)
constexpr int kProjRows = 256;
// bf16 (MFMA) workgroups take 128 or 256 rows of W but always store one
// partial per 128 rows, so every caller sums the same partials in the same
// order: the fused layer's first kernel spans 128 rows when it carries no
// top-k (256 workgroups at hidden 4096; B4 x 32K: that kernel 4.2 vs 5.1 us),
// 256 rows beside the top-k, and the standalone projection 256.
constexpr int kProjPartRows = 128;
constexpr int kProjPass = 4;     // batch rows per pass
constexpr int kProjMaxB = 16;    // batch rows staged in LDS per round

struct ProjSmem {
  float xs[kProjMaxB][kProjRows];
  float red[16][kProjPass][132];
};

template <typename T>
__host__ __device__ constexpr int proj_tile_cols_host() { return 16 * VecN<T>::N; }

template <typename T>
__device__ __forceinline__ void proj_partial_wg(const T* __restrict__ x, const T* __restrict__ w, int B, int hidden, int N, int tile,
                                int split, float* __restrict__ part, ProjSmem& sm) {
  constexpr int VEC = VecN<T>::N;
  constexpr int TC = 16 * VEC;
  constexpr int RPT = kProjRows / 16;   // rows of W per thread
  const int c = threadIdx.x & 15, rl = threadIdx.x >> 4;
  const int r_begin = split * kProjRows;
  const int col0 = tile * TC + c * VEC;
  uint4 raw[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) raw[i] = ld16_nt(w + (int64_t)(r_begin + rl + 16 * i) * N + col0);
  for (int b0 = 0; b0 < B; b0 += kProjMaxB) {
    const int nb = min(kProjMaxB, B - b0);
    // stage x[b0 .. b0+nb)[r_begin .. +kProjRows) as fp32 (16-byte loads)
    constexpr int XV = kProjRows / VEC;   // 16-byte vectors per batch row
    for (int i = threadIdx.x; i < nb * XV; i += kThreads) {
      const int bb = i / XV, cv = i % XV;
      float xv[VEC];
      cvt16<T>(ld16(x + (int64_t)(b0 + bb) * hidden + r_begin + cv * VEC), xv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm.xs[bb][cv * VEC + e] = xv[e];
    }
    __syncthreads();
    for (int p0 = 0; p0 < nb; p0 += kProjPass) {
      float acc[kProjPass][VEC];
#pragma unroll
      for (int bb = 0; bb < kProjPass; ++bb)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[bb][e] = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        float wv[VEC];
        cvt16<T>(raw[i], wv);
        const int r = rl + 16 * i;
#pragma unroll
        for (int bb = 0; bb < kProjPass; ++bb) {
          const float xv = (p0 + bb < nb) ? sm.xs[p0 + bb][r] : 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[bb][e] += xv * wv[e];
        }
      }
#pragma unroll
      for (int bb = 0; bb < kProjPass; ++bb)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm.red[rl][bb][c * VEC + e] = acc[bb][e];
      __syncthreads();
      for (int t = threadIdx.x; t < kProjPass * TC; t += kThreads) {
        const int bb = t / TC, col = t % TC;
        if (p0 + bb < nb) {
          float s = 0.f;
#pragma unroll
          for (int q = 0; q < 16; ++q) s += sm.red[q][bb][col];
          part[((int64_t)split * B + b0 + p0 + bb) * N + tile * TC + col] = s;
        }
      }
      __syncthreads();
    }
  }
}

// bf16 projection partials on MFMA (v_mfma_f32_16x16x32_bf16) for one tile
// of 128 rows x 128 columns of W:  F^T[n][b] = sum_k W^T[n][k] x^T[k][b].
// W is staged row-major in LDS (rows padded to 288 bytes) and read as the A
// operand with transposing reads: within each 16-lane group, lane 4r+c reads
// row r, columns 4c..4c+3, and ds_read_b64_tr_b16 hands lane i element i%4
// of lane 4r+i/4, so lane (m, g) gets column m at rows 4g..4g+3 (and, from a
// second read 16 rows down, 16+4g..16+4g+3).  x^T is the B operand, loaded
// from memory in the same row order (lane: batch row m).  Wave w owns column
// tiles 2w and 2w+1; one pass, no cross-lane reduction.
constexpr int kProjWStr = 128 + 16;
struct ProjMfmaSmem {
  bf16_bits w[kProjRows * kProjWStr];
};

// ROWS (128 or 256) rows of W from row span * ROWS; one partial per
// kProjPartRows rows: partial index r / kProjPartRows.
template <int ROWS>
__device__ __forceinline__ void proj_partial_mfma_wg(const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ w, int B,
                                     int hidden, int N, int tile, int span, float* __restrict__ part,
                                     ProjMfmaSmem& sm) {
  static_assert(ROWS % kProjPartRows == 0 && ROWS <= kProjRows, "row span");
  constexpr int TC = 128;
  constexpr int CPT = ROWS * TC / 8 / kThreads;   // 16-byte chunks of the tile per thread
  constexpr int KPP = kProjPartRows / 32;         // k-steps per partial
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int r_begin = span * ROWS, n0 = tile * TC;
  // x^T fragments (B operand) of batch rows b0 + l16, in the row order of
  // the transposed W reads
  auto load_x = [&](int b0, bf16x8_t (&xb)[ROWS / 32]) {
    const int b = b0 + l16;
#pragma unroll
    for (int ks = 0; ks < ROWS / 32; ++ks) {
      uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
      if (b < B) {
        const bf16_bits* xp = x + (int64_t)b * hidden + r_begin + 32 * ks + 4 * lg;
        lo = *reinterpret_cast<const uint2*>(xp);
        hi = *reinterpret_cast<const uint2*>(xp + 16);
      }
      xb[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  };
  uint4 raw[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = tid + i * kThreads, r = ch >> 4, cc = ch & 15;
    raw[i] = ld16_nt(w + (int64_t)(r_begin + r) * N + n0 + cc * 8);
  }
  // the first 16 batch rows travel beside the W tile, not after it
  bf16x8_t xb[ROWS / 32];
  load_x(0, xb);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = tid + i * kThreads, r = ch >> 4, cc = ch & 15;
    *reinterpret_cast<uint4*>(&sm.w[r * kProjWStr + cc * 8]) = raw[i];
  }
  __syncthreads();
  const int tr_row = 4 * lg + (l16 >> 2), tr_col = 4 * (l16 & 3);
  for (int b0 = 0; b0 < B; b0 += 16) {
    const int b = b0 + l16;
    if (b0 > 0) load_x(b0, xb);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int nt = 2 * wid + t;
#pragma unroll
      for (int pp = 0; pp < ROWS / kProjPartRows; ++pp) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KPP; ++kk) {
          const int ks = pp * KPP + kk;
          const bf16_bits* v0 = &sm.w[(32 * ks + tr_row) * kProjWStr + 16 * nt + tr_col];
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)v0);
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v0 + 16 * kProjWStr));
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[ks], acc, 0, 0, 0);
        }
        // lane (b, lg) holds F^T[n0 + 16 nt + 4 lg + i][b], i = 0..3, over
        // the partial's 128 rows
        const int64_t part_id = r_begin / kProjPartRows + pp;
        if (b < B)
          *reinterpret_cast<float4*>(&part[(part_id * B + b) * N + n0 + 16 * nt + 4 * lg]) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
  }
}

// F[b, n] = sum over splits of the partials, in split order (up to 32 loads
// issued before any is added: one round trip for hidden sizes up to 4096).
__device__ __forceinline__ float proj_reduce_one(const float* __restrict__ part, int n_splits, int B, int N, int b,
                                                 int n) {
  float s = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += 32) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = (s0 + i < n_splits) ? part[((int64_t)(s0 + i) * B + b) * N + n] : 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += v[i];
  }
  return s;
}

// ---------------------------------------------------------------------------
// Mean-pool one 64-token block of keys (one workgroup).
// ---------------------------------------------------------------------------
template <typename T, int D>
struct MeanpoolSmem {
  float red[kThreads / (D / VecN<T>::N)][D + 4];
};

// ROWS consecutive token rows (a 64-token block, or a 32-token window)
template <typename T, int D, int ROWS = kBlk>
__device__ __forceinline__ void meanpool_wg(const T* __restrict__ kblock, int64_t st, float* __restrict__ kc_row,
                            MeanpoolSmem<T, D>& sm) {
  constexpr int VEC = VecN<T>::N;
  constexpr int CPR = D / VEC;
  constexpr int RPP = kThreads / CPR;
  const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "rows must fill the row lanes");
  uint4 raw[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) raw[i] = ld16_nt(kblock + (int64_t)(r0 + i * RPP) * st + c * VEC);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float x[VEC];
    cvt16<T>(raw[i], x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sm.red[r0][c * VEC + e] = acc[e];
  __syncthreads();
  for (int t = threadIdx.x; t < D; t += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += sm.red[r][t];
    kc_row[t] = s / (float)ROWS;
  }
}

// ---------------------------------------------------------------------------
// Decode scoring of one slice of the candidate range of one (b, g).
// fvec: the fp32 Forecast of (b, g) in LDS.  Writes raw scores sc[j].
// 8 lanes per compressed-key row, every load of the slice issued before use.
// ---------------------------------------------------------------------------
struct DecodeCands {
  int cur, c0, c1;   // query block; candidates are [c0, c1)
};

// An empty sequence (L < 1) has no query block: cur = -1, and the union
// then holds no initial, local or candidate block (cnt 0).
__device__ __forceinline__ DecodeCands decode_cands(int64_t L, int64_t nb_cap, int n_init, int n_local) {
  int64_t cur = L < 1 ? -1 : (L - 1) / kBlk;
  if (cur > nb_cap - 1 + n_local) cur = nb_cap - 1 + n_local;   // never read past the cache
  DecodeCands r;
  r.cur = (int)cur;
  r.c0 = n_init;
  r.c1 = (int)min((int64_t)(cur - n_local + 1), nb_cap);
  if (r.c1 < r.c0) r.c1 = r.c0;
  return r;
}

// Agent-coherent 32-bit store and load (relaxed atomics at device scope):
// every XCD sees the value without cache maintenance, so workgroups of one
// launch can hand results to each other through an arrival counter (the
// writer waits for its stores to complete before it counts).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// CO: the scores are stored agent-coherent (read by another workgroup of the
// same launch)
template <int D, bool CO = false>
__device__ __forceinline__ void score_slice_wg(const float* fvec, const float* __restrict__ kc_bg, int lo, int hi,
                               float* __restrict__ sc) {
  constexpr int LPR = 8;
  constexpr int F4 = D / 4 / LPR;
  constexpr int RPP = kThreads / LPR;   // 32 rows per pass
  const int sub = threadIdx.x % LPR, row0 = threadIdx.x / LPR;
  float4 fv[F4];
#pragma unroll
  for (int i = 0; i < F4; ++i) fv[i] = *reinterpret_cast<const float4*>(fvec + (i * LPR + sub) * 4);
  constexpr int UNR = 4;
  for (int base = lo; base < hi; base += RPP * UNR) {
    float4 kv[UNR][F4];
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int j = base + row0 + uu * RPP;
      if (j < hi) {
#pragma unroll
        for (int i = 0; i < F4; ++i)
          kv[uu][i] = ld16f_nt(kc_bg + (int64_t)j * D + (i * LPR + sub) * 4);
      }
    }
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int j = base + row0 + uu * RPP;
      float acc = 0.f;
      if (j < hi) {
#pragma unroll
        for (int i = 0; i < F4; ++i) {
          acc += fv[i].x * kv[uu][i].x;
          acc += fv[i].y * kv[uu][i].y;
          acc += fv[i].z * kv[uu][i].z;
          acc += fv[i].w * kv[uu][i].w;
        }
      }
      acc = sum8(acc);   // the 8 lanes of the row (all active together)
      if (sub == 0 && j < hi) {
        if constexpr (CO) st_agent(sc + j, acc);
        else sc[j] = acc;
      }
    }
  }
}

// Scoring of one slice of a (b, g)'s candidates with the Forecast taken
// from the projection splits (written by an earlier kernel).  The loads of
// the slice's first rows are issued before the splits are added, so both
// round trips overlap; then as score_slice_wg.  CO: the scores are stored
// agent-coherent (read by another workgroup of the same launch); else plain
// stores (read by a later kernel).
template <int D, bool CO>
__device__ __forceinline__ void score_slice_proj_wg(const float* __restrict__ part, int n_splits, int B, int N, int b,
                                                    int g, const float* __restrict__ kc_bg, int lo, int hi,
                                                    float* __restrict__ sc, float* fvec) {
  constexpr int LPR = 8;
  constexpr int F4 = D / 4 / LPR;
  constexpr int RPP = kThreads / LPR;   // 32 rows per pass
  // one pass of rows in flight: next to the attention workgroups of the same
  // launch, fewer score rows in flight shorten the memory queues the
  // attention's dependent block loads wait in (B8 x 128K fused layer: one
  // pass 2-3% faster per step than two; 6% faster than four)
  constexpr int UNR = 1;
  const int sub = threadIdx.x % LPR, row0 = threadIdx.x / LPR;
  float4 kv[UNR][F4];
  auto issue = [&](int base) {
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int j = base + row0 + uu * RPP;
      if (j < hi) {
#pragma unroll
        for (int i = 0; i < F4; ++i) kv[uu][i] = ld16f_nt(kc_bg + (int64_t)j * D + (i * LPR + sub) * 4);
      }
    }
  };
  issue(lo);
  for (int i = threadIdx.x; i < D; i += kThreads) fvec[i] = proj_reduce_one(part, n_splits, B, N, b, g * D + i);
  __syncthreads();
  float4 fv[F4];
#pragma unroll
  for (int i = 0; i < F4; ++i) fv[i] = *reinterpret_cast<const float4*>(fvec + (i * LPR + sub) * 4);
  for (int base = lo; base < hi; base += RPP * UNR) {
    if (base != lo) issue(base);
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int j = base + row0 + uu * RPP;
      float acc = 0.f;
      if (j < hi) {
#pragma unroll
        for (int i = 0; i < F4; ++i) {
          acc += fv[i].x * kv[uu][i].x;
          acc += fv[i].y * kv[uu][i].y;
          acc += fv[i].z * kv[uu][i].z;
          acc += fv[i].w * kv[uu][i].w;
        }
      }
      acc = sum8(acc);   // the 8 lanes of the row (all active together)
      if (sub == 0 && j < hi) {
        if constexpr (CO) st_agent(sc + j, acc);
        else sc[j] = acc;
      }
    }
  }
}

// Top-k + union of one decode problem from its score row (written by an
// earlier kernel, or agent-coherent by this one when CO).  keys: LDS, at
// least (c1 - c0) entries.
template <bool CO = false>
__device__ __forceinline__ void topk_decode_wg(const float* __restrict__ sc, int64_t row_len, DecodeCands dc, int topk,
                                               int n_init,
                                               int n_local, int U,
                               int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out, uint32_t* keys,
                               TopkShared& sh) {
  const int n = dc.c1 - dc.c0;
  if (!CO && dc.c1 <= 8 * kThreads && (row_len & 3) == 0 && ((uintptr_t)sc & 15) == 0) {
    // thread t's eight row entries (block ids 8t .. 8t+7) in two aligned
    // 16-byte loads, none past the row (its length is a multiple of four);
    // ids outside the candidates are masked
    const int i0 = 8 * (int)threadIdx.x;
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (i0 < dc.c1) x0 = *reinterpret_cast<const float4*>(sc + i0);
    if (i0 + 4 < dc.c1) x1 = *reinterpret_cast<const float4*>(sc + i0 + 4);
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t kin[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kin[e] = orderable_key(v[e]);
    topk_union_fast(0, dc.c0, dc.c1, topk, dc.cur, n_init, n_local, U, idx_out, cnt_out, sh, kin);
    return;
  }
  if (n <= 8 * kThreads) {
    // thread t's eight candidates (c0 + 8t .. c0 + 8t + 7) straight into registers
    uint32_t kin[8];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * (int)threadIdx.x + e;
      v[e] = i < n ? (CO ? ld_agent(sc + dc.c0 + i) : sc[dc.c0 + i]) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) kin[e] = orderable_key(v[e]);
    topk_union_fast(dc.c0, dc.c0, dc.c1, topk, dc.cur, n_init, n_local, U, idx_out, cnt_out, sh, kin);
    return;
  }
  constexpr int PB = 8;   // loads in flight per thread
  for (int base = 0; base < n; base += PB * kThreads) {
    float v[PB];
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int i = base + e * kThreads + threadIdx.x;
      v[e] = i < n ? (CO ? ld_agent(sc + dc.c0 + i) : sc[dc.c0 + i]) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int i = base + e * kThreads + threadIdx.x;
      if (i < n) keys[i] = orderable_key(v[e]);
    }
  }
  __syncthreads();
  topk_union(keys, n, dc.c0, topk, dc.cur, n_init, n_local, U, idx_out, cnt_out, sh);
}

// ---------------------------------------------------------------------------
// Decode attention: one split (a run of listed blocks) of one KV head for
// its G query heads, one block at a time (one register set; other
// workgroups on the SIMD cover the load latency).  Writes the split's
// unnormalised output o[G][D] and its running max m / sum l (base-2 logits).
// ---------------------------------------------------------------------------
struct AttnDecodeParams {
  const void* q; const void* k; const void* v;
  int64_t sb, sg, st, kv_len;
  int ring;
  const int32_t* slot;   // block cache: listed block u sits in slot[u] (nullptr: cache or ring)
  const int32_t* idx; const int32_t* cnt; const int64_t* seq_len;
  int Hkv, U;
  float qscale;        // scale * log2(e)
  int bps, n_splits;   // listed blocks per split, number of splits
  float* out;          // [B, Hq, D] fp32
  float* ws_o;         // [B*Hkv, n_splits, G, D]
  float* ws_ml;        // [B*Hkv, n_splits, G, 2]
};

template <int D, int G>
struct AttnSmem {
  float qs[G][D];        // fp32 path: scaled query
  float sraw[G][kBlk];
  float ps[G][kBlk];
  float alpha[G];
  float red[4][G][D];
};

// bf16 path (attn_split_mfma_wg): each wave's 16 V rows of the current
// block, XOR-swizzled in 16-byte chunks; after the block loop the same bytes
// hold the four waves' unnormalised outputs for the merge.
template <int D, int G>
struct AttnMfmaSmem {
  static_assert(4 * G * D * sizeof(float) <= 4 * 16 * 2 * D, "merge buffer fits the V rows");
  union {
    unsigned char v[4][16 * 2 * D];
    float mo[4][G][D];
  };
  float ml[4][G][2];
};

template <typename T, int D, int G> struct AttnSmemSel { using type = AttnSmem<D, G>; };
template <int D, int G> struct AttnSmemSel<bf16_bits, D, G> { using type = AttnMfmaSmem<D, G>; };


// Register set of one 64-token K/V block.
//   bf16: K as the MFMA A operand of S^T = K Q^T -- wave w owns keys
//         16w..16w+15, lane l loads key 16w + l%16, dims 32ks + 8(l/16) ..+7
//   fp32: 4 lanes per key, each 4 x 16-byte loads interleaved over the row
//   V (both): lane = (16-byte column chunk, token lane) for the PV sums
template <typename T, int D, int G>
struct AttnRegs {
  static constexpr bool kMfma = std::is_same<T, bf16_bits>::value;
  static constexpr int VEC = VecN<T>::N;
  static constexpr int NKL = kMfma ? D / 32 : D / 4 / VEC;   // K loads per lane
  static constexpr int DCH = D / VEC;                          // 16-byte chunks per row
  static constexpr int TL = kThreads / DCH;                    // token lanes in PV
  static constexpr int TPL = kBlk / TL;                        // tokens per lane in PV
  uint4 k[NKL];
  uint4 v[TPL];
};

template <typename T, int D, int G>
__device__ __forceinline__ void attn_load(AttnRegs<T, D, G>& r, const T* kb, const T* vb, int64_t st) {
  using R = AttnRegs<T, D, G>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if constexpr (R::kMfma) {
    const T* kp = kb + (int64_t)(16 * w + (lane & 15)) * st + 8 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < R::NKL; ++i) r.k[i] = ld16_nt(kp + 32 * i);
  } else {
    const int tok = threadIdx.x >> 2, part = threadIdx.x & 3;
#pragma unroll
    for (int i = 0; i < R::NKL; ++i) r.k[i] = ld16_nt(kb + (int64_t)tok * st + (i * 4 + part) * R::VEC);
  }
  const int dc = threadIdx.x % R::DCH, tl = threadIdx.x / R::DCH;
#pragma unroll
  for (int i = 0; i < R::TPL; ++i) r.v[i] = ld16_nt(vb + (int64_t)(tl + i * R::TL) * st + dc * R::VEC);
}

// bf16 block loads through buffer resources: the resource holds the
// (b, g) base and the byte count of its K (or V) rows, each lane a fixed
// 32-bit offset, each block a wave-uniform offset.  No per-block address
// arithmetic lands in vector registers, so no such register can be one a
// load in flight still owes (which would make the compiler wait for every
// load), and accesses past the rows read zero.
struct BufBlock {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t ko, vo;     // per-lane byte offsets of the K fragment and V rows
  uint32_t vstep;      // bytes between the V rows one lane loads
};

template <int D>
__device__ __forceinline__ BufBlock make_buf_block(const bf16_bits* kb, const bf16_bits* vb, int64_t st,
                                                   int64_t kv_len) {
  constexpr int VEC = 8, DCH = D / VEC, TL = kThreads / DCH;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t span = kv_len > 0 ? ((kv_len - 1) * st + D) * 2 : 0;
  const int nrec = (int)(span < 0x7fffffff ? span : 0x7fffffff);
  BufBlock bb;
  bb.rk = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, nrec, 0x00020000);
  bb.rv = __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, nrec, 0x00020000);
  bb.ko = (uint32_t)(((16 * w + (lane & 15)) * (uint32_t)st + 8 * (lane >> 4)) * 2);
  const int dc = threadIdx.x % DCH, tl = threadIdx.x / DCH;
  bb.vo = (uint32_t)((tl * (uint32_t)st + dc * VEC) * 2);
  bb.vstep = (uint32_t)(TL * st * 2);
  return bb;
}

template <int D, int G>
__device__ __forceinline__ void attn_load_buf(AttnRegs<bf16_bits, D, G>& r, const BufBlock& bb, uint32_t boff) {
  using R = AttnRegs<bf16_bits, D, G>;
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < R::NKL; ++i) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(bb.rk, bb.ko + 64 * i, (int)boff, 2);
    r.k[i] = make_uint4(x[0], x[1], x[2], x[3]);
  }
#pragma unroll
  for (int i = 0; i < R::TPL; ++i) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(bb.rv, bb.vo, (int)(boff + i * bb.vstep), 2);
    r.v[i] = make_uint4(x[0], x[1], x[2], x[3]);
  }
}

// q fragments of the MFMA path: lane l holds q[head l%16][32ks + 8(l/16) ..+7]
// (zero for the padding heads G..15), already in bf16.
template <int D>
struct QFrag {
  bf16x8_t f[D / 32];
};

template <typename T, int D, int G>
__device__ __forceinline__ void attn_block(const AttnRegs<T, D, G>& r, int nvalid, AttnSmem<D, G>& sm,
                                           const QFrag<D>& qf, float qscale, float (&acc)[G][VecN<T>::N],
                                           float* m_run, float* l_run) {
  using R = AttnRegs<T, D, G>;
  constexpr int VEC = R::VEC;
  constexpr int HW = (G + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int tl = tid / R::DCH;
  if constexpr (R::kMfma) {
    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < R::NKL; ++ks)
      s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[ks]), qf.f[ks], s4, 0, 0, 0);
    const int h = lane & 15;
    if (h < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * wid + 4 * (lane >> 4) + i;
        sm.sraw[h][key] = key < nvalid ? s4[i] * qscale : -INFINITY;
      }
    }
  } else {
    const int tok = tid >> 2, part = tid & 3;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int i = 0; i < R::NKL; ++i) {
      float kf[VEC];
      cvt16<T>(r.k[i], kf);
      const int d0 = (i * 4 + part) * VEC;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[h] += kf[e] * sm.qs[h][d0 + e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = sum4(s[h]);
#pragma unroll
    for (int h = 0; h < G; ++h)
      if ((h & 3) == part) sm.sraw[h][tok] = (tok < nvalid) ? s[h] : -INFINITY;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const int h = wid + 4 * i;
    if (h < G) {
      const float x = sm.sraw[h][lane];
      const float mn = fmaxf(m_run[i], wave_max(x));
      float p, al;
      if (mn == -INFINITY) { p = 0.f; al = 1.f; }
      else { p = __builtin_amdgcn_exp2f(x - mn); al = __builtin_amdgcn_exp2f(m_run[i] - mn); }
      l_run[i] = l_run[i] * al + wave_sum(p);
      m_run[i] = mn;
      sm.ps[h][lane] = p;
      if (lane == 0) sm.alpha[h] = al;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float al = sm.alpha[h];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] *= al;
  }
#pragma unroll
  for (int i = 0; i < R::TPL; ++i) {
    const int t = tl + i * R::TL;
    if (t < nvalid) {
      float vf[VEC];
      cvt16<T>(r.v[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = sm.ps[h][t];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] += p * vf[e];
      }
    }
  }
}

// End of a split: sum the PV token lanes (inside the wave, then across the
// 4 waves) and write the unnormalised output and (m, l) of every head.
template <typename T, int D, int G, bool CO>
__device__ __forceinline__ void attn_split_finish(const AttnDecodeParams& p, int bg, int split, AttnSmem<D, G>& sm,
                                                  float (&acc)[G][VecN<T>::N], const float* m_run,
                                                  const float* l_run) {
  using R = AttnRegs<T, D, G>;
  constexpr int VEC = R::VEC;
  constexpr int HW = (G + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // token lanes are the lane bits at and above DCH (a power of two >= 8)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float v = acc[h][e], a, b;
      if constexpr (R::DCH <= 8) v += dpp_mov<0x128>(v);   // row_ror:8 = lane ^ 8 inside the row
      if constexpr (R::DCH <= 16) { swap16(v, a, b); v = a + b; }
      swap32(v, a, b);
      acc[h][e] = a + b;
    }
  const int dc = tid % R::DCH;
  if (lane < R::DCH) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm.red[wid][h][dc * VEC + e] = acc[h][e];
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)bg * p.n_splits + split) * G;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    const float o = sm.red[0][h][d] + sm.red[1][h][d] + sm.red[2][h][d] + sm.red[3][h][d];
    if constexpr (CO) st_agent(p.ws_o + (pbase + h) * D + d, o);
    else p.ws_o[(pbase + h) * D + d] = o;
  }
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const int h = wid + 4 * i;
    if (h < G && lane == 0) {
      if constexpr (CO) {
        st_agent(p.ws_ml + (pbase + h) * 2 + 0, m_run[i]);
        st_agent(p.ws_ml + (pbase + h) * 2 + 1, l_run[i]);
      } else {
        p.ws_ml[(pbase + h) * 2 + 0] = m_run[i];
        p.ws_ml[(pbase + h) * 2 + 1] = l_run[i];
      }
    }
  }
}

// bf16 decode attention of one split on the matrix cores, one online
// softmax per wave.  Wave w owns keys 16w..16w+15 of every listed block:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, K straight from 16-byte loads
//                 (lane: key 16w + l%16, dims 32ks + 8(l/16)..+7), q padded
//                 to 16 heads; lane l gets keys 4(l/16)+i of head l%16
//   P^T           the exponentials of those scores, rounded to bf16, are
//                 already the B operand of v_mfma_f32_16x16x16_bf16 (lane:
//                 keys 4(l/16)..+3 of head l%16)
//   O^T += V^T P^T  per 16-column tile of V; V^T comes from the wave's 16 V
//                 rows staged in its own LDS region and read back with the
//                 transposing ds_read_b64_tr_b16 (lane 4r+c of each 16-lane
//                 group reads row r, columns 4c..4c+3; lane i receives column
//                 i of the four rows)
// Two register sets: the next block's K/V rows are in flight while the
// current block is computed (~155 VGPRs: three workgroups per SIMD).
// No barrier inside the block loop: a wave touches only its own LDS rows,
// and LDS operations of one wave complete in order.  The running maximum
// is lazy: it moves only when some lane's block maximum exceeds it by more
// than kLazyTau (base 2), so most blocks exchange nothing across lanes and
// rescale nothing; the four lanes of a head agree on it whenever it moves.
// The waves' (m, l, O) are merged through LDS once per split.
constexpr float kLazyTau = 8.f;

template <int D, int G, bool CO>
__device__ __forceinline__ void attn_split_mfma_wg(const AttnDecodeParams& p, int bg, int split,
                                                   AttnMfmaSmem<D, G>& sm) {
  static_assert(G <= 16, "query heads of a group fit the 16 MFMA columns");
  constexpr int RB = 2 * D;          // bytes of one K/V row
  constexpr int KS = D / 32;         // k-steps of the QK product
  constexpr int DT = D / 16;         // 16-column tiles of V
  constexpr int NVC = D / 32;        // 16-byte V loads per lane (16 rows x D/8 chunks over 64 lanes)
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int Hq = p.Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int c = min(p.cnt[bg], p.U);
  const int u0 = split * p.bps, u1 = min(c, u0 + p.bps);
  const int64_t L = (p.ring || p.slot) ? p.seq_len[b] : min(p.seq_len[b], p.kv_len);

  // q as the B operand: lane l holds q[head l%16][dims 32ks + 8(l/16) ..+7]
  const bf16_bits* q = (const bf16_bits*)p.q;
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (l16 < G) raw = ld16(q + ((int64_t)b * Hq + g * G + l16) * D + 32 * ks + 8 * lg);
    qf[ks] = __builtin_bit_cast(bf16x8_t, raw);
  }

  // buffer resources over this (b, g)'s K and V rows; per-lane byte offsets
  const bf16_bits* kbase = (const bf16_bits*)p.k + b * p.sb + g * p.sg;
  const bf16_bits* vbase = (const bf16_bits*)p.v + b * p.sb + g * p.sg;
  const int64_t span = p.kv_len > 0 ? ((p.kv_len - 1) * p.st + D) * 2 : 0;
  const int nrec = (int)(span < 0x7fffffff ? span : 0x7fffffff);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nrec, 0x00020000);
  const uint32_t ko = (uint32_t)(((16 * w + l16) * (uint32_t)p.st + 8 * lg) * 2);
  // V: each load instruction of the wave reads whole rows (1 KB contiguous
  // at D = 128): load i, lane l -> row i * RPI + l / CPR, chunk l % CPR
  constexpr int CPR = D / 8;                          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                       // rows per load instruction
  const int vrow = lane / CPR, vch = lane % CPR;
  const uint32_t vo = (uint32_t)(((16 * w + vrow) * (uint32_t)p.st + 8 * vch) * 2);
  const uint32_t vstep = (uint32_t)(RPI * p.st * 2);
  // LDS: row r, logical chunk c at chunk c ^ 2(r mod D/16)
  unsigned char* vs = sm.v[w];
  const int tr_r = 4 * lg + (l16 >> 2);               // row of this lane's transposing read
  const int tr_off = tr_r * RB + 8 * (l16 & 3);
  const int tr_sw = 2 * (tr_r % (D / 16));

  float m_run = -1e30f, l_part = 0.f;                 // finite start: a masked key gives p = 0
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* list = p.idx + (int64_t)bg * p.U;
  const int nblk_buf = (int)min(p.kv_len / kBlk, (int64_t)0x7fffffff);
  const int Lc = (int)min(L, (int64_t)0x7fffffff - kBlk);
  const int jend = (Lc + kBlk - 1) / kBlk;
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  // list entries through the constant address space: scalar loads, which
  // do not wait behind the vector loads in flight
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  const cint_ptr clist = (cint_ptr)list;
  const cint_ptr cslot = (cint_ptr)(p.slot ? p.slot + (int64_t)bg * p.U : list);
  // a descriptor with no records: loads through it return zeros and touch
  // no memory (list slots that name no block)
  const __amdgpu_buffer_rsrc_t rnull = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, 0, 0x00020000);
  // Requests the K/V rows of list slot u into (kr, vr) and returns the
  // slot's valid key count (-1: no block).  Every call issues the same eight
  // loads in the same order (scheduling barriers keep that order), so the
  // compiler's wait counts stay exact while the next slot is in flight.
  auto issue = [&](int u, uint4 (&kr)[KS], uint4 (&vr)[NVC]) -> int {
    int nv = -1;
    uint32_t boff = 0;
    bool none = true;
    if (u < u1) {
      const int j = clist[u];
      const int loc = p.slot ? cslot[u] : (p.ring ? u : j);
      if (!(j < 0 || loc < 0 || loc >= nblk_buf || j >= jend)) {
        nv = min(kBlk, Lc - j * kBlk);
        boff = __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)loc * kBlk * p.st * 2));
        none = false;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(none ? rnull : rk, ko + 64 * ks, (int)boff, 2);
      kr[ks] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(none ? rnull : rv, vo + i * vstep, (int)boff, 2);
      vr[i] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    return nv;
  };
  // One block: scores, lazy softmax update, P V.  A slot with no block runs
  // with every key masked (p = 0, V rows zero), so it adds nothing.
  auto compute = [&](const uint4 (&kr)[KS], const uint4 (&vr)[NVC], int nv) {
    const int nvalid = nv < 0 ? 0 : nv;
    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[ks]), qf[ks], s4, 0, 0, 0);
    float sv[4], lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (16 * w + 4 * lg + i < nvalid) ? s4[i] * p.qscale : -INFINITY;
      lmax = fmaxf(lmax, sv[i]);
    }
    if (__any(lmax > m_run + kLazyTau)) {
      float a, bb;
      swap16(lmax, a, bb);
      float mx = fmaxf(a, bb);
      swap32(mx, a, bb);
      mx = fmaxf(a, bb);
      const bool up = mx > m_run + kLazyTau;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = up ? mx : m_run;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    s16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h = (__bf16)__builtin_amdgcn_exp2f(sv[i] - m_run);
      l_part += (float)h;
      pb[i] = __builtin_bit_cast(short, h);
    }
    // V rows of the wave's keys into its LDS rows (rows past the valid keys
    // as zeros: they meet p = 0, and 0 * NaN would not vanish)
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const int r = i * RPI + vrow;
      *reinterpret_cast<uint4*>(vs + r * RB + (vch ^ (2 * (r % (D / 16)))) * 16) =
          (16 * w + r < nvalid) ? vr[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs + tr_off + ((2 * dt) ^ tr_sw) * 16));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[dt], 0, 0, 0);
    }
  };
  // two register sets: slot u + 1 is requested before slot u is computed
  uint4 kA[KS], vA[NVC], kB[KS], vB[NVC];
  int nA = issue(u0, kA, vA), nB;
  for (int u = u0; u < u1; u += 2) {
    nB = issue(u + 1, kB, vB);
    compute(kA, vA, nA);
    if (u + 1 >= u1) break;
    nA = issue(u + 2, kA, vA);
    compute(kB, vB, nB);
  }
  // merge the four waves: lane l holds O[head l%16][d = 16dt + 4(l/16) + i]
  {
    float a, bb;
    swap16(l_part, a, bb);
    const float l2 = a + bb;
    swap32(l2, a, bb);
    l_part = a + bb;
  }
  __syncthreads();                                    // every wave is done with its V rows
  if (l16 < G) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(&sm.mo[w][l16][16 * dt + 4 * lg]) = o[dt];
    if (lg == 0) {
      sm.ml[w][l16][0] = m_run;
      sm.ml[w][l16][1] = l_part;
    }
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)bg * p.n_splits + split) * G;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    const float M = fmaxf(fmaxf(sm.ml[0][h][0], sm.ml[1][h][0]), fmaxf(sm.ml[2][h][0], sm.ml[3][h][0]));
    float acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) acc += __builtin_amdgcn_exp2f(sm.ml[ww][h][0] - M) * sm.mo[ww][h][d];
    if constexpr (CO) st_agent(p.ws_o + (pbase + h) * D + d, acc);
    else p.ws_o[(pbase + h) * D + d] = acc;
  }
  if (tid < G) {
    const int h = tid;
    const float M = fmaxf(fmaxf(sm.ml[0][h][0], sm.ml[1][h][0]), fmaxf(sm.ml[2][h][0], sm.ml[3][h][0]));
    float l = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) l += __builtin_amdgcn_exp2f(sm.ml[ww][h][0] - M) * sm.ml[ww][h][1];
    if constexpr (CO) {
      st_agent(p.ws_ml + (pbase + h) * 2 + 0, M);
      st_agent(p.ws_ml + (pbase + h) * 2 + 1, l);
    } else {
      p.ws_ml[(pbase + h) * 2 + 0] = M;
      p.ws_ml[(pbase + h) * 2 + 1] = l;
    }
  }
}

// fp32 decode attention of one split (VALU): one block at a time for the
// whole workgroup, scores and softmax weights exchanged through LDS.
template <typename T, int D, int G, bool CO>
__device__ __forceinline__ void attn_split_valu_wg(const AttnDecodeParams& p, int bg, int split, AttnSmem<D, G>& sm) {
  using R = AttnRegs<T, D, G>;
  constexpr int VEC = R::VEC;
  constexpr int HW = (G + 3) / 4;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int Hq = p.Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c = min(p.cnt[bg], p.U);
  const int u0 = split * p.bps, u1 = min(c, u0 + p.bps);
  // tokens of the sequence; a ring or a block cache holds only some blocks,
  // so its length bounds positions in it, not the sequence
  const int64_t L = (p.ring || p.slot) ? p.seq_len[b] : min(p.seq_len[b], p.kv_len);
  const T* q = (const T*)p.q;
  QFrag<D> qf;
  if constexpr (R::kMfma) {
    const int h = lane & 15;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (h < G) raw = ld16(q + ((int64_t)b * Hq + g * G + h) * D + 32 * ks + 8 * (lane >> 4));
      qf.f[ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  } else {
    for (int i = tid; i < G * D; i += kThreads)
      sm.qs[i / D][i % D] = to_f32<T>(q[((int64_t)b * Hq + g * G) * D + i]) * p.qscale;
  }
  const float sscale = R::kMfma ? p.qscale : 1.f;
  float m_run[HW], l_run[HW];
#pragma unroll
  for (int i = 0; i < HW; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  float acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  const T* kbase = (const T*)p.k + b * p.sb + g * p.sg;
  const T* vbase = (const T*)p.v + b * p.sb + g * p.sg;
  const int32_t* list = p.idx + (int64_t)bg * p.U;

  // block u -> (block slot in the buffer, valid token count); invalid ids
  // read nothing.  The tests run in 32-bit scalar arithmetic on per-split
  // constants: 64-bit compares would go through vector registers, and the
  // compiler may pick one that a load in flight still owes, waiting for all.
  const int nblk_buf = (int)min(p.kv_len / kBlk, (int64_t)0x7fffffff);       // whole blocks in the buffer
  const int Lc = (int)min(L, (int64_t)0x7fffffff - kBlk);
  const int jend = (Lc + kBlk - 1) / kBlk;                                    // blocks holding tokens
  auto locate = [&](int u, int64_t& tb, int& nvalid) {
    const int j = list[u];
    const int loc = p.slot ? p.slot[(int64_t)bg * p.U + u] : (p.ring ? u : j);
    tb = (int64_t)loc * kBlk;
    if (j < 0 || loc < 0 || loc >= nblk_buf) { nvalid = -1; return; }
    nvalid = j >= jend ? 0 : min(kBlk, Lc - j * kBlk);
  };
  // One register set: each block is requested, then computed.  With ~100
  // VGPRs four workgroups share a SIMD and cover each other's load latency;
  // two register sets (the next block requested before the current one is
  // computed) need ~190 VGPRs, two workgroups per SIMD, and measured slower
  // (B8 x 128K: 44.7 vs 40.7 us for the fused layer's kernel).  A block outside
  // the buffer is masked whole (nothing is read); K/V shorter than one block
  // hold no valid block.
  AttnRegs<T, D, G> ra;
  int64_t tba = 0;
  int nva = -1;
  BufBlock bb;
  if constexpr (R::kMfma) bb = make_buf_block<D>((const bf16_bits*)kbase, (const bf16_bits*)vbase, p.st, p.kv_len);
  __syncthreads();
  for (int u = u0; u < u1; ++u) {
    locate(u, tba, nva);
    if (nva >= 0) {
      if constexpr (R::kMfma)
        attn_load_buf<D, G>(ra, bb, __builtin_amdgcn_readfirstlane((uint32_t)(tba * p.st * 2)));
      else
        attn_load<T, D, G>(ra, kbase + tba * p.st, vbase + tba * p.st, p.st);
    }
    attn_block<T, D, G>(ra, nva < 0 ? 0 : nva, sm, qf, sscale, acc, m_run, l_run);
  }

  attn_split_finish<T, D, G, CO>(p, bg, split, sm, acc, m_run, l_run);
}

// CO: the partials are stored agent-coherent (merged by another workgroup
// of the same launch)
template <typename T, int D, int G, bool CO = false>
__device__ __forceinline__ void attn_split_wg(const AttnDecodeParams& p, int bg, int split,
                                              typename AttnSmemSel<T, D, G>::type& sm) {
  if constexpr (std::is_same<T, bf16_bits>::value) {
    attn_split_mfma_wg<D, G, CO>(p, bg, split, sm);
  } else {
    attn_split_valu_wg<T, D, G, CO>(p, bg, split, sm);
  }
}

// Merge the splits of one KV head (written by an earlier kernel), in split
// order: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int D, int G>
struct CombineSmem {
  float ml[kMaxSplitsDecode][G][2];
  float wts[kMaxSplitsDecode][G];
  float den[G];
};

template <int D, int G, bool CO = false>
__device__ __forceinline__ void attn_combine_wg(const AttnDecodeParams& p, int bg, CombineSmem<D, G>& sm) {
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int Hq = p.Hkv * G;
  const int ns = p.n_splits;
  const int64_t sbase = (int64_t)bg * ns * G;
  const int tid = threadIdx.x;
  // every partial this thread needs is requested first, together with the
  // (m, l) pairs: one round trip to memory
  constexpr int OPT = (G * D + kThreads - 1) / kThreads;   // outputs per thread
  float v[OPT][kMaxSplitsDecode];
#pragma unroll
  for (int o = 0; o < OPT; ++o) {
    const int i = tid + o * kThreads;
    const int h = i / D, d = i % D;
#pragma unroll
    for (int sp = 0; sp < kMaxSplitsDecode; ++sp)
      v[o][sp] = (i < G * D && sp < ns)
                     ? (CO ? ld_agent(p.ws_o + (sbase + sp * G + h) * D + d) : p.ws_o[(sbase + sp * G + h) * D + d])
                     : 0.f;
  }
  for (int i = tid; i < ns * G * 2; i += kThreads)
    (&sm.ml[0][0][0])[i] = CO ? ld_agent(p.ws_ml + sbase * 2 + i) : p.ws_ml[sbase * 2 + i];
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, sm.ml[sp][tid][0]);
    float den = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float m = sm.ml[sp][tid][0];
      const float w = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
      sm.wts[sp][tid] = w;
      den += w * sm.ml[sp][tid][1];
    }
    sm.den[tid] = den;
  }
  __syncthreads();
#pragma unroll
  for (int o = 0; o < OPT; ++o) {
    const int i = tid + o * kThreads;
    if (i >= G * D) break;
    const int h = i / D, d = i % D;
    float num = 0.f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplitsDecode; ++sp)
      if (sp < ns) num += sm.wts[sp][h] * v[o][sp];
    const float den = sm.den[h];
    p.out[((int64_t)b * Hq + g * G + h) * D + d] = den > 0.f ? num / den : 0.f;
  }
}

// Split plan of the decode attention: about `target` workgroups, at most
// kMaxSplitsDecode splits, every split the same number of listed blocks.
// With two blocks in flight per wave (three workgroups per SIMD: 768 slots)
// the attention needs fewer, longer splits: measured inside the fused decode
// layer at B8 x 128K (64 (b, g) units, U = 69), 256 workgroups (4 splits of
// 18 blocks) beside 512 score workgroups fill the 768 slots and ran the step
// 6% faster than 192 or 512 attention workgroups, 13% faster than 320, 22%
// faster than 128 (same box, top-k in the launch's tail).  Above 64
// units the earlier 768 is kept (at B16 it gives 6 splits).  `reserve`:
// workgroups of other work in the same launch; the attention then keeps to
// the 768 slots left beside them (at most one split per unit fewer than
// without), so none of its workgroups waits for a slot to free up.
__host__ __device__ inline void attn_split_plan(int n_bg, int U, int& n_splits, int& bps, int reserve = 0) {
  int target = n_bg <= 64 ? 256 : 768;
  if (reserve > 0 && target > 768 - reserve) target = 768 - reserve;
  int ns = target / n_bg;
  if (reserve <= 0 || ns < 1) ns = (target + n_bg - 1) / n_bg;
  if (ns > U) ns = U;
  if (ns > kMaxSplitsDecode) ns = kMaxSplitsDecode;
  if (ns < 1) ns = 1;
  bps = (U + ns - 1) / ns;
  n_splits = (U + bps - 1) / bps;
}

// Score split plan: about 512 workgroups (768 above 64 (b, g) units), at
// least 64 candidate rows each.
__host__ __device__ inline int score_split_plan(int n_bg, int64_t nb_cap) {
  const int target = n_bg <= 64 ? 512 : 768;
  int s = (target + n_bg - 1) / n_bg;
  const int max_s = (int)((nb_cap + 63) / 64);
  if (s > max_s) s = max_s;
  return s < 1 ? 1 : s;
}

}  // namespace bskv
