// Device helpers shared by the gfx950 kernels of libbskv: 16-byte vector
// loads with bf16/fp32 conversion, global-to-LDS copies, wavefront (64-lane)
// reductions, a 256-thread block scan, and the order-preserving float ->
// uint32 key used by the top-k selection.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bskv {

constexpr int kThreads = 256;   // 4 wavefronts of 64 lanes
constexpr int kWave = 64;

typedef uint16_t bf16_bits;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, h);
}

// Elements of T in one 16-byte vector.
template <typename T> struct VecN;
template <> struct VecN<float> { static constexpr int N = 4; };
template <> struct VecN<bf16_bits> { static constexpr int N = 8; };

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streamed 16-byte load (nontemporal): for data read once per step -- the
// selected K/V blocks, compressed keys, Forecast weights -- so it does not
// displace reusable lines.  On gfx950 streaming reads this way reach ~6.5 TB/s
// against ~6.0 TB/s for plain loads.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld16f_nt(const float* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

template <typename T> __device__ __forceinline__ void cvt16(const uint4& r, float* o);
template <> __device__ __forceinline__ void cvt16<float>(const uint4& r, float* o) {
  o[0] = __uint_as_float(r.x); o[1] = __uint_as_float(r.y);
  o[2] = __uint_as_float(r.z); o[3] = __uint_as_float(r.w);
}
template <> __device__ __forceinline__ void cvt16<bf16_bits>(const uint4& r, float* o) {
  o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x); o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
  o[4] = bf16_lo(r.z); o[5] = bf16_hi(r.z); o[6] = bf16_lo(r.w); o[7] = bf16_hi(r.w);
}

// Sum of n (<= 64) consecutive token rows of D values (a query block's
// Forecast vectors): 16-byte column chunks per lane, rows strided over the
// workgroup, partial sums reduced through LDS.  Result in sm.fpool; ends with
// a barrier.
template <typename T, int D>
struct PoolRowsSmem {
  static constexpr int RPP = kThreads / (D / VecN<T>::N);
  float red[RPP][D + 4];
  float fpool[D];
};

template <typename T, int D>
__device__ __forceinline__ void pool_rows(const T* __restrict__ rows, int n, PoolRowsSmem<T, D>& sm) {
  constexpr int VEC = VecN<T>::N;
  constexpr int CPR = D / VEC;
  constexpr int RPP = PoolRowsSmem<T, D>::RPP;
  const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int t = r0; t < n; t += RPP) {
    float x[VEC];
    cvt16<T>(ld16(rows + (int64_t)t * D + c * VEC), x);
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
    sm.fpool[t] = s;
  }
  __syncthreads();
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_bits>(bf16_bits x) { return __uint_as_float(((uint32_t)x) << 16); }

// Cross-lane reductions without LDS traffic: DPP inside rows of 16 lanes
// (quad permutes, then the half-row and row mirrors), and gfx950's
// v_permlane16_swap / v_permlane32_swap across rows.  A swap of a register
// with itself leaves each lane holding its own value and that of lane l^16
// (resp. l^32) in the two results, so combining them is an all-reduce step.
// Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16 lanes

__device__ __forceinline__ float sum4(float v) {
  v += dpp_mov<kDppXor1>(v);
  return v + dpp_mov<kDppXor2>(v);
}
__device__ __forceinline__ float sum8(float v) {
  v = sum4(v);
  return v + dpp_mov<kDppHalfMirror>(v);
}
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  return v + dpp_mov<kDppMirror>(v);
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppMirror>(v));
}
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  float a, b;
  v = max16(v);
  swap16(v, a, b);
  v = fmaxf(a, b);
  swap32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum(float v) {
  float a, b;
  v = sum16(v);
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP: shifts by 1, 2,
// 4, 8 inside each row of 16 lanes (zero from outside the row), then lane 15
// of row r added to row r+1 (rows 1 and 3) and lane 31 to rows 2 and 3.
// Every lane of the wave must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sum over the 256 threads of a block (thread order).
// `tmp` is 4 ints of shared memory; `total` receives the sum of all values.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int s = tmp[w];
    off += (w < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// Monotone map float -> uint32 (larger float -> larger key).  -0.0 maps like
// +0.0 so that equal scores tie exactly.
__device__ __forceinline__ uint32_t orderable_key(float f) {
  uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Shared scratch of topk_union.  The radix histogram is double buffered
// (pass p counts into buffer p % 2 while the previous one is cleared) and has
// kHistCopies private copies (lane l counts into copy l % kHistCopies, copies
// 257 words apart) so that atomic adds of lanes that share a bin -- scores
// share sign and exponent bits -- spread over several banks.
constexpr int kHistCopies = 4;
constexpr int kHistStride = 257;
struct TopkShared {
  union {
    int hist[2][kHistCopies * kHistStride];   // topk_union_regs (keys re-read from LDS)
    int whist[2][4][2][256];                  // topk_union_fast: [pass & 1][wave][lane & 1][digit]
  };
  int scan_tmp[4];
  int pick[3];
};

// Exclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_excl_scan(int v) { return wave_incl_scan(v) - v; }

// Top-k + union for one selection problem, run by all 256 threads.  Thread
// t owns candidates t*KPT .. t*KPT+KPT-1 (so its keys are in block-id order);
// with KPT <= 8 they are held in registers, above that re-read from LDS.
template <int KPT>
__device__ __forceinline__ void topk_union_regs(const uint32_t* keys, int n, int c0, int topk, int cur, int n_init,
                                                int n_local,
                                int U, int32_t* idx_out, int32_t* cnt_out, TopkShared& sh,
                                const uint32_t* kin = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i0 = tid * KPT;
  constexpr bool kRegs = KPT <= 8;
  uint32_t kr[kRegs ? KPT : 1];
  if constexpr (kRegs) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) kr[e] = (i0 + e < n) ? (kin ? kin[e] : keys[i0 + e]) : 0u;
  }
  auto key = [&](int e) -> uint32_t {
    if constexpr (kRegs) return kr[e];
    else return keys[i0 + e];
  };

  const bool take_none = topk <= 0 || n <= 0;
  const bool take_all = !take_none && n <= topk;
  uint32_t prefix = 0, mask = 0;
  int kk = topk;
  if (!take_none && !take_all) {
    // MSB-first radix select of the topk-th largest key, 8 bits per pass,
    // stopping as soon as the bucket holding it is taken whole.
    for (int i = tid; i < kHistCopies * kHistStride; i += kThreads) sh.hist[0][i] = 0;
    __syncthreads();
    int* mine = nullptr;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      int* h = sh.hist[pass & 1];
      mine = h + (tid & (kHistCopies - 1)) * kHistStride;
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t k = key(e);
        if (i0 + e < n && (k & mask) == prefix) atomicAdd(&mine[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      if (wid == 0) {
        // lane l looks at digits 255-4l .. 252-4l (descending)
        int c[4], ls = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int D = 255 - 4 * lane - r;
          int v = 0;
#pragma unroll
          for (int cp = 0; cp < kHistCopies; ++cp) v += h[cp * kHistStride + D];
          c[r] = v;
          ls += v;
        }
        int run = wave_excl_scan(ls);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (run < kk && kk <= run + c[r]) {
            sh.pick[0] = 255 - 4 * lane - r;
            sh.pick[1] = run;
            sh.pick[2] = c[r];
          }
          run += c[r];
        }
      } else {
        int* hn = sh.hist[(pass + 1) & 1];
        for (int i = tid - 64; i < kHistCopies * kHistStride; i += kThreads - 64) hn[i] = 0;
      }
      __syncthreads();
      prefix |= ((uint32_t)sh.pick[0]) << shift;
      mask |= 255u << shift;
      kk -= sh.pick[1];
      const bool whole = (kk == sh.pick[2]);
      __syncthreads();   // pick is rewritten by the next pass
      if (whole) break;
    }
  }
  // ties: keys whose masked value equals the threshold bucket; the kk of
  // them with the lowest block ids are taken
  const int need = kk;
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    if (i0 + e < n && !take_none) {
      if (take_all) ++gt;
      else {
        const uint32_t km = key(e) & mask;
        gt += km > prefix;
        eq += km == prefix;
      }
    }
  }
  int tot;
  const int ex = block_excl_scan((gt << 16) | eq, sh.scan_tmp, tot);
  int gt_b = ex >> 16, eq_b = ex & 0xffff;
  const int n_sel = take_none ? 0 : (take_all ? n : topk);
  const int local_lo = max(0, cur - n_local + 1);
  const int a = min(n_init, local_lo);          // initial blocks below the local window
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    if (i0 + e < n && !take_none) {
      bool sel;
      int pos;
      if (take_all) {
        sel = true;
        pos = a + gt_b++;
      } else {
        const uint32_t km = key(e) & mask;
        if (km > prefix) { sel = true; pos = a + gt_b + min(eq_b, need); ++gt_b; }
        else if (km == prefix) { sel = eq_b < need; pos = a + gt_b + eq_b; ++eq_b; }
        else { sel = false; pos = 0; }
      }
      if (sel && pos < U) idx_out[pos] = c0 + i0 + e;
    }
  }
  const int n_loc = cur - local_lo + 1;
  const int total = a + n_sel + n_loc;
  for (int j = tid; j < a; j += kThreads) idx_out[j] = j;
  for (int j = tid; j < n_loc; j += kThreads)
    if (a + n_sel + j < U) idx_out[a + n_sel + j] = local_lo + j;
  for (int p = total + tid; p < U; p += kThreads) idx_out[p] = -1;
  if (tid == 0) *cnt_out = min(total, U);
}

// Top-k + union for one selection problem of at most 8 * kThreads
// candidates, run by all 256 threads, thread t holding the keys of block ids
// base + 8t .. base + 8t + 7 in registers (so its keys are in block-id
// order); ids outside the candidates [c0, c1) take no part.  Same result as
// topk_union_regs<8> (MSB-first radix select, 8 bits per pass, stopping once
// the bucket holding the topk-th key is taken whole; ties to the lowest
// block ids), with one barrier per radix pass and one for the output
// positions: each wave counts into its own histogram copies (two per wave,
// double buffered over passes, cleared by the wave itself, 16 bytes per
// lane), and every wave scans all copies (16-byte reads: four digits per
// lane and copy) and finds the threshold bucket on its own, so nothing is
// broadcast.
__device__ __forceinline__ void topk_union_fast(int base, int c0, int c1, int topk, int cur, int n_init, int n_local,
                                                int U, int32_t* idx_out, int32_t* cnt_out, TopkShared& sh,
                                                const uint32_t (&kin)[8]) {
  constexpr int KPT = 8;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i0 = base + tid * KPT;   // block id of this thread's first key
  const int n = c1 - c0;
  uint32_t kr[KPT];
  bool valid[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    valid[e] = i0 + e >= c0 && i0 + e < c1;
    kr[e] = valid[e] ? kin[e] : 0u;
  }
  const bool take_none = topk <= 0 || n <= 0;
  const bool take_all = !take_none && n <= topk;
  uint32_t prefix = 0, mask = 0;
  int kk = topk;
  if (!take_none && !take_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      int(*h)[2][256] = sh.whist[pass & 1];
      // this wave's two copies: cleared in order before its own adds (LDS
      // operations of one wave complete in order); the other waves read them
      // only after the barrier, and reuse of this buffer two passes later is
      // behind the next pass's barrier
      *reinterpret_cast<int4*>(&h[wid][0][4 * lane]) = make_int4(0, 0, 0, 0);
      *reinterpret_cast<int4*>(&h[wid][1][4 * lane]) = make_int4(0, 0, 0, 0);
      int* mine = h[wid][lane & 1];
#pragma unroll
      for (int e = 0; e < KPT; ++e)
        if (valid[e] && (kr[e] & mask) == prefix) atomicAdd(&mine[(kr[e] >> shift) & 255u], 1);
      __syncthreads();
      // lane l looks at digits 255-4l .. 252-4l (descending): bins 252-4l ..
      // 255-4l of every copy
      int4 sum = make_int4(0, 0, 0, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
          const int4 x = *reinterpret_cast<const int4*>(&h[w][cp][252 - 4 * lane]);
          sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
        }
      const int c[4] = {sum.w, sum.z, sum.y, sum.x};
      int run = wave_excl_scan(sum.x + sum.y + sum.z + sum.w);
      int pick = -1, below = 0, in_bucket = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (run < kk && kk <= run + c[r]) {
          pick = 255 - 4 * lane - r;
          below = run;
          in_bucket = c[r];
        }
        run += c[r];
      }
      const uint64_t found = __ballot(pick >= 0);
      if (found == 0) break;   // unreachable: kk never exceeds the keys under the prefix
      const int src = __builtin_ctzll(found);
      pick = __builtin_amdgcn_readlane(pick, src);
      below = __builtin_amdgcn_readlane(below, src);
      in_bucket = __builtin_amdgcn_readlane(in_bucket, src);
      prefix |= ((uint32_t)pick) << shift;
      mask |= 255u << shift;
      kk -= below;
      if (kk == in_bucket) break;   // the bucket is taken whole
    }
  }
  // ties: keys whose masked value equals the threshold bucket; the kk of
  // them with the lowest block ids are taken
  const int need = kk;
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    if (valid[e] && !take_none) {
      if (take_all) ++gt;
      else {
        const uint32_t km = kr[e] & mask;
        gt += km > prefix;
        eq += km == prefix;
      }
    }
  }
  // exclusive scan of (gt, eq) over the workgroup in thread order: one barrier
  const int v = (gt << 16) | eq;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh.scan_tmp[wid] = inc;
  __syncthreads();
  int ex = inc - v;
#pragma unroll
  for (int w = 0; w < 4; ++w) ex += (w < wid) ? sh.scan_tmp[w] : 0;
  int gt_b = ex >> 16, eq_b = ex & 0xffff;
  const int n_sel = take_none ? 0 : (take_all ? n : topk);
  const int local_lo = max(0, cur - n_local + 1);
  const int a = min(n_init, local_lo);          // initial blocks below the local window
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    if (valid[e] && !take_none) {
      bool sel;
      int pos;
      if (take_all) {
        sel = true;
        pos = a + gt_b++;
      } else {
        const uint32_t km = kr[e] & mask;
        if (km > prefix) { sel = true; pos = a + gt_b + min(eq_b, need); ++gt_b; }
        else if (km == prefix) { sel = eq_b < need; pos = a + gt_b + eq_b; ++eq_b; }
        else { sel = false; pos = 0; }
      }
      if (sel && pos < U) idx_out[pos] = i0 + e;
    }
  }
  const int n_loc = cur - local_lo + 1;
  const int total = a + n_sel + n_loc;
  for (int j = tid; j < a; j += kThreads) idx_out[j] = j;
  for (int j = tid; j < n_loc; j += kThreads)
    if (a + n_sel + j < U) idx_out[a + n_sel + j] = local_lo + j;
  for (int q = total + tid; q < U; q += kThreads) idx_out[q] = -1;
  if (tid == 0) *cnt_out = min(total, U);
}

// Causal top-k + union for one selection problem, run by all 256 threads.
//   keys[0..n)  orderable scores of the candidate blocks c0 .. c0+n-1 (LDS)
//   cur         the query's block; candidates are the causal blocks that are
//               neither initial (< n_init) nor local (> cur - n_local)
// Writes idx_out[0..U) (ascending block ids of init | top-k | local, padded
// with -1) and *cnt_out.  Ranking: key descending, block id ascending.
__device__ __forceinline__ void topk_union(const uint32_t* keys, int n, int c0, int topk, int cur, int n_init,
                                           int n_local, int U, int32_t* idx_out, int32_t* cnt_out, TopkShared& sh) {
  if (n <= 8 * kThreads) {
    uint32_t kin[8];
    const int i0 = (int)threadIdx.x * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) kin[e] = (i0 + e < n) ? keys[i0 + e] : 0u;
    topk_union_fast(c0, c0, c0 + n, topk, cur, n_init, n_local, U, idx_out, cnt_out, sh, kin);
  } else {
    topk_union_regs<48>(keys, n, c0, topk, cur, n_init, n_local, U, idx_out, cnt_out, sh);
  }
}

// Copy of 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i of the wave writes bytes [16 i, 16 i + 16)
// after the wave-uniform LDS address `lds`.  The copy is counted by the
// wave's vmcnt like any load and has no register result; the caller waits
// for it (s_waitcnt vmcnt) and then synchronises the workgroup before any
// wave reads the bytes.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
#pragma clang diagnostic pop
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with vmcnt = n (n < 64) and the other counters left open
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace bskv
