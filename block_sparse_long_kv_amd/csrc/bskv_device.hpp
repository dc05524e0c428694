// Device helpers shared by the gfx950 kernels of libbskv: 16-byte vector
// loads with bf16/fp32 conversion, wavefront (64-lane) reductions, a
// 256-thread block scan, and the order-preserving float -> uint32 key used by
// the top-k selection.
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

// Streamed 16-byte load that should not displace reusable lines (KV blocks
// read once per step).
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 r;
  r.x = __builtin_nontemporal_load(&q->x);
  r.y = __builtin_nontemporal_load(&q->y);
  r.z = __builtin_nontemporal_load(&q->z);
  r.w = __builtin_nontemporal_load(&q->w);
  return r;
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

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_bits>(bf16_bits x) { return __uint_as_float(((uint32_t)x) << 16); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Exclusive prefix sum over the 256 threads of a block (thread order).
// `tmp` is 4 ints of shared memory; `total` receives the sum of all values.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
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

// Shared scratch of topk_union.
struct TopkShared {
  int hist[256];
  int scan_tmp[4];
  int pick[2];
};

// Causal top-k + union for one selection problem, run by all 256 threads.
//   keys[0..n)  orderable scores of the candidate blocks c0 .. c0+n-1 (LDS)
//   cur         the query's block; blocks 0..cur are the causal range
// Writes idx_out[0..U) (ascending block ids of init | local | top-k, padded
// with -1) and *cnt_out.  Ranking: key descending, block id ascending.
__device__ void topk_union(const uint32_t* keys, int n, int c0, int topk, int cur, int n_init, int n_local,
                           int U, int32_t* idx_out, int32_t* cnt_out, TopkShared& sh) {
  const int tid = threadIdx.x;
  uint32_t thr = 0;
  int need = 0;
  const bool take_none = (topk <= 0);
  const bool take_all = !take_none && (n <= topk);
  if (!take_all && !take_none) {
    // MSB-first radix select of the topk-th largest key, 8 bits per pass.
    uint32_t prefix = 0, mask = 0;
    int kk = topk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      sh.hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kThreads) {
        const uint32_t key = keys[i];
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // Thread tid looks at digit D = 255 - tid; incl = #keys with digit >= D.
      const int D = 255 - tid;
      const int h = sh.hist[D];
      int tot;
      const int excl = block_excl_scan(h, sh.scan_tmp, tot);
      const int above = excl;          // # with digit > D
      const int incl = excl + h;       // # with digit >= D
      if (above < kk && kk <= incl) {
        sh.pick[0] = D;
        sh.pick[1] = above;
      }
      __syncthreads();
      prefix |= ((uint32_t)sh.pick[0]) << shift;
      mask |= 255u << shift;
      kk -= sh.pick[1];
      __syncthreads();
    }
    thr = prefix;   // key of the topk-th best candidate
    need = kk;      // how many candidates equal to thr are taken (lowest ids first)
  }

  // Ordered pass over block ids 0..cur in contiguous per-thread chunks.
  const int N = cur + 1;
  const int E = (N + kThreads - 1) / kThreads;
  const int j_lo = min(N, tid * E), j_hi = min(N, j_lo + E);
  const int local_lo = cur - n_local + 1;
  int my_ties = 0;
  if (!take_all && !take_none) {
    for (int j = j_lo; j < j_hi; ++j) {
      const int i = j - c0;
      if (i >= 0 && i < n && keys[i] == thr) ++my_ties;
    }
  }
  int tot;
  int tie_rank = block_excl_scan(my_ties, sh.scan_tmp, tot);
  int my_sel = 0;
  for (int j = j_lo; j < j_hi; ++j) {
    const int i = j - c0;
    bool s = (j < n_init) || (j >= local_lo);
    if (i >= 0 && i < n && !take_none) {
      if (take_all) s = true;
      else {
        const uint32_t key = keys[i];
        if (key > thr) s = true;
        else if (key == thr) { if (tie_rank < need) s = true; ++tie_rank; }
      }
    }
    my_sel += s ? 1 : 0;
  }
  int total;
  int pos = block_excl_scan(my_sel, sh.scan_tmp, total);
  // second walk: recompute the same flags and write the positions
  tie_rank = tie_rank - my_ties;  // restore this thread's starting tie rank
  for (int j = j_lo; j < j_hi; ++j) {
    const int i = j - c0;
    bool s = (j < n_init) || (j >= local_lo);
    if (i >= 0 && i < n && !take_none) {
      if (take_all) s = true;
      else {
        const uint32_t key = keys[i];
        if (key > thr) s = true;
        else if (key == thr) { if (tie_rank < need) s = true; ++tie_rank; }
      }
    }
    if (s) {
      if (pos < U) idx_out[pos] = j;
      ++pos;
    }
  }
  for (int p = total + tid; p < U; p += kThreads) idx_out[p] = -1;
  if (tid == 0) *cnt_out = min(total, U);
}

}  // namespace bskv
