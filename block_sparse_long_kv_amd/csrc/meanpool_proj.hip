// Block mean-pooling of keys into compressed keys, and the Forecast
// projection GEMV.
//
// Sources: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The problem InfLLM-V2 leaves on the table" (keys are
// mean-pooled per block), "The fourth projection" (Eq. 3: the projection also
// emits the Forecast; Alg. 2: incremental compressed-key update), "One
// Forecast head per GQA group" (one Forecast head per KV head).
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

// ---------------------------------------------------------------------------
// kv_block_meanpool: one workgroup per (block j, kv head g, batch b).
// 256 threads = RPP row lanes x CPR 16-byte chunks of a token row; each lane
// sums its rows in fp32, then the RPP partial rows are added in a fixed order
// through LDS.  HBM-bound: reads block*D elements, writes D floats.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void meanpool_kernel(const T* __restrict__ k, int64_t sb, int64_t sg,
                                                          int64_t st, int64_t kv_len, int H, int block,
                                                          const int64_t* __restrict__ seq_len, int64_t j0,
                                                          int64_t j1, int newest_only, float* __restrict__ kc,
                                                          int64_t nb_cap) {
  constexpr int VEC = VecN<T>::N;
  constexpr int CPR = D / VEC;          // 16-byte chunks per token row
  constexpr int RPP = kThreads / CPR;   // rows per pass
  __shared__ float red[RPP][D + 4];

  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t L = min(seq_len[b], kv_len);
  int64_t j;
  if (newest_only) {
    if (L <= 0 || (L % block) != 0) return;
    j = L / block - 1;
    if (j < j0 || j >= j1) return;
  } else {
    j = j0 + blockIdx.x;
    if (j >= j1 || (j + 1) * (int64_t)block > L) return;
  }
  const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  const T* base = k + b * sb + g * sg + j * (int64_t)block * st + c * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int r = r0; r < block; r += RPP) {
    float x[VEC];
    cvt16<T>(ld16(base + r * st), x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[r0][c * VEC + e] = acc[e];
  __syncthreads();
  for (int t = threadIdx.x; t < D; t += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][t];
    kc[((int64_t)(b * H + g) * nb_cap + j) * D + t] = s / (float)block;
  }
}

template <typename T, int D>
static hipError_t launch_meanpool_t(const MeanpoolArgs& a) {
  const int64_t nx = a.newest_only ? 1 : (a.blk_end - a.blk_begin);
  if (nx <= 0) return hipSuccess;
  dim3 grid((unsigned)nx, (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((meanpool_kernel<T, D>), grid, dim3(kThreads), 0, a.stream, (const T*)a.k, a.sb, a.sg,
                     a.st, a.kv_len, a.H, a.block, a.seq_len, a.blk_begin, a.blk_end, a.newest_only, a.kc, a.nb_cap);
  return hipGetLastError();
}

hipError_t launch_meanpool(const MeanpoolArgs& a) {
  if (a.dtype == 0) return a.D == 64 ? launch_meanpool_t<float, 64>(a) : launch_meanpool_t<float, 128>(a);
  return a.D == 64 ? launch_meanpool_t<bf16_bits, 64>(a) : launch_meanpool_t<bf16_bits, 128>(a);
}

// ---------------------------------------------------------------------------
// forecast_proj: F[b, n] = sum_r x[b, r] W[r, n], W row-major [hidden, N].
// Workgroup (tile, split): a tile of TC = 16*VEC columns and a run of
// rows_per_split rows.  Thread = (row lane 0..15, column chunk 0..15); each
// lane walks every 16th row of the run with 16-byte loads of W and keeps
// MAXB x VEC fp32 sums.  Row lanes are added through LDS, the split partial
// goes to the workspace, and the last workgroup of a tile (atomic counter)
// adds the splits in split order: deterministic.  HBM-bound on W.
// ---------------------------------------------------------------------------
constexpr int kProjMaxB = 8;   // batch rows per pass (more spill registers)
constexpr int kProjRowsPerSplit = 128;

template <typename T, int MAXB>
__global__ __launch_bounds__(kThreads) void proj_kernel(const T* __restrict__ x, const T* __restrict__ w, int B,
                                                      int hidden, int N, int n_splits, float* __restrict__ f,
                                                      float* __restrict__ part, int* __restrict__ counters) {
  constexpr int VEC = VecN<T>::N;
  constexpr int TC = 16 * VEC;   // columns per tile
  __shared__ float xs[MAXB][kProjRowsPerSplit];
  __shared__ float red[16][TC + 4];
  __shared__ int is_last;

  const int tile = blockIdx.x, split = blockIdx.y;
  const int c = threadIdx.x & 15, rl = threadIdx.x >> 4;
  const int r_begin = split * kProjRowsPerSplit;
  const int col0 = tile * TC + c * VEC;

  for (int b0 = 0; b0 < B; b0 += MAXB) {
    const int nb = min(MAXB, B - b0);
    for (int i = threadIdx.x; i < MAXB * kProjRowsPerSplit; i += kThreads) {
      const int bb = i / kProjRowsPerSplit, r = i % kProjRowsPerSplit;
      xs[bb][r] = (bb < nb) ? to_f32<T>(x[(int64_t)(b0 + bb) * hidden + r_begin + r]) : 0.f;
    }
    __syncthreads();
    float acc[MAXB][VEC];
#pragma unroll
    for (int bb = 0; bb < MAXB; ++bb)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[bb][e] = 0.f;
#pragma unroll 4
    for (int r = rl; r < kProjRowsPerSplit; r += 16) {
      float wv[VEC];
      cvt16<T>(ld16(w + (int64_t)(r_begin + r) * N + col0), wv);
#pragma unroll
      for (int bb = 0; bb < MAXB; ++bb) {
        const float xv = xs[bb][r];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[bb][e] += xv * wv[e];
      }
    }
#pragma unroll
    for (int bb = 0; bb < MAXB; ++bb) {
      if (bb >= nb) break;
#pragma unroll
      for (int e = 0; e < VEC; ++e) red[rl][c * VEC + e] = acc[bb][e];
      __syncthreads();
      for (int t = threadIdx.x; t < TC; t += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) s += red[q][t];
        part[((int64_t)split * B + b0 + bb) * N + tile * TC + t] = s;
      }
      __syncthreads();
    }
  }
  // last workgroup of this column tile adds the split partials in order
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&counters[tile], 1) == n_splits - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int i = threadIdx.x; i < B * TC; i += kThreads) {
    const int bb = i / TC, t = i % TC;
    float s = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) s += part[((int64_t)sp * B + bb) * N + tile * TC + t];
    f[(int64_t)bb * N + tile * TC + t] = s;
  }
  if (threadIdx.x == 0) counters[tile] = 0;
}

int proj_splits(int hidden) { return hidden / kProjRowsPerSplit; }
int proj_tiles(int N, int dtype) { return N / (dtype == 0 ? 64 : 128); }

size_t proj_workspace_bytes(int B, int hidden, int N, int dtype) {
  const size_t part = (size_t)proj_splits(hidden) * B * N * sizeof(float);
  const size_t ctr = (size_t)proj_tiles(N, dtype) * sizeof(int);
  return ((part + 255) / 256) * 256 + ((ctr + 255) / 256) * 256;
}

template <typename T, int MAXB>
static void launch_proj_t(const ProjArgs& a, dim3 grid, int ns, float* part, int* ctr) {
  hipLaunchKernelGGL((proj_kernel<T, MAXB>), grid, dim3(kThreads), 0, a.stream, (const T*)a.x, (const T*)a.w,
                     a.B, a.hidden, a.N, ns, a.f, part, ctr);
}

template <typename T>
static void launch_proj_b(const ProjArgs& a, dim3 grid, int ns, float* part, int* ctr) {
  if (a.B <= 1) launch_proj_t<T, 1>(a, grid, ns, part, ctr);
  else if (a.B <= 2) launch_proj_t<T, 2>(a, grid, ns, part, ctr);
  else if (a.B <= 4) launch_proj_t<T, 4>(a, grid, ns, part, ctr);
  else launch_proj_t<T, kProjMaxB>(a, grid, ns, part, ctr);
}

hipError_t launch_proj(const ProjArgs& a) {
  const int ns = proj_splits(a.hidden), nt = proj_tiles(a.N, a.dtype);
  const size_t part_bytes = (size_t)ns * a.B * a.N * sizeof(float);
  float* part = (float*)a.ws;
  int* ctr = (int*)((char*)a.ws + ((part_bytes + 255) / 256) * 256);
  dim3 grid(nt, ns);
  if (a.dtype == 0) launch_proj_b<float>(a, grid, ns, part, ctr);
  else launch_proj_b<bf16_bits>(a, grid, ns, part, ctr);
  return hipGetLastError();
}

}  // namespace bskv
