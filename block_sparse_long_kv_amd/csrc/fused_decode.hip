// One decode layer with one-layer-ahead selection, as two kernels.
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Eq. 4 and Alg. 2: right
// after layer l's projection emits the Forecast F_l, it scores layer l+1's
// compressed keys and picks layer l+1's blocks, while layer l attends to the
// blocks picked one layer earlier.  Chinese SparDA overview
// (deepresearch2agi.pages.dev), 架构细节: the selection of the next layer runs
// beside the current layer's attention.
//
// The two launches keep the real data dependencies of a layer (the output
// of layer l feeds the next layer's input, hence its Forecast):
//   K1  Forecast projection partials of F_l (128-row splits)
//   K2  scores of layer l+1's candidates (each workgroup first adds the
//       projection splits of its (b, g) in order); the last score workgroup
//       of a (b, g) to finish runs that (b, g)'s top-k + union
//       + attention splits of layer l over its listed blocks; the last split
//       of a (b, g) to finish merges the splits and updates layer l's
//       compressed keys with the newest block
// K2 streams the compressed keys of l+1 and the selected K/V of l together,
// so the scoring and the attention share the HBM pipe instead of running
// back to back, and the per-(b, g) follow-up work (top-k, merge) runs while
// other workgroups still stream instead of in a third launch.  Roles are
// assigned by workgroup index; no workgroup waits for another: the last one
// to arrive at a (b, g)'s counter does the follow-up.
#include "bskv_launch.hpp"
#include "decode_ops.hpp"

namespace bskv {

struct LayerParams {
  // this layer: incremental compressed-key update
  const void* k; int64_t sb, sg, st, kv_len; const int64_t* seq_len;
  float* kc; int64_t nb_cap;
  // this layer: attention (q, k, v, idx, cnt, out inside)
  AttnDecodeParams attn;
  // lookahead: Forecast of this layer -> selection of the next layer
  int select;                       // 0: no next layer
  const void* x; const void* w; int hidden, N;
  float* proj_part; int proj_tiles, proj_splits;
  const float* kc_next; float* scores; int score_splits;
  int32_t* idx_next; int32_t* cnt_next;
  int B, H, topk, n_init, n_local, U;
  // arrival counters of K2: [0, B*H) score workgroups, [B*H, 2*B*H)
  // attention splits; zero before a launch (a zero-filled workspace) and
  // left at zero by each counter's last arrival
  int32_t* sync;
};

// Arrival of this workgroup at a counter shared by n workgroups of one
// launch.  Returns true in the last one to arrive, which resets the counter
// to zero.  What the others hand over is stored and loaded agent-coherent:
// each thread waits until its stores have completed (vmcnt 0) before the
// workgroup counts, and the last one loads only after it has seen the final
// count, so no cache write-back or invalidation is needed.
__device__ __forceinline__ bool arrive_last(int32_t* ctr, int n, int& flag) {
  __builtin_amdgcn_s_waitcnt(0);             // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(ctr, 1);
    flag = old == n - 1;
    if (flag) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // every arrival has counted
  }
  __syncthreads();
  return flag;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void layer_k1(LayerParams p) {
  if constexpr (std::is_same<T, bf16_bits>::value) {
    __shared__ ProjMfmaSmem sm;
    proj_partial_mfma_wg((const T*)p.x, (const T*)p.w, p.B, p.hidden, p.N, blockIdx.x % p.proj_tiles,
                         blockIdx.x / p.proj_tiles, p.proj_part, sm);
  } else {
    __shared__ ProjSmem sm;
    proj_partial_wg<T>((const T*)p.x, (const T*)p.w, p.B, p.hidden, p.N, blockIdx.x % p.proj_tiles,
                       blockIdx.x / p.proj_tiles, p.proj_part, sm);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void layer_k2(LayerParams p) {
  extern __shared__ uint32_t keys[];   // top-k keys of problems above 8 * kThreads candidates
  __shared__ __attribute__((aligned(16))) union {
    AttnSmem<D, G> attn;
    float fvec[D];
    TopkShared topk;
    CombineSmem<D, G> comb;
    MeanpoolSmem<T, D> mp;
  } sm;
  __shared__ int last_flag;
  const int n_bg = p.B * p.H;
  const int n_score = p.select ? p.score_splits * n_bg : 0;
  // attention workgroups (long chains of dependent loads) are dispatched
  // first; the short streaming score workgroups fill the tail
  const int n_attn = p.attn.n_splits * n_bg;
  const int bid = (int)blockIdx.x < n_attn ? (int)blockIdx.x + n_score : (int)blockIdx.x - n_attn;
  if (bid < n_score) {
    const int split = bid % p.score_splits, bg = bid / p.score_splits;
    const int b = bg / p.H, g = bg % p.H;
    for (int i = threadIdx.x; i < D; i += kThreads)
      sm.fvec[i] = proj_reduce_one(p.proj_part, p.proj_splits, p.B, p.N, b, g * D + i);
    __syncthreads();
    const DecodeCands dc = decode_cands(p.seq_len[b], p.nb_cap, p.n_init, p.n_local);
    const int n = dc.c1 - dc.c0;
    const int per = (n + p.score_splits - 1) / p.score_splits;
    const int lo = dc.c0 + split * per, hi = min(dc.c1, lo + per);
    score_slice_wg<D, true>(sm.fvec, p.kc_next + (int64_t)bg * p.nb_cap * D, lo, hi,
                            p.scores + (int64_t)bg * p.nb_cap);
    // the last score workgroup of (b, g): top-k + union of layer l+1
    if (arrive_last(p.sync + bg, p.score_splits, last_flag))
      topk_decode_wg<true>(p.scores + (int64_t)bg * p.nb_cap, dc, p.topk, p.n_init, p.n_local, p.U,
                     p.idx_next + (int64_t)bg * p.U, p.cnt_next + bg, keys, sm.topk);
    return;
  }
  const int a = bid - n_score;
  const int bg = a / p.attn.n_splits;
  attn_split_wg<T, D, G, true>(p.attn, bg, a % p.attn.n_splits, sm.attn);
  // the last attention split of (b, g): merge of the splits, then the
  // newest-block update of this layer's compressed keys (the block the
  // newest token completed)
  if (!arrive_last(p.sync + n_bg + bg, p.attn.n_splits, last_flag)) return;
  attn_combine_wg<D, G, true>(p.attn, bg, sm.comb);
  __syncthreads();
  const int b = bg / p.H, g = bg % p.H;
  const int64_t L = min(p.seq_len[b], p.kv_len);
  if (L <= 0 || (L % kBlk) != 0) return;
  const int64_t j = L / kBlk - 1;
  if (j >= p.nb_cap) return;
  meanpool_wg<T, D>((const T*)p.k + b * p.sb + g * p.sg + j * kBlk * p.st, p.st,
                    p.kc + ((int64_t)bg * p.nb_cap + j) * D, sm.mp);
}

size_t proj_workspace_bytes(int B, int hidden, int N, int dtype);
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int U);
AttnDecodeParams make_attn_params(const AttnDecodeArgs& a, void* ws);
int proj_splits(int hidden);
int proj_tiles(int N, int dtype);

static size_t al256(size_t x) { return ((x + 255) / 256) * 256; }

size_t layer_workspace_bytes(int B, int Hq, int Hkv, int D, int hidden, int64_t nb_cap, int U, int dtype) {
  return al256(proj_workspace_bytes(B, hidden, Hkv * D, dtype)) + al256((size_t)B * Hkv * nb_cap * sizeof(float)) +
         al256((size_t)2 * B * Hkv * sizeof(int32_t)) + attn_decode_workspace_bytes(B, Hq, Hkv, D, U);
}

template <typename T, int D, int G>
static void launch_layer_t(const LayerParams& p, int stages, hipStream_t s) {
  const int n_bg = p.B * p.H;
  const int n_proj = p.select ? p.proj_tiles * p.proj_splits : 0;
  if ((stages & 1) && n_proj > 0) hipLaunchKernelGGL((layer_k1<T>), dim3(n_proj), dim3(kThreads), 0, s, p);
  const int n_score = p.select ? p.score_splits * n_bg : 0;
  const int64_t cap = p.nb_cap < kMaxCandidates ? p.nb_cap : kMaxCandidates;
  const size_t lds = (p.select && cap > 8 * kThreads) ? (size_t)cap * sizeof(uint32_t) : 0;
  if (stages & 2)
    hipLaunchKernelGGL((layer_k2<T, D, G>), dim3(n_score + p.attn.n_splits * n_bg), dim3(kThreads), lds, s, p);
}

template <typename T, int D>
static void launch_layer_g(const LayerParams& p, int G, int stages, hipStream_t s) {
  switch (G) {
    case 1: launch_layer_t<T, D, 1>(p, stages, s); break;
    case 2: launch_layer_t<T, D, 2>(p, stages, s); break;
    case 4: launch_layer_t<T, D, 4>(p, stages, s); break;
    default: launch_layer_t<T, D, 8>(p, stages, s); break;
  }
}

hipError_t launch_decode_layer(const DecodeLayerArgs& a) {
  LayerParams p;
  p.k = a.attn.k; p.sb = a.attn.sb; p.sg = a.attn.sg; p.st = a.attn.st; p.kv_len = a.attn.kv_len;
  p.seq_len = a.attn.seq_len; p.kc = a.kc; p.nb_cap = a.nb_cap;
  const int H = a.attn.Hkv, D = a.attn.D, B = a.attn.B;
  const size_t proj_b = al256(proj_workspace_bytes(B, a.hidden, H * D, a.attn.dtype));
  const size_t score_b = al256((size_t)B * H * a.nb_cap * sizeof(float));
  const size_t sync_b = al256((size_t)2 * B * H * sizeof(int32_t));
  char* ws = (char*)a.attn.ws;
  p.sync = (int32_t*)(ws + proj_b + score_b);
  p.attn = make_attn_params(a.attn, ws + proj_b + score_b + sync_b);
  p.select = a.x != nullptr;
  p.x = a.x; p.w = a.w; p.hidden = a.hidden; p.N = H * D;
  p.proj_part = (float*)ws;
  p.proj_tiles = p.select ? proj_tiles(H * D, a.attn.dtype) : 0;
  p.proj_splits = p.select ? proj_splits(a.hidden) : 0;
  p.kc_next = a.kc_next; p.scores = (float*)(ws + proj_b);
  p.score_splits = score_split_plan(B * H, a.nb_cap);
  p.idx_next = a.idx_next; p.cnt_next = a.cnt_next;
  p.B = B; p.H = H; p.topk = a.topk; p.n_init = a.n_init; p.n_local = a.n_local; p.U = a.attn.U;
  const int G = a.attn.Hq / H;
  if (a.attn.dtype == 0) {
    if (D == 64) launch_layer_g<float, 64>(p, G, a.stages, a.attn.stream);
    else launch_layer_g<float, 128>(p, G, a.stages, a.attn.stream);
  } else {
    if (D == 64) launch_layer_g<bf16_bits, 64>(p, G, a.stages, a.attn.stream);
    else launch_layer_g<bf16_bits, 128>(p, G, a.stages, a.attn.stream);
  }
  return hipGetLastError();
}

}  // namespace bskv
