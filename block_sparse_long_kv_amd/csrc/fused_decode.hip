// One decode layer with one-layer-ahead selection, as two kernels.
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Eq. 4 and Alg. 2: right
// after layer l's projection emits the Forecast F_l, it scores layer l+1's
// compressed keys, which picks layer l+1's blocks, while layer l attends to
// the blocks picked one layer earlier.  Chinese SparDA overview
// (deepresearch2agi.pages.dev), 架构细节: the selection of the next layer runs
// beside the current layer's attention.
//
// The two launches keep the real data dependencies of a layer (the output
// of layer l feeds the next layer's input, hence its Forecast):
//   K1  the top-k + union of THIS layer's blocks, from the candidate scores
//       the previous layer's call left (when given), beside the Forecast
//       projection partials of F_l (128-row splits)
//   K2  scores of layer l+1's candidates (each workgroup first adds the
//       projection splits of its (b, g) in order), stored for the next
//       layer's call
//       + attention splits of layer l over its listed blocks; the last split
//       of a (b, g) to finish merges the splits, and the (b, g)'s last split
//       in list order updates layer l's compressed keys with the newest block
// The top-k of layer l+1 then runs in the next call's K1, where it shares a
// short, latency-bound launch with the projection (deferred mode).  In the
// immediate mode the scores go to the workspace instead and the last score
// workgroup of each (b, g) to finish runs that (b, g)'s top-k inside K2,
// while the long attention chains are still streaming.  K2 streams the
// compressed keys of l+1 and the selected K/V of l together, so the scoring
// and the attention share the HBM pipe.  Roles are assigned by workgroup
// index; no workgroup waits for another: the last attention split to arrive
// at a (b, g)'s counter does the merge.
#include "bskv_launch.hpp"
#include "decode_ops.hpp"

namespace bskv {

struct LayerParams {
  // this layer: incremental compressed-key update
  const void* k; int64_t sb, sg, st, kv_len; const int64_t* seq_len;
  float* kc; int64_t nb_cap;
  // this layer: top-k + union from the previous call's scores (nullptr: the
  // lists are given), then attention (q, k, v, idx, cnt, out inside)
  const float* scores_in; int32_t* idx; int32_t* cnt;
  AttnDecodeParams attn;
  // lookahead: Forecast of this layer -> scores of the next layer
  int select;                       // 0: no next layer
  const void* x; const void* w; int hidden, N;
  // proj_splits partials (kProjPartRows rows each for bf16); the first
  // kernel's projection workgroups span proj_rows rows of W each
  float* proj_part; int proj_tiles, proj_splits, proj_rows;
  const float* kc_next; float* scores_next; int score_splits;
  // immediate mode (idx_next != nullptr): the scores go to the workspace
  // and the last score workgroup of each (b, g) runs the next layer's top-k
  int32_t* idx_next; int32_t* cnt_next;
  int B, H, topk, n_init, n_local, U;
  // arrival counters of K2: [0, B*H) attention splits, [B*H, 2*B*H) score
  // slices (immediate mode), one per (b, g); zero before a launch (a
  // zero-filled workspace) and left at zero by each counter's last arrival
  int32_t* sync;
};

// The counter region opens every workspace with a fixed size, the counters
// of the largest B * H the calls accept, whatever this call's B * H is:
// only counters ever use those bytes, so a workspace shared by calls of
// different shapes still finds them zero.
constexpr size_t kSyncWords = (size_t)2 * 65535;

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
  extern __shared__ uint32_t keys[];   // top-k keys of problems above 8 * kThreads candidates
  constexpr bool kMfma = std::is_same<T, bf16_bits>::value;
  __shared__ __attribute__((aligned(16))) union {
    typename std::conditional<kMfma, ProjMfmaSmem, ProjSmem>::type proj;
    TopkShared topk;
  } sm;
  const int n_topk = p.scores_in ? p.B * p.H : 0;
  if ((int)blockIdx.x < n_topk) {
    // this layer's top-k + union (the longer chain: its workgroups go first)
    const int bg = blockIdx.x;
    const DecodeCands dc = decode_cands(p.seq_len[bg / p.H], p.nb_cap, p.n_init, p.n_local);
    topk_decode_wg(p.scores_in + (int64_t)bg * p.nb_cap, p.nb_cap, dc, p.topk, p.n_init, p.n_local, p.U,
                   p.idx + (int64_t)bg * p.U, p.cnt + bg, keys, sm.topk);
    return;
  }
  const int pid = (int)blockIdx.x - n_topk;
  if constexpr (kMfma) {
    if (p.proj_rows == kProjPartRows)
      proj_partial_mfma_wg<kProjPartRows>((const T*)p.x, (const T*)p.w, p.B, p.hidden, p.N, pid % p.proj_tiles,
                                          pid / p.proj_tiles, p.proj_part, sm.proj);
    else
      proj_partial_mfma_wg<kProjRows>((const T*)p.x, (const T*)p.w, p.B, p.hidden, p.N, pid % p.proj_tiles,
                                      pid / p.proj_tiles, p.proj_part, sm.proj);
  } else
    proj_partial_wg<T>((const T*)p.x, (const T*)p.w, p.B, p.hidden, p.N, pid % p.proj_tiles, pid / p.proj_tiles,
                       p.proj_part, sm.proj);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads, 3) void layer_k2(LayerParams p) {
  extern __shared__ uint32_t keys[];   // immediate mode: top-k keys of problems above 8 * kThreads candidates
  __shared__ __attribute__((aligned(16))) union {
    typename AttnSmemSel<T, D, G>::type attn;
    float fvec[D];
    CombineSmem<D, G> comb;
    MeanpoolSmem<T, D> mp;
    TopkShared topk;
  } sm;
  __shared__ int last_flag;
  const int n_bg = p.B * p.H;
  const int n_score = p.select ? p.score_splits * n_bg : 0;
  // attention workgroups (long chains of dependent loads) are dispatched
  // first; the short streaming score workgroups fill the tail
  const int n_attn = p.attn.n_splits * n_bg;
  const int bid = (int)blockIdx.x < n_attn ? (int)blockIdx.x + n_score : (int)blockIdx.x - n_attn;
  if (bid < n_score) {
    const int split = bid / n_bg, bg = bid % n_bg;   // split-major, as the attention below
    const int b = bg / p.H, g = bg % p.H;
    const DecodeCands dc = decode_cands(p.seq_len[b], p.nb_cap, p.n_init, p.n_local);
    const int n = dc.c1 - dc.c0;
    const int per = (n + p.score_splits - 1) / p.score_splits;
    const int lo = dc.c0 + split * per, hi = min(dc.c1, lo + per);
    float* sc = p.scores_next + (int64_t)bg * p.nb_cap;
    if (!p.idx_next) {
      score_slice_proj_wg<D, false>(p.proj_part, p.proj_splits, p.B, p.N, b, g, p.kc_next + (int64_t)bg * p.nb_cap * D,
                                    lo, hi, sc, sm.fvec);
      return;
    }
    score_slice_proj_wg<D, true>(p.proj_part, p.proj_splits, p.B, p.N, b, g, p.kc_next + (int64_t)bg * p.nb_cap * D,
                                 lo, hi, sc, sm.fvec);
    // the last score workgroup of (b, g): top-k + union of the next layer
    if (arrive_last(p.sync + n_bg + bg, p.score_splits, last_flag))
      topk_decode_wg<true>(sc, p.nb_cap, dc, p.topk, p.n_init, p.n_local, p.U, p.idx_next + (int64_t)bg * p.U, p.cnt_next + bg,
                           keys, sm.topk);
    return;
  }
  // Split-major: consecutive workgroups, which the dispatcher deals out to
  // the XCDs in turn, are different (b, g) units of one split, so every XCD
  // gets the same mix of long and short splits, and with B * H a multiple
  // of 8 all the attention splits and score slices of one (b, g) share an
  // XCD.  Measured in alternating runs against (b, g)-major attention and
  // slice-major scores (where the shorter last split of every unit landed
  // on the same two XCDs): B8 x 128K deferred 1.37-1.41 vs 1.41-1.43 ms
  // per step; B4 x 32K 22.1-22.4 vs 22.8-23.1 us per layer-step deferred,
  // 21.9-22.1 vs 22.3-22.6 immediate.
  const int a = bid - n_score;
  const int bg = a % n_bg, split = a / n_bg;
  attn_split_wg<T, D, G, true>(p.attn, bg, split, sm.attn);
  // the newest-block update of this layer's compressed keys (the block the
  // newest token completed) by the (b, g)'s last split, which has the
  // fewest blocks: off the merge's critical path.  No split reads that row
  // (the newest block is local, never a scored candidate).
  if (split == p.attn.n_splits - 1) {
    const int b = bg / p.H, g = bg % p.H;
    const int64_t L = min(p.seq_len[b], p.kv_len);
    const int64_t j = L / kBlk - 1;
    if (L > 0 && (L % kBlk) == 0 && j < p.nb_cap) {
      __syncthreads();
      meanpool_wg<T, D>((const T*)p.k + b * p.sb + g * p.sg + j * kBlk * p.st, p.st,
                        p.kc + ((int64_t)bg * p.nb_cap + j) * D, sm.mp);
    }
  }
  // the last attention split of (b, g) to finish merges the splits
  if (!arrive_last(p.sync + bg, p.attn.n_splits, last_flag)) return;
  attn_combine_wg<D, G, true>(p.attn, bg, sm.comb);
}

size_t proj_workspace_bytes(int B, int hidden, int N, int dtype);
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int U);
AttnDecodeParams make_attn_params(const AttnDecodeArgs& a, void* ws);
int proj_splits(int hidden, int dtype);
int proj_tiles(int N, int dtype);

static size_t al256(size_t x) { return ((x + 255) / 256) * 256; }

// Workspace layout: the counter region first (kSyncWords int32, the same
// size for every call), so one workspace can serve layers with and without
// a lookahead (whose projection partials are absent) and calls of any
// shape, and the counters always land on words every earlier call left at
// zero; then the projection partials, the next layer's candidate scores
// (immediate mode) and the attention split partials, which every call
// writes before it reads them.
size_t layer_workspace_bytes(int B, int Hq, int Hkv, int D, int hidden, int64_t nb_cap, int U, int dtype) {
  return al256(kSyncWords * sizeof(int32_t)) + al256(proj_workspace_bytes(B, hidden, Hkv * D, dtype)) +
         al256((size_t)B * Hkv * nb_cap * sizeof(float)) + attn_decode_workspace_bytes(B, Hq, Hkv, D, U);
}

template <typename T, int D, int G>
static void launch_layer_t(const LayerParams& p, int stages, hipStream_t s) {
  const int n_bg = p.B * p.H;
  const int n_topk = p.scores_in ? n_bg : 0;
  const int n_proj = p.select ? p.proj_tiles * (p.hidden / p.proj_rows) : 0;
  const int64_t cap = p.nb_cap < kMaxCandidates ? p.nb_cap : kMaxCandidates;
  const size_t lds = (n_topk > 0 && cap > 8 * kThreads) ? (size_t)cap * sizeof(uint32_t) : 0;
  if ((stages & 1) && n_topk + n_proj > 0)
    hipLaunchKernelGGL((layer_k1<T>), dim3(n_topk + n_proj), dim3(kThreads), lds, s, p);
  const int n_score = p.select ? p.score_splits * n_bg : 0;
  const size_t lds2 = (p.select && p.idx_next && cap > 8 * kThreads) ? (size_t)cap * sizeof(uint32_t) : 0;
  if (stages & 2)
    hipLaunchKernelGGL((layer_k2<T, D, G>), dim3(n_score + p.attn.n_splits * n_bg), dim3(kThreads), lds2, s, p);
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
  p.scores_in = a.scores; p.idx = a.idx; p.cnt = a.cnt;
  const int H = a.attn.Hkv, D = a.attn.D, B = a.attn.B;
  const size_t sync_b = al256(kSyncWords * sizeof(int32_t));
  const size_t proj_b = al256(proj_workspace_bytes(B, a.hidden, H * D, a.attn.dtype));
  const size_t score_b = al256((size_t)B * H * a.nb_cap * sizeof(float));
  char* ws = (char*)a.attn.ws;
  p.sync = (int32_t*)ws;
  p.attn = make_attn_params(a.attn, ws + sync_b + proj_b + score_b);
  p.select = a.x != nullptr;
  p.x = a.x; p.w = a.w; p.hidden = a.hidden; p.N = H * D;
  p.proj_part = (float*)(ws + sync_b);
  p.proj_tiles = p.select ? proj_tiles(H * D, a.attn.dtype) : 0;
  p.proj_splits = p.select ? proj_splits(a.hidden, a.attn.dtype) : 0;
  // bf16 without this layer's top-k in the first kernel: 128-row spans (twice
  // the workgroups, each with half the bytes in flight); beside the top-k
  // 256-row spans, so that both roles find a CU each
  p.proj_rows = (a.attn.dtype != 0 && !a.scores) ? kProjPartRows : kProjRows;
  p.kc_next = a.kc_next;
  p.idx_next = a.idx_next; p.cnt_next = a.cnt_next;
  p.scores_next = a.idx_next ? (float*)(ws + sync_b + proj_b) : a.scores_next;
  p.score_splits = score_split_plan(B * H, a.nb_cap);
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
