// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Arguments here are already validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bskv {

struct MeanpoolArgs {
  const void* k; int dtype; int64_t sb, sg, st; int64_t kv_len;
  int B, H, D, block;
  const int64_t* seq_len; int64_t blk_begin, blk_end; int newest_only;
  float* kc; int64_t nb_cap;
  hipStream_t stream;
};
hipError_t launch_meanpool(const MeanpoolArgs& a);

struct ProjArgs {
  const void* x; const void* w; int dtype;
  int B, hidden, N;
  float* f; void* ws;
  hipStream_t stream;
};
size_t proj_workspace_bytes(int B, int hidden, int N, int dtype);
hipError_t launch_proj(const ProjArgs& a);
int proj_splits(int hidden, int dtype);
template <typename T>
void launch_proj_partial(const void* x, const void* w, int B, int hidden, int N, float* part, hipStream_t s);

// Widened projection (Q, K, V, F) = X [W_Q | W_K | W_V | W_F], bf16.
struct QkvfDecodeArgs {
  const void* x; const void* w;
  int B, hidden, Hq, H, D;
  void* q; void* k; void* v; int64_t sb, sg, st, kv_len; const int64_t* seq_len;
  float* f;
  hipStream_t stream;
};
hipError_t launch_qkvf_decode(const QkvfDecodeArgs& a);
struct QkvfPrefillArgs {
  const void* x; const void* w;
  int B, Tq, hidden, Hq, H, D; int64_t q_start;
  void* q; void* k; void* v; int64_t sb, sg, st, kv_len;
  float* f_pooled;
  hipStream_t stream;
};
hipError_t launch_qkvf_prefill(const QkvfPrefillArgs& a);
hipError_t launch_score_topk_pooled(const float* f_pooled, int n_qb, int64_t q_start, const float* kc,
                                   int64_t nb_cap, int B, int H, int D, int topk, int n_init, int n_local,
                                   int32_t* idx, int32_t* cnt, void* ws, hipStream_t stream);
size_t prefill_select_workspace_bytes(int n_bg, int n_qb, int64_t nb_cap, int D, bool pooled);

struct ScoreTopkArgs {
  const void* f; int f_dtype; int n_q_tokens; int64_t q_start;
  const float* kc; int64_t nb_cap; const int64_t* seq_len;
  int B, H, D, block, topk, n_init, n_local, U;
  int32_t* idx; int32_t* cnt; float* scores;
  void* ws;
  hipStream_t stream;
};
size_t score_topk_workspace_bytes(int B, int H, int n_q_tokens, int64_t nb_cap, int D);
hipError_t launch_score_topk(const ScoreTopkArgs& a);
constexpr int kMaxCandidates = 12288;  // candidate blocks per problem (48 KB of LDS keys)

struct WindowMeanpoolArgs {
  const void* k; int dtype; int64_t sb, sg, st; int64_t kv_len;
  int B, H, D, window, stride;
  const int64_t* seq_len; int64_t w_begin, w_end; int newest_only;
  float* kcw; int64_t nw_cap;
  hipStream_t stream;
};
hipError_t launch_window_meanpool(const WindowMeanpoolArgs& a);

struct WindowSelectArgs {
  const void* f; int f_dtype; int n_q_tokens; int64_t q_start;
  const float* kcw; int64_t nw_cap; int64_t nb_cap; const int64_t* seq_len;
  int B, H, D, window, stride, topk, n_init, n_local, U;
  int32_t* idx; int32_t* cnt; float* scores;
  void* ws;
  hipStream_t stream;
};
size_t window_select_workspace_bytes(int B, int H, int n_q_tokens, int64_t nw_cap);
hipError_t launch_window_select(const WindowSelectArgs& a);

struct MultiheadSelectArgs {
  const void* q; int q_dtype;
  const float* kc; int64_t nb_cap; const int64_t* seq_len;
  int B, H, G, D, topk, n_init, n_local, U; float scale;
  int32_t* idx; int32_t* cnt; float* weights;
  void* ws;
  hipStream_t stream;
};
size_t multihead_select_workspace_bytes(int B, int H, int64_t nb_cap);
hipError_t launch_multihead_select(const MultiheadSelectArgs& a);

struct CacheFillArgs;
struct CacheFillParams;

struct AttnDecodeArgs {
  const void* q; const void* k; const void* v; int dtype;
  int64_t sb, sg, st; int64_t kv_len; int ring;
  const int32_t* idx; const int32_t* cnt; const int64_t* seq_len;
  int B, Hq, Hkv, D, block, U; float scale;
  float* out; void* ws;
  hipStream_t stream;
  const int32_t* slot = nullptr;     // block cache: listed block u is read from slot[u] of k, v
  const CacheFillArgs* fill = nullptr;   // another layer's cache fill in the split kernel's launch
};
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int U);
hipError_t launch_attn_decode(const AttnDecodeArgs& a);

struct AttnPrefillArgs {
  const void* q; const void* k; const void* v;
  int64_t sb, sg, st; int64_t kv_len;
  const int32_t* idx; const int32_t* cnt;
  int64_t q_start; int Tq;
  int B, Hq, Hkv, D, block, U; float scale;
  void* out;
  hipStream_t stream;
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a);

struct GatherArgs {
  const void* src_k; const void* src_v; int64_t sb, sg, st;  // element strides
  int64_t src_len;
  int esize;
  const int32_t* idx; const int32_t* cnt;
  void* ring_k; void* ring_v;
  int B, H, D, block, U, n_workgroups;
  hipStream_t stream;
};
hipError_t launch_gather(const GatherArgs& a);

// Resident block cache (least recently used, per (b, g)).
struct CachePlanArgs {
  const int32_t* idx; const int32_t* cnt; int U;
  int32_t* tags; int64_t* stamps; int64_t* clock; int S;
  int32_t* slot; int32_t* fill; int32_t* n_fill;
  int n_bg;
  hipStream_t stream;
};
hipError_t launch_cache_plan(const CachePlanArgs& a);
struct CacheFillArgs {
  const void* src_k; const void* src_v; int64_t sb, sg, st;  // element strides
  int64_t src_len;
  int esize;
  const int32_t* idx; const int32_t* slot; const int32_t* fill; const int32_t* n_fill;
  void* cache_k; void* cache_v;
  int B, H, D, block, U, S, n_workgroups;
  hipStream_t stream;
};
hipError_t launch_cache_fill(const CacheFillArgs& a);
CacheFillParams make_fill_params(const CacheFillArgs& a);
hipError_t launch_cache_reset(int32_t* tags, int64_t* stamps, int64_t* clock, int n_bg, int S, hipStream_t stream);

// One decode layer with lookahead selection of the next layer (3 kernels).
struct DecodeLayerArgs {
  AttnDecodeArgs attn;               // this layer's attention (ring must be 0); ws = the whole workspace
  float* kc; int64_t nb_cap;         // this layer's compressed keys (newest block updated)
  const float* scores;               // this layer's candidate scores (nullptr: idx/cnt are given)
  int32_t* idx; int32_t* cnt;        // this layer's lists (written from scores when given)
  const void* x; const void* w; int hidden;               // Forecast projection (x == nullptr: no next layer)
  const float* kc_next; float* scores_next;           // deferred mode: the next layer's scores
  int32_t* idx_next; int32_t* cnt_next;                 // immediate mode: the next layer's lists
  int topk, n_init, n_local;
  int stages;                        // bit mask of the two launches
};
size_t layer_workspace_bytes(int B, int Hq, int Hkv, int D, int hidden, int64_t nb_cap, int U, int dtype);
hipError_t launch_decode_layer(const DecodeLayerArgs& a);

}  // namespace bskv
