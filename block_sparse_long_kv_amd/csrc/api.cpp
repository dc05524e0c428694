// C ABI of libbskv: host-side argument checks, workspace sizing and
// dispatch to the gfx950 kernels.  Nothing here allocates, frees or
// synchronises; every failed check returns before any launch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "bskv_launch.hpp"
#include "../../include/bskv.h"

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e) {
  const char* s = hipGetErrorString(e);
  strncpy(g_last_error, s ? s : "unknown HIP error", sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = 0;
  return BSKV_EHIP;
}

int finish(hipError_t e) { return e == hipSuccess ? BSKV_OK : hip_fail(e); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize_of(int dtype) { return dtype == BSKV_F32 ? 4 : (dtype == BSKV_BF16 ? 2 : 0); }

bool dtype_ok(int dtype) { return dtype == BSKV_F32 || dtype == BSKV_BF16; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// K/V strides (elements) must keep every 16-byte row chunk aligned.
bool strides_ok(const int64_t* s, int dtype) {
  if (!s) return false;
  const int64_t m = 16 / esize_of(dtype);
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] % m) return false;
  // 64 rows of one block span less than 2 GiB (32-bit per-lane load offsets)
  if (s[2] * 64 * esize_of(dtype) >= (int64_t(1) << 31)) return false;
  return true;
}

// the decode attention reads K/V of one (b, g) through 32-bit byte offsets
bool span_ok(int64_t kv_len, const int64_t* s, int dtype) {
  return kv_len * s[2] * esize_of(dtype) < (int64_t(1) << 31);
}

bool group_ok(int hq, int hkv) {
  if (hq <= 0 || hkv <= 0 || hq % hkv) return false;
  const int G = hq / hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

}  // namespace

namespace bskv {
// for other translation units of the library (the allocation-free entry point)
void set_last_error(const char* msg) {
  strncpy(g_last_error, msg ? msg : "", sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = 0;
}
int report_hip(hipError_t e) { return finish(e); }
}  // namespace bskv

extern "C" {

int bskv_version(void) { return (0 << 16) | 1; }

const char* bskv_strerror(int status) {
  switch (status) {
    case BSKV_OK: return "ok";
    case BSKV_EINVAL: return "invalid argument (null pointer, size, stride or alignment)";
    case BSKV_EDTYPE: return "dtype not supported by this call";
    case BSKV_EUNSUPPORTED: return "configuration outside what the kernels handle";
    case BSKV_ENOSPC: return "workspace too small";
    case BSKV_EHIP: return "HIP error (see bskv_last_error)";
    default: return "unknown status";
  }
}

const char* bskv_last_error(void) { return g_last_error; }

size_t bskv_forecast_proj_workspace(int B, int hidden, int n_kv_heads, int head_dim, int dtype) {
  if (B <= 0 || hidden <= 0 || n_kv_heads <= 0 || head_dim <= 0 || !dtype_ok(dtype)) return 0;
  return bskv::proj_workspace_bytes(B, hidden, n_kv_heads * head_dim, dtype);
}

int bskv_forecast_proj(const void* x, const void* w, int dtype, int B, int hidden, int n_kv_heads, int head_dim,
                       float* f_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (B <= 0 || hidden <= 0 || n_kv_heads <= 0 || head_dim <= 0) return BSKV_EINVAL;
  if (!x || !w || !f_out || !ws) return BSKV_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(ws)) return BSKV_EINVAL;
  const int N = n_kv_heads * head_dim;
  const int tile = dtype == BSKV_F32 ? 64 : 128;
  if (hidden % 256 || N % tile) return BSKV_EUNSUPPORTED;
  if (ws_bytes < bskv::proj_workspace_bytes(B, hidden, N, dtype)) return BSKV_ENOSPC;
  bskv::ProjArgs a{x, w, dtype, B, hidden, N, f_out, ws, stream};
  return finish(bskv::launch_proj(a));
}

int bskv_kv_block_meanpool(const void* k, int dtype, const int64_t* kv_strides, int64_t kv_len, int B, int n_kv_heads,
                           int head_dim,
                           int block, const int64_t* seq_len, int64_t blk_begin, int64_t blk_end, int newest_only,
                           float* kc, int64_t kc_nb_cap, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!k || !kc || !seq_len || !aligned16(k) || !aligned16(kc)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || kc_nb_cap <= 0 || kv_len < 0) return BSKV_EINVAL;
  if (!strides_ok(kv_strides, dtype)) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (blk_begin < 0 || blk_end < blk_begin || blk_end > kc_nb_cap) return BSKV_EINVAL;
  if (!newest_only && blk_end - blk_begin > 0x7fffffff) return BSKV_EUNSUPPORTED;
  bskv::MeanpoolArgs a{k, dtype, kv_strides[0], kv_strides[1], kv_strides[2], kv_len, B, n_kv_heads, head_dim, block,
                       seq_len, blk_begin, blk_end, newest_only ? 1 : 0, kc, kc_nb_cap, stream};
  return finish(bskv::launch_meanpool(a));
}

size_t bskv_score_topk_workspace(int B, int n_kv_heads, int n_q_tokens, int64_t kc_nb_cap, int head_dim) {
  if (B <= 0 || n_kv_heads <= 0 || kc_nb_cap <= 0 || n_q_tokens < 0) return 0;
  return bskv::score_topk_workspace_bytes(B, n_kv_heads, n_q_tokens, kc_nb_cap, head_dim);
}

int bskv_forecast_block_score_topk(const void* f, int f_dtype, int n_q_tokens, int64_t q_start, const float* kc,
                                   int64_t kc_nb_cap, const int64_t* seq_len, int B, int n_kv_heads, int head_dim,
                                   int block, int topk, int n_init, int n_local, int32_t* idx_out, int32_t* cnt_out,
                                   float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(f_dtype)) return BSKV_EDTYPE;
  if (!f || !kc || !idx_out || !cnt_out || !aligned16(f) || !aligned16(kc)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || kc_nb_cap <= 0 || n_q_tokens < 0) return BSKV_EINVAL;
  if (topk < 0 || n_init < 1 || n_local < 1) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (kc_nb_cap > bskv::kMaxCandidates) return BSKV_EUNSUPPORTED;
  if ((int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  const int U = topk + n_init + n_local;
  if (n_q_tokens == 0) {
    if (f_dtype != BSKV_F32) return BSKV_EDTYPE;
    if (!seq_len || !ws) return BSKV_EINVAL;
    if (ws_bytes < bskv::score_topk_workspace_bytes(B, n_kv_heads, 0, kc_nb_cap, head_dim)) return BSKV_ENOSPC;
  } else {
    if (q_start < 0 || q_start % block) return BSKV_EINVAL;
    if (scores_out || !ws || !aligned16(ws)) return BSKV_EINVAL;
    const int64_t n_qb = (n_q_tokens + block - 1) / block;
    if (n_qb > 65535 || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
    if (ws_bytes < bskv::score_topk_workspace_bytes(B, n_kv_heads, n_q_tokens, kc_nb_cap, head_dim))
      return BSKV_ENOSPC;
  }
  bskv::ScoreTopkArgs a{f, f_dtype, n_q_tokens, q_start, kc, kc_nb_cap, seq_len, B, n_kv_heads, head_dim, block,
                        topk, n_init, n_local, U, idx_out, cnt_out, scores_out, ws, stream};
  return finish(bskv::launch_score_topk(a));
}

namespace {
bool window_grid_ok(int window, int stride) {
  return (window == 32 || window == 64) && (stride == 16 || stride == 32 || stride == 64) && stride <= window &&
         window % stride == 0;
}
// 64-token blocks whose windows all lie inside a window array of nw entries
int64_t window_blocks(int64_t nw, int window, int stride) { return ((nw - 1) * stride + window) / 64; }
}  // namespace

int bskv_kv_window_meanpool(const void* k, int dtype, const int64_t* kv_strides, int64_t kv_len, int B,
                            int n_kv_heads, int head_dim, int window, int stride, const int64_t* seq_len,
                            int64_t w_begin, int64_t w_end, int newest_only, float* kcw, int64_t kcw_nw_cap,
                            hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!k || !kcw || !seq_len || !aligned16(k) || !aligned16(kcw)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || kcw_nw_cap <= 0 || kv_len < 0) return BSKV_EINVAL;
  if (!strides_ok(kv_strides, dtype)) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || !window_grid_ok(window, stride)) return BSKV_EUNSUPPORTED;
  if (w_begin < 0 || w_end < w_begin || w_end > kcw_nw_cap) return BSKV_EINVAL;
  if (!newest_only && w_end - w_begin > 0x7fffffff) return BSKV_EUNSUPPORTED;
  if ((int64_t)B > 65535 || n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  bskv::WindowMeanpoolArgs a{k, dtype, kv_strides[0], kv_strides[1], kv_strides[2], kv_len, B, n_kv_heads, head_dim,
                             window, stride, seq_len, w_begin, w_end, newest_only ? 1 : 0, kcw, kcw_nw_cap, stream};
  return finish(bskv::launch_window_meanpool(a));
}

size_t bskv_window_score_topk_workspace(int B, int n_kv_heads, int n_q_tokens, int64_t kcw_nw_cap) {
  if (B <= 0 || n_kv_heads <= 0 || kcw_nw_cap <= 0 || n_q_tokens < 0) return 0;
  return bskv::window_select_workspace_bytes(B, n_kv_heads, n_q_tokens, kcw_nw_cap);
}

int bskv_forecast_window_score_topk(const void* f, int f_dtype, int n_q_tokens, int64_t q_start, const float* kcw,
                                    int64_t kcw_nw_cap, const int64_t* seq_len, int B, int n_kv_heads, int head_dim,
                                    int block, int window, int stride, int topk, int n_init, int n_local,
                                    int32_t* idx_out, int32_t* cnt_out, float* scores_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!dtype_ok(f_dtype)) return BSKV_EDTYPE;
  if (!f || !kcw || !idx_out || !cnt_out || !aligned16(f) || !aligned16(kcw)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || kcw_nw_cap <= 0 || n_q_tokens < 0) return BSKV_EINVAL;
  if (topk < 0 || n_init < 1 || n_local < 1) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || block != 64 || !window_grid_ok(window, stride)) return BSKV_EUNSUPPORTED;
  const int64_t nb_cap = window_blocks(kcw_nw_cap, window, stride);
  if (nb_cap < 1) return BSKV_EINVAL;
  if (nb_cap > bskv::kMaxCandidates || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  if (n_q_tokens == 0) {
    if (f_dtype != BSKV_F32) return BSKV_EDTYPE;
    if (!seq_len || !ws || !aligned16(ws)) return BSKV_EINVAL;
    if (ws_bytes < bskv::window_select_workspace_bytes(B, n_kv_heads, 0, kcw_nw_cap)) return BSKV_ENOSPC;
  } else {
    if (q_start < 0 || q_start % block) return BSKV_EINVAL;
    if (scores_out) return BSKV_EINVAL;
    if ((n_q_tokens + block - 1) / block > 65535) return BSKV_EUNSUPPORTED;
  }
  bskv::WindowSelectArgs a{f, f_dtype, n_q_tokens, q_start, kcw, kcw_nw_cap, nb_cap, seq_len, B, n_kv_heads,
                           head_dim, window, stride, topk, n_init, n_local, topk + n_init + n_local, idx_out, cnt_out,
                           scores_out, ws, stream};
  return finish(bskv::launch_window_select(a));
}

size_t bskv_multihead_score_topk_workspace(int B, int n_kv_heads, int64_t kc_nb_cap) {
  if (B <= 0 || n_kv_heads <= 0 || kc_nb_cap <= 0) return 0;
  return bskv::multihead_select_workspace_bytes(B, n_kv_heads, kc_nb_cap);
}

int bskv_multihead_block_score_topk(const void* q, int q_dtype, const float* kc, int64_t kc_nb_cap,
                                    const int64_t* seq_len, int B, int n_q_heads, int n_kv_heads, int head_dim,
                                    int block, int topk, int n_init, int n_local, float scale, int32_t* idx_out,
                                    int32_t* cnt_out, float* weights_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!dtype_ok(q_dtype)) return BSKV_EDTYPE;
  if (!q || !kc || !seq_len || !idx_out || !cnt_out || !ws) return BSKV_EINVAL;
  if (!aligned16(kc) || !aligned16(ws)) return BSKV_EINVAL;
  if (B <= 0 || kc_nb_cap <= 0 || topk < 0 || n_init < 1 || n_local < 1) return BSKV_EINVAL;
  if (!(scale > 0.f) || scale != scale) return BSKV_EINVAL;
  if (!group_ok(n_q_heads, n_kv_heads)) return BSKV_EUNSUPPORTED;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (kc_nb_cap > bskv::kMaxCandidates || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  if (ws_bytes < bskv::multihead_select_workspace_bytes(B, n_kv_heads, kc_nb_cap)) return BSKV_ENOSPC;
  bskv::MultiheadSelectArgs a{q, q_dtype, kc, kc_nb_cap, seq_len, B, n_kv_heads, n_q_heads / n_kv_heads, head_dim,
                              topk, n_init, n_local, topk + n_init + n_local, scale, idx_out, cnt_out, weights_out,
                              ws, stream};
  return finish(bskv::launch_multihead_select(a));
}

size_t bskv_attn_decode_workspace(int B, int n_q_heads, int n_kv_heads, int head_dim, int U) {
  if (B <= 0 || U <= 0 || !group_ok(n_q_heads, n_kv_heads) || head_dim <= 0) return 0;
  return bskv::attn_decode_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, U);
}

int bskv_block_sparse_attn_decode(const void* q, const void* k, const void* v, int dtype, const int64_t* kv_strides,
                                  int64_t kv_len, int kv_is_ring, const int32_t* idx, const int32_t* cnt, const int64_t* seq_len, int B,
                                  int n_q_heads, int n_kv_heads, int head_dim, int block, int U, float scale,
                                  float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!q || !k || !v || !idx || !cnt || !seq_len || !out || !ws) return BSKV_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(ws)) return BSKV_EINVAL;
  if (B <= 0 || U <= 0 || kv_len < 0 || !strides_ok(kv_strides, dtype)) return BSKV_EINVAL;
  if (kv_len % 64) return BSKV_EINVAL;   // the K/V buffers hold whole blocks
  if (!span_ok(kv_len, kv_strides, dtype)) return BSKV_EUNSUPPORTED;
  if (!group_ok(n_q_heads, n_kv_heads)) return BSKV_EUNSUPPORTED;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if ((int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  if (!(scale > 0.f) || scale != scale) return BSKV_EINVAL;
  if (ws_bytes < bskv::attn_decode_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, U)) return BSKV_ENOSPC;
  bskv::AttnDecodeArgs a{q, k, v, dtype, kv_strides[0], kv_strides[1], kv_strides[2], kv_len, kv_is_ring ? 1 : 0,
                         idx, cnt, seq_len, B, n_q_heads, n_kv_heads, head_dim, block, U, scale, out, ws, stream};
  return finish(bskv::launch_attn_decode(a));
}

int bskv_block_sparse_attn_prefill(const void* q, const void* k, const void* v, int dtype, const int64_t* kv_strides,
                                   int64_t kv_len, const int32_t* idx, const int32_t* cnt, int64_t q_start, int n_q_tokens, int B,
                                   int n_q_heads, int n_kv_heads, int head_dim, int block, int U, float scale,
                                   void* out, hipStream_t stream) {
  if (dtype != BSKV_BF16) return BSKV_EDTYPE;
  if (!q || !k || !v || !idx || !cnt || !out) return BSKV_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return BSKV_EINVAL;
  if (B <= 0 || U <= 0 || n_q_tokens <= 0 || kv_len < 0 || !strides_ok(kv_strides, dtype)) return BSKV_EINVAL;
  if (kv_len % 64) return BSKV_EINVAL;   // the K/V buffers hold whole blocks
  if (q_start < 0 || q_start % 64) return BSKV_EINVAL;
  if (!group_ok(n_q_heads, n_kv_heads)) return BSKV_EUNSUPPORTED;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (!(scale > 0.f) || scale != scale) return BSKV_EINVAL;
  // one workgroup per (query block, KV head, group of up to four query heads)
  const int64_t n_tiles = (int64_t)((n_q_tokens + 63) / 64) * B * n_kv_heads * ((n_q_heads / n_kv_heads + 3) / 4);
  if (n_tiles > 0x7fffffff) return BSKV_EUNSUPPORTED;
  bskv::AttnPrefillArgs a{q, k, v, kv_strides[0], kv_strides[1], kv_strides[2], kv_len, idx, cnt, q_start, n_q_tokens,
                          B, n_q_heads, n_kv_heads, head_dim, block, U, scale, out, stream};
  return finish(bskv::launch_attn_prefill(a));
}

int bskv_prefetch_selected_blocks(const void* src_k, const void* src_v, int dtype, const int64_t* src_strides,
                                  int64_t src_len, const int32_t* idx, const int32_t* cnt, void* ring_k, void* ring_v, int B,
                                  int n_kv_heads, int head_dim, int block, int U, int n_workgroups,
                                  hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!src_k || !src_v || !idx || !cnt || !ring_k || !ring_v) return BSKV_EINVAL;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(ring_k) || !aligned16(ring_v)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || U <= 0 || n_workgroups < 1 || src_len < 0 || !strides_ok(src_strides, dtype))
    return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if ((int64_t)B * n_kv_heads * U > 0x7fffffff || n_workgroups > 65535) return BSKV_EUNSUPPORTED;
  bskv::GatherArgs a{src_k, src_v, src_strides[0], src_strides[1], src_strides[2], src_len, esize_of(dtype), idx, cnt,
                     ring_k, ring_v, B, n_kv_heads, head_dim, block, U, n_workgroups, stream};
  return finish(bskv::launch_gather(a));
}

namespace {
constexpr int kCacheMaxSlots = 1024;   // slots per (b, g) of a block cache
}  // namespace

int bskv_block_cache_reset(int32_t* tags, int64_t* stamps, int64_t* clock, int B, int n_kv_heads, int n_slots,
                           hipStream_t stream) {
  if (!tags || !stamps || !clock) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || n_slots <= 0) return BSKV_EINVAL;
  if (n_slots > kCacheMaxSlots || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  return finish(bskv::launch_cache_reset(tags, stamps, clock, B * n_kv_heads, n_slots, stream));
}

int bskv_block_cache_plan(const int32_t* idx, const int32_t* cnt, int B, int n_kv_heads, int U, int32_t* tags,
                          int64_t* stamps, int64_t* clock, int n_slots, int32_t* slot_out, int32_t* fill_out,
                          int32_t* n_fill_out, hipStream_t stream) {
  if (!idx || !cnt || !tags || !stamps || !clock || !slot_out || !fill_out || !n_fill_out) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || U <= 0 || n_slots <= 0) return BSKV_EINVAL;
  if (U > n_slots) return BSKV_EINVAL;   // every listed block needs a slot
  if (n_slots > kCacheMaxSlots || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  bskv::CachePlanArgs a{idx, cnt, U, tags, stamps, clock, n_slots, slot_out, fill_out, n_fill_out,
                        B * n_kv_heads, stream};
  return finish(bskv::launch_cache_plan(a));
}

int bskv_prefetch_cache_fill(const void* src_k, const void* src_v, int dtype, const int64_t* src_strides,
                             int64_t src_len, const int32_t* idx, const int32_t* slot, const int32_t* fill,
                             const int32_t* n_fill, void* cache_k, void* cache_v, int B, int n_kv_heads, int head_dim,
                             int block, int U, int n_slots, int n_workgroups, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!src_k || !src_v || !idx || !slot || !fill || !n_fill || !cache_k || !cache_v) return BSKV_EINVAL;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(cache_k) || !aligned16(cache_v)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || U <= 0 || n_slots <= 0 || n_workgroups < 1 || src_len < 0 ||
      !strides_ok(src_strides, dtype))
    return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (n_slots > kCacheMaxSlots || (int64_t)B * n_kv_heads > 65535 || n_workgroups > 65535) return BSKV_EUNSUPPORTED;
  bskv::CacheFillArgs a{src_k, src_v, src_strides[0], src_strides[1], src_strides[2], src_len, esize_of(dtype), idx,
                        slot, fill, n_fill, cache_k, cache_v, B, n_kv_heads, head_dim, block, U, n_slots,
                        n_workgroups, stream};
  return finish(bskv::launch_cache_fill(a));
}

int bskv_block_sparse_attn_decode_cached(const void* q, const void* cache_k, const void* cache_v, int dtype,
                                         int n_slots, const int32_t* slot, const int32_t* idx, const int32_t* cnt,
                                         const int64_t* seq_len, int B, int n_q_heads, int n_kv_heads, int head_dim,
                                         int block, int U, float scale, float* out, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!q || !cache_k || !cache_v || !slot || !idx || !cnt || !seq_len || !out || !ws) return BSKV_EINVAL;
  if (!aligned16(q) || !aligned16(cache_k) || !aligned16(cache_v) || !aligned16(ws)) return BSKV_EINVAL;
  if (B <= 0 || U <= 0 || n_slots <= 0) return BSKV_EINVAL;
  if (!group_ok(n_q_heads, n_kv_heads)) return BSKV_EUNSUPPORTED;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (n_slots > kCacheMaxSlots || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  if (!(scale > 0.f) || scale != scale) return BSKV_EINVAL;
  if (ws_bytes < bskv::attn_decode_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, U)) return BSKV_ENOSPC;
  // cache layout [B, n_kv_heads, n_slots, block, head_dim], contiguous
  const int64_t st = head_dim, sg = (int64_t)n_slots * block * head_dim, sb = sg * n_kv_heads;
  bskv::AttnDecodeArgs a{q, cache_k, cache_v, dtype, sb, sg, st, (int64_t)n_slots * block, 1, idx, cnt, seq_len, B,
                         n_q_heads, n_kv_heads, head_dim, block, U, scale, out, ws, stream, slot};
  return finish(bskv::launch_attn_decode(a));
}

int bskv_block_sparse_attn_decode_cached_fill(
    const void* q, const void* cache_k, const void* cache_v, int dtype, int n_slots, const int32_t* slot,
    const int32_t* idx, const int32_t* cnt, const int64_t* seq_len, int B, int n_q_heads, int n_kv_heads, int head_dim,
    int block, int U, float scale, float* out, void* ws, size_t ws_bytes, const void* src_k, const void* src_v,
    const int64_t* src_strides, int64_t src_len, const int32_t* fill_idx, const int32_t* fill_slot,
    const int32_t* fill, const int32_t* n_fill, void* fill_cache_k, void* fill_cache_v, int fill_n_slots,
    int n_fill_workgroups, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!q || !cache_k || !cache_v || !slot || !idx || !cnt || !seq_len || !out || !ws) return BSKV_EINVAL;
  if (!src_k || !src_v || !fill_idx || !fill_slot || !fill || !n_fill || !fill_cache_k || !fill_cache_v)
    return BSKV_EINVAL;
  if (!aligned16(q) || !aligned16(cache_k) || !aligned16(cache_v) || !aligned16(ws) || !aligned16(src_k) ||
      !aligned16(src_v) || !aligned16(fill_cache_k) || !aligned16(fill_cache_v))
    return BSKV_EINVAL;
  // the filled cache is another layer's: this launch reads cache_k / cache_v
  if (fill_cache_k == cache_k || fill_cache_v == cache_v || fill_cache_k == cache_v || fill_cache_v == cache_k)
    return BSKV_EINVAL;
  if (B <= 0 || U <= 0 || n_slots <= 0 || fill_n_slots <= 0 || n_fill_workgroups < 1 || src_len < 0 ||
      !strides_ok(src_strides, dtype))
    return BSKV_EINVAL;
  if (!group_ok(n_q_heads, n_kv_heads)) return BSKV_EUNSUPPORTED;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (n_slots > kCacheMaxSlots || fill_n_slots > kCacheMaxSlots || (int64_t)B * n_kv_heads > 65535 ||
      n_fill_workgroups > 65535)
    return BSKV_EUNSUPPORTED;
  if (!(scale > 0.f) || scale != scale) return BSKV_EINVAL;
  if (ws_bytes < bskv::attn_decode_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, U)) return BSKV_ENOSPC;
  const bskv::CacheFillArgs f{src_k, src_v, src_strides[0], src_strides[1], src_strides[2], src_len, esize_of(dtype),
                              fill_idx, fill_slot, fill, n_fill, fill_cache_k, fill_cache_v, B, n_kv_heads, head_dim,
                              block, U, fill_n_slots, n_fill_workgroups, stream};
  const int64_t st = head_dim, sg = (int64_t)n_slots * block * head_dim, sb = sg * n_kv_heads;
  bskv::AttnDecodeArgs a{q, cache_k, cache_v, dtype, sb, sg, st, (int64_t)n_slots * block, 1, idx, cnt, seq_len, B,
                         n_q_heads, n_kv_heads, head_dim, block, U, scale, out, ws, stream, slot, &f};
  return finish(bskv::launch_attn_decode(a));
}

int bskv_qkvf_proj_decode(const void* x, const void* w_t, int B, int hidden, int n_q_heads, int n_kv_heads,
                          int head_dim, void* q_out, void* k_cache, void* v_cache, const int64_t* kv_strides,
                          int64_t kv_len, const int64_t* seq_len, float* f_out, hipStream_t stream) {
  if (!x || !w_t || !q_out || !k_cache || !v_cache || !seq_len || !f_out) return BSKV_EINVAL;
  if (!aligned16(x) || !aligned16(w_t)) return BSKV_EINVAL;
  if (B <= 0 || hidden <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || kv_len < 0) return BSKV_EINVAL;
  if (!strides_ok(kv_strides, BSKV_BF16)) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim)) return BSKV_EUNSUPPORTED;
  const int64_t N = (int64_t)(n_q_heads + 3 * n_kv_heads) * head_dim;
  // four waves split the hidden axis in steps of 8 x 32
  if (hidden % 1024 || B > 64 || N / 16 > 0x7fffffff) return BSKV_EUNSUPPORTED;
  bskv::QkvfDecodeArgs a{x, w_t, B, hidden, n_q_heads, n_kv_heads, head_dim, q_out, k_cache, v_cache, kv_strides[0],
                         kv_strides[1], kv_strides[2], kv_len, seq_len, f_out, stream};
  return finish(bskv::launch_qkvf_decode(a));
}

int bskv_qkvf_proj_prefill(const void* x, const void* w_t, int B, int n_q_tokens, int hidden, int n_q_heads,
                           int n_kv_heads, int head_dim, int64_t q_start, void* q_out, void* k_cache, void* v_cache,
                           const int64_t* kv_strides, int64_t kv_len, float* f_pooled, hipStream_t stream) {
  if (!x || !w_t || !q_out || !k_cache || !v_cache || !f_pooled) return BSKV_EINVAL;
  if (!aligned16(x) || !aligned16(w_t) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(f_pooled))
    return BSKV_EINVAL;
  if (B <= 0 || n_q_tokens <= 0 || hidden <= 0 || n_q_heads <= 0 || n_kv_heads <= 0) return BSKV_EINVAL;
  if (q_start < 0 || q_start % 64 || q_start + n_q_tokens > kv_len) return BSKV_EINVAL;
  if (!strides_ok(kv_strides, BSKV_BF16)) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim)) return BSKV_EUNSUPPORTED;
  // 128-column tiles never straddle the Q / K / V / F head groups
  if (hidden % 64 || ((int64_t)n_q_heads * head_dim) % 128 || ((int64_t)n_kv_heads * head_dim) % 128)
    return BSKV_EUNSUPPORTED;
  const int64_t n_tiles = (int64_t)(n_q_heads + 3 * n_kv_heads) * head_dim / 128 * ((n_q_tokens + 127) / 128) * B;
  if (n_tiles > 0x7fffffff) return BSKV_EUNSUPPORTED;
  bskv::QkvfPrefillArgs a{x, w_t, B, n_q_tokens, hidden, n_q_heads, n_kv_heads, head_dim, q_start, q_out, k_cache,
                          v_cache, kv_strides[0], kv_strides[1], kv_strides[2], kv_len, f_pooled, stream};
  return finish(bskv::launch_qkvf_prefill(a));
}

size_t bskv_score_topk_pooled_workspace(int B, int n_kv_heads, int n_qb, int64_t kc_nb_cap, int head_dim) {
  if (B <= 0 || n_kv_heads <= 0 || n_qb <= 0 || kc_nb_cap <= 0 || !head_dim_ok(head_dim)) return 0;
  return bskv::prefill_select_workspace_bytes(B * n_kv_heads, n_qb, kc_nb_cap, head_dim, true);
}

int bskv_forecast_block_score_topk_pooled(const float* f_pooled, int n_qb, int64_t q_start, const float* kc,
                                          int64_t kc_nb_cap, int B, int n_kv_heads, int head_dim, int block, int topk,
                                          int n_init, int n_local, int32_t* idx_out, int32_t* cnt_out, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  if (!f_pooled || !kc || !idx_out || !cnt_out || !ws) return BSKV_EINVAL;
  if (!aligned16(f_pooled) || !aligned16(kc) || !aligned16(ws)) return BSKV_EINVAL;
  if (B <= 0 || n_kv_heads <= 0 || n_qb <= 0 || kc_nb_cap <= 0) return BSKV_EINVAL;
  if (topk < 0 || n_init < 1 || n_local < 1) return BSKV_EINVAL;
  if (q_start < 0 || q_start % 64) return BSKV_EINVAL;
  if (!head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (kc_nb_cap > bskv::kMaxCandidates || n_qb > 65535 || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  if (ws_bytes < bskv::prefill_select_workspace_bytes(B * n_kv_heads, n_qb, kc_nb_cap, head_dim, true))
    return BSKV_ENOSPC;
  return finish(bskv::launch_score_topk_pooled(f_pooled, n_qb, q_start, kc, kc_nb_cap, B, n_kv_heads, head_dim, topk,
                                               n_init, n_local, idx_out, cnt_out, ws, stream));
}

size_t bskv_decode_layer_lookahead_workspace(int B, int n_q_heads, int n_kv_heads, int head_dim, int hidden,
                                             int64_t kc_nb_cap, int U, int dtype) {
  if (B <= 0 || U <= 0 || kc_nb_cap <= 0 || hidden < 0 || !group_ok(n_q_heads, n_kv_heads) || !dtype_ok(dtype) ||
      !head_dim_ok(head_dim))
    return 0;
  return bskv::layer_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, hidden, kc_nb_cap, U, dtype);
}

int bskv_decode_layer_lookahead(const void* q, const void* k, const void* v, int dtype, const int64_t* kv_strides,
                                int64_t kv_len, const int64_t* seq_len, float* kc, const float* scores, int32_t* idx,
                                int32_t* cnt, float scale, float* out, const void* x, const void* w_forecast,
                                int hidden, const float* kc_next, float* scores_next, int32_t* idx_next,
                                int32_t* cnt_next, int B, int n_q_heads,
                                int n_kv_heads, int head_dim, int block, int64_t kc_nb_cap, int topk, int n_init,
                                int n_local, int stages, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BSKV_EDTYPE;
  if (!q || !k || !v || !seq_len || !kc || !idx || !cnt || !out || !ws) return BSKV_EINVAL;
  if (stages < 1 || stages > 3) return BSKV_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(kc) || !aligned16(ws)) return BSKV_EINVAL;
  const bool sel = x != nullptr;
  const bool deferred = scores_next != nullptr, immediate = idx_next != nullptr || cnt_next != nullptr;
  if (sel != (w_forecast != nullptr) || sel != (kc_next != nullptr) || sel != (deferred || immediate))
    return BSKV_EINVAL;   // the lookahead arguments come all together or not at all
  if (deferred && immediate) return BSKV_EINVAL;           // one form of the next layer's selection
  if (immediate && (!idx_next || !cnt_next)) return BSKV_EINVAL;
  if (sel && (!aligned16(x) || !aligned16(w_forecast) || !aligned16(kc_next))) return BSKV_EINVAL;
  if (B <= 0 || kv_len < 0 || kc_nb_cap <= 0 || !strides_ok(kv_strides, dtype)) return BSKV_EINVAL;
  if (kv_len % 64) return BSKV_EINVAL;   // the K/V buffers hold whole blocks
  if (!span_ok(kv_len, kv_strides, dtype)) return BSKV_EUNSUPPORTED;
  if (topk < 0 || n_init < 1 || n_local < 1) return BSKV_EINVAL;
  if (!(scale > 0.f) || scale != scale) return BSKV_EINVAL;
  if (!group_ok(n_q_heads, n_kv_heads) || !head_dim_ok(head_dim) || block != 64) return BSKV_EUNSUPPORTED;
  if (kc_nb_cap > bskv::kMaxCandidates || (int64_t)B * n_kv_heads > 65535) return BSKV_EUNSUPPORTED;
  const int tile = dtype == BSKV_F32 ? 64 : 128;
  if (sel && (hidden <= 0 || hidden % 256 || (n_kv_heads * head_dim) % tile)) return BSKV_EUNSUPPORTED;
  const int U = topk + n_init + n_local;
  if (ws_bytes < bskv::layer_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, sel ? hidden : 0, kc_nb_cap, U,
                                             dtype))
    return BSKV_ENOSPC;
  bskv::DecodeLayerArgs a;
  a.attn = bskv::AttnDecodeArgs{q, k, v, dtype, kv_strides[0], kv_strides[1], kv_strides[2], kv_len, 0, idx, cnt,
                                seq_len, B, n_q_heads, n_kv_heads, head_dim, block, U, scale, out, ws, stream};
  a.kc = kc; a.nb_cap = kc_nb_cap;
  a.scores = scores; a.idx = idx; a.cnt = cnt;
  a.x = x; a.w = w_forecast; a.hidden = sel ? hidden : 0;
  a.kc_next = kc_next; a.scores_next = scores_next; a.idx_next = idx_next; a.cnt_next = cnt_next;
  a.topk = topk; a.n_init = n_init; a.n_local = n_local; a.stages = stages;
  return finish(bskv::launch_decode_layer(a));
}

int bskv_host_device_pointer(void* host_ptr, void** dev_ptr) {
  if (!host_ptr || !dev_ptr) return BSKV_EINVAL;
  return finish(hipHostGetDevicePointer(dev_ptr, host_ptr, 0));
}

}  // extern "C"
