/*
 * bskv.h -- C ABI of libbskv.so: Forecast-driven block-sparse attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (SparDA, built on InfLLM-V2-style block selection) is described
 * on these web pages, cited below by tag:
 *   [EXPL] "SparDA: a fourth projection that lets sparse attention prefetch
 *          its own KV cache" (ai.thesatyajit.com/articles/sparda)
 *   [OVW]  Chinese-language SparDA overview (deepresearch2agi.pages.dev),
 *          sections 架构细节 (architecture details) and 系统实现 (system
 *          implementation)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless a parameter says otherwise.  The
 *   caller allocates and owns every buffer, stream and workspace; the library
 *   never allocates, frees, synchronises or creates streams inside these
 *   calls.  Every compute call is asynchronous on `stream`.
 * - Return value: BSKV_OK (0) or a negative bskv_status.  All arguments are
 *   checked on the host before anything is launched; on any error nothing is
 *   launched.  BSKV_EHIP means a HIP launch failed (bskv_last_error() has the
 *   HIP message).  Faults inside a kernel surface at the caller's next
 *   synchronisation, as usual in HIP.
 * - Layouts: K/V caches are addressed as [B, Hkv, T, d] with element strides
 *   kv_strides = {batch, kv head, token}; head_dim elements are contiguous.
 *   Base pointers must be 16-byte aligned and strides multiples of
 *   16 bytes / element size; 64 token strides must span less than 2 GiB
 *   (else BSKV_EINVAL), and for the decode attention calls kv_len token
 *   strides of one (b, g) too (else BSKV_EUNSUPPORTED: its loads use 32-bit
 *   byte offsets).  A 64-token block j of (b, g) is the contiguous
 *   run of tokens 64j..64j+63, so the default contiguous layout is also
 *   [B, Hkv, T/64, 64, d].
 * - dtype: BSKV_F32 or BSKV_BF16 (raw bfloat16 bits, round-to-nearest-even).
 *   Accumulation is always fp32.
 * - head_dim must be 64 or 128; block must be 64 (the pages' block size).
 * - Workspaces: a call that takes `ws` needs at least the bytes returned by
 *   its *_workspace() query, 16-byte aligned.  Every partial result in it is
 *   written before it is read.  One exception holds state between calls:
 *   bskv_decode_layer_lookahead keeps arrival counters at the start of its
 *   workspace, which must be zero-filled once before its first use and which
 *   every complete call leaves at zero (see that call).  All other
 *   workspaces need no initialisation.  Calls that overlap in time must not
 *   share a workspace.
 * - kv_len / src_len: the number of tokens the K/V buffers hold (their
 *   allocation along the token axis).  For the attention calls and the
 *   decode layer it must be a whole number of blocks (else BSKV_EINVAL):
 *   allocate caches in whole blocks; tokens past seq_len (decode) or past
 *   the query position (prefill) are masked.  Kernels skip any listed block
 *   that would reach beyond kv_len, so a bad index list cannot make them
 *   read outside the buffers.
 * - Thread safety: the library holds no mutable state apart from the
 *   thread-local text of the last HIP error.
 */
#ifndef BSKV_H
#define BSKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSKV_OK = 0,
  BSKV_EINVAL = -1,       /* null pointer, bad size, bad stride or alignment */
  BSKV_EDTYPE = -2,       /* dtype not supported by this call */
  BSKV_EUNSUPPORTED = -3, /* valid but outside what the kernels handle */
  BSKV_ENOSPC = -4,       /* workspace too small */
  BSKV_EHIP = -5          /* a HIP call failed */
} bskv_status;

typedef enum { BSKV_F32 = 0, BSKV_BF16 = 1 } bskv_dtype;

/* Library version, (major << 16) | minor. */
int bskv_version(void);

/* Static description of a status code. */
const char* bskv_strerror(int status);

/* Text of the last HIP error seen by this thread ("" if none). */
const char* bskv_last_error(void);

/* ----------------------------------------------------------------------- *
 * a1  Forecast projection.  [EXPL] "The fourth projection", Eq. 3: the
 * layer's projection phi_l also emits the Forecast F; [EXPL] "One Forecast
 * head per GQA group": one Forecast head per KV head.
 *
 *   f_out[b, g, c] = sum_r x[b, r] * w[r, g*head_dim + c]
 *
 * x      [B, hidden]                 dtype, contiguous
 * w      [hidden, n_kv_heads*head_dim] dtype, contiguous (row-major)
 * f_out  [B, n_kv_heads, head_dim]   fp32, contiguous
 * hidden must be a multiple of 256.  ws: bskv_forecast_proj_workspace().
 * Two launches: partial products (per 128 rows of w for bf16, 256 for
 * fp32), then their sum in row order; the fused decode layer adds the same
 * partials in the same order, so both give bit-identical Forecasts.
 * The same call serves the separate layer-0 projection ([EXPL] "Training"):
 * pass that projection's weights.  Deterministic: fixed summation order.
 * ----------------------------------------------------------------------- */
size_t bskv_forecast_proj_workspace(int B, int hidden, int n_kv_heads, int head_dim, int dtype);
int bskv_forecast_proj(const void* x, const void* w, int dtype, int B, int hidden, int n_kv_heads,
                       int head_dim, float* f_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * a2  Block mean-pooling into compressed keys.  [EXPL] "The problem
 * InfLLM-V2 leaves on the table" (keys are mean-pooled into compressed
 * representations); [EXPL] "The fourth projection", Alg. 2 (a per-layer
 * compressed-key cache updated incrementally during decode).
 *
 *   kc[b, g, j, :] = (1/block) * sum_{r<block} k[b, g, block*j + r, :]
 *
 * written for every j in [blk_begin, blk_end) whose block is complete for
 * batch b (block*(j+1) <= min(seq_len[b], kv_len)); other rows are left
 * untouched.
 * newest_only != 0 selects the incremental decode update: for each b only
 * the block completed by the last token (j = seq_len[b]/block - 1, when
 * seq_len[b] is a multiple of block and j lies in the range) is written, so
 * the same launch can be replayed every step.
 *
 * k        cache, dtype, strides kv_strides (host array of 3 int64)
 * seq_len  [B] int64 (device): tokens held per batch element
 * kc       [B, n_kv_heads, kc_nb_cap, head_dim] fp32, contiguous
 * Requires 0 <= blk_begin <= blk_end <= kc_nb_cap.
 * ----------------------------------------------------------------------- */
int bskv_kv_block_meanpool(const void* k, int dtype, const int64_t* kv_strides, int64_t kv_len, int B, int n_kv_heads,
                           int head_dim, int block, const int64_t* seq_len, int64_t blk_begin,
                           int64_t blk_end, int newest_only, float* kc, int64_t kc_nb_cap,
                           hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * a3  Forecast block scoring, causal top-k and union.  [EXPL] "The fourth
 * projection", Eq. 4 and Algs. 1-2: B = B_init | B_local | f_top(F K~^T, k);
 * [EXPL] "One Forecast head per GQA group", Sec. 4.1 selector: one raw dot
 * product per block, ranking only (no 1/sqrt(d), no softmax); [EXPL]
 * "Training", Eq. 7 comment: the top-k is taken after the causal mask and
 * without the initial and local blocks.
 *
 * For a query in block cur:
 *   B_init  = {0 .. n_init-1}             (those <= cur)
 *   B_local = {max(0, cur-n_local+1) .. cur}
 *   cand    = {n_init .. cur-n_local}     (complete, causal, not init/local)
 *   s_j     = F . kc[j]   (fp32)
 *   B_topk  = the min(topk, |cand|) best j by (s_j descending, j ascending)
 * idx_out lists B_init | B_local | B_topk in ascending order, padded with -1
 * up to U = topk + n_init + n_local; cnt_out holds the list length.
 *
 * Decode (n_q_tokens == 0): f is the fp32 Forecast [B, n_kv_heads, head_dim]
 *   (f_dtype must be BSKV_F32); the query is the last cached token, so
 *   cur = (seq_len[b]-1)/block; an empty sequence (seq_len[b] 0) lists no
 *   block (cnt 0).  idx_out [B, Hkv, U], cnt_out [B, Hkv].
 *   scores_out (nullable) [B, Hkv, kc_nb_cap]: s_j for candidates, -inf
 *   elsewhere up to cur; rows beyond cur untouched.
 * Prefill (n_q_tokens > 0): f holds one Forecast per token
 *   [B, Hkv, n_q_tokens, head_dim] (f_dtype F32 or BF16) for the chunk
 *   starting at position q_start (a multiple of block).  Each query block
 *   qi (tokens qi*block ..) is one selection problem with cur = q_start/block
 *   + qi and s_j = sum over its tokens t of F_t . kc[j] (computed as
 *   (sum_t F_t) . kc[j]).  seq_len is ignored.  idx_out [B, Hkv, n_qb, U],
 *   cnt_out [B, Hkv, n_qb], n_qb = ceil(n_q_tokens/block); scores_out must
 *   be NULL.
 * kc must hold compressed keys for every candidate block; kc_nb_cap is
 * limited to 12288 blocks (a 786432-token context).
 * ws: bskv_score_topk_workspace() bytes, no initialisation needed (decode:
 * candidate scores; prefill: each query block's summed Forecast and its
 * score row).
 * Decode runs two launches: candidate scores in slices, then one top-k
 * workgroup per (b, g).  Prefill runs three: the Forecast sum of each query
 * block; the scores of all query blocks of the chunk against the causal
 * compressed keys as one fp32 MFMA contraction per (b, g); one top-k
 * workgroup per query block.
 * ----------------------------------------------------------------------- */
size_t bskv_score_topk_workspace(int B, int n_kv_heads, int n_q_tokens, int64_t kc_nb_cap, int head_dim);
int bskv_forecast_block_score_topk(const void* f, int f_dtype, int n_q_tokens, int64_t q_start,
                                   const float* kc, int64_t kc_nb_cap, const int64_t* seq_len, int B,
                                   int n_kv_heads, int head_dim, int block, int topk, int n_init,
                                   int n_local, int32_t* idx_out, int32_t* cnt_out, float* scores_out,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * Overlapping key compression and Forecast selection on it: the variant the
 * evaluated models run.
 * "SparDA: a fourth projection that lets sparse attention prefetch its own
 * KV cache" -- "One Forecast head per GQA group", closing paragraph (keys
 * pooled with a 32-token window at stride 16, blocks of 64) and "Training"
 * (window scores max-pooled to blocks in a final step).
 *
 * bskv_kv_window_meanpool: kcw[b, g, w, :] = mean of the keys at positions
 *   stride*w .. stride*w + window - 1, for the complete windows w (those with
 *   stride*w + window <= min(seq_len[b], kv_len)) in [w_begin, w_end); with
 *   newest_only != 0, only the window the newest token completed, if any.
 *   k as for bskv_kv_block_meanpool; kcw [B, n_kv_heads, kcw_nw_cap,
 *   head_dim] fp32; other rows untouched.
 * bskv_forecast_window_score_topk: bskv_forecast_block_score_topk (same
 *   arguments, candidates, ties, union, layouts and limits) with the score of
 *   candidate block j = the maximum of F . kcw[w] over the windows w that
 *   share a token with block j (w = 4j-1 .. 4j+3 on the 32/16 grid) and are
 *   visible to the query:
 *   decode (n_q_tokens == 0): the complete windows of the sequence; f fp32
 *     [B, n_kv_heads, head_dim]; scores_out (nullable) [B, n_kv_heads, nb]
 *     receives the candidates' block scores, other entries untouched;
 *   prefill (n_q_tokens > 0): F = the sum of the query block's Forecast
 *     vectors (f [B, n_kv_heads, n_q_tokens, head_dim], F32 or BF16), and
 *     only windows whose tokens all precede the query block take part;
 *     scores_out must be NULL; seq_len is ignored.
 *   The block capacity is nb = ((kcw_nw_cap-1)*stride + window)/64 (at most
 *   12288).  ws: bskv_window_score_topk_workspace() bytes (window scores in
 *   decode, none in prefill), no initialisation needed.  Decode runs two
 *   launches (window scores in slices, then one max-pool + top-k workgroup
 *   per (b, g)); prefill one workgroup per query block.
 * Both: (window, stride) with window 32 or 64, stride 16, 32 or 64 dividing
 * window; block 64; head_dim 64 or 128.  Errors as everywhere.
 * ----------------------------------------------------------------------- */
int bskv_kv_window_meanpool(const void* k, int dtype, const int64_t* kv_strides, int64_t kv_len, int B,
                            int n_kv_heads, int head_dim, int window, int stride, const int64_t* seq_len,
                            int64_t w_begin, int64_t w_end, int newest_only, float* kcw, int64_t kcw_nw_cap,
                            hipStream_t stream);
size_t bskv_window_score_topk_workspace(int B, int n_kv_heads, int n_q_tokens, int64_t kcw_nw_cap);
int bskv_forecast_window_score_topk(const void* f, int f_dtype, int n_q_tokens, int64_t q_start, const float* kcw,
                                    int64_t kcw_nw_cap, const int64_t* seq_len, int B, int n_kv_heads, int head_dim,
                                    int block, int window, int stride, int topk, int n_init, int n_local,
                                    int32_t* idx_out, int32_t* cnt_out, float* scores_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * Baseline multi-head block selector (decode), the comparison point of the
 * Forecast selector.
 * "SparDA: a fourth projection that lets sparse attention prefetch its own
 * KV cache" -- "One Forecast head per GQA group", baseline selector listing
 * (Sec. 3.1): every query head of a KV group scores every candidate block
 * against the compressed keys, the per-head scores are summed, a softmax of
 * the sum times `scale` (normally 1/sqrt(head_dim)) weights the candidates,
 * and the top-k of the weights is united with the initial and local blocks.
 *
 * q        [B, n_q_heads, head_dim], F32 or BF16 (q_dtype): the layer's own
 *          queries; query head h belongs to KV head h / (n_q_heads/n_kv_heads)
 * kc       [B, n_kv_heads, kc_nb_cap, head_dim] fp32 compressed keys
 * seq_len  [B] int64; the query is the last cached token (as in decode above)
 * Candidates, ties, union, padding, idx_out/cnt_out layouts and the 12288
 * block limit are those of bskv_forecast_block_score_topk (decode); the
 * ranking is by softmax weight (descending), then block id (ascending).
 * weights_out (nullable) [B, n_kv_heads, kc_nb_cap] fp32: the softmax weight
 *          of every candidate; other entries untouched.
 * n_q_heads/n_kv_heads must be 1, 2, 4 or 8; head_dim 64 or 128; block 64;
 * n_init >= 1, n_local >= 1, topk >= 0, scale > 0.
 * ws: bskv_multihead_score_topk_workspace() bytes (the shared scores); needs
 * no initialisation.  Two launches: score slices, then one softmax + top-k
 * workgroup per (b, g).  Errors as everywhere (nothing launched on error).
 * ----------------------------------------------------------------------- */
size_t bskv_multihead_score_topk_workspace(int B, int n_kv_heads, int64_t kc_nb_cap);
int bskv_multihead_block_score_topk(const void* q, int q_dtype, const float* kc, int64_t kc_nb_cap,
                                    const int64_t* seq_len, int B, int n_q_heads, int n_kv_heads, int head_dim,
                                    int block, int topk, int n_init, int n_local, float scale, int32_t* idx_out,
                                    int32_t* cnt_out, float* weights_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * a4  Block-sparse decode attention.  [EXPL] "The fourth projection", Eq. 5
 * and Alg. 2: the layer's own query attends to the K/V of its selected
 * blocks only.  For query head h (KV head g = h / (n_q_heads/n_kv_heads)):
 *
 *   out[b, h] = softmax_t(scale * q[b,h] . k_t) v_t
 *
 * over the tokens t of the listed blocks idx[b, g, 0..cnt-1] with position
 * < seq_len[b]; a head with no such token (cnt 0, or seq_len[b] 0) gets the
 * zero vector.  Two launches: splits over the listed blocks (fp32 online
 * softmax), then their merge in split order (deterministic).
 * q      [B, n_q_heads, head_dim] dtype, contiguous
 * k, v   cache (kv_is_ring == 0): block idx[u] is read at token idx[u]*block;
 *        ring  (kv_is_ring != 0): the u-th listed block is read at token
 *        u*block (a buffer filled by bskv_prefetch_selected_blocks).
 * idx    [B, Hkv, U] int32, cnt [B, Hkv] int32 (as written by a3)
 * out    [B, n_q_heads, head_dim] fp32
 * n_q_heads/n_kv_heads must be 1, 2, 4 or 8.  ws: bskv_attn_decode_workspace().
 * ----------------------------------------------------------------------- */
size_t bskv_attn_decode_workspace(int B, int n_q_heads, int n_kv_heads, int head_dim, int U);
int bskv_block_sparse_attn_decode(const void* q, const void* k, const void* v, int dtype,
                                  const int64_t* kv_strides, int64_t kv_len, int kv_is_ring, const int32_t* idx,
                                  const int32_t* cnt, const int64_t* seq_len, int B, int n_q_heads,
                                  int n_kv_heads, int head_dim, int block, int U, float scale,
                                  float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * a4p Block-sparse causal prefill attention (bf16 MFMA, fp32 accumulate).
 * [EXPL] "The fourth projection", Eq. 5 and Alg. 1.  The query token at
 * position p = q_start + t (chunk-relative t) attends to the tokens of its
 * query block's list idx[b, g, t/block, 0..cnt-1] at positions <= p: a
 * listed block before the query block is used whole, the query block itself
 * up to p, and a listed block after it not at all.  A token with no such key
 * (an empty list) gets the zero vector.
 * q      [B, n_q_heads, n_q_tokens, head_dim] bf16, contiguous
 * k, v   cache holding at least q_start + n_q_tokens tokens (bf16)
 * idx    [B, Hkv, n_qb, U] int32, cnt [B, Hkv, n_qb] int32
 * out    [B, n_q_heads, n_q_tokens, head_dim] bf16
 * dtype must be BSKV_BF16; head_dim 128 or 64; q_start multiple of block.
 * ----------------------------------------------------------------------- */
int bskv_block_sparse_attn_prefill(const void* q, const void* k, const void* v, int dtype,
                                   const int64_t* kv_strides, int64_t kv_len, const int32_t* idx, const int32_t* cnt,
                                   int64_t q_start, int n_q_tokens, int B, int n_q_heads, int n_kv_heads,
                                   int head_dim, int block, int U, float scale, void* out,
                                   hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * a5  Lookahead prefetch of the selected blocks.  [EXPL] "The fourth
 * projection", Alg. 2: the next layer's block set is fetched from CPU pinned
 * memory to the GPU on a dedicated prefetch stream while the current layer
 * computes; [OVW] 系统实现: the GPU reads host memory directly and the
 * number of thread blocks is tuned to the batch size.
 *
 *   ring_k[b, g, u] = src_k[b, g, idx[b,g,u]*block .. +block)   u < cnt[b,g]
 *   (same for v); slots u >= cnt are not written.
 *
 * src_k, src_v  device-accessible addresses of one layer's K and V: either
 *               device memory or host-pinned memory mapped for the device
 *               (see bskv_host_device_pointer), strides src_strides
 * ring_k/v      [B, Hkv, U, block, head_dim] contiguous, dtype
 * n_workgroups  number of workgroups of the copy kernel (>= 1): the pages'
 *               batch-dependent thread-block count
 * Ordering with the consumer is the caller's: record an event on `stream`
 * after this call and make the attention stream wait on it; make this
 * stream wait for the last reader of a ring slot before refilling it.
 * ----------------------------------------------------------------------- */
int bskv_prefetch_selected_blocks(const void* src_k, const void* src_v, int dtype,
                                  const int64_t* src_strides, int64_t src_len, const int32_t* idx, const int32_t* cnt,
                                  void* ring_k, void* ring_v, int B, int n_kv_heads, int head_dim,
                                  int block, int U, int n_workgroups, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * The layer's projection widened by the Forecast head group.  "SparDA: a
 * fourth projection that lets sparse attention prefetch its own KV cache"
 * -- "The fourth projection", Eq. 3: (Q, K, V, F) = phi_l(X), phi_l the
 * existing linear projection widened by one small head group.
 *
 * w_t  [N, hidden] bf16 row-major, N = (n_q_heads + 3 n_kv_heads) *
 *      head_dim: row n holds the weights of output column n (the layout a
 *      linear layer stores, out x in); the columns are the query heads, then
 *      the key, value and Forecast heads (head_dim columns per head).  All
 *      inputs and Q/K/V outputs bf16 (rounded to nearest even from fp32
 *      sums); F fp32.
 *
 * bskv_qkvf_proj_decode: one token per sequence, x [B, hidden], B <= 64.
 *   q_out [B, n_q_heads, head_dim]; the token's K and V are written into
 *   the caches (strides kv_strides, as for the attention calls) at position
 *   seq_len[b] - 1 (rows outside [0, kv_len) are not written); f_out
 *   [B, n_kv_heads, head_dim] fp32, ready for the decode selection.  One
 *   launch, no workspace.  hidden a multiple of 1024.
 * bskv_qkvf_proj_prefill: a chunk of n_q_tokens tokens per sequence,
 *   x [B, n_q_tokens, hidden], starting at position q_start (a multiple of
 *   64; q_start + n_q_tokens <= kv_len).  q_out [B, n_q_heads, n_q_tokens,
 *   head_dim]; K and V written into the caches at positions q_start + t;
 *   f_pooled [B, n_kv_heads, ceil(n_q_tokens/64), head_dim] fp32 receives
 *   each 64-token query block's Forecast sum (the last block may be
 *   partial) instead of per-token Forecasts.  hidden a multiple of 64;
 *   n_q_heads * head_dim and n_kv_heads * head_dim multiples of 128.  All
 *   pointers 16-byte aligned.  No workspace.
 * bskv_forecast_block_score_topk_pooled: the prefill selection of
 *   bskv_forecast_block_score_topk from f_pooled (n_qb query blocks starting
 *   at global block q_start/64), same candidates, ties, union and outputs;
 *   ws: bskv_score_topk_pooled_workspace() bytes (score rows).
 * ----------------------------------------------------------------------- */
int bskv_qkvf_proj_decode(const void* x, const void* w_t, int B, int hidden, int n_q_heads, int n_kv_heads,
                          int head_dim, void* q_out, void* k_cache, void* v_cache, const int64_t* kv_strides,
                          int64_t kv_len, const int64_t* seq_len, float* f_out, hipStream_t stream);
int bskv_qkvf_proj_prefill(const void* x, const void* w_t, int B, int n_q_tokens, int hidden, int n_q_heads,
                           int n_kv_heads, int head_dim, int64_t q_start, void* q_out, void* k_cache, void* v_cache,
                           const int64_t* kv_strides, int64_t kv_len, float* f_pooled, hipStream_t stream);
size_t bskv_score_topk_pooled_workspace(int B, int n_kv_heads, int n_qb, int64_t kc_nb_cap, int head_dim);
int bskv_forecast_block_score_topk_pooled(const float* f_pooled, int n_qb, int64_t q_start, const float* kc,
                                          int64_t kc_nb_cap, int B, int n_kv_heads, int head_dim, int block, int topk,
                                          int n_init, int n_local, int32_t* idx_out, int32_t* cnt_out, void* ws,
                                          size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * Resident block cache for offloaded decode.  The pages do not describe
 * one; their offloaded decode throughput at batch 64 and 128K ("SparDA: a
 * fourth projection that lets sparse attention prefetch its own KV cache"
 * -- "Three speedups, three different baselines", Table 4) needs most
 * selected blocks to stay on the GPU between decode steps.  Per (b, g) the
 * cache has n_slots block slots (<= 1024) in
 *   cache_k, cache_v  [B, n_kv_heads, n_slots, block, head_dim] contiguous
 * and a slot table owned by the caller:
 *   tags   int32 [B, n_kv_heads, n_slots]  block id held by the slot, -1 empty
 *   stamps int64 [B, n_kv_heads, n_slots]  last use (lookup * U + list position)
 *   clock  int64 [B, n_kv_heads]           lookups so far
 * bskv_block_cache_reset empties the table (a kernel: safe under graph
 * capture).
 * bskv_block_cache_plan looks one layer's list up (idx [B, Hkv, U]: distinct
 *   ascending block ids, as the selectors write them; cnt [B, Hkv]) and
 *   updates the table, least recently used first: listed blocks already held
 *   keep their slot; the others take, in list order, the unlisted slots in
 *   order of (stamp, slot), empty slots first.  Writes slot_out [B, Hkv, U]
 *   (the slot of each listed block, -1 past cnt), n_fill_out [B, Hkv] (the
 *   number of blocks to copy) and fill_out [B, Hkv, U]: its first n_fill
 *   entries are the list positions u of the blocks to copy (the listed blocks
 *   not held before), ascending; the rest -1.  Requires U <= n_slots.  One
 *   workgroup per (b, g).
 * bskv_prefetch_cache_fill copies those blocks (idx[u], from a layer's K/V
 *   in device or host-mapped memory, as for bskv_prefetch_selected_blocks)
 *   into their slots slot[u].  Workgroup w serves the (b, g) w, w +
 *   n_workgroups, ...; a (b, g) with nothing to copy costs one load.
 * bskv_block_sparse_attn_decode_cached: bskv_block_sparse_attn_decode with
 *   listed block u (logical id idx[u], masked by seq_len) read from cache slot
 *   slot[u]; ws as bskv_attn_decode_workspace().
 * bskv_block_sparse_attn_decode_cached_fill: bskv_block_sparse_attn_decode_cached
 *   of one layer with the copy of another layer's missing blocks
 *   (bskv_prefetch_cache_fill's arguments, prefixed fill_: the source K/V,
 *   that layer's list fill_idx, fill_slot, fill, n_fill from its plan, and
 *   its cache fill_cache_k / fill_cache_v of fill_n_slots slots; same dtype,
 *   B, heads, head_dim, block and U) in the same launch: the first
 *   n_fill_workgroups workgroups copy while the rest attend.  For a
 *   one-layer-ahead schedule on one stream: attention of layer l carries the
 *   copy of layer l+1's blocks, so no second stream and no cross-stream wait
 *   is needed.  The filled cache must not be the one this call reads
 *   (EINVAL for the same pointers; partial overlap is not checked).
 * Ordering is the caller's: plan on the compute stream after the selection,
 * fill on the copy stream after the plan (or inside the previous layer's
 * attention launch), attend after the fill; a layer's plan must follow that
 * layer's previous attention (slots are reused).
 * ----------------------------------------------------------------------- */
int bskv_block_cache_reset(int32_t* tags, int64_t* stamps, int64_t* clock, int B, int n_kv_heads, int n_slots,
                           hipStream_t stream);
int bskv_block_cache_plan(const int32_t* idx, const int32_t* cnt, int B, int n_kv_heads, int U, int32_t* tags,
                          int64_t* stamps, int64_t* clock, int n_slots, int32_t* slot_out, int32_t* fill_out,
                          int32_t* n_fill_out, hipStream_t stream);
int bskv_prefetch_cache_fill(const void* src_k, const void* src_v, int dtype, const int64_t* src_strides,
                             int64_t src_len, const int32_t* idx, const int32_t* slot, const int32_t* fill,
                             const int32_t* n_fill, void* cache_k, void* cache_v, int B, int n_kv_heads, int head_dim,
                             int block, int U, int n_slots, int n_workgroups, hipStream_t stream);
int bskv_block_sparse_attn_decode_cached(const void* q, const void* cache_k, const void* cache_v, int dtype,
                                         int n_slots, const int32_t* slot, const int32_t* idx, const int32_t* cnt,
                                         const int64_t* seq_len, int B, int n_q_heads, int n_kv_heads, int head_dim,
                                         int block, int U, float scale, float* out, void* ws, size_t ws_bytes,
                                         hipStream_t stream);
int bskv_block_sparse_attn_decode_cached_fill(
    const void* q, const void* cache_k, const void* cache_v, int dtype, int n_slots, const int32_t* slot,
    const int32_t* idx, const int32_t* cnt, const int64_t* seq_len, int B, int n_q_heads, int n_kv_heads, int head_dim,
    int block, int U, float scale, float* out, void* ws, size_t ws_bytes, const void* src_k, const void* src_v,
    const int64_t* src_strides, int64_t src_len, const int32_t* fill_idx, const int32_t* fill_slot,
    const int32_t* fill, const int32_t* n_fill, void* fill_cache_k, void* fill_cache_v, int fill_n_slots,
    int n_fill_workgroups, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * One decode layer with one-layer-ahead selection.  [EXPL] "The fourth
 * projection", Alg. 2 and Eq. 4: right after layer l's projection emits the
 * Forecast F_l, it scores layer l+1's compressed keys, which picks layer
 * l+1's blocks, while layer l attends to the blocks picked one layer earlier.
 * Equivalent to this sequence of the calls above, in two kernels:
 *   [scores != NULL] top-k + union of this layer from `scores`
 *                                          -> idx, cnt     (this layer)
 *   kv_block_meanpool(k, newest_only=1)    -> kc           (this layer)
 *   forecast_proj(x, w_forecast)           -> F            (this layer's Forecast)
 *   the next layer's selection from F against kc_next, in one of two forms:
 *     immediate (idx_next, cnt_next given): forecast_block_score_topk(F,
 *       kc_next) -> idx_next, cnt_next; the top-k of each (b, g) runs inside
 *       the second kernel as soon as that (b, g)'s scores are complete
 *     deferred (scores_next given): only the raw scores of the next layer's
 *       candidate blocks, scores_next[b, g, j] = F[b, g] . kc_next[b, g, j]
 *       (the causal blocks that are neither initial nor local, see
 *       bskv_forecast_block_score_topk; other entries are not written); the
 *       next layer's call, given them as `scores`, turns them into its list
 *       in its first kernel, beside its projection
 *   block_sparse_attn_decode(q, k, v, idx, cnt) -> out     (this layer)
 * Both forms give the same lists (same ranking and union as
 * bskv_forecast_block_score_topk).  Pass scores = NULL when idx/cnt already
 * hold this layer's list (layer 0, selected by its own projection, or any
 * layer after an immediate-mode call).
 * Layouts as in those calls: kc, kc_next [B, Hkv, kc_nb_cap, d] fp32 (must
 * not overlap); scores, scores_next [B, Hkv, kc_nb_cap] fp32; idx, idx_next
 * [B, Hkv, U] int32 with U = topk + n_init + n_local, cnt, cnt_next [B, Hkv]
 * int32 (idx/cnt are outputs when scores != NULL, inputs otherwise).  The
 * attention's split partials are merged by the last split of each (b, g) to
 * finish, which then updates kc with the newest block.
 * x, w_forecast, kc_next and one form of the next layer's selection
 * (scores_next, or idx_next with cnt_next) are all given or all NULL (NULL:
 * the last layer, no lookahead); giving both forms is BSKV_EINVAL.  hidden
 * must be a multiple of 256.
 * ws: bskv_decode_layer_lookahead_workspace() with hidden = 0 when x is NULL,
 * zero-filled once before its first use: its first 2 * 65535 int32 words
 * (the same for every shape) are the second kernel's arrival counters, and
 * every complete call leaves them at zero again.  One ws may therefore
 * serve every layer of a model, last layer included, and calls of other
 * shapes (size it for the largest layout, i.e. with the lookahead's
 * hidden); calls that share one ws must not overlap in time.
 * stages: bit 0 = K1 (this layer's top-k when scores is given, projection
 * partials when x is given), bit 1 = K2 (next-layer scores [and top-k], this
 * layer's attention, merge and kc update); 3 runs the whole layer.  K2 reads
 * what K1 left in ws and idx/cnt, so a caller may launch them separately (to
 * place other work between them, or to time each), in order, with the same
 * ws and arguments.  Stages outside 1..3: BSKV_EINVAL.
 * ----------------------------------------------------------------------- */
size_t bskv_decode_layer_lookahead_workspace(int B, int n_q_heads, int n_kv_heads, int head_dim, int hidden,
                                             int64_t kc_nb_cap, int U, int dtype);
int bskv_decode_layer_lookahead(const void* q, const void* k, const void* v, int dtype,
                                const int64_t* kv_strides, int64_t kv_len, const int64_t* seq_len,
                                float* kc, const float* scores, int32_t* idx, int32_t* cnt, float scale,
                                float* out, const void* x, const void* w_forecast, int hidden,
                                const float* kc_next, float* scores_next, int32_t* idx_next,
                                int32_t* cnt_next, int B, int n_q_heads,
                                int n_kv_heads, int head_dim, int block, int64_t kc_nb_cap, int topk,
                                int n_init, int n_local, int stages, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * For callers that cannot allocate device memory -- code under HIP-graph
 * capture, tight serving loops, harnesses that forbid allocation: the fused
 * decode layer with its workspace in a static device array of the library
 * (bskv_decode_layer_lookahead_noalloc_capacity() bytes, 16 MiB, one per
 * GPU, held until the process ends) instead of a caller buffer.  Arguments
 * and results as bskv_decode_layer_lookahead without ws / ws_bytes; the
 * device is the one current on the calling thread (it must be the stream's).
 * Returns BSKV_ENOSPC, before touching the device, when the layer's
 * workspace (bskv_decode_layer_lookahead_workspace) exceeds the array.  The
 * first call on a device looks the array up and clears its arrival counters
 * with a small kernel on `stream`; no call allocates or frees anything.
 * Every call on one device shares that device's array and keeps its last
 * contents (the counters are left at zero): calls that overlap in time on
 * one device race, so they must be ordered (one stream, or events).
 * ----------------------------------------------------------------------- */
size_t bskv_decode_layer_lookahead_noalloc_capacity(void);
int bskv_decode_layer_lookahead_noalloc(const void* q, const void* k, const void* v, int dtype,
                                        const int64_t* kv_strides, int64_t kv_len, const int64_t* seq_len,
                                        float* kc, const float* scores, int32_t* idx, int32_t* cnt, float scale,
                                        float* out, const void* x, const void* w_forecast, int hidden,
                                        const float* kc_next, float* scores_next, int32_t* idx_next,
                                        int32_t* cnt_next, int B, int n_q_heads, int n_kv_heads, int head_dim,
                                        int block, int64_t kc_nb_cap, int topk, int n_init, int n_local,
                                        int stages, hipStream_t stream);

/* Device address of host memory allocated pinned (hipHostMalloc, or a torch
 * tensor created with pin_memory=True).  Returns BSKV_EHIP if the pointer is
 * not pinned host memory known to HIP. */
int bskv_host_device_pointer(void* host_ptr, void** dev_ptr);

#ifdef __cplusplus
}
#endif

#endif /* BSKV_H */
