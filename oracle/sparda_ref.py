"""Plain fp64 CPU oracle for Forecast-driven block-sparse attention.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The HIP library in ``block_sparse_long_kv_amd/`` never
imports it, and it imports nothing from the library: the two share no code.

Everything here is written for clarity, not speed: numpy float64, one loop per
(batch, head) or (batch, head, query block), a library matmul / dot / sort as
the only primitives.  Inputs may be any real numpy dtype (bf16 tensors are
upcast exactly by the caller); every result is float64 or int64.

Sources (web pages describing SparDA, cited below by tag):
  [EXPL] "SparDA: a fourth projection that lets sparse attention prefetch its
         own KV cache" (ai.thesatyajit.com/articles/sparda)
  [OVW]  Chinese-language SparDA overview, deepresearch2agi.pages.dev
         ("sparda_sparse_decoupled_attention"); sections named in Chinese.
  [ABS]  "SparDA: Sparse Decoupled Attention for Efficient Long-Context LLM
         Inference", abstract (chatpaper.ai / stacks.braintank.ai).

Readings taken where the pages leave a step open (each is repeated at the
function that uses it):
  R1  Compressed keys: one plain mean per complete 64-token block; a block that
      is not complete has no compressed key.
  R2  Decode query position: the cache holds seq_len tokens including the
      current one, so the query sits at position seq_len - 1 and its block is
      cur = (seq_len - 1) // block.
  R3  Local window: the n_local whole blocks ending at the query's block.
  R4  Top-k candidates exclude the initial and local blocks and every block
      after the causal cut: cand = { n_init <= j <= cur - n_local }.
  R5  Fewer candidates than k: take them all; the index list is padded with -1
      and the count carries the true size.
  R6  Equal scores: the lower block index ranks first.
  R7  Score: the raw dot product F . K~_j, no 1/sqrt(d), no softmax.
  R8  Prefill: one selection per 64-token query block; its score for block j
      is the sum over the block's tokens of F_t . K~_j.
  R9  Attention scale and GQA map are caller-given: scale (normally
      1/sqrt(d)); query head h reads KV head h // (Hq / Hkv).
  R10 Prefill causality is per token: a query at position p sees keys at
      positions <= p inside its selected blocks.
  R15 Overlapping compression (the variant the evaluated models run): a
      compressed key per window of `window` tokens every `stride` tokens
      (32 and 16), mean-pooled; only complete windows exist.  A block's score
      is the maximum of the scores of the windows that share at least one
      token with it (windows 4j-1 .. 4j+3 of block j at 32/16); with
      window = stride = block it is the plain block mean of R1.
  R16 Overlapping compression in prefill: query block qb scores window w by
      the sum over its tokens of F_t . K~w (R8 applied to windows) and
      max-pools as in R15; a window takes part only if all its tokens precede
      the query block (the decode rule of R15 at the block's first token).
  R17 Resident block cache for offloaded decode (not described on the pages;
      their offloaded decode throughput at batch 64 and 128K, [EXPL] "Three
      speedups, three different baselines" (Table 4), implies that most
      selected blocks are reused from one decode step to the next): per
      (batch, KV head) a cache of S block slots
      with least-recently-used replacement.  A call lists the blocks one
      layer needs: listed blocks already held keep their slot; the others
      take, in list order, the unlisted slots in order of (last use, slot),
      empty slots first; every listed slot is then stamped with
      (call number, list position).
  R18 Widened projection: the columns of the layer's projection matrix are
      the query heads, then the key, value and Forecast heads (head_dim
      columns each); in prefill only each query block's summed Forecast
      leaves the projection (R8).
  R14 Baseline multi-head selector (decode): the G query heads of a KV group
      each score the candidates against the compressed keys, the G score rows
      are summed, the sum times the attention scale goes through a softmax over
      the candidates, and the top-k of the softmax weights (R6 ties) is united
      with the initial and local blocks as in R3-R5.  The pages give the
      selector for one query; prefill is not covered.
Parity status: every function below is pinned by tests/test_oracle_pins.py
(brute force, closed forms, textbook special cases, hand-worked fixtures under
tests/golden/).  None is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# a1: the Forecast projection
# --------------------------------------------------------------------------
def forecast_proj(x, w, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """F[b, g, :] = x[b, :] @ w[:, g*d:(g+1)*d].

    [EXPL] "The fourth projection", Eq. 3: the per-layer projection phi_l
    also emits F_l; [OVW] 架构细节 and [EXPL] "One Forecast head per GQA
    group": one Forecast head per KV head, so w has n_kv_heads * head_dim
    columns and head g owns the g-th run of head_dim columns.
    x: [B, hidden]; w: [hidden, n_kv_heads*head_dim].  Returns [B, Hkv, d].
    """
    x = _f64(x)
    w = _f64(w)
    B, hidden = x.shape
    if w.shape != (hidden, n_kv_heads * head_dim):
        raise ValueError(f"w shape {w.shape} != ({hidden}, {n_kv_heads * head_dim})")
    return np.matmul(x, w).reshape(B, n_kv_heads, head_dim)


def qkvf_proj(x, w, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """The widened per-layer projection of one decode token:
    (Q, K, V, F) = x @ [W_Q | W_K | W_V | W_F].

    [EXPL] "The fourth projection", Eq. 3: the layer's existing linear
    projection, widened by one small head group, emits the Forecast next to
    Q, K and V.  Reading R18: the columns of w are the query heads, then the
    key heads, the value heads and the Forecast heads (n_kv_heads of each
    of the last three), head_dim columns per head.  x: [B, hidden]; w:
    [hidden, (n_q_heads + 3 n_kv_heads) * head_dim].  Returns q [B, Hq, d],
    k, v, f [B, Hkv, d] (float64).
    """
    x = _f64(x)
    w = _f64(w)
    B, hidden = x.shape
    Hq, H, d = n_q_heads, n_kv_heads, head_dim
    if w.shape != (hidden, (Hq + 3 * H) * d):
        raise ValueError(f"w shape {w.shape} != ({hidden}, {(Hq + 3 * H) * d})")
    y = np.matmul(x, w)
    q = y[:, : Hq * d].reshape(B, Hq, d)
    k = y[:, Hq * d: (Hq + H) * d].reshape(B, H, d)
    v = y[:, (Hq + H) * d: (Hq + 2 * H) * d].reshape(B, H, d)
    f = y[:, (Hq + 2 * H) * d:].reshape(B, H, d)
    return q, k, v, f


def qkvf_proj_prefill(x, w, n_q_heads: int, n_kv_heads: int, head_dim: int, block: int):
    """The widened projection of a prefill chunk, with the Forecast summed
    per query block instead of kept per token.

    [EXPL] "The fourth projection", Eq. 3 and Alg. 1; reading R8: a query
    block's selection uses the sum of its tokens' Forecast vectors, so only
    that sum leaves the projection.  x: [B, Tq, hidden].  Returns q
    [B, Hq, Tq, d], k, v [B, Hkv, Tq, d] and f_pooled [B, Hkv, ceil(Tq /
    block), d] (the last query block may be partial).
    """
    x = _f64(x)
    B, Tq, hidden = x.shape
    Hq, H, d = n_q_heads, n_kv_heads, head_dim
    q = np.zeros((B, Hq, Tq, d))
    k = np.zeros((B, H, Tq, d))
    v = np.zeros((B, H, Tq, d))
    n_qb = -(-Tq // block)
    f_pooled = np.zeros((B, H, n_qb, d))
    for t in range(Tq):
        qt, kt, vt, ft = qkvf_proj(x[:, t], w, Hq, H, d)
        q[:, :, t], k[:, :, t], v[:, :, t] = qt, kt, vt
        f_pooled[:, :, t // block] += ft
    return q, k, v, f_pooled


# --------------------------------------------------------------------------
# a2: block mean-pooling into compressed keys
# --------------------------------------------------------------------------
def kv_block_meanpool(k, block: int, seq_len=None) -> np.ndarray:
    """K~[b, g, j, :] = mean of the keys at positions block*j .. block*j+block-1.

    [EXPL] "The problem InfLLM-V2 leaves on the table": keys are mean-pooled
    into compressed representations; [OVW] 架构细节 (block selection uses the
    mean-compressed keys of the layer); [EXPL] "The fourth projection",
    Alg. 2 keeps them in a per-layer cache updated incrementally.
    Reading R1: only complete blocks get a compressed key.
    k: [B, Hkv, T, d]; seq_len: optional [B] valid token counts (default T).
    Returns [B, Hkv, T // block, d]; rows of blocks that are not complete for
    batch b are NaN so that any use of them shows.
    """
    k = _f64(k)
    B, H, T, d = k.shape
    nb = T // block
    lens = np.full(B, T, dtype=np.int64) if seq_len is None else np.asarray(seq_len, dtype=np.int64)
    out = np.full((B, H, nb, d), np.nan)
    for b in range(B):
        n_complete = min(int(lens[b]), T) // block
        for g in range(H):
            for j in range(n_complete):
                out[b, g, j] = k[b, g, block * j: block * (j + 1)].mean(axis=0)
    return out


def kv_window_meanpool(k, window: int, stride: int, seq_len=None) -> np.ndarray:
    """K~w[b, g, w, :] = mean of the keys at positions stride*w .. stride*w +
    window - 1, for every complete window.

    [EXPL] "One Forecast head per GQA group", closing paragraph: the
    evaluated models pool keys with a 32-token window at stride 16; reading
    R15.  k: [B, Hkv, T, d]; seq_len: optional [B].  Returns
    [B, Hkv, (T - window) // stride + 1, d]; windows that are not complete
    for batch b are NaN.
    """
    k = _f64(k)
    B, H, T, d = k.shape
    nw = (T - window) // stride + 1 if T >= window else 0
    lens = np.full(B, T, dtype=np.int64) if seq_len is None else np.asarray(seq_len, dtype=np.int64)
    out = np.full((B, H, nw, d), np.nan)
    for b in range(B):
        L = min(int(lens[b]), T)
        for g in range(H):
            for w in range(nw):
                if stride * w + window <= L:
                    out[b, g, w] = k[b, g, stride * w: stride * w + window].mean(axis=0)
    return out


def window_block_scores(f_vec, kcw_bg, blocks, block: int, window: int, stride: int) -> dict:
    """Block score = max over the windows sharing a token with the block of
    f . K~w (reading R15).  kcw_bg: [NW, d] (NaN rows are incomplete windows,
    which take no part); blocks: candidate block ids."""
    nw = kcw_bg.shape[0]
    lo = stride * np.arange(nw)                              # window w holds tokens [lo, lo + window)
    hi = lo + window
    done = ~np.isnan(kcw_bg[:, 0])
    s = np.full(nw, -np.inf)
    s[done] = kcw_bg[done] @ np.asarray(f_vec, dtype=np.float64)
    out = {}
    for j in blocks:
        touch = (hi > block * j) & (lo < block * (j + 1)) & done
        out[j] = float(s[touch].max()) if touch.any() else -np.inf
    return out


def decode_select_windows(f, kcw, seq_len, topk: int, n_init: int, n_local: int, block: int, window: int,
                          stride: int) -> Selection:
    """decode_select with the overlapping compression of R15: candidates,
    ties and union as in decode_select, block scores max-pooled from the
    window scores.  f: [B, Hkv, d]; kcw: [B, Hkv, NW, d]."""
    f = _f64(f)
    kcw = _f64(kcw)
    B, H, d = f.shape
    lens = np.asarray(seq_len, dtype=np.int64)
    cap = topk + n_init + n_local
    idx = np.full((B, H, cap), -1, dtype=np.int64)
    cnt = np.zeros((B, H), dtype=np.int64)
    tops, all_scores = [], []
    for b in range(B):
        cur = (int(lens[b]) - 1) // block
        init, local, cand = block_sets(cur, n_init, n_local)
        for g in range(H):
            scores = window_block_scores(f[b, g], kcw[b, g], cand, block, window, stride)
            top = rank_topk(scores, topk)
            idx[b, g], cnt[b, g] = _union(init, local, top, cap)
            tops.append(top)
            all_scores.append(scores)
    return Selection(idx, cnt, tops, all_scores)


# --------------------------------------------------------------------------
# a3: scoring, causal top-k, union with the initial and local blocks
# --------------------------------------------------------------------------
@dataclass
class Selection:
    """Block sets for one selection call.

    idx   int64 [..., U]  ascending block ids of B_init | B_local | B_topk,
                          padded with -1 (U = topk + n_init + n_local)
    cnt   int64 [...]     number of valid entries in idx
    top   list            per problem, the top-k block ids in rank order
    scores list           per problem, dict block id -> fp64 score (candidates only)
    """
    idx: np.ndarray
    cnt: np.ndarray
    top: list
    scores: list


def block_sets(cur: int, n_init: int, n_local: int):
    """Initial, local and candidate block ids for a query whose block is cur.

    [EXPL] "The problem InfLLM-V2 leaves on the table", block-set formula
    B_l(i) = B_init | B_local(i) | B_topk(i).  Readings R3 and R4: the local
    window is the n_local blocks ending at cur; the top-k candidates are the
    causal blocks that are neither initial nor local ([EXPL] "Training",
    the Eq. 7 selection is taken after the causal mask and without the
    initial/local blocks).
    """
    init = [j for j in range(n_init) if j <= cur]
    local = list(range(max(0, cur - n_local + 1), cur + 1))
    cand = list(range(n_init, cur - n_local + 1))
    return init, local, cand


def rank_topk(scores: dict, k: int) -> list:
    """f_top(s, k): the k best candidates by (score descending, id ascending).

    [EXPL] "The fourth projection", Eq. 4 (f_top) and "One Forecast head per
    GQA group" (Sec. 4.1 selector: a ranking of the raw scores).  Reading R6
    breaks ties toward the lower block id; R5 takes all when fewer than k.
    """
    order = sorted(scores.keys(), key=lambda j: (-scores[j], j))
    return order[:k]


def _union(init, local, top, cap: int) -> np.ndarray:
    u = sorted(set(init) | set(local) | set(top))
    row = np.full(cap, -1, dtype=np.int64)
    row[: len(u)] = u
    return row, len(u)


def decode_select(f, kc, seq_len, topk: int, n_init: int, n_local: int, block: int) -> Selection:
    """Block set of one decode step for every (batch, KV head).

    [EXPL] "The fourth projection", Eq. 4 and Alg. 2:
    B = B_init | B_local | f_top(F . K~^T, k), with F the Forecast that
    selects this layer (the previous layer's, or the separate layer-0
    projection, [EXPL] "Training").  Scores are raw dot products (R7,
    [EXPL] "One Forecast head per GQA group", Sec. 4.1).  Query position by
    R2.  f: [B, Hkv, d]; kc: [B, Hkv, NB, d]; seq_len: [B].
    """
    f = _f64(f)
    kc = _f64(kc)
    B, H, d = f.shape
    lens = np.asarray(seq_len, dtype=np.int64)
    cap = topk + n_init + n_local
    idx = np.full((B, H, cap), -1, dtype=np.int64)
    cnt = np.zeros((B, H), dtype=np.int64)
    tops, all_scores = [], []
    for b in range(B):
        cur = (int(lens[b]) - 1) // block
        init, local, cand = block_sets(cur, n_init, n_local)
        for g in range(H):
            scores = {j: float(np.dot(f[b, g], kc[b, g, j])) for j in cand}
            top = rank_topk(scores, topk)
            idx[b, g], cnt[b, g] = _union(init, local, top, cap)
            tops.append(top)
            all_scores.append(scores)
    return Selection(idx, cnt, tops, all_scores)


def multihead_select_decode(q, kc, seq_len, topk: int, n_init: int, n_local: int, block: int,
                            scale: float) -> Selection:
    """Baseline selector of the InfLLM-V2 / NSA / MoBA shape, one decode step.

    [EXPL] "One Forecast head per GQA group", the baseline selector listing
    (Sec. 3.1): every query head of the group scores every candidate block,
    the per-head scores are summed into a shared score, a softmax of the
    shared score divided by sqrt(d) weights the candidates, and the top-k of
    those weights is taken.  Reading R14 (scale given, normally 1/sqrt(d));
    candidate and union rules as decode_select.  q: [B, Hq, d] (the layer's
    own queries, query head h in group h // (Hq / Hkv)); kc: [B, Hkv, NB, d].
    Selection.scores holds the softmax weights.
    """
    q = _f64(q)
    kc = _f64(kc)
    B, Hq, d = q.shape
    H = kc.shape[1]
    G = Hq // H
    lens = np.asarray(seq_len, dtype=np.int64)
    cap = topk + n_init + n_local
    idx = np.full((B, H, cap), -1, dtype=np.int64)
    cnt = np.zeros((B, H), dtype=np.int64)
    tops, all_w = [], []
    for b in range(B):
        cur = (int(lens[b]) - 1) // block
        init, local, cand = block_sets(cur, n_init, n_local)
        for g in range(H):
            shared = {j: 0.0 for j in cand}
            for h in range(g * G, (g + 1) * G):          # G score rows, summed
                for j in cand:
                    shared[j] += float(np.dot(q[b, h], kc[b, g, j]))
            w = {}
            if cand:
                z = np.array([shared[j] * scale for j in cand])
                e = np.exp(z - z.max())
                e /= e.sum()
                w = {j: float(e[i]) for i, j in enumerate(cand)}
            top = rank_topk(w, topk)
            idx[b, g], cnt[b, g] = _union(init, local, top, cap)
            tops.append(top)
            all_w.append(w)
    return Selection(idx, cnt, tops, all_w)


def prefill_select(f_tok, kc, q_start: int, topk: int, n_init: int, n_local: int, block: int) -> Selection:
    """Block sets of a prefill chunk, one per 64-token query block.

    [EXPL] "The fourth projection", Alg. 1: top_k(F_prev @ K_compressed.T, k)
    unioned with the initial and local blocks.  Reading R8: the tokens of a
    query block share one selection and its score for block j is the sum of
    their raw scores F_t . K~_j.  The chunk starts at position q_start (a
    multiple of block); its query block qi is the global block
    q_start // block + qi.  f_tok: [B, Hkv, Tq, d]; kc: [B, Hkv, NB, d].
    Returns idx [B, Hkv, n_qb, U], cnt [B, Hkv, n_qb].
    """
    f_tok = _f64(f_tok)
    kc = _f64(kc)
    B, H, Tq, d = f_tok.shape
    if q_start % block:
        raise ValueError("q_start must be a multiple of block")
    n_qb = -(-Tq // block)
    cap = topk + n_init + n_local
    idx = np.full((B, H, n_qb, cap), -1, dtype=np.int64)
    cnt = np.zeros((B, H, n_qb), dtype=np.int64)
    tops, all_scores = [], []
    for b in range(B):
        for g in range(H):
            for qi in range(n_qb):
                qb = q_start // block + qi
                init, local, cand = block_sets(qb, n_init, n_local)
                rows = f_tok[b, g, qi * block: min(Tq, (qi + 1) * block)]
                scores = {}
                for j in cand:
                    per_token = rows @ kc[b, g, j]          # F_t . K~_j for each token t
                    scores[j] = float(per_token.sum())
                top = rank_topk(scores, topk)
                idx[b, g, qi], cnt[b, g, qi] = _union(init, local, top, cap)
                tops.append(top)
                all_scores.append(scores)
    return Selection(idx, cnt, tops, all_scores)


def prefill_select_windows(f_tok, kcw, q_start: int, topk: int, n_init: int, n_local: int, block: int, window: int,
                           stride: int) -> Selection:
    """prefill_select with the overlapping compression (reading R16).

    [EXPL] "One Forecast head per GQA group", closing paragraph (32-token
    windows at stride 16) and "Training" (window scores max-pooled to
    blocks).  Query block qb scores window w by the sum over its tokens of
    F_t . K~w; block j takes the maximum over the windows that share a token
    with it and whose tokens all precede the query block (start of window
    w + window <= qb * block).  Candidates, ties and union as prefill_select.
    f_tok: [B, Hkv, Tq, d]; kcw: [B, Hkv, NW, d] (NaN rows: incomplete).
    """
    f_tok = _f64(f_tok)
    kcw = _f64(kcw)
    B, H, Tq, d = f_tok.shape
    if q_start % block:
        raise ValueError("q_start must be a multiple of block")
    n_qb = -(-Tq // block)
    nw = kcw.shape[2]
    w_start = stride * np.arange(nw)                        # window w holds tokens [w_start, w_start + window)
    cap = topk + n_init + n_local
    idx = np.full((B, H, n_qb, cap), -1, dtype=np.int64)
    cnt = np.zeros((B, H, n_qb), dtype=np.int64)
    tops, all_scores = [], []
    for b in range(B):
        for g in range(H):
            done = ~np.isnan(kcw[b, g, :, 0])
            for qi in range(n_qb):
                qb = q_start // block + qi
                init, local, cand = block_sets(qb, n_init, n_local)
                rows = f_tok[b, g, qi * block: min(Tq, (qi + 1) * block)]
                seen = done & (w_start + window <= qb * block)
                wsc = np.full(nw, -np.inf)
                wsc[seen] = (rows @ kcw[b, g, seen].T).sum(axis=0)     # sum over tokens of F_t . K~w
                scores = {}
                for j in cand:
                    touch = seen & (w_start + window > block * j) & (w_start < block * (j + 1))
                    scores[j] = float(wsc[touch].max()) if touch.any() else -np.inf
                top = rank_topk(scores, topk)
                idx[b, g, qi], cnt[b, g, qi] = _union(init, local, top, cap)
                tops.append(top)
                all_scores.append(scores)
    return Selection(idx, cnt, tops, all_scores)


def prefill_select_pooled(f_pooled, kc, q_start: int, topk: int, n_init: int, n_local: int, block: int) -> Selection:
    """prefill_select from the summed Forecast of each query block.

    Reading R8: query block qi scores block j by F_pooled[qi] . K~_j, with
    F_pooled[qi] the sum of its tokens' Forecast vectors (as the widened
    projection delivers it).  f_pooled: [B, Hkv, n_qb, d]; kc:
    [B, Hkv, NB, d]; the chunk starts at q_start (a multiple of block).
    """
    f_pooled = _f64(f_pooled)
    kc = _f64(kc)
    B, H, n_qb, d = f_pooled.shape
    if q_start % block:
        raise ValueError("q_start must be a multiple of block")
    cap = topk + n_init + n_local
    idx = np.full((B, H, n_qb, cap), -1, dtype=np.int64)
    cnt = np.zeros((B, H, n_qb), dtype=np.int64)
    tops, all_scores = [], []
    for b in range(B):
        for g in range(H):
            for qi in range(n_qb):
                qb = q_start // block + qi
                init, local, cand = block_sets(qb, n_init, n_local)
                scores = {j: float(np.dot(f_pooled[b, g, qi], kc[b, g, j])) for j in cand}
                top = rank_topk(scores, topk)
                idx[b, g, qi], cnt[b, g, qi] = _union(init, local, top, cap)
                tops.append(top)
                all_scores.append(scores)
    return Selection(idx, cnt, tops, all_scores)


# --------------------------------------------------------------------------
# a4: attention over the selected blocks only
# --------------------------------------------------------------------------
def _softmax_attend(qrow, keys, vals, scale):
    # Reading R19: a query with no token to attend to (an empty block list,
    # or every listed token masked) gets the zero vector, the empty sum.
    if keys.shape[0] == 0:
        return np.zeros(vals.shape[-1])
    logits = (keys @ qrow) * scale
    w = np.exp(logits - logits.max())
    w /= w.sum()
    return w @ vals


def _block_tokens(blocks, block: int) -> np.ndarray:
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(block * j, block * (j + 1)) for j in blocks])


def attend_decode(q, k, v, idx, cnt, seq_len, scale: float, block: int) -> np.ndarray:
    """O = softmax(q . K[B]^T * scale) V[B] over the tokens of the block set.

    [EXPL] "The fourth projection", Eq. 5 and Alg. 2: the layer's own query
    attends to K/V of its selected blocks only.  Tokens at positions
    >= seq_len (unwritten cache) are excluded.  GQA map and scale by R9.
    q: [B, Hq, d]; k, v: [B, Hkv, T, d]; idx: [B, Hkv, U]; cnt: [B, Hkv].
    Returns [B, Hq, d].
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    lens = np.asarray(seq_len, dtype=np.int64)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            toks = _block_tokens(np.asarray(idx[b, g][: int(cnt[b, g])]), block)
            toks = toks[toks < lens[b]]
            out[b, h] = _softmax_attend(q[b, h], k[b, g, toks], v[b, g, toks], scale)
    return out


def attend_prefill(q, k, v, idx, cnt, q_start: int, scale: float, block: int, rows=None) -> np.ndarray:
    """Block-sparse causal attention for a prefill chunk.

    [EXPL] "The fourth projection", Eq. 5 and Alg. 1; causality per token
    (R10): the query at position p = q_start + t attends to the tokens of
    its query block's selected blocks at positions <= p.
    q: [B, Hq, Tq, d]; k, v: [B, Hkv, T, d] holding at least q_start + Tq
    tokens; idx: [B, Hkv, n_qb, U]; cnt: [B, Hkv, n_qb].
    rows: optional iterable of (b, h, t) to evaluate; the others stay 0.
    Returns [B, Hq, Tq, d].
    """
    q = _f64(q)
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, d))
    todo = rows if rows is not None else [(b, h, t) for b in range(B) for h in range(Hq) for t in range(Tq)]
    for b, h, t in todo:
        g = h // G
        qi = t // block
        pos = q_start + t
        toks = _block_tokens(np.asarray(idx[b, g, qi][: int(cnt[b, g, qi])]), block)
        toks = toks[toks <= pos]
        kk = _f64(k[b, g, toks])
        vv = _f64(v[b, g, toks])
        out[b, h, t] = _softmax_attend(q[b, h, t], kk, vv, scale)
    return out


# --------------------------------------------------------------------------
# a5: lookahead prefetch of the selected blocks
# --------------------------------------------------------------------------
def gather_selected_blocks(kv, idx, cnt, block: int) -> np.ndarray:
    """Copy of the selected blocks of one layer, in index-list order.

    [EXPL] "The fourth projection", Alg. 2 (fetch of the next layer's block
    set from CPU pinned memory into GPU memory on a prefetch stream) and
    [OVW] 系统实现 (the blocks a layer needs are in GPU memory when it starts).
    The prefetch is a pure copy: slot u of (b, g) holds block idx[b, g, u].
    kv: [B, Hkv, T, d] of any dtype; idx: [B, Hkv, U]; cnt: [B, Hkv].
    Returns [B, Hkv, U, block, d] of kv's dtype; slots u >= cnt are zero.
    """
    kv = np.asarray(kv)
    B, H, T, d = kv.shape
    U = idx.shape[-1]
    ring = np.zeros((B, H, U, block, d), dtype=kv.dtype)
    for b in range(B):
        for g in range(H):
            for u in range(int(cnt[b, g])):
                j = int(idx[b, g, u])
                ring[b, g, u] = kv[b, g, block * j: block * (j + 1)]
    return ring


def block_cache_plan(tags, stamps, clock, idx, cnt):
    """One lookup of a resident block cache (reading R17), updating the
    cache state in place.

    tags   int [B, Hkv, S]   block id held by each slot, -1 when empty
    stamps int [B, Hkv, S]   last use of each slot as call * U + list position,
                             -1 when never used
    clock  int [B, Hkv]      calls made so far
    idx    int [B, Hkv, U]   the blocks one layer needs (ascending, -1 padded)
    cnt    int [B, Hkv]      valid entries of idx
    Returns (slot [B, Hkv, U], fill [B, Hkv, U], n_fill [B, Hkv]): slot[u]
    is the slot that holds idx[u] after the call (-1 for u >= cnt); the
    listed blocks that were not held have to be copied into their slots:
    there are n_fill of them, and fill[:n_fill] lists their positions u in
    the list, ascending (-1 after).  Needs cnt <= S.
    """
    B, H, U = idx.shape
    S = tags.shape[-1]
    slot = np.full((B, H, U), -1, dtype=np.int64)
    fill = np.full((B, H, U), -1, dtype=np.int64)
    n_fill = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for g in range(H):
            c = int(cnt[b, g])
            if c > S:
                raise ValueError("more listed blocks than cache slots")
            listed = [int(j) for j in idx[b, g, :c]]
            held = {int(tags[b, g, s]): s for s in range(S) if tags[b, g, s] >= 0}
            kept = set()
            for u, j in enumerate(listed):           # listed blocks already held keep their slot
                if j in held:
                    slot[b, g, u] = held[j]
                    kept.add(held[j])
            free = sorted((int(stamps[b, g, s]), s) for s in range(S) if s not in kept)
            k = 0
            for u, j in enumerate(listed):           # the others take the least recently used slots
                if slot[b, g, u] < 0:
                    s_new = free[k][1]
                    tags[b, g, s_new] = j
                    slot[b, g, u] = s_new
                    fill[b, g, k] = u
                    k += 1
            n_fill[b, g] = k
            clock[b, g] += 1
            for u in range(c):
                stamps[b, g, slot[b, g, u]] = int(clock[b, g]) * U + u
    return slot, fill, n_fill


# --------------------------------------------------------------------------
# The layer-to-layer lookahead of one decode step
# --------------------------------------------------------------------------
def decode_step_lookahead(layers, topk: int, n_init: int, n_local: int, block: int, scale: float):
    """One decode step over L layers with one-layer-ahead selection.

    [EXPL] "The fourth projection", Eq. 4 and Alg. 2; [EXPL] "Training":
    layer 0 is selected by a separate projection because it has no previous
    layer.  Each element of ``layers`` is a dict with
      'x_sel'  [B, hidden]  the hidden state the selecting Forecast reads
                            (layer l-1's input for l >= 1, layer 0's own input
                            for the layer-0 projection)
      'w_sel'  [hidden, Hkv*d] the Forecast weights that select this layer
      'kc'     [B, Hkv, NB, d] this layer's compressed keys
      'q'      [B, Hq, d];  'k', 'v' [B, Hkv, T, d];  'seq_len' [B]
    Returns the list of (Selection, output) per layer.
    """
    results = []
    for lay in layers:
        Hkv, d = lay["kc"].shape[1], lay["kc"].shape[3]
        f = forecast_proj(lay["x_sel"], lay["w_sel"], Hkv, d)
        sel = decode_select(f, lay["kc"], lay["seq_len"], topk, n_init, n_local, block)
        out = attend_decode(lay["q"], lay["k"], lay["v"], sel.idx, sel.cnt, lay["seq_len"], scale, block)
        results.append((sel, out))
    return results


def kth_gap(scores: dict, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th best candidate scores.

    (s_k - s_{k+1}) / max(|s_k|, |s_{k+1}|); +inf when there is no (k+1)-th
    candidate (the selection is then forced).  Used by the parity checker to
    decide where selected ids must match exactly.
    """
    vals = sorted(scores.values(), reverse=True)
    if len(vals) <= k or k == 0:
        return float("inf")
    a, b = vals[k - 1], vals[k]
    den = max(abs(a), abs(b))
    if den == 0.0:
        return 0.0
    return (a - b) / den
