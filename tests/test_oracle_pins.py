"""Pins of the fp64 oracle against things other than itself.

Every oracle function is checked here against at least one of: a hand-worked
fixture (tests/golden/), a closed form, a brute force over all subsets or all
tokens, or a textbook library routine it reduces to (torch's scaled dot-product
attention in float64).  The cases are chosen so that a dropped term, a wrong
sign, an off-by-one block index, a transposed operand or a wrong GQA map in the
oracle fails at least one test.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
from workloads import WORKLOADS, decode_inputs, random_decode_case


def _np(t):
    return t.detach().to(torch.float64).cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as fh:
        return json.load(fh)


# --------------------------------------------------------------------------- a1
def test_forecast_proj_triple_loop():
    rng = np.random.default_rng(0)
    B, hidden, H, d = 3, 7, 2, 4
    x = rng.integers(-5, 6, size=(B, hidden)).astype(np.float64)
    w = rng.integers(-5, 6, size=(hidden, H * d)).astype(np.float64)
    f = orc.forecast_proj(x, w, H, d)
    for b in range(B):
        for g in range(H):
            for c in range(d):
                acc = 0.0
                for r in range(hidden):
                    acc += x[b, r] * w[r, g * d + c]
                assert f[b, g, c] == acc


def test_forecast_proj_head_columns():
    # W = identity: head g must read columns g*d .. g*d+d-1, i.e. x[b, g*d:(g+1)*d].
    B, H, d = 2, 3, 4
    x = np.arange(B * H * d, dtype=np.float64).reshape(B, H * d)
    f = orc.forecast_proj(x, np.eye(H * d), H, d)
    for b in range(B):
        for g in range(H):
            assert np.array_equal(f[b, g], x[b, g * d:(g + 1) * d])


# --------------------------------------------------------------------------- a2
def test_meanpool_closed_form_and_partial_blocks():
    B, H, T, d, blk = 2, 2, 40, 3, 8
    t = np.arange(T, dtype=np.float64)
    k = np.broadcast_to(t[None, None, :, None] * np.array([1.0, -2.0, 0.5]), (B, H, T, d)).copy()
    k[1, 1] += 3.0
    kc = orc.kv_block_meanpool(k, blk, seq_len=[40, 29])
    for j in range(5):
        mid = blk * j + (blk - 1) / 2.0           # mean of positions 8j .. 8j+7
        np.testing.assert_allclose(kc[0, 0, j], mid * np.array([1.0, -2.0, 0.5]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(kc[0, 1, j], mid * np.array([1.0, -2.0, 0.5]), rtol=0, atol=1e-12)
    for j in range(3):
        expect = (blk * j + 3.5) * np.array([1.0, -2.0, 0.5]) + 3.0
        np.testing.assert_allclose(kc[1, 1, j], expect, rtol=0, atol=1e-12)
    # seq_len 29 -> blocks 0..2 complete (24 tokens), block 3 (24..31) is not: no compressed key
    assert np.isnan(kc[1, :, 3:]).all()
    assert not np.isnan(kc[1, :, :3]).any()


def test_meanpool_linearity_with_scores():
    # F . K~_j equals the mean over the block's tokens of F . K_t (the scores of a pooled key)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, 1, 64 * 3, 5))
    f = rng.standard_normal(5)
    kc = orc.kv_block_meanpool(k, 64)
    for j in range(3):
        per_tok = [sum(f[c] * k[0, 0, 64 * j + r, c] for c in range(5)) for r in range(64)]
        assert abs(float(f @ kc[0, 0, j]) - sum(per_tok) / 64.0) < 1e-12


# --------------------------------------------------------------------------- a3 decode
def test_golden_decode_select_and_attend(golden_dir):
    gx = _load(golden_dir, "decode_select_attend_hand.json")
    blk, d, T = gx["block"], gx["d"], gx["T"]
    keys = np.array(gx["keys"], dtype=np.float64).reshape(1, 1, T, d)
    kc = orc.kv_block_meanpool(keys, blk, seq_len=[gx["seq_len"]])
    np.testing.assert_array_equal(kc[0, 0, :6], np.array(gx["kc_expected"], dtype=np.float64))
    f = np.array(gx["f"], dtype=np.float64).reshape(1, 1, d)
    sel = orc.decode_select(f, kc, [gx["seq_len"]], gx["topk"], gx["n_init"], gx["n_local"], blk)
    assert {str(j): s for j, s in sel.scores[0].items()} == gx["scores_expected"]
    assert sel.top[0] == gx["top_expected"]
    assert sel.idx[0, 0].tolist() == gx["idx_expected"]
    assert int(sel.cnt[0, 0]) == gx["cnt_expected"]
    v = np.zeros((1, 1, T, d))
    v[0, 0, :, 0] = np.arange(T)
    v[0, 0, 26:, 1] = 100.0
    q = np.array(gx["q"], dtype=np.float64).reshape(1, 1, d)
    out = orc.attend_decode(q, keys, v, sel.idx, sel.cnt, [gx["seq_len"]], gx["scale"], blk)
    np.testing.assert_allclose(out[0, 0], gx["out_expected"], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- widened projection (R18)
def test_qkvf_proj_triple_loop():
    """Small integer inputs, every output element from an explicit sum over
    the hidden axis with the column map written out: query heads first, then
    key, value and Forecast heads."""
    rng = np.random.default_rng(1)
    B, hidden, Hq, H, d = 2, 5, 4, 2, 3
    x = rng.integers(-4, 5, size=(B, hidden)).astype(np.float64)
    w = rng.integers(-4, 5, size=(hidden, (Hq + 3 * H) * d)).astype(np.float64)
    q, k, v, f = orc.qkvf_proj(x, w, Hq, H, d)

    def col_sum(b, c):
        return sum(x[b, i] * w[i, c] for i in range(hidden))
    for b in range(B):
        for h in range(Hq):
            for e in range(d):
                assert q[b, h, e] == col_sum(b, h * d + e)
        for g in range(H):
            for e in range(d):
                assert k[b, g, e] == col_sum(b, (Hq + g) * d + e)
                assert v[b, g, e] == col_sum(b, (Hq + H + g) * d + e)
                assert f[b, g, e] == col_sum(b, (Hq + 2 * H + g) * d + e)


def test_qkvf_forecast_part_is_the_forecast_projection():
    rng = np.random.default_rng(2)
    B, hidden, Hq, H, d = 3, 16, 8, 2, 4
    x = rng.standard_normal((B, hidden))
    w = rng.standard_normal((hidden, (Hq + 3 * H) * d))
    f = orc.qkvf_proj(x, w, Hq, H, d)[3]
    np.testing.assert_allclose(f, orc.forecast_proj(x, w[:, (Hq + 2 * H) * d:], H, d), rtol=1e-13, atol=1e-13)


def test_qkvf_prefill_pools_the_forecast_per_query_block():
    """Per-token Q/K/V equal the one-token projection; the pooled Forecast
    equals the plain sum of the tokens' Forecast vectors, block by block,
    with a partial last block."""
    rng = np.random.default_rng(3)
    B, Tq, hidden, Hq, H, d, blk = 2, 11, 6, 2, 1, 3, 4
    x = rng.standard_normal((B, Tq, hidden))
    w = rng.standard_normal((hidden, (Hq + 3 * H) * d))
    q, k, v, fp = orc.qkvf_proj_prefill(x, w, Hq, H, d, blk)
    assert fp.shape == (B, H, 3, d)
    f_tok = np.einsum("bth,hc->btc", x, w[:, (Hq + 2 * H) * d:]).reshape(B, Tq, H, d)
    for t in range(Tq):
        qt, kt, vt, _ = orc.qkvf_proj(x[:, t], w, Hq, H, d)
        np.testing.assert_allclose(q[:, :, t], qt, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(k[:, :, t], kt, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(v[:, :, t], vt, rtol=1e-13, atol=1e-13)
    for qi, (t0, t1) in enumerate([(0, 4), (4, 8), (8, 11)]):
        np.testing.assert_allclose(fp[:, :, qi], f_tok[:, t0:t1].sum(axis=1), rtol=1e-12, atol=1e-12)


def test_golden_prefill_select_pooled(golden_dir):
    """The hand-worked prefill chunk, selected from each query block's summed
    Forecast: the same scores and block sets as per-token scoring (R8)."""
    gx = _load(golden_dir, "prefill_select_attend_hand.json")
    blk, d, Tq = gx["block"], gx["d"], gx["Tq"]
    keys = np.array(gx["keys"], dtype=np.float64).reshape(1, 1, Tq, d)
    f = np.array(gx["f"], dtype=np.float64).reshape(1, 1, Tq // blk, blk, d).sum(axis=3)
    kc = orc.kv_block_meanpool(keys, blk)
    sel = orc.prefill_select_pooled(f, kc, gx["q_start"], gx["topk"], gx["n_init"], gx["n_local"], blk)
    assert {str(j): s for j, s in sel.scores[3].items()} == gx["scores_qb3_expected"]
    assert sel.idx[0, 0].tolist() == gx["idx_expected"]
    assert sel.cnt[0, 0].tolist() == gx["cnt_expected"]


@pytest.mark.parametrize("seed", range(3))
def test_prefill_select_pooled_equals_per_token_selection(seed):
    rng = np.random.default_rng(400 + seed)
    B, H, d, blk, T = 2, 2, 5, 4, 4 * 12
    q_start, Tq = 16, 27
    k = rng.standard_normal((B, H, T, d))
    f = rng.standard_normal((B, H, Tq, d))
    kc = orc.kv_block_meanpool(k, blk)
    n_qb = -(-Tq // blk)
    fp = np.zeros((B, H, n_qb, d))
    for t in range(Tq):
        fp[:, :, t // blk] += f[:, :, t]
    a = orc.prefill_select_pooled(fp, kc, q_start, 3, 1, 2, blk)
    b = orc.prefill_select(f, kc, q_start, 3, 1, 2, blk)
    np.testing.assert_array_equal(a.idx, b.idx)
    np.testing.assert_array_equal(a.cnt, b.cnt)
    for sa, sb in zip(a.scores, b.scores):
        assert sa.keys() == sb.keys()
        for j in sa:
            assert abs(sa[j] - sb[j]) <= 1e-12 * (1 + abs(sb[j]))


# --------------------------------------------------------------------------- overlapping compression (R15)
def test_golden_window_select(golden_dir):
    gx = _load(golden_dir, "window_select_hand.json")
    T = gx["T"]
    k = np.array(gx["keys"], dtype=np.float64).reshape(1, 1, T, 1)
    kcw = orc.kv_window_meanpool(k, gx["window"], gx["stride"], seq_len=[gx["seq_len"]])
    np.testing.assert_array_equal(kcw[0, 0, :, 0], np.array(gx["windows_expected"]))
    f = np.ones((1, 1, 1))
    for case in gx["cases"]:
        sel = orc.decode_select_windows(f, kcw, [gx["seq_len"]], case["topk"], gx["n_init"], gx["n_local"],
                                        gx["block"], gx["window"], gx["stride"])
        assert {str(j): v for j, v in sel.scores[0].items()} == gx["scores_expected"]
        assert sel.top[0] == case["top_expected"]
        assert sel.idx[0, 0].tolist()[: case["cnt_expected"]] == case["idx_expected"]
        assert int(sel.cnt[0, 0]) == case["cnt_expected"]


def test_window_meanpool_against_prefix_sums():
    """Window means from cumulative sums (an independent formula), ragged
    lengths: incomplete windows are NaN."""
    g = torch.Generator().manual_seed(3)
    k = torch.randn(2, 3, 64 * 9, 8, generator=g, dtype=torch.float64).numpy()
    lens = [64 * 9, 64 * 5 + 40]
    kcw = orc.kv_window_meanpool(k, 32, 16, seq_len=lens)
    cs = np.concatenate([np.zeros((2, 3, 1, 8)), np.cumsum(k, axis=2)], axis=2)
    for b, L in enumerate(lens):
        for w in range(kcw.shape[2]):
            if 16 * w + 32 <= L:
                np.testing.assert_allclose(kcw[b, :, w], (cs[b, :, 16 * w + 32] - cs[b, :, 16 * w]) / 32, rtol=1e-12)
            else:
                assert np.isnan(kcw[b, :, w]).all()


@pytest.mark.parametrize("seed", [0, 1])
def test_window_select_with_block_sized_windows_is_block_select(seed):
    """window = stride = block: every block has exactly one window, itself,
    so the variant is the plain block-mean selector (R1)."""
    c = random_decode_case(seed, B=2, Hq=4, Hkv=2, d=16, T=64 * 30, seq_len=[64 * 30, 64 * 21 + 5])
    k, f, lens = _np(c["k"]), _np(c["f"]), _np(c["seq_len"])
    kcw = orc.kv_window_meanpool(k, 64, 64, seq_len=lens)
    kc = orc.kv_block_meanpool(k, 64, seq_len=lens)
    np.testing.assert_array_equal(np.isnan(kcw), np.isnan(kc))
    np.testing.assert_allclose(np.nan_to_num(kcw), np.nan_to_num(kc), rtol=0, atol=1e-13)
    a = orc.decode_select_windows(f, kcw, lens, 6, 1, 2, 64, 64, 64)
    b = orc.decode_select(f, kc, lens, 6, 1, 2, 64)
    np.testing.assert_array_equal(a.idx, b.idx)
    assert a.top == b.top


def test_window_select_spike_reaches_exactly_the_blocks_of_its_windows():
    """A large key at token p enters the windows that contain p; with the
    32/16 grid those windows touch block p // 64 and, for the 16 tokens at
    either edge of a block, also the neighbouring block.  Brute force over
    positions: the blocks whose score jumps are exactly those."""
    T, d = 64 * 12, 4
    base = np.zeros((1, 1, T, d))
    f = np.ones((1, 1, d))
    for p in (64 * 5 + 3, 64 * 5 + 20, 64 * 5 + 50, 64 * 6 + 63, 64 * 3):
        k = base.copy()
        k[0, 0, p] = 100.0
        kcw = orc.kv_window_meanpool(k, 32, 16)
        sc = orc.window_block_scores(f[0, 0], kcw[0, 0], list(range(1, 10)), 64, 32, 16)
        hit = sorted(j for j, v in sc.items() if v > 1.0)
        w_with_p = [w for w in range(kcw.shape[2]) if 16 * w <= p < 16 * w + 32]
        expect = sorted({j for w in w_with_p for j in range(1, 10) if 16 * w < 64 * (j + 1) and 16 * w + 32 > 64 * j})
        assert hit == expect, (p, hit, expect)
        assert p // 64 in hit or p // 64 not in range(1, 10)


# --------------------------------------------------------------------------- overlapping compression in prefill (R16)
def test_golden_prefill_window_select(golden_dir):
    gx = _load(golden_dir, "prefill_window_select_hand.json")
    Tq = gx["Tq"]
    k = np.array(gx["keys"], dtype=np.float64).reshape(1, 1, Tq, 1)
    kcw = orc.kv_window_meanpool(k, gx["window"], gx["stride"])
    f = np.array(gx["f"], dtype=np.float64).reshape(1, 1, Tq, 1)
    for case in gx["cases"]:
        sel = orc.prefill_select_windows(f, kcw, gx["q_start"], case["topk"], gx["n_init"], gx["n_local"],
                                         gx["block"], gx["window"], gx["stride"])
        assert {str(j): v for j, v in sel.scores[2].items()} == gx["scores_qb2_expected"]
        assert {str(j): v for j, v in sel.scores[3].items()} == gx["scores_qb3_expected"]
        for qi, (want, c) in enumerate(zip(case["idx_expected"], case["cnt_expected"])):
            assert int(sel.cnt[0, 0, qi]) == c
            assert sel.idx[0, 0, qi].tolist()[:c] == want


def test_prefill_window_select_block_sized_windows_is_prefill_select():
    """window = stride = block: the windows are the blocks and every complete
    block precedes the query blocks that may select it, so the variant is the
    plain prefill selector (R8)."""
    g = torch.Generator().manual_seed(7)
    k = torch.randn(2, 2, 64 * 12, 8, generator=g, dtype=torch.float64).numpy()
    f = torch.randn(2, 2, 64 * 4 + 17, 8, generator=g, dtype=torch.float64).numpy()
    kc = orc.kv_block_meanpool(k, 64)
    kcw = orc.kv_window_meanpool(k, 64, 64)
    a = orc.prefill_select_windows(f, kcw, 64 * 7, 3, 1, 2, 64, 64, 64)
    b = orc.prefill_select(f, kc, 64 * 7, 3, 1, 2, 64)
    np.testing.assert_array_equal(a.idx, b.idx)
    np.testing.assert_array_equal(a.cnt, b.cnt)
    assert a.top == b.top
    for sa, sb in zip(a.scores, b.scores):
        assert sa.keys() == sb.keys()
        for j in sa:
            assert abs(sa[j] - sb[j]) <= 1e-12 * (1 + abs(sb[j]))


@pytest.mark.parametrize("window,stride,n_local", [(32, 16, 1), (32, 16, 3), (64, 16, 2), (32, 32, 1)])
def test_prefill_window_row_is_decode_at_the_blocks_first_token(window, stride, n_local):
    """Each query block's selection equals the decode selection of R15 for a
    query at the block's first token (seq_len = 64 qb + 1) with F = the sum of
    the block's Forecast vectors: the decode window rule, summed tokens (R8)."""
    g = torch.Generator().manual_seed(window + stride + n_local)
    T, d, q0 = 64 * 10, 8, 64 * 6
    k = torch.randn(1, 2, T, d, generator=g, dtype=torch.float64).numpy()
    f = torch.randn(1, 2, T - q0, d, generator=g, dtype=torch.float64).numpy()
    kcw = orc.kv_window_meanpool(k, window, stride)
    p = orc.prefill_select_windows(f, kcw, q0, 2, 1, n_local, 64, window, stride)
    n_qb = (T - q0) // 64
    for qi in range(n_qb):
        qb = q0 // 64 + qi
        fsum = f[:, :, 64 * qi: 64 * (qi + 1)].sum(axis=2)
        kv_seen = orc.kv_window_meanpool(k, window, stride, seq_len=[64 * qb + 1])
        dsel = orc.decode_select_windows(fsum, kv_seen, [64 * qb + 1], 2, 1, n_local, 64, window, stride)
        np.testing.assert_array_equal(p.idx[0, :, qi], dsel.idx[0])
        for h in range(2):
            sp, sd = p.scores[h * n_qb + qi], dsel.scores[h]
            assert sp.keys() == sd.keys()
            for j in sp:
                assert abs(sp[j] - sd[j]) <= 1e-10 * (1 + abs(sd[j]))


# --------------------------------------------------------------------------- resident block cache (R17)
def test_golden_block_cache_lru(golden_dir):
    gx = _load(golden_dir, "block_cache_lru_hand.json")
    S, U = gx["S"], gx["U"]
    tags = np.full((1, 1, S), -1, dtype=np.int64)
    stamps = np.full((1, 1, S), -1, dtype=np.int64)
    clock = np.zeros((1, 1), dtype=np.int64)
    for call in gx["calls"]:
        idx = np.array(call["idx"], dtype=np.int64).reshape(1, 1, U)
        cnt = np.array([[call["cnt"]]])
        slot, fill, n_fill = orc.block_cache_plan(tags, stamps, clock, idx, cnt)
        assert slot[0, 0].tolist() == call["slot"]
        assert fill[0, 0].tolist() == call["fill"]
        assert int(n_fill[0, 0]) == call["n_fill"]
        assert tags[0, 0].tolist() == call["tags"]
        assert stamps[0, 0].tolist() == call["stamps"]


def _lists_with_drift(rng, n_calls, B, H, U, universe, churn):
    """Sorted lists of U blocks per call; each call swaps `churn` of the
    previous list's blocks for others (a drifting working set)."""
    cur = [[sorted(rng.choice(universe, U, replace=False).tolist()) for _ in range(H)] for _ in range(B)]
    out = []
    for _ in range(n_calls):
        idx = np.full((B, H, U), -1, dtype=np.int64)
        cnt = np.zeros((B, H), dtype=np.int64)
        for b in range(B):
            for g in range(H):
                keep = set(rng.choice(cur[b][g], U - churn, replace=False).tolist())
                rest = [j for j in range(universe) if j not in keep]
                new = set(rng.choice(rest, churn, replace=False).tolist())
                cur[b][g] = sorted(keep | new)
                c = int(rng.integers(U - 2, U + 1))           # some lists shorter (padded)
                idx[b, g, :c] = cur[b][g][:c]
                cnt[b, g] = c
        out.append((idx, cnt))
    return out


@pytest.mark.parametrize("S,U,universe,churn", [(8, 5, 12, 2), (16, 6, 40, 3), (6, 6, 20, 1)])
def test_block_cache_is_a_textbook_lru(S, U, universe, churn):
    """Against an OrderedDict LRU of capacity S (most recent at the end):
    room is made for the missing blocks by evicting from the front, skipping
    listed blocks; then every listed block is touched (moved or inserted at
    the end) in list order.  The resident sets and the blocks copied agree
    call by call; and the slot map is consistent (each listed block sits in
    its slot, held blocks never move)."""
    from collections import OrderedDict
    rng = np.random.default_rng(S * 100 + U)
    B, H = 2, 3
    tags = np.full((B, H, S), -1, dtype=np.int64)
    stamps = np.full((B, H, S), -1, dtype=np.int64)
    clock = np.zeros((B, H), dtype=np.int64)
    lru = [[OrderedDict() for _ in range(H)] for _ in range(B)]
    for idx, cnt in _lists_with_drift(rng, 25, B, H, U, universe, churn):
        before = tags.copy()
        slot, fill, n_fill = orc.block_cache_plan(tags, stamps, clock, idx, cnt)
        for b in range(B):
            for g in range(H):
                c = int(cnt[b, g])
                listed = idx[b, g, :c].tolist()
                od = lru[b][g]
                missing = [j for j in listed if j not in od]
                victims = [j for j in od if j not in listed][:max(0, len(od) + len(missing) - S)]
                for j in victims:
                    del od[j]
                for j in listed:
                    od[j] = True
                    od.move_to_end(j)
                assert set(od) == {int(t) for t in tags[b, g] if t >= 0}
                nf = int(n_fill[b, g])
                assert nf == len(missing)
                assert [int(idx[b, g, u]) for u in fill[b, g, :nf]] == missing
                assert (fill[b, g, nf:] == -1).all()
                for u, j in enumerate(listed):
                    s = int(slot[b, g, u])
                    assert tags[b, g, s] == j
                    if j in before[b, g]:
                        assert before[b, g, s] == j            # a held block is never moved or copied again
                assert len(set(slot[b, g, :c].tolist())) == c
                assert (slot[b, g, c:] == -1).all()


# --------------------------------------------------------------------------- baseline multi-head selector
def test_golden_multihead_select(golden_dir):
    gx = _load(golden_dir, "multihead_select_hand.json")
    d = gx["d"]
    nb = gx["seq_len"] // gx["block"]
    kc = np.zeros((1, 1, nb, d))
    for j, row in gx["kc_rows"].items():
        kc[0, 0, int(j)] = row
    q = np.array(gx["q"], dtype=np.float64).reshape(1, 2, d)
    for case in gx["cases"]:
        sel = orc.multihead_select_decode(q, kc, [gx["seq_len"]], case["topk"], gx["n_init"], gx["n_local"],
                                          gx["block"], 1.0 / math.sqrt(d))
        assert sel.top[0] == case["top_expected"]
        assert sel.idx[0, 0].tolist()[: case["cnt_expected"]] == case["idx_expected"]
        assert int(sel.cnt[0, 0]) == case["cnt_expected"]
        for j, w in gx["weights_expected"].items():
            assert abs(sel.scores[0][int(j)] - w) < 2e-6


@pytest.mark.parametrize("seed,G", [(0, 4), (1, 2), (2, 8)])
def test_multihead_select_equals_forecast_select_of_summed_queries(seed, G):
    """Summing the G per-head score rows equals one dot product with the
    summed query (linearity), and the softmax is monotone: the baseline's
    sets equal the Forecast selector's with F = the group's summed query,
    grouped by the attention map (query head h in KV head h // G), computed
    here with torch from the same tensors."""
    B, H, d, T, k = 2, 2, 32, 64 * 40, 6
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H * G, d, generator=g, dtype=torch.float64)
    kc = torch.randn(B, H, T // 64, d, generator=g, dtype=torch.float64)
    lens = [T, T - 64 * 9 - 3]
    f = q.view(B, H, G, d).sum(2)
    base = orc.multihead_select_decode(q.numpy(), kc.numpy(), lens, k, 1, 2, 64, 1 / math.sqrt(d))
    ref = orc.decode_select(f.numpy(), kc.numpy(), lens, k, 1, 2, 64)
    np.testing.assert_array_equal(base.idx, ref.idx)
    np.testing.assert_array_equal(base.cnt, ref.cnt)
    assert base.top == ref.top
    # the weights are the softmax over the candidates of (summed score) * scale
    for i in range(B * H):
        cand = sorted(ref.scores[i])
        z = torch.tensor([ref.scores[i][j] for j in cand], dtype=torch.float64) / math.sqrt(d)
        w = torch.softmax(z, 0).numpy()
        np.testing.assert_allclose([base.scores[i][j] for j in cand], w, rtol=1e-12, atol=1e-15)


def test_multihead_select_single_head_and_head_order():
    """G = 1: the baseline ranks the query's raw scores, i.e. the Forecast
    selector with F = q.  Reordering the heads inside a group changes nothing;
    moving a head to another group does."""
    B, d, T, k = 1, 16, 64 * 30, 5
    g = torch.Generator().manual_seed(7)
    q = torch.randn(B, 2, d, generator=g, dtype=torch.float64)
    kc = torch.randn(B, 2, T // 64, d, generator=g, dtype=torch.float64)
    one = orc.multihead_select_decode(q.numpy(), kc.numpy(), [T], k, 1, 2, 64, 0.25)
    ref = orc.decode_select(q.numpy(), kc.numpy(), [T], k, 1, 2, 64)
    np.testing.assert_array_equal(one.idx, ref.idx)
    q4 = torch.randn(B, 4, d, generator=g, dtype=torch.float64)
    kc2 = kc.clone()
    a = orc.multihead_select_decode(q4[:, [0, 1, 2, 3]].numpy(), kc2.numpy(), [T], k, 1, 2, 64, 0.25)
    b = orc.multihead_select_decode(q4[:, [1, 0, 3, 2]].numpy(), kc2.numpy(), [T], k, 1, 2, 64, 0.25)
    np.testing.assert_array_equal(a.idx, b.idx)
    c = orc.multihead_select_decode(q4[:, [0, 2, 1, 3]].numpy(), kc2.numpy(), [T], k, 1, 2, 64, 0.25)
    assert not np.array_equal(a.idx, c.idx)


def test_golden_attention_gqa(golden_dir):
    gx = _load(golden_dir, "attention_gqa_hand.json")
    k = np.array(gx["keys"], dtype=np.float64)[None]         # [1, 2, 2, 2]
    v = np.array(gx["values"], dtype=np.float64)[None]
    q = np.array(gx["q"], dtype=np.float64)[None]            # [1, 4, 2]
    idx = np.array([[[0, -1], [0, -1]]])
    cnt = np.array([[1, 1]])
    out = orc.attend_decode(q, k, v, idx, cnt, [gx["seq_len"]], gx["scale"], gx["block"])
    np.testing.assert_allclose(out[0], np.array(gx["out_expected"]), rtol=0, atol=1e-12)


def _brute_topk(scores: dict, k: int):
    """Best k-subset by total score (unique when scores are distinct)."""
    best, best_sum = None, -math.inf
    for comb in itertools.combinations(sorted(scores), min(k, len(scores))):
        s = sum(scores[j] for j in comb)
        if s > best_sum:
            best, best_sum = set(comb), s
    return best or set()


@pytest.mark.parametrize("seed", range(6))
def test_decode_select_bruteforce_subsets(seed):
    rng = np.random.default_rng(seed)
    B, H, d, blk = 2, 2, 3, 4
    T = 4 * 12
    lens = [int(rng.integers(1, T + 1)) for _ in range(B)]
    kc = rng.standard_normal((B, H, T // blk, d))
    f = rng.standard_normal((B, H, d))
    topk, n_init, n_local = 3, 1, 2
    sel = orc.decode_select(f, kc, lens, topk, n_init, n_local, blk)
    for b in range(B):
        pos = lens[b] - 1
        cur = pos // blk
        for g in range(H):
            # enumerate candidates from first principles: causal, not initial, not local
            cands = [j for j in range(T // blk) if j <= cur and j >= n_init and j < cur - n_local + 1]
            scores = {j: sum(f[b, g, c] * kc[b, g, j, c] for c in range(d)) for j in cands}
            best = _brute_topk(scores, topk)
            got = set(sel.top[b * H + g])
            assert got == best
            want_union = sorted(set(range(min(n_init, cur + 1))) | set(range(max(0, cur - n_local + 1), cur + 1)) | best)
            row = sel.idx[b, g]
            assert row[: sel.cnt[b, g]].tolist() == want_union
            assert (row[sel.cnt[b, g]:] == -1).all()


def test_decode_select_ties_prefer_lower_index():
    kc = np.zeros((1, 1, 10, 2))
    kc[0, 0, :, 0] = [0, 5, 3, 5, 3, 5, 0, 0, 0, 0]
    f = np.array([[[1.0, 0.0]]])
    sel = orc.decode_select(f, kc, [10 * 4], 4, 1, 2, 4)   # cur=9, cand 1..7
    assert sel.top[0] == [1, 3, 5, 2]
    assert sel.idx[0, 0].tolist() == [0, 1, 2, 3, 5, 8, 9]


def test_decode_select_sign():
    # the largest raw dot products win, not the smallest (and no 1/sqrt(d) or softmax changes that)
    kc = np.zeros((1, 1, 8, 1))
    kc[0, 0, :, 0] = [0, -4, 1, 9, -2, 7, 0, 0]
    sel = orc.decode_select(np.ones((1, 1, 1)), kc, [32], 2, 1, 2, 4)   # cur=7, cand 1..5
    assert sel.top[0] == [3, 5]


@pytest.mark.parametrize("seed", range(4))
def test_decode_select_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    blk = 8
    for _ in range(30):
        B, H, d = 2, 3, 4
        T = blk * int(rng.integers(1, 20))
        lens = [int(rng.integers(1, T + 1)) for _ in range(B)]
        topk, n_init, n_local = int(rng.integers(0, 6)), int(rng.integers(1, 3)), int(rng.integers(1, 4))
        kc = rng.standard_normal((B, H, T // blk, d))
        f = rng.standard_normal((B, H, d))
        sel = orc.decode_select(f, kc, lens, topk, n_init, n_local, blk)
        U = topk + n_init + n_local
        assert sel.idx.shape == (B, H, U)
        for b in range(B):
            cur = (lens[b] - 1) // blk
            n_cand = max(0, cur - n_local + 1 - n_init)
            for g in range(H):
                c = int(sel.cnt[b, g])
                row = sel.idx[b, g, :c].tolist()
                assert row == sorted(set(row)), "sorted and unique"
                assert max(row) == cur and all(0 <= j <= cur for j in row), "no future block"
                assert 0 in row, "initial block always present"
                for j in range(max(0, cur - n_local + 1), cur + 1):
                    assert j in row, "local blocks always present"
                assert len(sel.top[b * H + g]) == min(topk, n_cand)
                assert c <= U and (sel.idx[b, g, c:] == -1).all()


def test_planted_tiny_fp32_is_topk():
    wl = WORKLOADS["tiny-decode-fp32"]
    lay = decode_inputs(wl, "cpu")[0]
    kc = orc.kv_block_meanpool(_np(lay["k"]), wl.block)
    sel = orc.decode_select(_np(lay["f"]), kc, _np(lay["seq_len"]).astype(np.int64), wl.topk, wl.n_init,
                            wl.n_local, wl.block)
    assert set(sel.top[0]) == set(lay["planted"][0, 0].tolist())
    assert orc.kth_gap(sel.scores[0], wl.topk) > 0.5


def test_planted_B4_32K_is_topk():
    wl = WORKLOADS["decode-B4-32K"]
    lay = decode_inputs(wl, "cpu")[0]
    f = orc.forecast_proj(_np(lay["x_sel"]), _np(lay["w_sel"]), wl.Hkv, wl.d)
    k = lay["k"]
    for b in (0, 3):
        kc = orc.kv_block_meanpool(_np(k[b:b + 1]), wl.block)
        sel = orc.decode_select(f[b:b + 1], kc, [wl.T], wl.topk, wl.n_init, wl.n_local, wl.block)
        for g in range(wl.Hkv):
            assert set(sel.top[g]) == set(lay["planted"][b, g].tolist())
            assert orc.kth_gap(sel.scores[g], wl.topk) > 0.5


# --------------------------------------------------------------------------- a3 prefill
def test_golden_prefill(golden_dir):
    gx = _load(golden_dir, "prefill_select_attend_hand.json")
    blk, d, Tq = gx["block"], gx["d"], gx["Tq"]
    keys = np.array(gx["keys"], dtype=np.float64).reshape(1, 1, Tq, d)
    f = np.array(gx["f"], dtype=np.float64).reshape(1, 1, Tq, d)
    kc = orc.kv_block_meanpool(keys, blk)
    sel = orc.prefill_select(f, kc, gx["q_start"], gx["topk"], gx["n_init"], gx["n_local"], blk)
    assert {str(j): s for j, s in sel.scores[3].items()} == gx["scores_qb3_expected"]
    assert sel.idx[0, 0].tolist() == gx["idx_expected"]
    assert sel.cnt[0, 0].tolist() == gx["cnt_expected"]
    v = np.zeros((1, 1, Tq, d))
    v[0, 0, :, 0] = np.arange(Tq)
    q = np.zeros((1, 1, Tq, d))
    out = orc.attend_prefill(q, keys, v, sel.idx, sel.cnt, gx["q_start"], gx["scale"], blk)
    for t, want in gx["out_first_coord_expected"].items():
        assert abs(out[0, 0, int(t), 0] - want) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_prefill_select_bruteforce(seed):
    rng = np.random.default_rng(200 + seed)
    B, H, d, blk = 1, 2, 3, 4
    T = 4 * 10
    q_start, Tq = 16, 22                            # chunk covers query blocks 4..9, the last one partial
    k = rng.standard_normal((B, H, T, d))
    f = rng.standard_normal((B, H, Tq, d))
    kc = orc.kv_block_meanpool(k, blk)
    topk, n_init, n_local = 2, 1, 2
    sel = orc.prefill_select(f, kc, q_start, topk, n_init, n_local, blk)
    p = 0
    for b in range(B):
        for g in range(H):
            for qi in range(-(-Tq // blk)):
                qb = q_start // blk + qi
                toks = [t for t in range(Tq) if (q_start + t) // blk == qb]
                cands = [j for j in range(qb + 1) if n_init <= j <= qb - n_local]
                # score = sum over the block's tokens of per-token scores against the block's mean key
                scores = {}
                for j in cands:
                    mean_key = [sum(k[b, g, blk * j + r, c] for r in range(blk)) / blk for c in range(d)]
                    scores[j] = sum(sum(f[b, g, t, c] * mean_key[c] for c in range(d)) for t in toks)
                assert set(sel.top[p]) == _brute_topk(scores, topk)
                for j, s in scores.items():
                    assert abs(sel.scores[p][j] - s) < 1e-9
                p += 1


# --------------------------------------------------------------------------- a4
def _dense_masked_decode(q, k, v, idx, cnt, lens, scale, blk):
    """Brute force: softmax over ALL T tokens with -inf where a token is not attended."""
    B, Hq, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            allowed = set(int(j) for j in idx[b, g, : cnt[b, g]])
            logits = np.full(T, -np.inf)
            for t in range(T):
                if t // blk in allowed and t < lens[b]:
                    logits[t] = scale * sum(q[b, h, c] * k[b, g, t, c] for c in range(d))
            m = logits.max()
            w = np.array([math.exp(x - m) if x > -np.inf else 0.0 for x in logits])
            w /= w.sum()
            for c in range(d):
                out[b, h, c] = sum(w[t] * v[b, g, t, c] for t in range(T))
    return out


@pytest.mark.parametrize("seed", range(3))
def test_attend_decode_vs_dense_mask_bruteforce(seed):
    c = random_decode_case(seed, B=2, Hq=4, Hkv=2, d=4, T=40, block=8, seq_len=[40, 21])
    q, k, v = _np(c["q"]), _np(c["k"]), _np(c["v"])
    lens = _np(c["seq_len"]).astype(np.int64)
    kc = orc.kv_block_meanpool(k, 8, seq_len=lens)
    sel = orc.decode_select(_np(c["f"]), kc, lens, 1, 1, 1, 8)
    got = orc.attend_decode(q, k, v, sel.idx, sel.cnt, lens, 0.37, 8)
    want = _dense_masked_decode(q, k, v, sel.idx, sel.cnt, lens, 0.37, 8)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _sdpa64(q, k, v, scale, causal):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("seed", range(3))
def test_decode_full_budget_equals_dense_attention(seed):
    # with k >= number of candidates every causal block is selected: plain softmax attention
    c = random_decode_case(seed, B=2, Hq=8, Hkv=2, d=16, T=256, block=16, seq_len=[256, 201])
    q, k, v = _np(c["q"]), _np(c["k"]), _np(c["v"])
    lens = _np(c["seq_len"]).astype(np.int64)
    kc = orc.kv_block_meanpool(k, 16, seq_len=lens)
    sel = orc.decode_select(_np(c["f"]), kc, lens, 100, 1, 2, 16)
    scale = 1 / math.sqrt(16)
    got = orc.attend_decode(q, k, v, sel.idx, sel.cnt, lens, scale, 16)
    for b in range(2):
        L = int(lens[b])
        kk = np.repeat(k[b, :, :L], 4, axis=0)[None]
        vv = np.repeat(v[b, :, :L], 4, axis=0)[None]
        want = _sdpa64(q[b][None, :, None, :], kk, vv, scale, False)[0, :, 0]
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(2))
def test_prefill_full_budget_equals_causal_attention(seed):
    rng = np.random.default_rng(300 + seed)
    B, Hq, Hkv, d, T, blk = 1, 4, 2, 8, 96, 8
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    f = rng.standard_normal((B, Hkv, T, d))
    kc = orc.kv_block_meanpool(k, blk)
    sel = orc.prefill_select(f, kc, 0, 64, 1, 2, blk)
    scale = 1 / math.sqrt(d)
    got = orc.attend_prefill(q, k, v, sel.idx, sel.cnt, 0, scale, blk)
    want = _sdpa64(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), scale, True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_chunked_prefill_equals_unchunked():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d, T, blk = 1, 2, 1, 4, 64, 4
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    f = rng.standard_normal((B, Hkv, T, d))
    kc = orc.kv_block_meanpool(k, blk)
    whole_sel = orc.prefill_select(f, kc, 0, 3, 1, 2, blk)
    whole = orc.attend_prefill(q, k, v, whole_sel.idx, whole_sel.cnt, 0, 0.5, blk)
    for q0 in range(0, T, 16):
        s = orc.prefill_select(f[:, :, q0:q0 + 16], kc, q0, 3, 1, 2, blk)
        np.testing.assert_array_equal(s.idx, whole_sel.idx[:, :, q0 // blk:(q0 + 16) // blk])
        part = orc.attend_prefill(q[:, :, q0:q0 + 16], k, v, s.idx, s.cnt, q0, 0.5, blk)
        np.testing.assert_allclose(part, whole[:, :, q0:q0 + 16], rtol=0, atol=1e-13)


def test_empty_token_sets_give_zero_rows():
    """Reading R19: a query with nothing to attend to (an empty sequence, a
    group whose list is empty, a prefill query block with an empty list)
    gets the zero vector; every other row is the brute-force dense-mask
    result, so the convention touches the empty rows only."""
    c = random_decode_case(11, B=3, Hq=4, Hkv=2, d=4, T=40, block=8)
    q, k, v = _np(c["q"]), _np(c["k"]), _np(c["v"])
    lens = np.array([40, 0, 21])
    kc = orc.kv_block_meanpool(k, 8, seq_len=lens)
    sel = orc.decode_select(_np(c["f"]), kc, lens, 1, 1, 1, 8)
    # the empty sequence selects nothing: no initial, local or candidate block
    assert (sel.cnt[1] == 0).all() and (sel.idx[1] == -1).all()
    idx, cnt = sel.idx.copy(), sel.cnt.copy()
    cnt[2, 1] = 0                                   # a caller's empty list for one group
    got = orc.attend_decode(q, k, v, idx, cnt, lens, 0.37, 8)
    assert (got[1] == 0).all() and (got[2, 2:] == 0).all()
    keep = [(0, h) for h in range(4)] + [(2, 0), (2, 1)]
    with np.errstate(invalid="ignore"):   # the brute force's emptied rows are 0/0 and are not compared
        want = _dense_masked_decode(q[[0, 2]], k[[0, 2]], v[[0, 2]], idx[[0, 2]], cnt[[0, 2]], lens[[0, 2]], 0.37, 8)
    for b, h in keep:
        np.testing.assert_allclose(got[b, h], want[0 if b == 0 else 1, h], rtol=0, atol=1e-12)
    # prefill: query block 1's list emptied, query block 0 untouched
    rng = np.random.default_rng(12)
    qq = rng.standard_normal((1, 2, 16, 4))
    kk = rng.standard_normal((1, 1, 16, 4))
    vv = rng.standard_normal((1, 1, 16, 4))
    ps = orc.prefill_select(rng.standard_normal((1, 1, 16, 4)), orc.kv_block_meanpool(kk, 8), 0, 1, 1, 1, 8)
    pc = ps.cnt.copy()
    pc[0, 0, 1] = 0
    out = orc.attend_prefill(qq, kk, vv, ps.idx, pc, 0, 0.5, 8)
    assert (out[:, :, 8:] == 0).all()
    ref = orc.attend_prefill(qq, kk, vv, ps.idx, ps.cnt, 0, 0.5, 8)
    np.testing.assert_array_equal(out[:, :, :8], ref[:, :, :8])
    assert np.abs(ref[:, :, 8:]).max() > 0


def test_attention_is_convex_combination():
    c = random_decode_case(5, B=1, Hq=4, Hkv=1, d=8, T=128, block=16)
    q, k, v = _np(c["q"]) * 4, _np(c["k"]), _np(c["v"])
    kc = orc.kv_block_meanpool(k, 16)
    sel = orc.decode_select(_np(c["f"]), kc, [128], 2, 1, 1, 16)
    out = orc.attend_decode(q, k, v, sel.idx, sel.cnt, [128], 1.0, 16)
    toks = np.concatenate([np.arange(16 * j, 16 * j + 16) for j in sel.idx[0, 0, : sel.cnt[0, 0]]])
    sub = v[0, 0, toks]
    assert (out[0] >= sub.min(axis=0) - 1e-12).all() and (out[0] <= sub.max(axis=0) + 1e-12).all()


# --------------------------------------------------------------------------- a5
def test_gather_selected_blocks_bytes():
    rng = np.random.default_rng(9)
    kv = rng.integers(0, 2 ** 16, size=(2, 2, 32, 3), dtype=np.uint16)
    idx = np.array([[[0, 3, 5, -1], [1, 2, -1, -1]], [[7, -1, -1, -1], [0, 1, 2, 3]]])
    cnt = np.array([[3, 2], [1, 4]])
    ring = orc.gather_selected_blocks(kv, idx, cnt, 4)
    assert ring.dtype == np.uint16
    for b in range(2):
        for g in range(2):
            for u in range(4):
                if u < cnt[b, g]:
                    j = idx[b, g, u]
                    assert ring[b, g, u].tobytes() == kv[b, g, 4 * j:4 * j + 4].tobytes()
                else:
                    assert not ring[b, g, u].any()


# --------------------------------------------------------------------------- lookahead
def test_lookahead_uses_each_layers_own_forecast_and_keys():
    wl = WORKLOADS["decode-B4-32K"]
    rng = np.random.default_rng(11)
    L, B, H, d, hidden, T, blk = 3, 1, 2, 4, 6, 64, 8
    layers = []
    for _ in range(L):
        k = rng.standard_normal((B, H, T, d))
        layers.append({"x_sel": rng.standard_normal((B, hidden)), "w_sel": rng.standard_normal((hidden, H * d)),
                       "kc": orc.kv_block_meanpool(k, blk), "q": rng.standard_normal((B, 2 * H, d)), "k": k,
                       "v": rng.standard_normal((B, H, T, d)), "seq_len": [T]})
    res = orc.decode_step_lookahead(layers, 2, 1, 1, blk, 0.5)
    for lay, (sel, out) in zip(layers, res):
        # recompute from scratch with explicit loops: F = x W (GEMV), scores vs that layer's pooled keys
        f = np.array([[sum(lay["x_sel"][0, r] * lay["w_sel"][r, g * d + c] for r in range(hidden))
                       for c in range(d)] for g in range(H)])
        for g in range(H):
            sc = {j: float(f[g] @ lay["kc"][0, g, j]) for j in range(1, (T - 1) // blk)}
            assert set(sel.top[g]) == _brute_topk(sc, 2)
    assert wl.U == 35


def test_kth_gap_values():
    assert orc.kth_gap({1: 4.0, 2: 3.0, 3: 1.0}, 2) == pytest.approx((3.0 - 1.0) / 3.0)
    assert orc.kth_gap({1: 4.0, 2: 3.0}, 2) == math.inf
    assert orc.kth_gap({1: 2.0, 2: 2.0, 3: 2.0}, 1) == 0.0
