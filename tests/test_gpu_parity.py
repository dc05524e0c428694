"""GPU parity: every C-ABI call against the fp64 oracle on seeded inputs.

Tolerances: selection ids bit-exact outside a 1e-3 relative k-th score gap
(near-ties: rescored in fp64, see parity.check_selection); attention 1e-4
absolute for fp32 inputs, 2e-2 absolute for bf16 inputs; compressed keys
(fp32 means of 64 values of magnitude below ~5) 1e-4 absolute; Forecast
vectors and raw scores (fp32 sums of `hidden`, 64 * `hidden` or d products)
within parity.fp32_sum_tol of the fp64 value, a bound computed per output
from the sum of the products' magnitudes and the number of terms.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_long_kv_amd as bskv
import oracle as orc
from parity import check_selection, fp32_sum_close, max_abs, np64
from workloads import WORKLOADS, decode_inputs, random_decode_case, random_prefill_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _gpu(case):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in case.items()}


def _kc_gpu(k, seq_len, nb_cap=None):
    B, H, T, d = k.shape
    nb_cap = nb_cap or T // 64
    kc = torch.full((B, H, nb_cap, d), float("nan"), dtype=torch.float32, device=DEV)
    bskv.kv_block_meanpool(k, seq_len, kc)
    return kc


# ----------------------------------------------------------------------------- a2
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_meanpool_range_ragged(dtype, d):
    lens = [64 * 20, 64 * 20 - 1, 64 * 5 + 3, 1]
    c = _gpu(random_decode_case(1, B=4, Hq=2, Hkv=2, d=d, T=64 * 20, dtype=dtype, seq_len=lens))
    kc = _kc_gpu(c["k"], c["seq_len"])
    torch.cuda.synchronize()
    want = orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens)
    got = np64(kc)
    done = ~np.isnan(want)
    assert np.array_equal(done, ~np.isnan(got)), "exactly the complete blocks are written"
    assert max_abs(got[done], want[done]) < 1e-4


def test_meanpool_newest_only_and_subrange():
    lens = [64 * 9, 64 * 9 + 5, 64 * 3, 64 * 12]
    c = _gpu(random_decode_case(2, B=4, Hq=4, Hkv=1, d=128, T=64 * 12, dtype="bf16", seq_len=lens))
    kc = torch.full((4, 1, 12, 128), 7.0, dtype=torch.float32, device=DEV)
    bskv.kv_block_meanpool(c["k"], c["seq_len"], kc, 0, 12, newest_only=True)
    torch.cuda.synchronize()
    want = orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens)
    got = np64(kc)
    for b, L in enumerate(lens):
        for j in range(12):
            if L % 64 == 0 and j == L // 64 - 1:
                assert max_abs(got[b, 0, j], want[b, 0, j]) < 1e-4
            else:
                assert (got[b, 0, j] == 7.0).all(), (b, j)
    kc.fill_(7.0)
    bskv.kv_block_meanpool(c["k"], c["seq_len"], kc, 2, 5)
    torch.cuda.synchronize()
    got = np64(kc)
    for b, L in enumerate(lens):
        for j in range(12):
            if 2 <= j < 5 and 64 * (j + 1) <= L:
                assert max_abs(got[b, 0, j], want[b, 0, j]) < 1e-4
            else:
                assert (got[b, 0, j] == 7.0).all(), (b, j)


# ----------------------------------------------------------------------------- a1
@pytest.mark.parametrize("B", [1, 3, 4, 8, 16, 20])
def test_forecast_proj_bf16(B):
    g = torch.Generator().manual_seed(10 + B)
    x = torch.randn(B, 4096, generator=g).to(torch.bfloat16)
    w = (torch.randn(4096, 1024, generator=g) * 0.02).to(torch.bfloat16)
    f = bskv.forecast_proj(x.to(DEV), w.to(DEV), 8, 128)
    torch.cuda.synchronize()
    want = orc.forecast_proj(np64(x), np64(w), 8, 128)
    mag = (np.abs(np64(x)) @ np.abs(np64(w))).reshape(want.shape)
    assert fp32_sum_close(np64(f), want, mag, 4096)


@pytest.mark.parametrize("B,hidden,H,d", [(2, 512, 2, 64), (5, 768, 1, 128), (17, 256, 4, 64)])
def test_forecast_proj_bf16_shapes(B, hidden, H, d):
    """Other tile counts: hidden 256..768 (2..6 row splits), 128..256 columns."""
    g = torch.Generator().manual_seed(hidden + B)
    x = torch.randn(B, hidden, generator=g).to(torch.bfloat16)
    w = (torch.randn(hidden, H * d, generator=g) * 0.05).to(torch.bfloat16)
    f = bskv.forecast_proj(x.to(DEV), w.to(DEV), H, d)
    torch.cuda.synchronize()
    mag = (np.abs(np64(x)) @ np.abs(np64(w))).reshape(B, H, d)
    assert fp32_sum_close(np64(f), orc.forecast_proj(np64(x), np64(w), H, d), mag, hidden)


def test_forecast_proj_f32_and_repeat():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(5, 256, generator=g)
    w = torch.randn(256, 128, generator=g)
    xd, wd = x.to(DEV), w.to(DEV)
    f1 = bskv.forecast_proj(xd, wd, 2, 64).clone()
    f2 = bskv.forecast_proj(xd, wd, 2, 64)
    torch.cuda.synchronize()
    assert torch.equal(f1, f2), "deterministic and the split counters are reset"
    mag = (np.abs(np64(x)) @ np.abs(np64(w))).reshape(5, 2, 64)
    assert fp32_sum_close(np64(f1), orc.forecast_proj(np64(x), np64(w), 2, 64), mag, 256)


# ----------------------------------------------------------------------------- a3 decode
def _decode_select_both(c, topk, n_init, n_local, hidden=None):
    B, H, T, d = c["k"].shape
    if "f" in c:
        f = c["f"]
        f_or = np64(c["f"])
    else:
        f = bskv.forecast_proj(c["x_sel"], c["w_sel"], H, d)
        f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), H, d)
    kc = _kc_gpu(c["k"], c["seq_len"])
    idx, cnt, sc = bskv.forecast_block_score_topk(f, kc, topk, n_init, n_local, seq_len=c["seq_len"],
                                                  return_scores=True)
    torch.cuda.synchronize()
    lens = c["seq_len"].cpu().numpy()
    kc_or = orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens)
    sel = orc.decode_select(f_or, kc_or, lens, topk, n_init, n_local, 64)
    return idx, cnt, sc, sel


def test_decode_selection_tiny_fp32():
    wl = WORKLOADS["tiny-decode-fp32"]
    lay = _gpu(decode_inputs(wl, "cpu")[0])
    idx, cnt, sc, sel = _decode_select_both(lay, wl.topk, wl.n_init, wl.n_local)
    assert check_selection(idx, cnt, sel, wl.topk) == 0
    assert set(sel.top[0]) == set(lay["planted"][0, 0].tolist())
    got = np64(sc)[0, 0]
    for j, s in sel.scores[0].items():
        assert abs(got[j] - s) <= 1e-5 * max(1.0, abs(s))
    cur = (wl.T - 1) // 64
    for j in list(range(wl.n_init)) + list(range(cur - wl.n_local + 1, cur + 1)):
        assert got[j] == -math.inf


def test_decode_selection_B4_32K():
    wl = WORKLOADS["decode-B4-32K"]
    lay = _gpu(decode_inputs(wl, "cpu")[0])
    idx, cnt, _, sel = _decode_select_both(lay, wl.topk, wl.n_init, wl.n_local)
    assert check_selection(idx, cnt, sel, wl.topk) == 0
    top = [set(t) for t in sel.top]
    for b in range(wl.B):
        for g in range(wl.Hkv):
            assert top[b * wl.Hkv + g] == set(lay["planted"][b, g].tolist())


@pytest.mark.parametrize("seed,d,topk,n_local", [(0, 64, 3, 1), (1, 128, 8, 2), (2, 128, 40, 4), (3, 64, 0, 3),
                                                 (4, 128, 5, 1)])
def test_decode_selection_ragged(seed, d, topk, n_local):
    lens = [64 * 37, 64 * 37 - 13, 65, 64, 1, 64 * 10 + 1]
    c = _gpu(random_decode_case(seed, B=6, Hq=4, Hkv=2, d=d, T=64 * 37, seq_len=lens, plant=topk // 2,
                                topk=topk, n_local=n_local))
    idx, cnt, _, sel = _decode_select_both(c, topk, 1, n_local)
    check_selection(idx, cnt, sel, topk)


def test_decode_selection_exact_ties_take_lower_index():
    B, H, d, nb = 2, 2, 64, 300
    kc = torch.zeros(B, H, nb, d)
    g = torch.Generator().manual_seed(5)
    kc[..., 0] = torch.randint(-3, 4, (B, H, nb), generator=g).float()   # many exactly equal scores
    f = torch.zeros(B, H, d)
    f[..., 0] = 1.0
    lens = torch.tensor([64 * nb, 64 * 200 + 7], dtype=torch.int64)
    idx, cnt = bskv.forecast_block_score_topk(f.to(DEV), kc.to(DEV), 17, 1, 3, seq_len=lens.to(DEV))
    torch.cuda.synchronize()
    sel = orc.decode_select(f.numpy(), kc.numpy(), lens.numpy(), 17, 1, 3, 64)
    assert np.array_equal(idx.cpu().numpy(), sel.idx)
    assert np.array_equal(cnt.cpu().numpy(), sel.cnt)


def test_decode_selection_repeatable():
    wl = WORKLOADS["decode-B4-32K"]
    lay = _gpu(decode_inputs(wl, "cpu", B=2, T=8192)[0])
    f = bskv.forecast_proj(lay["x_sel"], lay["w_sel"], wl.Hkv, wl.d)
    kc = _kc_gpu(lay["k"], lay["seq_len"])
    a = bskv.forecast_block_score_topk(f, kc, wl.topk, 1, 2, seq_len=lay["seq_len"])
    a = [t.clone() for t in a]
    b = bskv.forecast_block_score_topk(f, kc, wl.topk, 1, 2, seq_len=lay["seq_len"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------------------- baseline multi-head selector
@pytest.mark.parametrize("dtype,d,G,topk,lens", [("bf16", 128, 4, 32, [64 * 512] * 4),
                                                 ("f32", 64, 2, 8, [64 * 40, 64 * 33 + 17, 100, 64 * 40 - 1]),
                                                 ("bf16", 64, 8, 16, [64 * 300, 64 * 150 + 1]),
                                                 ("f32", 128, 1, 64, [64 * 2048]),
                                                 ("bf16", 64, 2, 32, [64 * 2100 + 5, 64 * 1000])])
def test_multihead_select_decode(dtype, d, G, topk, lens):
    """The baseline selector (per-head scores summed, softmax, top-k) against
    the oracle: lists equal outside the near-tie band, softmax weights to
    float32 accuracy.  Ragged lengths, one with fewer candidates than k, one
    with more than 2048 candidates (the top-k's keys through LDS)."""
    B, Hkv = len(lens), 2
    T = max(lens) + 64
    g = torch.Generator().manual_seed(100 + d + G)
    q = torch.randn(B, Hkv * G, d, generator=g).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    k = torch.randn(B, Hkv, T, d, generator=g).to(q.dtype)
    seq_len = torch.tensor(lens, dtype=torch.int64)
    kc = _kc_gpu(k.to(DEV), seq_len.to(DEV))
    idx, cnt, w = bskv.multihead_block_score_topk(q.to(DEV), kc, topk, 1, 4, seq_len.to(DEV), return_weights=True)
    torch.cuda.synchronize()
    kc_or = orc.kv_block_meanpool(np64(k), 64, seq_len=seq_len.numpy())
    sel = orc.multihead_select_decode(np64(q), kc_or, seq_len.numpy(), topk, 1, 4, 64, 1.0 / math.sqrt(d))
    assert check_selection(idx, cnt, sel, topk) == 0
    wn = w.cpu().numpy()
    for i, ws in enumerate(sel.scores):
        b, gg = divmod(i, Hkv)
        for j, wt in ws.items():
            assert abs(wn[b, gg, j] - wt) < 1e-5 + 1e-4 * wt, (b, gg, j)


def test_multihead_select_matches_forecast_select_on_summed_queries():
    """Linearity on the GPU path: the baseline's lists equal the Forecast
    selector's with F = the fp32 sum of each group's queries."""
    B, Hkv, G, d, T = 4, 8, 4, 128, 64 * 1024
    g = torch.Generator().manual_seed(5)
    q = torch.randn(B, Hkv * G, d, generator=g)
    k = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    seq_len = torch.full((B,), T, dtype=torch.int64, device=DEV)
    kc = _kc_gpu(k.to(DEV), seq_len)
    i1, c1 = bskv.multihead_block_score_topk(q.to(DEV), kc, 64, 1, 4, seq_len)
    i2, c2 = bskv.forecast_block_score_topk(q.view(B, Hkv, G, d).sum(2).to(DEV).contiguous(), kc, 64, 1, 4,
                                            seq_len=seq_len)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    # the two paths add the same products in different fp32 orders: a row may
    # differ only by a swap at the k-th place
    a, b = i1.cpu().numpy(), i2.cpu().numpy()
    rows = [(set(a[r, h]) ^ set(b[r, h])) for r in range(B) for h in range(Hkv)]
    assert all(len(x) <= 2 for x in rows)
    assert sum(1 for x in rows if x) <= 2


# ----------------------------------------------------------------------------- a2'/a3' windows
def _kcw_gpu(k, seq_len, window, stride, nw_cap=None):
    B, H, T, d = k.shape
    nw_cap = nw_cap or (T - window) // stride + 1
    kcw = torch.full((B, H, nw_cap, d), float("nan"), dtype=torch.float32, device=DEV)
    bskv.kv_window_meanpool(k, seq_len, kcw, window, stride)
    return kcw


@pytest.mark.parametrize("dtype,d,window,stride", [("bf16", 128, 32, 16), ("f32", 64, 32, 16), ("bf16", 64, 64, 16),
                                                   ("f32", 128, 32, 32), ("bf16", 128, 64, 64)])
def test_window_meanpool_ragged(dtype, d, window, stride):
    """Exactly the complete windows are written, each the mean of its keys."""
    lens = [64 * 20, 64 * 20 - 1, 64 * 5 + 3, 1, 31, 48]
    c = _gpu(random_decode_case(11, B=6, Hq=2, Hkv=2, d=d, T=64 * 20, dtype=dtype, seq_len=lens))
    kcw = _kcw_gpu(c["k"], c["seq_len"], window, stride)
    torch.cuda.synchronize()
    want = orc.kv_window_meanpool(np64(c["k"]), window, stride, seq_len=lens)
    got = np64(kcw)
    done = ~np.isnan(want)
    assert np.array_equal(done, ~np.isnan(got)), "exactly the complete windows are written"
    assert max_abs(got[done], want[done]) < 1e-4


def test_window_meanpool_newest_only_and_subrange():
    lens = [64 * 9, 64 * 9 + 16, 64 * 3 + 5, 32, 16]
    T, W, S = 64 * 12, 32, 16
    nw = (T - W) // S + 1
    c = _gpu(random_decode_case(12, B=5, Hq=4, Hkv=1, d=128, T=T, dtype="bf16", seq_len=lens))
    want = orc.kv_window_meanpool(np64(c["k"]), W, S, seq_len=lens)
    kcw = torch.full((5, 1, nw, 128), 7.0, dtype=torch.float32, device=DEV)
    bskv.kv_window_meanpool(c["k"], c["seq_len"], kcw, W, S, newest_only=True)
    torch.cuda.synchronize()
    got = np64(kcw)
    for b, L in enumerate(lens):
        newest = (L - W) // S if L >= W and (L - W) % S == 0 else None
        for w in range(nw):
            if w == newest:
                assert max_abs(got[b, 0, w], want[b, 0, w]) < 1e-4
            else:
                assert (got[b, 0, w] == 7.0).all(), (b, w)
    kcw.fill_(7.0)
    bskv.kv_window_meanpool(c["k"], c["seq_len"], kcw, W, S, w_begin=5, w_end=20)
    torch.cuda.synchronize()
    got = np64(kcw)
    for b, L in enumerate(lens):
        for w in range(nw):
            if 5 <= w < 20 and S * w + W <= L:
                assert max_abs(got[b, 0, w], want[b, 0, w]) < 1e-4
            else:
                assert (got[b, 0, w] == 7.0).all(), (b, w)


@pytest.mark.parametrize("dtype,d,window,stride,topk,lens", [
    ("bf16", 128, 32, 16, 16, [64 * 300, 64 * 150 + 1, 64 * 150 + 16, 64 * 150 + 40]),
    ("f32", 64, 32, 16, 8, [64 * 40, 64 * 33 + 17, 100, 64 * 40 - 1]),
    ("bf16", 64, 64, 16, 12, [64 * 200, 64 * 77 + 63]),
    ("f32", 128, 32, 32, 64, [64 * 2048, 64 * 1000 + 31]),
    ("bf16", 64, 32, 16, 32, [64 * 2100 + 5, 64 * 2048])])
def test_window_select_decode(dtype, d, window, stride, topk, lens):
    """Selection on window-compressed keys against the oracle: lists equal
    outside the near-tie band, block scores (max over each block's complete
    windows) to float32 accuracy.  Ragged lengths: the newest block's last
    window may or may not be complete; one sequence has fewer candidates than k."""
    B, Hkv = len(lens), 4
    T = max(lens) + 64
    g = torch.Generator().manual_seed(200 + d + window + stride)
    f = torch.randn(B, Hkv, d, generator=g)
    k = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    seq_len = torch.tensor(lens, dtype=torch.int64)
    kcw = _kcw_gpu(k.to(DEV), seq_len.to(DEV), window, stride)
    idx, cnt, bs = bskv.forecast_window_score_topk(f.to(DEV), kcw, topk, 1, 4, seq_len.to(DEV), window, stride,
                                                   return_scores=True)
    torch.cuda.synchronize()
    kcw_or = orc.kv_window_meanpool(np64(k), window, stride, seq_len=seq_len.numpy())
    sel = orc.decode_select_windows(np64(f), kcw_or, seq_len.numpy(), topk, 1, 4, 64, window, stride)
    assert check_selection(idx, cnt, sel, topk) <= 1
    bn = bs.cpu().numpy()
    for i, sc in enumerate(sel.scores):
        b, gg = divmod(i, Hkv)
        for j, want in sc.items():
            assert abs(bn[b, gg, j] - want) < 1e-4 * (1 + abs(want)), (b, gg, j)


def test_window_select_block_sized_windows_equal_block_selector():
    """With 64-token windows at stride 64 the windows are the blocks: the
    window path gives the block selector's compressed keys, lists and scores
    bit for bit."""
    B, Hkv, d, T = 3, 8, 128, 64 * 700
    lens = [T, T - 30, 64 * 333]
    g = torch.Generator().manual_seed(21)
    f = torch.randn(B, Hkv, d, generator=g).to(DEV)
    k = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16).to(DEV)
    seq_len = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kc = _kc_gpu(k, seq_len)
    kcw = _kcw_gpu(k, seq_len, 64, 64)
    i1, c1, s1 = bskv.forecast_window_score_topk(f, kcw, 32, 1, 4, seq_len, 64, 64, return_scores=True)
    i2, c2 = bskv.forecast_block_score_topk(f, kc, 32, 1, 4, seq_len=seq_len)
    torch.cuda.synchronize()
    assert torch.equal(kc.nan_to_num(-1.0), kcw.nan_to_num(-1.0))
    assert torch.equal(c1, c2) and torch.equal(i1, i2)
    f64, kc64 = np64(f), np64(kc)
    sc = np.einsum("bgd,bgjd->bgj", f64, kc64)
    mag = np.einsum("bgd,bgjd->bgj", np.abs(f64), np.abs(kc64))
    assert torch.isfinite(s1[:, :, 1:300]).all()
    assert fp32_sum_close(np64(s1[:, :, 1:300]), sc[:, :, 1:300], mag[:, :, 1:300], d)


@pytest.mark.parametrize("dtype,d,window,stride,n_local,q_start,Tq", [
    ("bf16", 128, 32, 16, 32, 64 * 64, 2048), ("f32", 64, 32, 16, 1, 64 * 3, 64 * 9 + 17),
    ("bf16", 64, 64, 16, 2, 0, 64 * 20), ("f32", 128, 32, 32, 1, 64 * 40, 64 * 6)])
def test_window_select_prefill(dtype, d, window, stride, n_local, q_start, Tq):
    """Prefill selection on window-compressed keys against the oracle: each
    query block sums its Forecast vectors, max-pools the visible windows'
    scores per candidate block; a ragged last query block; n_local = 1 makes
    the windows that reach into the query block matter."""
    B, Hkv, topk = 2, 2, 8
    T = q_start + Tq
    g = torch.Generator().manual_seed(300 + d + window + n_local)
    cdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    f = torch.randn(B, Hkv, Tq, d, generator=g).to(cdt)
    k = torch.randn(B, Hkv, T, d, generator=g).to(cdt)
    seq_len = torch.full((B,), T, dtype=torch.int64)
    kcw = _kcw_gpu(k.to(DEV), seq_len.to(DEV), window, stride)
    idx, cnt = bskv.forecast_window_score_topk(f.to(DEV), kcw, topk, 1, n_local, None, window, stride, q_start=q_start)
    torch.cuda.synchronize()
    kcw_or = orc.kv_window_meanpool(np64(k), window, stride)
    sel = orc.prefill_select_windows(np64(f), kcw_or, q_start, topk, 1, n_local, 64, window, stride)
    assert check_selection(idx, cnt, sel, topk) <= 2


def test_window_select_prefill_block_sized_windows_equal_block_selector():
    """Block-sized windows give the block selector's prefill lists: both
    GPU paths (per-query-block window scoring; the MFMA score contraction)
    against the oracle's block selection, near-tie swaps only."""
    B, Hkv, d, T, q0 = 2, 4, 128, 64 * 300, 64 * 200
    g = torch.Generator().manual_seed(31)
    f = torch.randn(B, Hkv, T - q0, d, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16).to(DEV)
    seq_len = torch.full((B,), T, dtype=torch.int64, device=DEV)
    kc = _kc_gpu(k, seq_len)
    kcw = _kcw_gpu(k, seq_len, 64, 64)
    i1, c1 = bskv.forecast_window_score_topk(f, kcw, 16, 1, 3, None, 64, 64, q_start=q0)
    i2, c2 = bskv.forecast_block_score_topk(f, kc, 16, 1, 3, q_start=q0, prefill=True)
    torch.cuda.synchronize()
    sel = orc.prefill_select(np64(f), orc.kv_block_meanpool(np64(k), 64), q0, 16, 1, 3, 64)
    assert check_selection(i1, c1, sel, 16) <= 2 and check_selection(i2, c2, sel, 16) <= 2


# ----------------------------------------------------------------------------- a4 decode
def _attn_case(seed, B, Hq, Hkv, d, T, dtype, lens, topk, n_local):
    c = _gpu(random_decode_case(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, dtype=dtype, seq_len=lens, plant=topk,
                                topk=topk, n_local=n_local))
    lens_np = c["seq_len"].cpu().numpy()
    kc_or = orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens_np)
    sel = orc.decode_select(np64(c["f"]), kc_or, lens_np, topk, 1, n_local, 64)
    return c, sel, lens_np


@pytest.mark.parametrize("dtype,d,G,tol", [("f32", 64, 4, 1e-4), ("f32", 128, 1, 1e-4), ("bf16", 128, 4, 2e-2),
                                           ("bf16", 64, 8, 2e-2), ("bf16", 128, 2, 2e-2), ("f32", 64, 8, 1e-4)])
def test_attn_decode_on_oracle_lists(dtype, d, G, tol):
    Hkv = 2
    lens = [64 * 40, 64 * 33 + 17, 100, 64 * 40 - 1]
    c, sel, lens_np = _attn_case(7, 4, Hkv * G, Hkv, d, 64 * 40, dtype, lens, topk=9, n_local=2)
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    scale = 1.0 / math.sqrt(d)
    out = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"], scale)
    torch.cuda.synchronize()
    want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), sel.idx, sel.cnt, lens_np, scale, 64)
    assert max_abs(np64(out), want) < tol


@pytest.mark.parametrize("dtype,d,G,tol", [("bf16", 128, 4, 2e-2), ("bf16", 64, 8, 2e-2), ("f32", 64, 2, 1e-4)])
def test_attn_decode_long_splits(dtype, d, G, tol):
    """One KV head per sequence and 155 listed blocks: 32 splits of 5 blocks
    each, i.e. the double-buffered online-softmax loop rather than the
    all-at-once path of short splits.  Ragged lengths."""
    lens = [64 * 300, 64 * 251 + 30]
    c, sel, lens_np = _attn_case(13, 2, G, 1, d, 64 * 300, dtype, lens, topk=150, n_local=4)
    assert int(sel.cnt.max()) == 155
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    scale = 1.0 / math.sqrt(d)
    out = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"], scale)
    torch.cuda.synchronize()
    want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), sel.idx, sel.cnt, lens_np, scale, 64)
    assert max_abs(np64(out), want) < tol


def test_attn_decode_tiny_fp32_end_to_end():
    wl = WORKLOADS["tiny-decode-fp32"]
    lay = _gpu(decode_inputs(wl, "cpu")[0])
    idx, cnt, _, sel = _decode_select_both(lay, wl.topk, wl.n_init, wl.n_local)
    assert check_selection(idx, cnt, sel, wl.topk) == 0
    out = bskv.block_sparse_attn_decode(lay["q"], lay["k"], lay["v"], idx, cnt, lay["seq_len"], wl.scale)
    torch.cuda.synchronize()
    want = orc.attend_decode(np64(lay["q"]), np64(lay["k"]), np64(lay["v"]), sel.idx, sel.cnt, [wl.T], wl.scale, 64)
    assert max_abs(np64(out), want) < 1e-4


def test_attn_decode_B4_32K_end_to_end():
    wl = WORKLOADS["decode-B4-32K"]
    lay = _gpu(decode_inputs(wl, "cpu")[0])
    idx, cnt, _, sel = _decode_select_both(lay, wl.topk, wl.n_init, wl.n_local)
    assert check_selection(idx, cnt, sel, wl.topk) == 0
    out = bskv.block_sparse_attn_decode(lay["q"], lay["k"], lay["v"], idx, cnt, lay["seq_len"], wl.scale)
    torch.cuda.synchronize()
    want = orc.attend_decode(np64(lay["q"]), np64(lay["k"]), np64(lay["v"]), sel.idx, sel.cnt, [wl.T] * wl.B,
                             wl.scale, 64)
    assert max_abs(np64(out), want) < 2e-2


def test_attn_decode_full_budget_is_dense_attention():
    lens = [64 * 12, 64 * 7 + 9]
    c, sel, lens_np = _attn_case(11, 2, 8, 2, 128, 64 * 12, "bf16", lens, topk=64, n_local=2)
    idx, cnt = bskv.forecast_block_score_topk(c["f"], _kc_gpu(c["k"], c["seq_len"]), 64, 1, 2, seq_len=c["seq_len"])
    out = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"])
    torch.cuda.synchronize()
    q, k, v = np64(c["q"]), np64(c["k"]), np64(c["v"])
    for b, L in enumerate(lens):
        for h in range(8):
            g = h // 4
            lg = k[b, g, :L] @ q[b, h] / math.sqrt(128)
            w = np.exp(lg - lg.max())
            w /= w.sum()
            assert max_abs(np64(out)[b, h], w @ v[b, g, :L]) < 2e-2


# ----------------------------------------------------------------------------- a3p / a4p prefill
def _prefill_case(seed, B, Hq, Hkv, d, T, q_start, Tq, topk, n_local, n_plant=3):
    c = _gpu(random_prefill_case(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, n_plant=n_plant))
    lens = torch.full((B,), T, dtype=torch.int64, device=DEV)
    kc = _kc_gpu(c["k"], lens)
    f_chunk = c["f"][:, :, q_start:q_start + Tq].contiguous()
    q_chunk = c["q"][:, :, q_start:q_start + Tq].contiguous()
    idx, cnt = bskv.forecast_block_score_topk(f_chunk, kc, topk, 1, n_local, q_start=q_start, prefill=True)
    torch.cuda.synchronize()
    kc_or = orc.kv_block_meanpool(np64(c["k"]), 64)
    sel = orc.prefill_select(np64(f_chunk), kc_or, q_start, topk, 1, n_local, 64)
    return c, q_chunk, idx, cnt, sel


@pytest.mark.parametrize("q_start,Tq", [(0, 1024), (1024, 1024), (512, 300)])
def test_prefill_selection(q_start, Tq):
    c, _, idx, cnt, sel = _prefill_case(21, 2, 8, 2, 128, 2048, q_start, Tq, topk=6, n_local=4)
    check_selection(idx, cnt, sel, 6)


@pytest.mark.parametrize("d,q_start,Tq,n_local", [(128, 64 * 2500, 64 * 40 + 5, 2), (64, 64 * 70, 64 * 33, 1)])
def test_prefill_selection_long_context(d, q_start, Tq, n_local):
    """Query blocks with more than 2048 candidates (the top-k's streaming
    path), more than 32 query blocks per chunk (two query-block tiles of the
    score contraction), a ragged last query block."""
    B, Hkv, T = 1, 2, q_start + Tq
    g = torch.Generator().manual_seed(d + Tq)
    f = torch.randn(B, Hkv, Tq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    lens = torch.full((B,), T, dtype=torch.int64, device=DEV)
    kc = _kc_gpu(k.to(DEV), lens)
    idx, cnt = bskv.forecast_block_score_topk(f.to(DEV), kc, 16, 1, n_local, q_start=q_start, prefill=True)
    torch.cuda.synchronize()
    sel = orc.prefill_select(np64(f), orc.kv_block_meanpool(np64(k), 64), q_start, 16, 1, n_local, 64)
    assert check_selection(idx, cnt, sel, 16) <= 4


@pytest.mark.parametrize("d,G,q_start,Tq", [(128, 4, 0, 1024), (128, 4, 1024, 1024), (128, 2, 512, 300),
                                            (64, 8, 256, 448), (128, 1, 0, 200), (64, 4, 1536, 512)])
def test_prefill_attention_on_oracle_lists(d, G, q_start, Tq):
    Hkv = 2
    c, q_chunk, _, _, sel = _prefill_case(31, 2, Hkv * G, Hkv, d, 2048, q_start, Tq, topk=5, n_local=3)
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    out = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt, q_start)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = [(b, h, t) for b in range(2) for h in range(Hkv * G) for t in rng.choice(Tq, 24, replace=False)]
    rows += [(0, 0, Tq - 1), (1, Hkv * G - 1, 0)]
    want = orc.attend_prefill(np64(q_chunk), np64(c["k"]), np64(c["v"]), sel.idx, sel.cnt, q_start,
                              1.0 / math.sqrt(d), 64, rows=rows)
    got = np64(out)
    err = max(max_abs(got[r], want[r]) for r in rows)
    assert err < 2e-2, err


@pytest.mark.parametrize("d,G", [(128, 4), (128, 8), (64, 2)])
def test_prefill_attention_wide_score_range(d, G):
    """Queries scaled up so that scaled scores span tens of units in base 2
    and each row's maximum keeps growing along its block list: the running
    maximum moves many times (also mid-list), and long lists (24 blocks)
    cover many ping-pong slots."""
    Hkv, T, q_start, Tq = 1, 4096, 2048, 1024
    c, q_chunk, _, _, sel = _prefill_case(61, 1, Hkv * G, Hkv, d, T, q_start, Tq, topk=16, n_local=8)
    ramp = torch.linspace(0.5, 6.0, Tq, device=DEV).view(1, 1, Tq, 1)
    q_chunk = (q_chunk.float() * ramp * 3.0).to(torch.bfloat16).contiguous()
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    assert int(cnt.max()) == 25
    out = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt, q_start)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = [(0, h, t) for h in range(Hkv * G) for t in rng.choice(Tq, 16, replace=False)]
    rows += [(0, 0, Tq - 1), (0, Hkv * G - 1, 0), (0, 0, 63), (0, 0, 64)]
    want = orc.attend_prefill(np64(q_chunk), np64(c["k"]), np64(c["v"]), sel.idx, sel.cnt, q_start,
                              1.0 / math.sqrt(d), 64, rows=rows)
    got = np64(out)
    err = max(max_abs(got[r], want[r]) for r in rows)
    assert err < 2e-2, err


@pytest.mark.parametrize("d,G", [(128, 4), (64, 2)])
def test_prefill_attention_ignores_listed_future_blocks(d, G):
    """A list passed through the boundary may name blocks after the query
    block: none of their tokens is attended (all lie after every query
    position of the block), while the query block itself stays causal per
    token.  Each query block's list gets two future blocks in place of two
    top-k entries (kept ascending, the count unchanged)."""
    Hkv, T, q_start, Tq = 2, 2048, 512, 1024
    c, q_chunk, _, _, sel = _prefill_case(71, 1, Hkv * G, Hkv, d, T, q_start, Tq, topk=6, n_local=3)
    NB = T // 64
    idx_np, cnt_np = sel.idx.copy(), sel.cnt.copy()
    n_future = 0
    for g in range(Hkv):
        for qi in range(idx_np.shape[2]):
            qb = q_start // 64 + qi
            c0 = int(cnt_np[0, g, qi])
            lst = [int(j) for j in idx_np[0, g, qi, :c0]]
            keep = [j for j in lst if j >= qb - 2 or j == 0]       # initial + local blocks
            top = [j for j in lst if j not in keep]
            fut = [j for j in (qb + 1, qb + 7) if j < NB][: len(top)]
            new = sorted(keep + top[: len(top) - len(fut)] + fut)
            assert len(new) == c0
            idx_np[0, g, qi, :c0] = new
            n_future += len(fut)
    assert n_future > 0
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(cnt_np.astype(np.int32)).to(DEV)
    out = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt, q_start)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = [(0, h, t) for h in range(Hkv * G) for t in rng.choice(Tq, 24, replace=False)]
    rows += [(0, 0, 0), (0, 0, 63), (0, Hkv * G - 1, Tq - 1)]
    want = orc.attend_prefill(np64(q_chunk), np64(c["k"]), np64(c["v"]), idx_np, cnt_np, q_start,
                              1.0 / math.sqrt(d), 64, rows=rows)
    got = np64(out)
    err = max(max_abs(got[r], want[r]) for r in rows)
    assert err < 2e-2, err


def test_partial_kv_blocks_are_rejected():
    """K/V buffers whose token axis is not a whole number of blocks are
    refused (the binding raises before calling; the C ABI returns
    BSKV_EINVAL), instead of silently dropping the partial block."""
    c = _gpu(random_decode_case(3, B=1, Hq=4, Hkv=1, d=128, T=300, dtype="bf16", seq_len=[300]))
    idx = torch.tensor([[[0, 4]]], dtype=torch.int32, device=DEV)
    cnt = torch.tensor([[2]], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="whole 64-token blocks"):
        bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"])
    q = torch.zeros(1, 4, 300, 128, dtype=torch.bfloat16, device=DEV)
    pidx = torch.zeros(1, 1, 5, 2, dtype=torch.int32, device=DEV)
    pcnt = torch.ones(1, 1, 5, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="whole 64-token blocks"):
        bskv.block_sparse_attn_prefill(q, c["k"], c["v"], pidx, pcnt, 0)
    # a cache allocated in whole blocks with a ragged length works
    kp = torch.zeros(1, 1, 320, 128, dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    kp[:, :, :300], vp[:, :, :300] = c["k"], c["v"]
    out = bskv.block_sparse_attn_decode(c["q"], kp, vp, idx, cnt, c["seq_len"])
    torch.cuda.synchronize()
    want = orc.attend_decode(np64(c["q"]), np64(kp), np64(vp), idx.cpu().numpy(), cnt.cpu().numpy(), [300],
                             1 / math.sqrt(128), 64)
    assert max_abs(np64(out), want) < 2e-2


def test_prefill_full_budget_is_causal_attention():
    B, Hq, Hkv, d, T = 1, 4, 1, 128, 512
    c, q_chunk, idx, cnt, _ = _prefill_case(41, B, Hq, Hkv, d, T, 0, T, topk=64, n_local=2)
    out = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt, 0)
    torch.cuda.synchronize()
    want = torch.nn.functional.scaled_dot_product_attention(
        q_chunk.double().cpu(), c["k"].double().cpu().repeat_interleave(4, 1),
        c["v"].double().cpu().repeat_interleave(4, 1), is_causal=True).numpy()
    assert max_abs(np64(out), want) < 2e-2


def test_chunked_prefill_matches_single_chunk():
    c, q_all, idx_all, cnt_all, _ = _prefill_case(51, 1, 4, 1, 128, 1024, 0, 1024, topk=4, n_local=2)
    whole = bskv.block_sparse_attn_prefill(q_all, c["k"], c["v"], idx_all, cnt_all, 0)
    lens = torch.full((1,), 1024, dtype=torch.int64, device=DEV)
    kc = _kc_gpu(c["k"], lens)
    parts = []
    for q0 in range(0, 1024, 256):
        f = c["f"][:, :, q0:q0 + 256].contiguous()
        i, n = bskv.forecast_block_score_topk(f, kc, 4, 1, 2, q_start=q0, prefill=True)
        assert torch.equal(i, idx_all[:, :, q0 // 64:(q0 + 256) // 64])
        parts.append(bskv.block_sparse_attn_prefill(q_all[:, :, q0:q0 + 256].contiguous(), c["k"], c["v"], i, n, q0))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=2), whole)


# ----------------------------------------------------------------------------- a5
def test_prefetch_from_pinned_host_and_ring_attention():
    """The ring holds U blocks, far fewer than the sequence has: blocks whose id
    lies past the ring's length must still be attended (ring position u holds
    list entry u).  Ragged lengths, one with a partial newest block."""
    wl = WORKLOADS["offload-decode-B16-128K-32L"]
    B, T = 3, 64 * 200
    lay = decode_inputs(wl, DEV, layers=1, B=B, T=T)[0]
    lay["seq_len"] = torch.tensor([T, T - 64 * 37 - 5, 64 * 90], dtype=torch.int64, device=DEV)
    assert wl.U * 64 < T - 64 * 40
    kc = _kc_gpu(lay["k"], lay["seq_len"])
    f = bskv.forecast_proj(lay["x_sel"], lay["w_sel"], wl.Hkv, wl.d)
    idx, cnt = bskv.forecast_block_score_topk(f, kc, wl.topk, wl.n_init, wl.n_local, seq_len=lay["seq_len"])
    hk = torch.empty(lay["k"].shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(lay["v"].shape, dtype=torch.bfloat16, pin_memory=True)
    hk.copy_(lay["k"])
    hv.copy_(lay["v"])
    U = wl.U
    ring_k = torch.full((B, wl.Hkv, U, 64, wl.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ring_v = torch.full_like(ring_k, float("nan"))
    side = torch.cuda.Stream(DEV)
    ev = torch.cuda.Event()
    ev.record()
    side.wait_event(ev)
    bskv.prefetch_selected_blocks(hk, hv, idx, cnt, ring_k, ring_v, n_workgroups=64, stream=side)
    done = torch.cuda.Event()
    done.record(side)
    torch.cuda.current_stream().wait_event(done)
    out_ring = bskv.block_sparse_attn_decode(lay["q"], ring_k, ring_v, idx, cnt, lay["seq_len"], ring=True)
    out_res = bskv.block_sparse_attn_decode(lay["q"], lay["k"], lay["v"], idx, cnt, lay["seq_len"])
    torch.cuda.synchronize()
    want = orc.gather_selected_blocks(hk.view(torch.int16).numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), 64)
    got = ring_k.view(torch.int16).cpu().numpy()
    cn = cnt.cpu().numpy()
    for b in range(B):
        for g in range(wl.Hkv):
            assert np.array_equal(got[b, g, :cn[b, g]], want[b, g, :cn[b, g]])
    assert torch.equal(out_ring, out_res), "ring read must equal resident read bit for bit"
    gi = idx.cpu().numpy()
    lens = lay["seq_len"].cpu().numpy()
    assert (gi[cn > 0] >= wl.U).any(), "some selected block must lie past the ring's length"
    want_o = orc.attend_decode(np64(lay["q"]), np64(lay["k"]), np64(lay["v"]), gi, cn, lens, wl.scale, 64)
    assert max_abs(np64(out_ring), want_o) < 2e-2


# ----------------------------------------------------------------------------- widened projection
def _bf16_close(got, want, rel=2.0 ** -8, abs_tol=1e-3):
    """bf16 outputs of fp32 sums against the fp64 oracle: one rounding to
    bf16 (half an ulp, 2^-9 relative) plus the fp32 summation error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return bool(np.all(np.abs(got - want) <= rel * np.abs(want) + abs_tol))


@pytest.mark.parametrize("B,hidden,Hq,Hkv,d", [(3, 1024, 8, 2, 128), (16, 4096, 32, 8, 128), (5, 2048, 4, 4, 64),
                                           (40, 1024, 8, 2, 64), (64, 1024, 4, 1, 128), (7, 4096, 16, 4, 64),
                                           (1, 4096, 32, 8, 128)])
def test_qkvf_proj_decode(B, hidden, Hq, Hkv, d):
    g = torch.Generator().manual_seed(B + hidden)
    x = torch.randn(B, hidden, generator=g).to(torch.bfloat16)
    w = (torch.randn(hidden, (Hq + 3 * Hkv) * d, generator=g) * 0.02).to(torch.bfloat16)
    T = 64 * 4
    kc = torch.full((B, Hkv, T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    lens = torch.tensor([(37 * b) % T + 1 for b in range(B)], dtype=torch.int64)
    q, f = bskv.qkvf_proj_decode(x.to(DEV), w.t().contiguous().to(DEV), Hq, Hkv, kc, vc, lens.to(DEV))
    torch.cuda.synchronize()
    wq, wk, wv, wf = orc.qkvf_proj(np64(x), np64(w), Hq, Hkv, d)
    assert _bf16_close(np64(q), wq)
    mag = (np.abs(np64(x)) @ np.abs(np64(w)))[:, (Hq + 2 * Hkv) * d:].reshape(wf.shape)
    assert fp32_sum_close(np64(f), wf, mag, hidden)
    kn, vn = np64(kc), np64(vc)
    for b, L in enumerate(lens.tolist()):
        assert _bf16_close(kn[b, :, L - 1], wk[b]) and _bf16_close(vn[b, :, L - 1], wv[b])
        rest = np.delete(kn[b], L - 1, axis=1)
        assert np.isnan(rest).all(), "only the new token's row is written"


@pytest.mark.parametrize("B,Tq,hidden,Hq,Hkv,d,q_start", [(2, 256, 512, 8, 2, 128, 0), (1, 64 * 5 + 17, 512, 8, 2, 128, 128),
                                                         (2, 512, 256, 32, 8, 128, 64), (3, 200, 192, 4, 2, 64, 0)])
def test_qkvf_proj_prefill(B, Tq, hidden, Hq, Hkv, d, q_start):
    """Q/K/V per token (bf16) and each query block's Forecast sum (fp32)
    against the oracle; a ragged last block; an 8 x 8 tile case takes the
    XCD-aware tile order."""
    g = torch.Generator().manual_seed(Tq + hidden + Hq)
    x = torch.randn(B, Tq, hidden, generator=g).to(torch.bfloat16)
    w = (torch.randn(hidden, (Hq + 3 * Hkv) * d, generator=g) * 0.05).to(torch.bfloat16)
    T = q_start + Tq + 64
    kc = torch.full((B, Hkv, T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    q, fp = bskv.qkvf_proj_prefill(x.to(DEV), w.t().contiguous().to(DEV), Hq, Hkv, kc, vc, q_start=q_start)
    torch.cuda.synchronize()
    wq, wk, wv, wfp = orc.qkvf_proj_prefill(np64(x), np64(w), Hq, Hkv, d, 64)
    assert _bf16_close(np64(q), wq)
    kn, vn = np64(kc), np64(vc)
    assert _bf16_close(kn[:, :, q_start:q_start + Tq], wk) and _bf16_close(vn[:, :, q_start:q_start + Tq], wv)
    assert np.isnan(kn[:, :, :q_start]).all() and np.isnan(kn[:, :, q_start + Tq:]).all()
    # magnitude of each query block's Forecast sum: sum over its tokens of |x_t| @ |W_F|
    per_tok = (np.abs(np64(x)) @ np.abs(np64(w))[:, (Hq + 2 * Hkv) * d:]).reshape(B, Tq, Hkv, d)
    n_qb = (Tq + 63) // 64
    mag = np.zeros((B, Hkv, n_qb, d))
    for t in range(Tq):
        mag[:, :, t // 64] += per_tok[:, t]
    assert fp32_sum_close(np64(fp), wfp, mag, 64 * hidden)


def test_qkvf_prefill_chunk_end_to_end():
    """One prefill chunk through the widened projection: its K/V land in the
    cache, the compressed keys are pooled, each query block is selected from
    its summed Forecast and attends with the projected queries; against the
    oracle chain on the same bf16 inputs."""
    B, Hq, Hkv, d, hidden, T = 2, 8, 2, 128, 256, 64 * 24
    q_start, Tq = 64 * 8, 64 * 16
    g = torch.Generator().manual_seed(77)
    x = torch.randn(B, Tq, hidden, generator=g).to(torch.bfloat16)
    w = (torch.randn(hidden, (Hq + 3 * Hkv) * d, generator=g) * 0.05).to(torch.bfloat16)
    k_prev = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    v_prev = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    kc_cache, vc_cache = k_prev.clone().to(DEV), v_prev.clone().to(DEV)
    q, fp = bskv.qkvf_proj_prefill(x.to(DEV), w.t().contiguous().to(DEV), Hq, Hkv, kc_cache, vc_cache, q_start=q_start)
    seq_len = torch.full((B,), q_start + Tq, dtype=torch.int64, device=DEV)
    kcmp = _kc_gpu(kc_cache, seq_len)
    idx, cnt = bskv.forecast_block_score_topk_pooled(fp, kcmp, 4, 1, 2, q_start=q_start)
    out = bskv.block_sparse_attn_prefill(q, kc_cache, vc_cache, idx, cnt, q_start)
    torch.cuda.synchronize()
    # oracle chain on the GPU's bf16 Q/K/V (the bf16 rounding of the projection is the kernel's)
    k_all, v_all = np64(kc_cache), np64(vc_cache)
    wq, wk, wv, wfp = orc.qkvf_proj_prefill(np64(x), np64(w), Hq, Hkv, d, 64)
    kc_or = orc.kv_block_meanpool(k_all, 64, seq_len=seq_len.cpu().numpy())
    sel = orc.prefill_select_pooled(wfp, kc_or, q_start, 4, 1, 2, 64)
    assert check_selection(idx, cnt, sel, 4) <= 2
    want = orc.attend_prefill(np64(q), k_all, v_all, idx.cpu().numpy(), cnt.cpu().numpy(), q_start, 1 / math.sqrt(d), 64)
    assert max_abs(np64(out), want) < 2e-2


# ----------------------------------------------------------------------------- resident block cache
def _drifting_lists(rng, n_calls, B, H, U, universe, churn):
    """Sorted distinct lists of up to U blocks per (b, g); each call swaps
    `churn` blocks of the previous list for others; some lists are short."""
    cur = [[sorted(rng.choice(universe, U, replace=False).tolist()) for _ in range(H)] for _ in range(B)]
    out = []
    for _ in range(n_calls):
        idx = np.full((B, H, U), -1, dtype=np.int32)
        cnt = np.zeros((B, H), dtype=np.int32)
        for b in range(B):
            for g in range(H):
                keep = set(rng.choice(cur[b][g], U - churn, replace=False).tolist())
                pool = np.setdiff1d(np.arange(universe), np.array(sorted(keep)))
                new = set(rng.choice(pool, churn, replace=False).tolist())
                cur[b][g] = sorted(keep | new)
                c = int(rng.integers(max(0, U - 3), U + 1))
                idx[b, g, :c] = cur[b][g][:c]
                cnt[b, g] = c
        out.append((idx, cnt))
    return out


@pytest.mark.parametrize("S,U,universe,churn,calls", [(8, 5, 14, 2, 30), (128, 69, 2043, 4, 40),
                                                      (96, 96, 400, 10, 12), (1024, 1000, 5000, 50, 6)])
def test_block_cache_plan_matches_oracle(S, U, universe, churn, calls):
    """The slot table, slot map, copies and counts equal the oracle's LRU
    exactly, lookup after lookup (integer work: bit-exact)."""
    rng = np.random.default_rng(S + U)
    B, H = 2, 3
    cache = bskv.BlockCache(B, H, S, 64, device=DEV)
    tags = np.full((B, H, S), -1, dtype=np.int64)
    stamps = np.full((B, H, S), -1, dtype=np.int64)
    clock = np.zeros((B, H), dtype=np.int64)
    for idx, cnt in _drifting_lists(rng, calls, B, H, U, universe, churn):
        slot, fill, n_fill = bskv.block_cache_plan(cache, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV))
        torch.cuda.synchronize()
        w_slot, w_fill, w_n = orc.block_cache_plan(tags, stamps, clock, idx, cnt)
        assert np.array_equal(slot.cpu().numpy(), w_slot)
        assert np.array_equal(fill.cpu().numpy(), w_fill)
        assert np.array_equal(n_fill.cpu().numpy(), w_n)
        assert np.array_equal(cache.tags.cpu().numpy(), tags)
        assert np.array_equal(cache.stamps.cpu().numpy(), stamps)
        assert np.array_equal(cache.clock.cpu().numpy(), clock)
    cache.reset()
    torch.cuda.synchronize()
    assert (cache.tags == -1).all() and (cache.stamps == -1).all() and (cache.clock == 0).all()


@pytest.mark.parametrize("B,n_wg", [(500, 300), (520, 300), (6, 5)])
def test_cache_fill_copies_every_missing_block(B, n_wg):
    """The fill deals a layer's missing blocks out over its workgroups (up
    to 4096 (b, g) units; above that each workgroup copies whole units):
    every listed block lands in its slot, bytewise, at 4000 units, at 4160
    units and with fewer workgroups than blocks; ragged list lengths."""
    H, D, nb, U = 8, 64, 6, 4
    g = torch.Generator(device=DEV).manual_seed(71 + B)
    k = torch.randn(B, H, nb * 64, D, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(B, H, nb * 64, D, generator=g, device=DEV).to(torch.bfloat16)
    # each unit lists cnt distinct ascending blocks of the nb (cnt 0..U), padded with -1
    cnt = torch.randint(0, U + 1, (B, H), generator=g, device=DEV).to(torch.int32)
    perm = torch.rand(B, H, nb, generator=g, device=DEV).argsort(-1)[..., :U].sort(-1).values
    pos = torch.arange(U, device=DEV)
    idx = torch.where(pos < cnt[..., None], perm, -1).to(torch.int32).contiguous()
    cache = bskv.BlockCache(B, H, U + 1, D, device=DEV)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    slot, fill, n_fill = bskv.block_cache_plan(cache, idx, cnt)
    bskv.prefetch_cache_fill(k, v, idx, slot, fill, n_fill, cache, n_workgroups=n_wg)
    torch.cuda.synchronize()
    assert torch.equal(n_fill, cnt), "a first lookup copies every listed block"
    valid = pos < cnt[..., None].long()
    j = idx.long().clamp(min=0)
    s_ = slot.long().clamp(min=0)
    for src, dst in ((k, cache.k), (v, cache.v)):
        want = src.view(B, H, nb, 64, D).gather(2, j[..., None, None].expand(-1, -1, -1, 64, D))
        got = dst.gather(2, s_[..., None, None].expand(-1, -1, -1, 64, D))
        m = valid[..., None, None].expand_as(got)
        assert torch.equal(got.view(torch.int16)[m], want.view(torch.int16)[m])


@pytest.mark.parametrize("host", [True, False])
def test_cache_fill_and_cached_attention_over_steps(host):
    """Three decode steps of one layer through a block cache smaller than the
    sequence: lookup, copy of the missing blocks (from pinned host memory or
    from device memory), attention from the cache.  The cache slots hold the
    listed blocks bytewise, the cached attention equals the resident one bit
    for bit and the oracle within bf16 tolerance.  Ragged lengths, a partial
    newest block."""
    wl = WORKLOADS["offload-decode-B16-128K-32L"]
    B, T, S = 3, 64 * 200, 96
    lay = decode_inputs(wl, DEV, layers=1, B=B, T=T)[0]
    lay["seq_len"] = torch.tensor([T, T - 64 * 37 - 5, 64 * 90], dtype=torch.int64, device=DEV)
    kc = _kc_gpu(lay["k"], lay["seq_len"])
    if host:
        src_k = torch.empty(lay["k"].shape, dtype=torch.bfloat16, pin_memory=True)
        src_v = torch.empty(lay["v"].shape, dtype=torch.bfloat16, pin_memory=True)
        src_k.copy_(lay["k"])
        src_v.copy_(lay["v"])
    else:
        src_k, src_v = lay["k"], lay["v"]
    cache = bskv.BlockCache(B, wl.Hkv, S, wl.d, device=DEV)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    g = torch.Generator(device=DEV).manual_seed(9)
    resident = [set() for _ in range(B * wl.Hkv)]
    kh = lay["k"].view(torch.int16).cpu().numpy()
    f0 = bskv.forecast_proj(lay["x_sel"], lay["w_sel"], wl.Hkv, wl.d)
    # step 0 fills the cache; step 1's unrelated Forecast lists other blocks
    # (evictions); step 2 returns to the first lists (part resident, part refetched)
    forecasts = [f0, torch.randn(f0.shape, generator=g, device=DEV), f0]
    for step, f in enumerate(forecasts):
        idx, cnt = bskv.forecast_block_score_topk(f.contiguous(), kc, wl.topk, wl.n_init, wl.n_local,
                                                  seq_len=lay["seq_len"])
        slot, fill, n_fill = bskv.block_cache_plan(cache, idx, cnt)
        side = torch.cuda.Stream(DEV)
        ev = torch.cuda.Event()
        ev.record()
        side.wait_event(ev)
        bskv.prefetch_cache_fill(src_k, src_v, idx, slot, fill, n_fill, cache, n_workgroups=17, stream=side)
        done = torch.cuda.Event()
        done.record(side)
        torch.cuda.current_stream().wait_event(done)
        out_c = bskv.block_sparse_attn_decode_cached(lay["q"], cache, slot, idx, cnt, lay["seq_len"])
        out_r = bskv.block_sparse_attn_decode(lay["q"], lay["k"], lay["v"], idx, cnt, lay["seq_len"])
        torch.cuda.synchronize()
        gi, cn, sl = idx.cpu().numpy(), cnt.cpu().numpy(), slot.cpu().numpy()
        fl, nf = fill.cpu().numpy(), n_fill.cpu().numpy()
        ck = cache.k.view(torch.int16).cpu().numpy()
        for b in range(B):
            for h in range(wl.Hkv):
                c = int(cn[b, h])
                listed = set(gi[b, h, :c].tolist())
                assert int(nf[b, h]) == len(listed - resident[b * wl.Hkv + h])
                assert {int(gi[b, h, u]) for u in fl[b, h, :nf[b, h]]} == listed - resident[b * wl.Hkv + h]
                resident[b * wl.Hkv + h] = set(cache.tags[b, h].cpu().numpy().tolist()) - {-1}
                for u in range(c):
                    j = int(gi[b, h, u])
                    assert np.array_equal(ck[b, h, sl[b, h, u]], kh[b, h, 64 * j: 64 * (j + 1)]), (step, b, h, u)
        assert torch.equal(out_c, out_r), "cached read must equal resident read bit for bit"
        want = orc.attend_decode(np64(lay["q"]), np64(lay["k"]), np64(lay["v"]), gi, cn,
                                 lay["seq_len"].cpu().numpy(), wl.scale, 64)
        assert max_abs(np64(out_c), want) < 2e-2
        if step > 0:
            assert 0 < nf.sum() < cn.sum(), "a later step reuses some resident blocks and fetches others"


# ----------------------------------------------------------------------------- fused decode layer
def _layer_case(dtype, d, G, B, T, lens, seed):
    wl = WORKLOADS["decode-B4-32K"]
    Hkv = 4
    c = _gpu(random_decode_case(seed, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype=dtype, hidden=512, seq_len=lens))
    c2 = _gpu(random_decode_case(seed + 100, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype=dtype, seq_len=lens))
    kc = _kc_gpu(c["k"], c["seq_len"])
    kc_next = _kc_gpu(c2["k"], c2["seq_len"])
    # this layer's own block lists (from any Forecast: the oracle's, on the pooled keys)
    sel = orc.decode_select(np64(c2["f"]), orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens), lens, 6, 1, 2, 64)
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    return c, c2, kc, kc_next, idx, cnt


def _next_lists(c, kc, scores, topk, n_init, n_local, ws=None):
    """The next layer's lists from the scores a lookahead call left: the
    top-k stage alone (stage 1, scores given, no lookahead)."""
    U = topk + n_init + n_local
    B, Hkv = kc.shape[0], kc.shape[1]
    idx = torch.full((B, Hkv, U), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
    kw = {} if ws is None else {"ws": ws}
    bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc, idx, cnt, scores=scores, topk=topk,
                                n_init=n_init, n_local=n_local, stages=1, **kw)
    return idx, cnt


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f32", 64, 2), ("bf16", 64, 8)])
def test_decode_layer_equals_the_per_op_calls(dtype, d, G):
    lens = [64 * 30, 64 * 30 - 5, 64 * 17, 64 * 30]
    c, c2, kc, kc_next, idx, cnt = _layer_case(dtype, d, G, 4, 64 * 30, lens, 3)
    # stale rows where the newest blocks go, to see them rewritten
    kc_a = kc.clone()
    kc_a[:, :, 29] = float("nan")
    kc_a[:, :, 16] = float("nan")
    kc_b = kc_a.clone()
    scale = 1.0 / math.sqrt(d)
    bskv.kv_block_meanpool(c["k"], c["seq_len"], kc_a, 0, kc.shape[2], newest_only=True)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], 4, d)
    idx_a, cnt_a = bskv.forecast_block_score_topk(f, kc_next, 6, 1, 2, seq_len=c["seq_len"])
    out_a = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"], scale)
    out_b, sc_next = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc_b, idx, cnt, scale,
                                                 x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=6, n_init=1,
                                                 n_local=2)
    idx_b, cnt_b = _next_lists(c2, kc_next, sc_next, 6, 1, 2)
    torch.cuda.synchronize()
    assert torch.equal(kc_a.nan_to_num(7.0), kc_b.nan_to_num(7.0))
    assert torch.equal(idx_a, idx_b) and torch.equal(cnt_a, cnt_b)
    assert torch.equal(out_a, out_b)
    # and against the oracle
    lens_np = np.array(lens)
    f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), 4, d)
    kc_next_or = orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens)
    sel = orc.decode_select(f_or, kc_next_or, lens_np, 6, 1, 2, 64)
    check_selection(idx_b, cnt_b, sel, 6)
    # the raw candidate scores handed to the next call, against the oracle's
    sc = np64(sc_next)
    for bg in range(sc.shape[0] * sc.shape[1]):
        b, g = divmod(bg, sc.shape[1])
        for j, v in sel.scores[bg].items():
            assert abs(sc[b, g, j] - v) <= 1e-4 * max(1.0, abs(v)), (b, g, j)
    want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(), lens_np,
                             scale, 64)
    assert max_abs(np64(out_b), want) < (1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f32", 64, 2)])
def test_decode_layer_short_sequences(dtype, d, G):
    """Sequences of 1, 64 and 65 tokens beside a long one: no candidates
    (only the local and initial blocks), a just-completed first block (the
    newest-block update writes block 0) and one token past it.  The fused
    layer (deferred, then the next call ranking those scores) equals the
    per-op calls bit for bit and the oracle."""
    lens = [1, 64, 65, 64 * 30]
    c, c2, kc, kc_next, idx, cnt = _layer_case(dtype, d, G, 4, 64 * 30, lens, 17)
    scale = 1.0 / math.sqrt(d)
    kc_a, kc_b = kc.clone(), kc.clone()
    kc_a[:, :, 0] = float("nan")
    kc_b[:, :, 0] = float("nan")
    bskv.kv_block_meanpool(c["k"], c["seq_len"], kc_a, 0, kc.shape[2], newest_only=True)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], 4, d)
    idx_a, cnt_a = bskv.forecast_block_score_topk(f, kc_next, 6, 1, 2, seq_len=c["seq_len"])
    out_a = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"], scale)
    out_b, sc_next = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc_b, idx, cnt, scale,
                                                 x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=6, n_init=1,
                                                 n_local=2)
    idx_b, cnt_b = _next_lists(c2, kc_next, sc_next, 6, 1, 2)
    torch.cuda.synchronize()
    assert torch.equal(kc_a.nan_to_num(7.0), kc_b.nan_to_num(7.0))
    assert torch.equal(idx_a, idx_b) and torch.equal(cnt_a, cnt_b)
    assert torch.equal(out_a, out_b)
    lens_np = np.array(lens)
    assert int(cnt_b[0].max()) == 1 and int(cnt_b[1].max()) == 1, "one block, no candidates: the local block alone"
    sel = orc.decode_select(orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), 4, d),
                            orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens), lens_np, 6, 1, 2, 64)
    check_selection(idx_b, cnt_b, sel, 6)
    want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(), lens_np,
                             scale, 64)
    assert max_abs(np64(out_b), want) < (1e-4 if dtype == "f32" else 2e-2)
    pooled = orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens)
    assert max_abs(np64(kc_b)[1, :, 0], pooled[1, :, 0]) < 1e-4, "block 0 of the 64-token sequence"


def test_decode_layer_top_k_from_scores_in_the_same_call():
    """A call given the previous call's scores writes its own lists first
    and attends over them: equal to the lists and output of the per-op
    selection and attention."""
    lens = [64 * 30, 64 * 23 + 9]
    c, c2, kc, kc_next, idx, cnt = _layer_case("bf16", 128, 4, 2, 64 * 30, lens, 13)
    scale = 1.0 / math.sqrt(128)
    _, sc1 = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt, scale,
                                         x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=6, n_init=1, n_local=2)
    # layer 1 (c2's q/k/v), selected by layer 0's scores, is also the last layer
    i1 = torch.full_like(idx, -7)
    n1 = torch.full_like(cnt, -7)
    out1, none = bskv.decode_layer_lookahead(c2["q"], c2["k"], c2["v"], c2["seq_len"], kc_next.clone(), i1, n1, scale,
                                             scores=sc1, topk=6, n_init=1, n_local=2)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], 4, 128)
    i_ref, n_ref = bskv.forecast_block_score_topk(f, kc_next, 6, 1, 2, seq_len=c["seq_len"])
    out_ref = bskv.block_sparse_attn_decode(c2["q"], c2["k"], c2["v"], i_ref, n_ref, c2["seq_len"], scale)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(i1, i_ref) and torch.equal(n1, n_ref) and torch.equal(out1, out_ref)


def test_decode_layer_graph_replays():
    """The merge of the last attention split hands results over through
    arrival counters in the workspace, which every launch leaves at zero:
    replays of a captured pair of layer calls (lookahead, then the next
    layer from its scores), with eager calls between them, match the eager
    result exactly."""
    lens = [64 * 20, 64 * 20 - 3]
    c, c2, kc, kc_next, idx, cnt = _layer_case("bf16", 128, 4, 2, 64 * 20, lens, 21)
    ws = torch.zeros(bskv.workspace_bytes("layer", 2, 16, 4, 128, 512, kc.shape[2], 9, 1), dtype=torch.uint8,
                     device=DEV)
    kc_g, kcn_g = kc.clone(), kc_next.clone()
    out_g, out2_g = torch.empty(2, 16, 128, device=DEV), torch.empty(2, 16, 128, device=DEV)
    sc = torch.empty(2, 4, kc.shape[2], device=DEV)
    i_g, n_g = torch.empty_like(idx), torch.empty_like(cnt)

    def call():
        bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc_g, idx, cnt, out=out_g, x=c["x_sel"],
                                    w=c["w_sel"], kc_next=kc_next, scores_next=sc, topk=6, n_init=1, n_local=2, ws=ws)
        bskv.decode_layer_lookahead(c2["q"], c2["k"], c2["v"], c2["seq_len"], kcn_g, i_g, n_g, out=out2_g, scores=sc,
                                    topk=6, n_init=1, n_local=2, ws=ws)
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out_g, out2_g, i_g, n_g, kc_g, kcn_g)]
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        call()
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out_g.zero_()
        out2_g.zero_()
        i_g.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = (out_g, out2_g, i_g, n_g, kc_g, kcn_g)
        for a_, b_ in zip(got, ref):
            assert torch.equal(torch.nan_to_num(a_, nan=7.0), torch.nan_to_num(b_, nan=7.0)), rep
        call()                     # eager work between the replays, on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(out2_g, ref[1]) and torch.equal(i_g, ref[2]), rep


def test_decode_layer_stages_and_last_layer():
    lens = [64 * 20] * 2
    c, c2, kc, kc_next, idx, cnt = _layer_case("bf16", 128, 4, 2, 64 * 20, lens, 9)
    kc1, kc2 = kc.clone(), kc.clone()
    out1, s1 = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc1, idx, cnt, x=c["x_sel"],
                                           w=c["w_sel"], kc_next=kc_next, topk=6, n_init=1, n_local=2)
    s2 = torch.empty_like(s1)
    out2 = torch.empty_like(out1)
    for st in (1, 2):
        bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc2, idx, cnt, out=out2, x=c["x_sel"],
                                    w=c["w_sel"], kc_next=kc_next, scores_next=s2, topk=6, n_init=1, n_local=2,
                                    stages=st)
    out3, none = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt, topk=6,
                                             n_init=1, n_local=2)
    torch.cuda.synchronize()
    # scores are written for the candidates only; compare those
    cand = slice(1, 20 - 2)
    assert torch.equal(out1, out2) and torch.equal(s1[:, :, cand], s2[:, :, cand]) and torch.equal(kc1, kc2)
    assert none is None and torch.equal(out3, out1)


def test_decode_layer_shared_workspace_across_lookahead_and_last_layer():
    """One workspace serves a layer with a lookahead, a last layer (no
    projection partials in its layout) and another lookahead layer, in that
    order, as a model's layers share it: each call must equal the same call
    on a fresh zero-filled workspace."""
    lens = [64 * 40, 64 * 40 - 9]
    c, _, kc, kc_next, idx, cnt = _layer_case("bf16", 128, 4, 2, 64 * 40, lens, 31)
    nb = kc.shape[2]
    ws = torch.zeros(bskv.workspace_bytes("layer", 2, 16, 4, 128, 512, nb, 9, 1), dtype=torch.uint8, device=DEV)

    def run(shared, sel):
        kw = dict(x=c["x_sel"], w=c["w_sel"], kc_next=kc_next) if sel else {}
        own = ws if shared else torch.zeros_like(ws)
        out, sc = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt, topk=6,
                                              n_init=1, n_local=2, ws=own, **kw)
        return out, (sc[:, :, 1:nb - 2] if sel else None)
    for rnd in range(2):
        for sel in (True, False, True):
            got = run(True, sel)
            want = run(False, sel)
            torch.cuda.synchronize()
            assert torch.equal(got[0], want[0]), (rnd, sel)
            if sel:
                assert torch.equal(got[1], want[1]), (rnd, sel)
    # every complete call leaves the counter region (the first 2 * 65535 words) at zero
    assert int(ws[: 2 * 65535 * 4].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("lens", [[64 * 300, 64 * 300 - 17], [64 * 300 - 63, 64 * 131 + 5]])
def test_decode_layer_multi_slice_multi_block_splits(lens):
    """B2 x 4 KV heads with 300 blocks and top-64: several score slices per
    (b, g), and each attention split covers several blocks.  The next
    layer's compressed keys are pooled by the oracle, not taken from the
    GPU; the next layer's lists come from the scores by its own call."""
    T, topk = 64 * 300, 64
    c = _gpu(random_decode_case(41, B=2, Hq=16, Hkv=4, d=128, T=T, dtype="bf16", hidden=512, seq_len=lens))
    c2 = _gpu(random_decode_case(42, B=2, Hq=16, Hkv=4, d=128, T=T, dtype="bf16", seq_len=lens, plant=20,
                                 n_local=2))
    kc = _kc_gpu(c["k"], c["seq_len"])
    kc_next = _kc_gpu(c2["k"], c2["seq_len"])
    lens_np = np.array(lens)
    kc_or = orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens)
    kc_next_or = orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens)
    own = orc.decode_select(np64(c2["f"]), kc_or, lens_np, topk, 1, 2, 64)
    idx = torch.from_numpy(own.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(own.cnt.astype(np.int32)).to(DEV)
    U = topk + 3
    ws = torch.zeros(bskv.workspace_bytes("layer", 2, 16, 4, 128, 512, 300, U, 1), dtype=torch.uint8, device=DEV)
    for rep in range(2):                      # the second call reuses the counters the first left at zero
        kc_l = kc.clone()
        out, sc = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc_l, idx, cnt, x=c["x_sel"],
                                              w=c["w_sel"], kc_next=kc_next, topk=topk, n_init=1, n_local=2, ws=ws)
        i_n, c_n = _next_lists(c2, kc_next, sc, topk, 1, 2, ws=ws)
        torch.cuda.synchronize()
        f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), 4, 128)
        sel = orc.decode_select(f_or, kc_next_or, lens_np, topk, 1, 2, 64)
        check_selection(i_n, c_n, sel, topk)
        want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), own.idx, own.cnt, lens_np,
                                 1 / math.sqrt(128), 64)
        assert max_abs(np64(out), want) < 2e-2, rep
        done = ~np.isnan(kc_or)
        assert max_abs(np64(kc_l)[done], kc_or[done]) < 1e-4


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f32", 64, 2)])
def test_decode_layer_immediate_mode_equals_deferred_and_per_op(dtype, d, G):
    """Immediate mode (the next layer's top-k inside the second kernel, from
    agent-coherent scores handed over through an arrival counter) gives the
    lists of the deferred mode and of the per-op selection, with several
    score slices per (b, g), and leaves its counters at zero for a reused
    workspace."""
    lens = [64 * 300, 64 * 300 - 17, 64 * 131 + 5, 64 * 300]
    B, Hkv, T, topk = 4, 4, 64 * 300, 32
    c = _gpu(random_decode_case(51, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype=dtype, hidden=512, seq_len=lens))
    c2 = _gpu(random_decode_case(52, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype=dtype, seq_len=lens))
    kc, kc_next = _kc_gpu(c["k"], c["seq_len"]), _kc_gpu(c2["k"], c2["seq_len"])
    own = orc.decode_select(np64(c2["f"]), orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens), np.array(lens),
                            topk, 1, 2, 64)
    idx = torch.from_numpy(own.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(own.cnt.astype(np.int32)).to(DEV)
    U = topk + 3
    ws = torch.zeros(bskv.workspace_bytes("layer", B, Hkv * G, Hkv, d, 512, 300, U, 1 if dtype == "bf16" else 0),
                     dtype=torch.uint8, device=DEV)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], Hkv, d)
    i_ref, n_ref = bskv.forecast_block_score_topk(f, kc_next, topk, 1, 2, seq_len=c["seq_len"])
    for rep in range(2):
        i_im = torch.full_like(idx, -7)
        n_im = torch.full_like(cnt, -7)
        out_im, none = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt,
                                                   x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, idx_next=i_im,
                                                   cnt_next=n_im, topk=topk, n_init=1, n_local=2, ws=ws)
        out_de, sc = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt,
                                                 x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=topk, n_init=1,
                                                 n_local=2, ws=ws)
        i_de, n_de = _next_lists(c2, kc_next, sc, topk, 1, 2, ws=ws)
        torch.cuda.synchronize()
        assert none is None
        assert torch.equal(i_im, i_ref) and torch.equal(n_im, n_ref), rep
        assert torch.equal(i_de, i_ref) and torch.equal(n_de, n_ref), rep
        assert torch.equal(out_im, out_de), rep
    assert int(ws[: 2 * 65535 * 4].view(torch.int32).abs().sum()) == 0
    sel = orc.decode_select(orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), Hkv, d),
                            orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens), np.array(lens), topk, 1, 2, 64)
    check_selection(i_im, n_im, sel, topk)


@pytest.mark.gpu
def test_decode_layer_projection_spans_give_identical_scores():
    """The first kernel's projection workgroups span 128 rows of W when the
    kernel carries no top-k and 256 rows beside one; partials are stored per
    128 rows either way, so the next layer's raw candidate scores are bit for
    bit the same in both forms, rank to the per-op selection's lists, and
    match the oracle's scores to the fp32-sum bound."""
    lens = [64 * 300, 64 * 300 - 17, 64 * 131 + 5, 64 * 300]
    B, Hkv, G, d, T, topk, hidden = 4, 4, 4, 128, 64 * 300, 32, 1024
    c = _gpu(random_decode_case(61, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype="bf16", hidden=hidden, seq_len=lens))
    c2 = _gpu(random_decode_case(62, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype="bf16", seq_len=lens))
    kc, kc_next = _kc_gpu(c["k"], c["seq_len"]), _kc_gpu(c2["k"], c2["seq_len"])
    nb = kc.shape[2]
    # this layer's own raw candidate scores (from c2's Forecast), for the form
    # that ranks them in its first kernel
    i_own, n_own, sc_own = bskv.forecast_block_score_topk(c2["f"].contiguous(), kc, topk, 1, 2, seq_len=c["seq_len"],
                                                          return_scores=True)
    nan = lambda: torch.full((B, Hkv, nb), float("nan"), dtype=torch.float32, device=DEV)  # noqa: E731
    sc_a, sc_b = nan(), nan()
    # 128-row spans: no top-k in the first kernel, this layer's lists given
    out_a, _ = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), i_own, n_own,
                                           x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, scores_next=sc_a, topk=topk,
                                           n_init=1, n_local=2)
    # 256-row spans: the first kernel also ranks sc_own into this layer's lists
    i_b = torch.full_like(i_own, -7)
    n_b = torch.full_like(n_own, -7)
    out_b, _ = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), i_b, n_b,
                                           scores=sc_own, x=c["x_sel"], w=c["w_sel"], kc_next=kc_next,
                                           scores_next=sc_b, topk=topk, n_init=1, n_local=2)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], Hkv, d)
    i_ref, n_ref = bskv.forecast_block_score_topk(f, kc_next, topk, 1, 2, seq_len=c["seq_len"])
    i_a, n_a = _next_lists(c2, kc_next, sc_a, topk, 1, 2)
    torch.cuda.synchronize()
    assert torch.equal(i_b, i_own) and torch.equal(n_b, n_own)
    assert torch.equal(out_a, out_b)
    assert torch.equal(sc_a.nan_to_num(7.0), sc_b.nan_to_num(7.0)), "128- and 256-row spans differ"
    assert torch.equal(i_a, i_ref) and torch.equal(n_a, n_ref)
    f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), Hkv, d)
    kc_next_or = orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens)
    sel = orc.decode_select(f_or, kc_next_or, np.array(lens), topk, 1, 2, 64)
    check_selection(i_a, n_a, sel, topk)
    sc = np64(sc_a)
    for bg, row in enumerate(sel.scores):
        b, g = divmod(bg, Hkv)
        for j, v in row.items():
            assert abs(sc[b, g, j] - v) <= 1e-4 * max(1.0, abs(v)), (b, g, j)


def test_empty_sequence_selects_nothing_and_attends_to_nothing():
    """An empty sequence in the batch (seq_len 0) has no query block: the
    Forecast, multi-head and window selectors list no block for it (cnt 0),
    as the oracle does, and attention gives it the zero vector (reading R19);
    a caller's empty list for one group zeroes that group's heads only.  The
    fused decode layer does the same.  Every other row matches the oracle."""
    B, Hkv, G, d, T, topk = 3, 2, 4, 128, 64 * 40, 8
    lens = [64 * 40, 0, 64 * 17 + 3]
    c = _gpu(random_decode_case(71, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype="bf16", hidden=512))
    c2 = _gpu(random_decode_case(72, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype="bf16"))
    seq_len = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kc, kc_next = _kc_gpu(c["k"], seq_len), _kc_gpu(c2["k"], seq_len)
    scale = 1.0 / math.sqrt(d)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], Hkv, d)
    idx, cnt = bskv.forecast_block_score_topk(f, kc, topk, 1, 2, seq_len=seq_len)
    mi, mc = bskv.multihead_block_score_topk(c["q"], kc, topk, 1, 2, seq_len, scale)
    kcw = _kcw_gpu(c["k"], seq_len, 32, 16)
    wi, wc = bskv.forecast_window_score_topk(f, kcw, topk, 1, 2, seq_len=seq_len)
    cnt_e = cnt.clone()
    cnt_e[2, 1] = 0
    out = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt_e, seq_len, scale)
    out_l, sc_next = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], seq_len, kc.clone(), idx, cnt, scale,
                                                 x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=topk, n_init=1,
                                                 n_local=2)
    i_next, n_next = _next_lists(c2 | {"seq_len": seq_len}, kc_next, sc_next, topk, 1, 2)
    torch.cuda.synchronize()
    k64 = np64(c["k"])
    f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), Hkv, d)
    sel = orc.decode_select(f_or, orc.kv_block_meanpool(k64, 64, seq_len=lens), np.array(lens), topk, 1, 2, 64)
    msel = orc.multihead_select_decode(np64(c["q"]), orc.kv_block_meanpool(k64, 64, seq_len=lens), np.array(lens),
                                       topk, 1, 2, 64, scale)
    wsel = orc.decode_select_windows(f_or, orc.kv_window_meanpool(k64, 32, 16, seq_len=lens), np.array(lens), topk,
                                     1, 2, 64, 32, 16)
    nsel = orc.decode_select(f_or, orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens), np.array(lens), topk, 1,
                             2, 64)
    for (i_, c_), s in (((idx, cnt), sel), ((mi, mc), msel), ((wi, wc), wsel), ((i_next, n_next), nsel)):
        assert int(c_[1].abs().sum()) == 0 and bool((i_[1] == -1).all())
        check_selection(i_, c_, s, topk)
    want = orc.attend_decode(np64(c["q"]), k64, np64(c["v"]), idx.cpu().numpy(), cnt_e.cpu().numpy(), lens, scale, 64)
    got = np64(out)
    assert (got[1] == 0).all() and (got[2, G:] == 0).all()
    assert max_abs(got, want) < 2e-2
    want_l = orc.attend_decode(np64(c["q"]), k64, np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(), lens, scale, 64)
    assert (np64(out_l)[1] == 0).all()
    assert max_abs(np64(out_l), want_l) < 2e-2


def test_prefill_empty_list_gives_zero_rows():
    """A query block whose list a caller leaves empty (cnt 0) gets zero
    output rows (reading R19); the other query blocks are unchanged."""
    d, G, Hkv, q_start, Tq = 128, 4, 2, 1024, 256
    c, q_chunk, _, _, sel = _prefill_case(33, 1, Hkv * G, Hkv, d, 2048, q_start, Tq, topk=5, n_local=3)
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    cnt_e = cnt.clone()
    cnt_e[0, 1, 2] = 0                          # KV head 1, third query block of the chunk
    out = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt_e, q_start)
    ref = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt, q_start)
    torch.cuda.synchronize()
    got, full = np64(out), np64(ref)
    assert (got[0, G:2 * G, 128:192] == 0).all()
    mask = np.ones(got.shape, dtype=bool)
    mask[0, G:2 * G, 128:192] = False
    assert np.array_equal(got[mask], full[mask])
    rows = [(0, h, t) for h in range(Hkv * G) for t in (0, 127, 128, 191, 192, 255)]
    want = orc.attend_prefill(np64(q_chunk), np64(c["k"]), np64(c["v"]), sel.idx, cnt_e.cpu().numpy(), q_start,
                              1.0 / math.sqrt(d), 64, rows=rows)
    assert max(max_abs(got[r], want[r]) for r in rows) < 2e-2


def test_prefill_attention_lists_longer_than_128_blocks():
    """Block lists of up to 159 entries (top-k 150 + 1 initial + 8 local):
    the prefill kernel's ring runs through more than a hundred blocks per
    query block; sampled rows against the oracle."""
    d, G, Hkv, T, q_start, Tq, topk, n_local = 128, 4, 1, 64 * 300, 64 * 280, 256, 150, 8
    c, q_chunk, idx, cnt, sel = _prefill_case(81, 1, Hkv * G, Hkv, d, T, q_start, Tq, topk=topk, n_local=n_local)
    check_selection(idx, cnt, sel, topk)
    assert int(cnt.max()) == topk + 1 + n_local
    out = bskv.block_sparse_attn_prefill(q_chunk, c["k"], c["v"], idx, cnt, q_start)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = [(0, h, int(t)) for h in range(Hkv * G) for t in rng.choice(Tq, 6, replace=False)]
    rows += [(0, 0, 0), (0, Hkv * G - 1, Tq - 1)]
    want = orc.attend_prefill(np64(q_chunk), np64(c["k"]), np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(),
                              q_start, 1.0 / math.sqrt(d), 64, rows=rows)
    got = np64(out)
    assert max(max_abs(got[r], want[r]) for r in rows) < 2e-2


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f32", 64, 2)])
def test_decode_attention_lists_longer_than_128_blocks(dtype, d, G):
    """Decode selection and attention with U = 203 (top-k 200): many blocks
    per attention split, against the oracle."""
    B, Hkv, T, topk = 2, 2, 64 * 400, 200
    lens = [64 * 400, 64 * 371 + 9]
    c = _gpu(random_decode_case(91, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype=dtype, seq_len=lens))
    kc = _kc_gpu(c["k"], c["seq_len"])
    idx, cnt = bskv.forecast_block_score_topk(c["f"], kc, topk, 1, 2, seq_len=c["seq_len"])
    scale = 1.0 / math.sqrt(d)
    out = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"], scale)
    torch.cuda.synchronize()
    sel = orc.decode_select(np64(c["f"]), orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens), np.array(lens), topk,
                            1, 2, 64)
    check_selection(idx, cnt, sel, topk)
    assert int(cnt.max()) == topk + 3
    want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(), lens,
                             scale, 64)
    assert max_abs(np64(out), want) < (1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("immediate", [False, True])
def test_decode_layer_above_64_units(immediate):
    """The fused layer above 64 (b, g) units (B20 x 8 KV heads = 160), where
    its plans take 768 score and 768 attention workgroups, more than the
    chip holds at once: lists, raw scores and outputs equal the per-op path
    and the oracle, ragged lengths, and the counters end at zero."""
    B, Hkv, G, d, T, topk = 20, 8, 4, 128, 64 * 60, 16
    lens = [64 * 60 - (7 * b) % 200 for b in range(B)]
    c = _gpu(random_decode_case(95, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype="bf16", hidden=1024, seq_len=lens))
    c2 = _gpu(random_decode_case(96, B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dtype="bf16", seq_len=lens))
    kc, kc_next = _kc_gpu(c["k"], c["seq_len"]), _kc_gpu(c2["k"], c2["seq_len"])
    nb = kc.shape[2]
    scale = 1.0 / math.sqrt(d)
    f = bskv.forecast_proj(c["x_sel"], c["w_sel"], Hkv, d)
    idx, cnt = bskv.forecast_block_score_topk(c2["f"], kc, topk, 1, 2, seq_len=c["seq_len"])
    i_ref, n_ref = bskv.forecast_block_score_topk(f, kc_next, topk, 1, 2, seq_len=c["seq_len"])
    out_ref = bskv.block_sparse_attn_decode(c["q"], c["k"], c["v"], idx, cnt, c["seq_len"], scale)
    ws = torch.zeros(bskv.workspace_bytes("layer", B, Hkv * G, Hkv, d, 1024, nb, topk + 3, 1), dtype=torch.uint8,
                     device=DEV)
    if immediate:
        i_next = torch.full_like(idx, -7)
        n_next = torch.full_like(cnt, -7)
        out, _ = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt, scale,
                                             x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, idx_next=i_next,
                                             cnt_next=n_next, topk=topk, n_init=1, n_local=2, ws=ws)
    else:
        out, sc = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kc.clone(), idx, cnt, scale,
                                              x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=topk, n_init=1,
                                              n_local=2, ws=ws)
        i_next, n_next = _next_lists(c2, kc_next, sc, topk, 1, 2, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(i_next, i_ref) and torch.equal(n_next, n_ref)
    assert int(ws[: 2 * 65535 * 4].view(torch.int32).abs().sum()) == 0
    f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), Hkv, d)
    sel = orc.decode_select(f_or, orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens), np.array(lens), topk, 1, 2,
                            64)
    check_selection(i_next, n_next, sel, topk)
    want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(), lens,
                             scale, 64)
    assert max_abs(np64(out), want) < 2e-2
