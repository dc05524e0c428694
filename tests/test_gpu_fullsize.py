"""GPU parity at full workload sizes, in the launch configuration bench.py
times, checked against the fp64 oracle on sampled batch elements."""
import numpy as np
import pytest
import torch

import block_sparse_long_kv_amd as bskv
import oracle as orc
from parity import check_selection, fp32_sum_close, max_abs, np64
from workloads import WORKLOADS, decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_decode_B8_128K_two_layers_sampled():
    """B8, T=131072, top-64 + 1 + 4: layer 0 selected by the layer-0
    projection, layer 1 by layer 0's Forecast (the fused layer calls: layer
    0's call scores layer 1's candidates, layer 1's call selects from them).
    Every batch element of both layers is checked against the oracle, which
    pools its own compressed keys from the inputs."""
    wl = WORKLOADS["decode-B8-128K-32L"]
    L = 2
    layers = decode_inputs(wl, DEV, layers=L)
    nb = wl.NB
    kc = []
    for lay in layers:
        k = torch.empty(wl.B, wl.Hkv, nb, wl.d, dtype=torch.float32, device=DEV)
        bskv.kv_block_meanpool(lay["k"], lay["seq_len"], k)
        kc.append(k)
    f0 = bskv.forecast_proj(layers[0]["x_sel"], layers[0]["w_sel"], wl.Hkv, wl.d)
    idx0, cnt0 = bskv.forecast_block_score_topk(f0, kc[0], wl.topk, wl.n_init, wl.n_local, seq_len=layers[0]["seq_len"])
    l0, l1 = layers
    out0, sc1 = bskv.decode_layer_lookahead(l0["q"], l0["k"], l0["v"], l0["seq_len"], kc[0], idx0, cnt0,
                                            wl.scale, x=l1["x_sel"], w=l1["w_sel"], kc_next=kc[1],
                                            topk=wl.topk, n_init=wl.n_init, n_local=wl.n_local)
    idx1, cnt1 = torch.empty_like(idx0), torch.empty_like(cnt0)
    out1, _ = bskv.decode_layer_lookahead(l1["q"], l1["k"], l1["v"], l1["seq_len"], kc[1], idx1, cnt1, wl.scale,
                                          scores=sc1, topk=wl.topk, n_init=wl.n_init, n_local=wl.n_local)
    torch.cuda.synchronize()
    sel_gpu = [(idx0, cnt0, out0), (idx1, cnt1, out1)]
    for b in range(wl.B):
        for l, lay in enumerate(layers):
            idx, cnt, out = sel_gpu[l]
            k = np64(lay["k"][b:b + 1])
            v = np64(lay["v"][b:b + 1])
            f = orc.forecast_proj(np64(lay["x_sel"][b:b + 1]), np64(lay["w_sel"]), wl.Hkv, wl.d)
            sel = orc.decode_select(f, orc.kv_block_meanpool(k, 64), [wl.T], wl.topk, wl.n_init, wl.n_local, 64)
            assert check_selection(idx[b:b + 1], cnt[b:b + 1], sel, wl.topk) == 0
            for g in range(wl.Hkv):
                assert set(sel.top[g]) == set(lay["planted"][b, g].tolist())
            want = orc.attend_decode(np64(lay["q"][b:b + 1]), k, v, idx[b:b + 1].cpu().numpy(),
                                     cnt[b:b + 1].cpu().numpy(), [wl.T], wl.scale, 64)
            assert max_abs(np64(out[b:b + 1]), want) < 2e-2


def test_prefill_B4_128K_chunks_sampled():
    """B4, T=131072, 2048-token chunks, top-64 + 1 + 32 local: selection and
    attention on sampled (batch, KV head, query block) problems of the first,
    a middle and the last chunk, at the kernels' full launch size.  Every
    token of each sampled query block, for every query head of the KV head,
    is compared (2 x 3 x 7 x 4 x 64 = 10,752 rows), on the oracle's own lists
    whenever the GPU's selection equals them (no near-tie swap), else on the
    GPU's lists."""
    import math
    from workloads import prefill_inputs
    wl = WORKLOADS["prefill-B4-128K"]
    inp = prefill_inputs(wl, DEV)
    lens = torch.full((wl.B,), wl.T, dtype=torch.int64, device=DEV)
    kc = torch.empty(wl.B, wl.Hkv, wl.NB, wl.d, dtype=torch.float32, device=DEV)
    bskv.kv_block_meanpool(inp["k"], lens, kc)
    samples = [(0, 0), (wl.B - 1, wl.Hkv - 1)]
    kc_or = {s: orc.kv_block_meanpool(np64(inp["k"][s[0]:s[0] + 1, s[1]:s[1] + 1]), 64) for s in samples}
    kv_or = {s: (np64(inp["k"][s[0]:s[0] + 1, s[1]:s[1] + 1]), np64(inp["v"][s[0]:s[0] + 1, s[1]:s[1] + 1]))
             for s in samples}
    rows_checked, on_oracle_lists = 0, 0
    for q0 in (0, wl.T // 2, wl.T - wl.chunk):
        f = inp["f"][:, :, q0:q0 + wl.chunk].contiguous()
        q = inp["q"][:, :, q0:q0 + wl.chunk].contiguous()
        idx, cnt = bskv.forecast_block_score_topk(f, kc, wl.topk, wl.n_init, wl.n_local, q_start=q0, prefill=True)
        out = bskv.block_sparse_attn_prefill(q, inp["k"], inp["v"], idx, cnt, q0, wl.scale)
        torch.cuda.synchronize()
        for (b, g) in samples:
            k1, v1 = kv_or[(b, g)]
            for qi in (0, 5, 11, 17, 23, 29, 31):
                fq = np64(f[b:b + 1, g:g + 1, qi * 64:(qi + 1) * 64])
                sel = orc.prefill_select(fq, kc_or[(b, g)], q0 + qi * 64, wl.topk, wl.n_init, wl.n_local, 64)
                swaps = check_selection(idx[b:b + 1, g:g + 1, qi:qi + 1], cnt[b:b + 1, g:g + 1, qi:qi + 1], sel,
                                        wl.topk)
                if swaps == 0:
                    li, lc = sel.idx, sel.cnt
                    on_oracle_lists += 1
                else:
                    li = idx[b:b + 1, g:g + 1, qi:qi + 1].cpu().numpy()
                    lc = cnt[b:b + 1, g:g + 1, qi:qi + 1].cpu().numpy()
                heads = list(range(g * wl.G, (g + 1) * wl.G))
                qq = np64(q[b:b + 1, heads[0]:heads[-1] + 1, qi * 64:(qi + 1) * 64])
                want = orc.attend_prefill(qq, k1, v1, li, lc, q0 + qi * 64, 1.0 / math.sqrt(wl.d), 64)
                got = np64(out[b:b + 1, heads[0]:heads[-1] + 1, qi * 64:(qi + 1) * 64])
                err = max_abs(got, want)
                assert err < 2e-2, (q0, b, g, qi, err)
                rows_checked += want.shape[1] * want.shape[2]
    assert rows_checked >= 10_000 and on_oracle_lists > 0


def test_offload_B16_128K_sampled():
    """B16, T=131072 with the KV cache in host-pinned memory: the layer-0
    projection selects layer 0, its blocks are gathered from the host pool
    into the ring on a side stream, and attention reads the ring.  Checked on
    sampled batch elements against the oracle and bytewise against the host."""
    wl = WORKLOADS["offload-decode-B16-128K-32L"]
    lay = decode_inputs(wl, DEV, layers=1)[0]
    kc = torch.empty(wl.B, wl.Hkv, wl.NB, wl.d, dtype=torch.float32, device=DEV)
    bskv.kv_block_meanpool(lay["k"], lay["seq_len"], kc)
    hk = torch.empty(lay["k"].shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(lay["v"].shape, dtype=torch.bfloat16, pin_memory=True)
    hk.copy_(lay["k"])
    hv.copy_(lay["v"])
    q = lay["q"]
    del lay["k"], lay["v"]
    f = bskv.forecast_proj(lay["x_sel"], lay["w_sel"], wl.Hkv, wl.d)
    idx, cnt = bskv.forecast_block_score_topk(f, kc, wl.topk, wl.n_init, wl.n_local, seq_len=lay["seq_len"])
    ring_k = torch.empty(wl.B, wl.Hkv, wl.U, 64, wl.d, dtype=torch.bfloat16, device=DEV)
    ring_v = torch.empty_like(ring_k)
    side = torch.cuda.Stream(DEV)
    sel_done = torch.cuda.Event()
    sel_done.record()
    side.wait_event(sel_done)
    bskv.prefetch_selected_blocks(hk, hv, idx, cnt, ring_k, ring_v, n_workgroups=256, stream=side)
    copied = torch.cuda.Event()
    copied.record(side)
    torch.cuda.current_stream().wait_event(copied)
    out = bskv.block_sparse_attn_decode(q, ring_k, ring_v, idx, cnt, lay["seq_len"], wl.scale, ring=True)
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        k = hk[b:b + 1].to(torch.float64).numpy()
        v = hv[b:b + 1].to(torch.float64).numpy()
        fo = orc.forecast_proj(np64(lay["x_sel"][b:b + 1]), np64(lay["w_sel"]), wl.Hkv, wl.d)
        sel = orc.decode_select(fo, orc.kv_block_meanpool(k, 64), [wl.T], wl.topk, wl.n_init, wl.n_local, 64)
        assert check_selection(idx[b:b + 1], cnt[b:b + 1], sel, wl.topk) == 0
        gi, gc = idx[b:b + 1].cpu().numpy(), cnt[b:b + 1].cpu().numpy()
        ring = orc.gather_selected_blocks(hk[b:b + 1].view(torch.int16).numpy(), gi, gc, 64)
        got = ring_k[b:b + 1].view(torch.int16).cpu().numpy()
        for g in range(wl.Hkv):
            assert np.array_equal(got[0, g, :gc[0, g]], ring[0, g, :gc[0, g]])
        want = orc.attend_decode(np64(q[b:b + 1]), k, v, gi, gc, [wl.T], wl.scale, 64)
        assert max_abs(np64(out[b:b + 1]), want) < 2e-2


def test_steady_offload_cache_full_size():
    """B16, T=131072, the KV cache in host-pinned memory and a 128-slot cache
    per (b, g): two decode steps with different Forecasts.  The lookups equal
    the oracle's LRU exactly for every (b, g); the slots hold the host blocks
    bytewise and the cached attention matches the oracle on sampled batch
    elements."""
    wl = WORKLOADS["offload-steady-B16-128K-32L"]
    lay = decode_inputs(wl, DEV, layers=1)[0]
    kc = torch.empty(wl.B, wl.Hkv, wl.NB, wl.d, dtype=torch.float32, device=DEV)
    bskv.kv_block_meanpool(lay["k"], lay["seq_len"], kc)
    hk = torch.empty(lay["k"].shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(lay["v"].shape, dtype=torch.bfloat16, pin_memory=True)
    hk.copy_(lay["k"])
    hv.copy_(lay["v"])
    q = lay["q"]
    del lay["k"], lay["v"]
    S = 128
    cache = bskv.BlockCache(wl.B, wl.Hkv, S, wl.d, device=DEV)
    tags = np.full((wl.B, wl.Hkv, S), -1, dtype=np.int64)
    stamps = np.full((wl.B, wl.Hkv, S), -1, dtype=np.int64)
    clock = np.zeros((wl.B, wl.Hkv), dtype=np.int64)
    f0 = bskv.forecast_proj(lay["x_sel"], lay["w_sel"], wl.Hkv, wl.d)
    g = torch.Generator(device=DEV).manual_seed(3)
    for f in (f0, f0 + 0.3 * f0.norm(dim=-1, keepdim=True) * torch.randn(f0.shape, generator=g, device=DEV) / 11.3):
        idx, cnt = bskv.forecast_block_score_topk(f.contiguous(), kc, wl.topk, wl.n_init, wl.n_local,
                                                  seq_len=lay["seq_len"])
        slot, fill, n_fill = bskv.block_cache_plan(cache, idx, cnt)
        bskv.prefetch_cache_fill(hk, hv, idx, slot, fill, n_fill, cache, n_workgroups=64)
        out = bskv.block_sparse_attn_decode_cached(q, cache, slot, idx, cnt, lay["seq_len"], wl.scale)
        torch.cuda.synchronize()
        gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
        w_slot, w_fill, w_n = orc.block_cache_plan(tags, stamps, clock, gi, gc)
        assert np.array_equal(slot.cpu().numpy(), w_slot) and np.array_equal(fill.cpu().numpy(), w_fill)
        assert np.array_equal(n_fill.cpu().numpy(), w_n)
        assert np.array_equal(cache.tags.cpu().numpy(), tags)
        for b in (0, wl.B - 1):
            ck = cache.k[b].view(torch.int16).cpu().numpy()
            hb = hk[b].view(torch.int16).numpy()
            for h in range(wl.Hkv):
                for u in range(int(gc[b, h])):
                    j = int(gi[b, h, u])
                    assert np.array_equal(ck[h, w_slot[b, h, u]], hb[h, 64 * j: 64 * (j + 1)])
            k = hk[b:b + 1].to(torch.float64).numpy()
            v = hv[b:b + 1].to(torch.float64).numpy()
            want = orc.attend_decode(np64(q[b:b + 1]), k, v, gi[b:b + 1], gc[b:b + 1], [wl.T], wl.scale, 64)
            assert max_abs(np64(out[b:b + 1]), want) < 2e-2


def test_window_select_B8_128K_sampled():
    """B8, T=131072: 32-token windows at stride 16 over every (b, g), decode
    selection with block scores max-pooled from the windows, checked on two
    sampled batch elements (all KV heads) against the oracle."""
    wl = WORKLOADS["decode-B8-128K-32L"]
    lay = decode_inputs(wl, DEV, layers=1)[0]
    nw = (wl.T - 32) // 16 + 1
    kcw = torch.empty(wl.B, wl.Hkv, nw, wl.d, dtype=torch.float32, device=DEV)
    bskv.kv_window_meanpool(lay["k"], lay["seq_len"], kcw, 32, 16)
    f = bskv.forecast_proj(lay["x_sel"], lay["w_sel"], wl.Hkv, wl.d)
    idx, cnt = bskv.forecast_window_score_topk(f, kcw, wl.topk, wl.n_init, wl.n_local, lay["seq_len"], 32, 16)
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        k = np64(lay["k"][b:b + 1])
        kw_or = orc.kv_window_meanpool(k, 32, 16)
        fo = orc.forecast_proj(np64(lay["x_sel"][b:b + 1]), np64(lay["w_sel"]), wl.Hkv, wl.d)
        sel = orc.decode_select_windows(fo, kw_or, [wl.T], wl.topk, wl.n_init, wl.n_local, 64, 32, 16)
        assert check_selection(idx[b:b + 1], cnt[b:b + 1], sel, wl.topk) <= 1
        assert max_abs(np64(kcw[b:b + 1, :, :64]), kw_or[:, :, :64]) < 1e-5


def test_widened_projection_full_size_sampled():
    """Decode: x [8 x 4096] @ W [4096 x 7168] (32 query heads, 8 KV and 8
    Forecast heads of 128), every output against the oracle.  Prefill: one
    2048-token chunk of four sequences, sampled tokens' Q/K/V and sampled
    query blocks' Forecast sums."""
    g = torch.Generator(device=DEV).manual_seed(11)
    B, hid, Hq, H, d = 8, 4096, 32, 8, 128
    N = (Hq + 3 * H) * d
    w_t = (torch.randn(N, hid, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    x = torch.randn(B, hid, generator=g, device=DEV).to(torch.bfloat16)
    T = 4096
    kc = torch.zeros(B, H, T, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    lens = torch.full((B,), T, dtype=torch.int64, device=DEV)
    q, f = bskv.qkvf_proj_decode(x, w_t, Hq, H, kc, vc, lens)
    torch.cuda.synchronize()
    w64 = np64(w_t).T
    wq, wk, wv, wf = orc.qkvf_proj(np64(x), w64, Hq, H, d)
    assert np.all(np.abs(np64(q) - wq) <= 2.0 ** -8 * np.abs(wq) + 1e-3)
    assert np.all(np.abs(np64(kc[:, :, T - 1]) - wk) <= 2.0 ** -8 * np.abs(wk) + 1e-3)
    mag_f = (np.abs(np64(x)) @ np.abs(w64))[:, (Hq + 2 * H) * d:].reshape(wf.shape)
    assert fp32_sum_close(np64(f), wf, mag_f, hid)
    Bp, C, q0, Tc = 4, 2048, 4096, 8192
    xp = torch.randn(Bp, C, hid, generator=g, device=DEV).to(torch.bfloat16)
    kcp = torch.zeros(Bp, H, Tc, d, dtype=torch.bfloat16, device=DEV)
    vcp = torch.zeros_like(kcp)
    qp, fp = bskv.qkvf_proj_prefill(xp, w_t, Hq, H, kcp, vcp, q_start=q0)
    torch.cuda.synchronize()
    for b, qi in ((0, 0), (Bp - 1, 31), (2, 13)):
        xs = np64(xp[b:b + 1, 64 * qi:64 * (qi + 1)])
        oq, ok_, ov, of = orc.qkvf_proj_prefill(xs, w64, Hq, H, d, 64)
        gq = np64(qp[b:b + 1, :, 64 * qi:64 * (qi + 1)])
        assert np.all(np.abs(gq - oq) <= 2.0 ** -8 * np.abs(oq) + 1e-3)
        gk = np64(kcp[b:b + 1, :, q0 + 64 * qi:q0 + 64 * (qi + 1)])
        assert np.all(np.abs(gk - ok_) <= 2.0 ** -8 * np.abs(ok_) + 1e-3)
        mag_p = (np.abs(xs[0]) @ np.abs(w64)[:, (Hq + 2 * H) * d:]).sum(0).reshape(of.shape)
        assert fp32_sum_close(np64(fp[b:b + 1, :, qi:qi + 1]), of, mag_p, 64 * hid)
