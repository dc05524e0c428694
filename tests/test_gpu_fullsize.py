"""GPU parity at full workload sizes, in the launch configuration bench.py
times, checked against the fp64 oracle on sampled batch elements."""
import numpy as np
import pytest
import torch

import block_sparse_long_kv_amd as bskv
import oracle as orc
from parity import check_selection, max_abs, np64
from workloads import CONFIGS, decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_config3_two_layers_sampled():
    """B8, T=131072, top-64 + 1 + 4: layer 0 selected by the layer-0
    projection, layer 1 by layer 0's Forecast (fused layer call)."""
    wl = CONFIGS[3]
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
    out0, idx1, cnt1 = bskv.decode_layer_lookahead(l0["q"], l0["k"], l0["v"], l0["seq_len"], kc[0], idx0, cnt0,
                                                   wl.scale, x=l1["x_sel"], w=l1["w_sel"], kc_next=kc[1],
                                                   topk=wl.topk, n_init=wl.n_init, n_local=wl.n_local)
    out1, _, _ = bskv.decode_layer_lookahead(l1["q"], l1["k"], l1["v"], l1["seq_len"], kc[1], idx1, cnt1, wl.scale,
                                             topk=wl.topk, n_init=wl.n_init, n_local=wl.n_local)
    torch.cuda.synchronize()
    sel_gpu = [(idx0, cnt0, out0), (idx1, cnt1, out1)]
    for b in (0, wl.B - 1):
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


def test_config4_prefill_chunks_sampled():
    """B4, T=131072, 2048-token chunks, top-64 + 1 + 32 local: selection and
    attention on sampled (batch, KV head, query block) problems of the first,
    a middle and the last chunk, at the kernels' full launch size."""
    import math
    from workloads import prefill_inputs
    wl = CONFIGS[4]
    inp = prefill_inputs(wl, DEV)
    lens = torch.full((wl.B,), wl.T, dtype=torch.int64, device=DEV)
    kc = torch.empty(wl.B, wl.Hkv, wl.NB, wl.d, dtype=torch.float32, device=DEV)
    bskv.kv_block_meanpool(inp["k"], lens, kc)
    samples = [(0, 0), (wl.B - 1, wl.Hkv - 1)]
    kc_or = {s: orc.kv_block_meanpool(np64(inp["k"][s[0]:s[0] + 1, s[1]:s[1] + 1]), 64) for s in samples}
    kv_or = {s: (np64(inp["k"][s[0]:s[0] + 1, s[1]:s[1] + 1]), np64(inp["v"][s[0]:s[0] + 1, s[1]:s[1] + 1]))
             for s in samples}
    for q0 in (0, wl.T // 2, wl.T - wl.chunk):
        f = inp["f"][:, :, q0:q0 + wl.chunk].contiguous()
        q = inp["q"][:, :, q0:q0 + wl.chunk].contiguous()
        idx, cnt = bskv.forecast_block_score_topk(f, kc, wl.topk, wl.n_init, wl.n_local, q_start=q0, prefill=True)
        out = bskv.block_sparse_attn_prefill(q, inp["k"], inp["v"], idx, cnt, q0, wl.scale)
        torch.cuda.synchronize()
        for (b, g) in samples:
            for qi in (0, 17, 31):
                fq = np64(f[b:b + 1, g:g + 1, qi * 64:(qi + 1) * 64])
                sel = orc.prefill_select(fq, kc_or[(b, g)], q0 + qi * 64, wl.topk, wl.n_init, wl.n_local, 64)
                check_selection(idx[b:b + 1, g:g + 1, qi:qi + 1], cnt[b:b + 1, g:g + 1, qi:qi + 1], sel, wl.topk)
                # attention of two query heads of this KV head on a few tokens, on the GPU's list
                k1, v1 = kv_or[(b, g)]
                gi = idx[b:b + 1, g:g + 1, qi:qi + 1].cpu().numpy()
                gc = cnt[b:b + 1, g:g + 1, qi:qi + 1].cpu().numpy()
                for h in (g * wl.G, g * wl.G + wl.G - 1):
                    qq = np64(q[b:b + 1, h:h + 1, qi * 64:(qi + 1) * 64])
                    rows = [(0, 0, t) for t in (0, 31, 63)]
                    want = orc.attend_prefill(qq, k1, v1, gi, gc, q0 + qi * 64, 1.0 / math.sqrt(wl.d), 64, rows=rows)
                    got = np64(out[b:b + 1, h:h + 1, qi * 64:(qi + 1) * 64])
                    for r in rows:
                        assert max_abs(got[r], want[r]) < 2e-2


def test_config5_offload_sampled():
    """B16, T=131072 with the KV cache in host-pinned memory: the layer-0
    projection selects layer 0, its blocks are gathered from the host pool
    into the ring on a side stream, and attention reads the ring.  Checked on
    sampled batch elements against the oracle and bytewise against the host."""
    wl = CONFIGS[5]
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
