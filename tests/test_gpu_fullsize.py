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
