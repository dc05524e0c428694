"""The allocation-free fused decode layer (workspace in the library's
static device array) against the same call with a caller workspace: equal
outputs, on two calls in a row, the second with a smaller input."""
import math

import numpy as np
import pytest
import torch

import block_sparse_long_kv_amd as bskv
import oracle as orc
from parity import check_selection, max_abs, np64
from workloads import random_decode_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(seed, B, T, lens, topk):
    c = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
         for k, v in random_decode_case(seed, B=B, Hq=16, Hkv=4, d=128, T=T, dtype="bf16", hidden=512,
                                        seq_len=lens).items()}
    c2 = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
          for k, v in random_decode_case(seed + 1, B=B, Hq=16, Hkv=4, d=128, T=T, dtype="bf16", seq_len=lens,
                                         plant=topk, n_local=2).items()}
    kc = torch.full((B, 4, T // 64, 128), float("nan"), dtype=torch.float32, device=DEV)
    kc_next = torch.full_like(kc, float("nan"))
    bskv.kv_block_meanpool(c["k"], c["seq_len"], kc)
    bskv.kv_block_meanpool(c2["k"], c2["seq_len"], kc_next)
    sel = orc.decode_select(np64(c2["f"]), orc.kv_block_meanpool(np64(c["k"]), 64, seq_len=lens), np.array(lens),
                            topk, 1, 2, 64)
    idx = torch.from_numpy(sel.idx.astype(np.int32)).to(DEV)
    cnt = torch.from_numpy(sel.cnt.astype(np.int32)).to(DEV)
    return c, c2, kc, kc_next, idx, cnt


@pytest.mark.parametrize("mode", ["deferred", "immediate"])
def test_noalloc_layer_equals_the_workspace_call(mode):
    topk = 16
    # the second call is smaller; a third, larger again, finds the counters
    # the smaller layout left at zero
    for B, T, lens in ((4, 64 * 300, [64 * 300, 64 * 300 - 11, 64 * 150, 64 * 299 + 1]),
                       (2, 64 * 120, [64 * 120, 64 * 77 + 3]),
                       (6, 64 * 200, [64 * 200] * 5 + [64 * 100 + 1])):
        c, c2, kc, kc_next, idx, cnt = _case(60 + B, B, T, lens, topk)
        U = topk + 3
        kw = dict(x=c["x_sel"], w=c["w_sel"], kc_next=kc_next, topk=topk, n_init=1, n_local=2)
        res = []
        for fn in ("noalloc", "ws"):
            kcl = kc.clone()
            extra = {}
            if mode == "immediate":
                extra = {"idx_next": torch.full_like(idx, -7), "cnt_next": torch.full_like(cnt, -7)}
            if fn == "noalloc":
                out, sc = bskv.decode_layer_lookahead_noalloc(c["q"], c["k"], c["v"], c["seq_len"], kcl, idx, cnt,
                                                              **kw, **extra)
            else:
                ws = torch.zeros(bskv.workspace_bytes("layer", B, 16, 4, 128, 512, T // 64, U, 1), dtype=torch.uint8,
                                 device=DEV)
                out, sc = bskv.decode_layer_lookahead(c["q"], c["k"], c["v"], c["seq_len"], kcl, idx, cnt, ws=ws,
                                                      **kw, **extra)
            torch.cuda.synchronize()
            res.append((out, sc, kcl, extra))
        (o1, s1, k1, e1), (o2, s2, k2, e2) = res
        assert torch.equal(o1, o2), (mode, B)
        assert torch.equal(k1.nan_to_num(7.0), k2.nan_to_num(7.0)), (mode, B)
        if mode == "immediate":
            assert torch.equal(e1["idx_next"], e2["idx_next"]) and torch.equal(e1["cnt_next"], e2["cnt_next"])
            nxt_idx, nxt_cnt = e1["idx_next"], e1["cnt_next"]
        else:
            for b, L in enumerate(lens):       # only each sequence's candidates are written
                c1 = min((L - 1) // 64 - 2 + 1, T // 64)
                assert torch.equal(s1[b, :, 1:c1], s2[b, :, 1:c1]), (mode, B, b)
            nxt_idx, nxt_cnt = torch.full_like(idx, -7), torch.full_like(cnt, -7)
            bskv.decode_layer_lookahead_noalloc(c2["q"], c2["k"], c2["v"], c2["seq_len"], kc_next.clone(), nxt_idx,
                                                nxt_cnt, scores=s1, topk=topk, n_init=1, n_local=2, stages=1)
            torch.cuda.synchronize()
        # and against the oracle
        f_or = orc.forecast_proj(np64(c["x_sel"]), np64(c["w_sel"]), 4, 128)
        sel = orc.decode_select(f_or, orc.kv_block_meanpool(np64(c2["k"]), 64, seq_len=lens), np.array(lens), topk,
                                1, 2, 64)
        check_selection(nxt_idx, nxt_cnt, sel, topk)
        want = orc.attend_decode(np64(c["q"]), np64(c["k"]), np64(c["v"]), idx.cpu().numpy(), cnt.cpu().numpy(),
                                 np.array(lens), 1 / math.sqrt(128), 64)
        assert max_abs(np64(o1), want) < 2e-2


def test_noalloc_layer_rejects_a_layer_too_large_for_the_array():
    cap = bskv.lib.bskv_decode_layer_lookahead_noalloc_capacity()
    # the smallest compressed-key capacity (a multiple of 1024 blocks) whose
    # layer workspace exceeds the array
    nb = 1024
    while bskv.workspace_bytes("layer", 64, 32, 8, 128, 4096, nb, 69, 1) <= cap:
        nb += 1024
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(64, 8, 64 * 64, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(64, 8, nb, 128, dtype=torch.float32, device=DEV)
    idx = torch.zeros(64, 8, 69, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(64, 8, dtype=torch.int32, device=DEV)
    lens = torch.full((64,), 64 * 64, dtype=torch.int64, device=DEV)
    x = torch.zeros(64, 4096, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(4096, 1024, dtype=torch.bfloat16, device=DEV)
    assert bskv.workspace_bytes("layer", 64, 32, 8, 128, 4096, nb, 69, 1) > cap
    with pytest.raises(bskv.BskvError) as ei:
        bskv.decode_layer_lookahead_noalloc(q, k, k, lens, kc, idx, cnt, x=x, w=w, kc_next=kc.clone(), topk=64,
                                            n_init=1, n_local=4)
    assert ei.value.status == -4
