"""GPU parity of the offloaded decode schedules (block_sparse_long_kv_amd.offload)
against the fp64 oracle's one-layer-ahead decode step.

The KV cache of every layer sits in host-pinned memory; the ring schedule
copies each layer's whole union into one of two device slots on a copy
stream while the previous layer computes, the cached schedule copies only
the blocks a resident cache misses.  Each ring slot is filled with NaN on the
copy stream right before every refill (after the slot-reuse wait), so a
layer that read a slot before its copy landed, or a copy that overwrote a
slot still being read, shows up as NaN or a wrong output.  A second run puts
a fixed delay on the copy stream ahead of every copy, so the compute stream
must really wait for it.  Tolerances: selection ids as in parity.check_selection,
attention 2e-2 absolute (bf16 K/V).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_long_kv_amd as bskv
import oracle as orc
from block_sparse_long_kv_amd.offload import CachedLookahead, LookaheadRing, OffloadLayer
from parity import check_selection, max_abs, np64
from workloads import drift_walk, random_decode_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
B, HQ, HKV, D, HID = 2, 16, 4, 128, 512
TOPK, N_INIT, N_LOCAL = 16, 1, 2
U = TOPK + N_INIT + N_LOCAL
T = 64 * 210
LENS = [64 * 210, 64 * 210 - 37]
SCALE = 1.0 / math.sqrt(D)
DELAY_CYCLES = 1_000_000        # about half a millisecond of spinning on the copy stream per copy


def _layers(n_layers, seed0, plant=TOPK):
    """Per layer: host-pinned K/V, GPU compressed keys, the selecting
    Forecast input/weights and the query; `plant` planted blocks along that
    Forecast, so the top-k is well separated."""
    cases, layers = [], []
    for l in range(n_layers):
        c = random_decode_case(seed0 + l, B=B, Hq=HQ, Hkv=HKV, d=D, T=T, dtype="bf16", hidden=HID, seq_len=LENS,
                               plant=plant, topk=TOPK, n_init=N_INIT, n_local=N_LOCAL)
        hk = torch.empty(c["k"].shape, dtype=torch.bfloat16, pin_memory=True)
        hv = torch.empty(c["v"].shape, dtype=torch.bfloat16, pin_memory=True)
        hk.copy_(c["k"])
        hv.copy_(c["v"])
        seq_len = c["seq_len"].to(DEV)
        kc = torch.full((B, HKV, T // 64, D), float("nan"), dtype=torch.float32, device=DEV)
        bskv.kv_block_meanpool(c["k"].to(DEV), seq_len, kc)
        layers.append(OffloadLayer(
            hk, hv, kc, c["x_sel"].to(DEV), c["w_sel"].to(DEV), c["q"].to(DEV), seq_len,
            f=torch.empty(B, HKV, D, dtype=torch.float32, device=DEV),
            idx=torch.empty(B, HKV, U, dtype=torch.int32, device=DEV),
            cnt=torch.empty(B, HKV, dtype=torch.int32, device=DEV),
            out=torch.empty(B, HQ, D, dtype=torch.float32, device=DEV)))
        cases.append(c)
    torch.cuda.synchronize()
    return cases, layers


def _workspaces():
    z = lambda n: torch.zeros(max(int(n), 256), dtype=torch.uint8, device=DEV)  # noqa: E731
    return {"ws_proj": z(bskv.workspace_bytes("proj", B, HID, HKV, D, 1)),
            "ws_score": z(bskv.workspace_bytes("score", B, HKV, 0, T // 64, D)),
            "ws_attn": z(bskv.workspace_bytes("attn", B, HQ, HKV, D, U))}


def _oracle_layers(cases, x_override=None):
    out = []
    for l, c in enumerate(cases):
        k = np64(c["k"])
        out.append({"x_sel": np64(c["x_sel"] if x_override is None else x_override[l]), "w_sel": np64(c["w_sel"]),
                    "kc": orc.kv_block_meanpool(k, 64, seq_len=LENS), "q": np64(c["q"]), "k": k,
                    "v": np64(c["v"]), "seq_len": np.array(LENS)})
    return out


def _check_layer(lay, sel, want, o_lay):
    check_selection(lay.idx, lay.cnt, sel, TOPK)
    got = np64(lay.out)
    assert np.isfinite(got).all()
    gi, gc = lay.idx.cpu().numpy(), lay.cnt.cpu().numpy()
    if np.array_equal(gi, sel.idx):
        assert max_abs(got, want) < 2e-2
    else:   # a legitimate near-tie swap: attention on the GPU's own lists
        alt = orc.attend_decode(o_lay["q"], o_lay["k"], o_lay["v"], gi, gc, o_lay["seq_len"], SCALE, 64)
        assert max_abs(got, alt) < 2e-2


@pytest.mark.parametrize("delay", [0, DELAY_CYCLES])
def test_ring_schedule_matches_lookahead_oracle(delay):
    n_layers = 5
    cases, layers = _layers(n_layers, 500)
    ring = LookaheadRing(B, HKV, U, D, device=DEV, n_workgroups=24)
    refills = []

    def poison_then_wait(l, slot, stream):
        ring.ring_k[slot].fill_(float("nan"))
        ring.ring_v[slot].fill_(float("nan"))
        if delay:
            torch.cuda._sleep(delay)
        refills.append((l, slot))

    for lay in layers:
        lay.out.fill_(float("nan"))
    ring.step(layers, TOPK, N_INIT, N_LOCAL, SCALE, on_refill=poison_then_wait)
    torch.cuda.synchronize()
    assert refills == [(l, l % 2) for l in range(n_layers)]
    results = orc.decode_step_lookahead(_oracle_layers(cases), TOPK, N_INIT, N_LOCAL, 64, SCALE)
    o_layers = _oracle_layers(cases)
    for l, (sel, want) in enumerate(results):
        _check_layer(layers[l], sel, want, o_layers[l])
    # the ring equals the resident path bit for bit (same kernel, same order)
    for l, lay in enumerate(layers):
        k_dev, v_dev = lay.host_k.to(DEV), lay.host_v.to(DEV)
        res = bskv.block_sparse_attn_decode(lay.q, k_dev, v_dev, lay.idx, lay.cnt, lay.seq_len, SCALE)
        torch.cuda.synchronize()
        assert torch.equal(res, lay.out), l


def test_ring_schedule_graph_replays():
    """The ring step captured in a HIP graph (poisoning and delay inside):
    every replay, with eager work between replays, gives the eager outputs."""
    n_layers = 4
    cases, layers = _layers(n_layers, 600)
    ring = LookaheadRing(B, HKV, U, D, device=DEV, n_workgroups=16)
    ws = _workspaces()       # caller-owned: nothing is allocated while the graph is captured

    def poison(l, slot, stream):
        ring.ring_k[slot].fill_(float("nan"))
        ring.ring_v[slot].fill_(float("nan"))
        torch.cuda._sleep(DELAY_CYCLES // 4)

    ring.step(layers, TOPK, N_INIT, N_LOCAL, SCALE, on_refill=poison, **ws)
    torch.cuda.synchronize()
    eager = [(lay.idx.clone(), lay.cnt.clone(), lay.out.clone()) for lay in layers]
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ring.step(layers, TOPK, N_INIT, N_LOCAL, SCALE, on_refill=poison, **ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ring.step(layers, TOPK, N_INIT, N_LOCAL, SCALE, on_refill=poison, **ws)
    for rep in range(3):
        for lay in layers:
            lay.out.fill_(float("nan"))
            lay.idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for l, lay in enumerate(layers):
            i, c, o = eager[l]
            assert torch.equal(lay.idx, i) and torch.equal(lay.cnt, c) and torch.equal(lay.out, o), (rep, l)
        ring.step(layers, TOPK, N_INIT, N_LOCAL, SCALE, **ws)        # eager work between replays
        torch.cuda.synchronize()
    results = orc.decode_step_lookahead(_oracle_layers(cases), TOPK, N_INIT, N_LOCAL, 64, SCALE)
    o_layers = _oracle_layers(cases)
    for l, (sel, want) in enumerate(results):
        _check_layer(layers[l], sel, want, o_layers[l])


@pytest.mark.parametrize("fused", [False, True])
def test_cached_schedule_over_steps_matches_oracle(fused):
    """Steady state: 4 layers, 3 decode steps with the Forecast inputs
    drifting, a resident cache of 2U slots per (b, g) and layer, a delay on
    the copy stream ahead of every fill (fused: the copy of layer l+1 inside
    layer l's attention launch, the delay on the compute stream before it).
    Every layer of every step matches the oracle's one-layer-ahead step on
    that step's inputs, and later steps copy only part of each union (no
    planted blocks here, so the drift moves some selections)."""
    n_layers, n_steps, S = 4, 3, 2 * U
    cases, layers = _layers(n_layers, 700, plant=0)
    x0 = torch.stack([c["x_sel"] for c in cases])                      # [L, B, hidden]
    xs = drift_walk(x0, n_steps, 0.3, 77)                             # [steps, L, B, hidden]
    xbuf = torch.empty(n_layers, B, HID, dtype=torch.bfloat16, device=DEV)
    for l, lay in enumerate(layers):
        lay.x_sel = xbuf[l]
    caches = [bskv.BlockCache(B, HKV, S, D, device=DEV) for _ in range(n_layers)]
    slot = [torch.empty(B, HKV, U, dtype=torch.int32, device=DEV) for _ in range(n_layers)]
    fill = [torch.empty(B, HKV, U, dtype=torch.int32, device=DEV) for _ in range(n_layers)]
    n_fill = [torch.empty(B, HKV, dtype=torch.int32, device=DEV) for _ in range(n_layers)]
    sched = CachedLookahead(caches, slot, fill, n_fill, device=DEV, n_workgroups=8, fused_fill=fused)

    def delay(l, stream):
        torch.cuda._sleep(DELAY_CYCLES // 2)

    fetched = []
    for t in range(n_steps):
        xbuf.copy_(xs[t].to(DEV))
        for lay in layers:
            lay.out.fill_(float("nan"))
        sched.step(layers, TOPK, N_INIT, N_LOCAL, SCALE, on_fill=delay)
        torch.cuda.synchronize()
        fetched.append(sum(int(n.sum()) for n in n_fill))
        o_layers = _oracle_layers(cases, x_override=[xs[t, l] for l in range(n_layers)])
        results = orc.decode_step_lookahead(o_layers, TOPK, N_INIT, N_LOCAL, 64, SCALE)
        for l, (sel, want) in enumerate(results):
            _check_layer(layers[l], sel, want, o_layers[l])
    total = n_layers * B * HKV * U
    assert fetched[0] == total, "the first step copies every listed block"
    assert all(0 < f < total for f in fetched[1:]), fetched


def test_cached_attention_with_fill_equals_separate_calls():
    """One launch (attention of layer 0 from its cache + copy of layer 1's
    missing blocks) gives the same attention output and the same layer-1
    cache, bit for bit, as the fill and the attention called separately."""
    cases, layers = _layers(2, 800)
    S = 2 * U
    ws = _workspaces()
    outs, cache_bytes = [], []
    for fused in (False, True):
        caches = [bskv.BlockCache(B, HKV, S, D, device=DEV) for _ in range(2)]
        slot = [torch.empty(B, HKV, U, dtype=torch.int32, device=DEV) for _ in range(2)]
        fill = [torch.empty(B, HKV, U, dtype=torch.int32, device=DEV) for _ in range(2)]
        n_fill = [torch.empty(B, HKV, dtype=torch.int32, device=DEV) for _ in range(2)]
        sched = CachedLookahead(caches, slot, fill, n_fill, device=DEV, n_workgroups=5)
        for l in range(2):
            sched.plan(layers[l], l, TOPK, N_INIT, N_LOCAL, ws["ws_proj"], ws["ws_score"])
        sched.fill_cache(layers[0], 0)
        layers[0].out.fill_(float("nan"))
        if fused:
            sched.attend_and_fill(layers[0], 0, layers[1], SCALE, ws["ws_attn"])
        else:
            sched.fill_cache(layers[1], 1)
            sched.attend(layers[0], 0, SCALE, ws["ws_attn"])
        torch.cuda.synchronize()
        outs.append(layers[0].out.clone())
        # the listed slots of layer 1 (the rest of the cache is never written)
        sl = slot[1].long().clamp(min=0)
        got = [c.gather(2, sl[..., None, None].expand(-1, -1, -1, 64, D)) for c in (caches[1].k, caches[1].v)]
        cache_bytes.append(got)
        assert int(n_fill[1].sum()) == B * HKV * U, "a first lookup copies every listed block"
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(cache_bytes[0][0], cache_bytes[1][0]) and torch.equal(cache_bytes[0][1], cache_bytes[1][1])
    # and the filled blocks are the host blocks the list names
    idx1 = layers[1].idx.cpu().long()
    hk = layers[1].host_k.view(B, HKV, T // 64, 64, D)
    want = torch.stack([torch.stack([hk[b, g, idx1[b, g]] for g in range(HKV)]) for b in range(B)])
    assert torch.equal(cache_bytes[1][0].cpu(), want)


def test_cached_attention_with_fill_short_lists_and_many_fill_workgroups():
    """Short sequences (fewer candidates than k: lists padded with -1 past
    cnt) and more fill workgroups than (b, g) units: the fused call still
    equals the separate calls bit for bit, and its attention matches the
    oracle on the GPU's lists."""
    T2, lens2 = 64 * 12, [64 * 12, 64 * 7 - 5]
    layers, cases = [], []
    for l in range(2):
        c = random_decode_case(900 + l, B=B, Hq=HQ, Hkv=HKV, d=D, T=T2, dtype="bf16", hidden=HID, seq_len=lens2,
                               topk=TOPK, n_init=N_INIT, n_local=N_LOCAL)
        hk = torch.empty(c["k"].shape, dtype=torch.bfloat16, pin_memory=True)
        hv = torch.empty(c["v"].shape, dtype=torch.bfloat16, pin_memory=True)
        hk.copy_(c["k"])
        hv.copy_(c["v"])
        seq_len = c["seq_len"].to(DEV)
        kc = torch.full((B, HKV, T2 // 64, D), float("nan"), dtype=torch.float32, device=DEV)
        bskv.kv_block_meanpool(c["k"].to(DEV), seq_len, kc)
        layers.append(OffloadLayer(
            hk, hv, kc, c["x_sel"].to(DEV), c["w_sel"].to(DEV), c["q"].to(DEV), seq_len,
            f=torch.empty(B, HKV, D, dtype=torch.float32, device=DEV),
            idx=torch.empty(B, HKV, U, dtype=torch.int32, device=DEV),
            cnt=torch.empty(B, HKV, dtype=torch.int32, device=DEV),
            out=torch.empty(B, HQ, D, dtype=torch.float32, device=DEV)))
        cases.append(c)
    z = lambda n: torch.zeros(max(int(n), 256), dtype=torch.uint8, device=DEV)  # noqa: E731
    ws = {"ws_proj": z(bskv.workspace_bytes("proj", B, HID, HKV, D, 1)),
          "ws_score": z(bskv.workspace_bytes("score", B, HKV, 0, T2 // 64, D)),
          "ws_attn": z(bskv.workspace_bytes("attn", B, HQ, HKV, D, U))}
    S = U
    outs, filled = [], []
    for fused in (False, True):
        caches = [bskv.BlockCache(B, HKV, S, D, device=DEV) for _ in range(2)]
        slot = [torch.empty(B, HKV, U, dtype=torch.int32, device=DEV) for _ in range(2)]
        fill = [torch.empty(B, HKV, U, dtype=torch.int32, device=DEV) for _ in range(2)]
        n_fill = [torch.empty(B, HKV, dtype=torch.int32, device=DEV) for _ in range(2)]
        sched = CachedLookahead(caches, slot, fill, n_fill, device=DEV, n_workgroups=1000)
        for l in range(2):
            sched.plan(layers[l], l, TOPK, N_INIT, N_LOCAL, ws["ws_proj"], ws["ws_score"])
        sched.fill_cache(layers[0], 0)
        layers[0].out.fill_(float("nan"))
        if fused:
            sched.attend_and_fill(layers[0], 0, layers[1], SCALE, ws["ws_attn"])
        else:
            sched.fill_cache(layers[1], 1)
            sched.attend(layers[0], 0, SCALE, ws["ws_attn"])
        torch.cuda.synchronize()
        outs.append(layers[0].out.clone())
        cnt1 = layers[1].cnt.cpu()
        assert int(cnt1.min()) < U, "some lists are padded"
        assert torch.equal(n_fill[1].cpu(), cnt1), "a first lookup copies every listed block"
        # the listed slots of layer 1 (entries past cnt name no slot)
        got = []
        sl, c1 = slot[1].cpu(), cnt1
        for b in range(B):
            for g in range(HKV):
                for u in range(int(c1[b, g])):
                    s_ = int(sl[b, g, u])
                    got.append((caches[1].k[b, g, s_].cpu(), caches[1].v[b, g, s_].cpu()))
        filled.append(got)
    assert torch.equal(outs[0], outs[1])
    assert all(torch.equal(a[0], b_[0]) and torch.equal(a[1], b_[1]) for a, b_ in zip(filled[0], filled[1]))
    gi, gc = layers[0].idx.cpu().numpy(), layers[0].cnt.cpu().numpy()
    k0, v0 = np64(cases[0]["k"]), np64(cases[0]["v"])
    want = orc.attend_decode(np64(cases[0]["q"]), k0, v0, gi, gc, np.array(lens2), SCALE, 64)
    got = np64(outs[1])
    assert np.isfinite(got).all()
    assert max_abs(got, want) < 2e-2
