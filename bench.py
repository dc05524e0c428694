"""Benchmark of the Forecast-driven block-sparse attention hot path on one GPU.

Default workload (one JSON line on stdout): a decode step of batch 8 at a
131072-token context through 32 layers.  The layer-0 projection selects
layer 0's blocks; then each layer l runs (bskv_decode_layer_lookahead,
two kernels)
  Forecast projection F_l
  -> layer l+1's scores (F_l against its compressed keys), then its top-k /
     union per (b, g) once that (b, g)'s scores are written
     + layer l's block-sparse attention, then the merge of its splits and
     the incremental compressed-key update (newest block) per (b, g)
with every input resident in HBM.  The step is captured once in a HIP graph
and replayed.  `value` = batch tokens per second of the whole step.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload decode|decode-b4] [--per-op]

Per-kernel durations come from HIP events around back-to-back launches of
one kernel over all layers; the roofline object reports the dominant kernel
(`traffic`: HBM bytes per launch from rocprofv3 counters, while the kernel
sources match those they were measured on).  Also reported: the rate without
the Forecast projection, the box's measured device-copy rate, the selection
cost per layer at 32K/64K/128K context, and the fp64 oracle on the host
(`cpu_baseline`, also on one thread).

  --workload decode-b4   B4 x 32K, one layer, rotated over 8 replicas so the
                         45 MB working set is not served from the 256 MB cache
  --workload decode-tiny B1 x 4096 fp32 (correctness configuration; us per step)
  --workload prefill     B4 x 128K chunked prefill (MFMA-bound attention; the
                         vendor bf16 GEMM rate on the box is reported beside it)
  --workload offload     B16 x 128K decode with the KV cache in host memory
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "decode select+sparse-attn tokens/s at B×T (e.g. B8,128K); % HBM peak"

# HBM bytes per launch measured with rocprofv3 counters on the default
# workloads (FETCH_SIZE and WRITE_SIZE in separate passes, KiB per dispatch,
# averaged over the kernel's dispatches in `bench.py --steps 2 --warmup 1
# --no-cpu-baseline --copy-probe-gib 1`), each scaled by what the same counter
# reads for a copy kernel of known size using the same kind of loads: the
# runtime's device copy (nontemporal loads) and an elementwise kernel (plain
# loads) each read 1 GiB and FETCH_SIZE reports 512 MiB for both, so fetches
# take x2; WRITE_SIZE reports the 1 GiB written exactly (x1).
# An entry holds the digest of the sources it was measured on and is reported
# only while they are unchanged.
PMC_TRAFFIC = {
    "layer_k2": {"fetch_kib": 103802.4, "write_kib": 1194.6, "fetch_scale": 2.0, "write_scale": 1.0,
                 "sources": ['block_sparse_long_kv_amd/csrc/fused_decode.hip', 'block_sparse_long_kv_amd/csrc/decode_ops.hpp', 'block_sparse_long_kv_amd/csrc/bskv_device.hpp', 'block_sparse_long_kv_amd/csrc/bskv_launch.hpp'],
                 "sha256": "7d5d7755f940a734ca4621627c724962321d0f4cd7463db6939bb6a426c72319"},
    "attn_prefill": {"fetch_kib": 366793.8, "write_kib": 65537.0, "fetch_scale": 2.0, "write_scale": 1.0,
                     "sources": ['block_sparse_long_kv_amd/csrc/attn_prefill.hip', 'block_sparse_long_kv_amd/csrc/bskv_device.hpp', 'block_sparse_long_kv_amd/csrc/bskv_launch.hpp'],
                     "sha256": "8579e641ec7c6cd782d2afd4e69ede7a0b13a6e53a14d83f5abfd243e51e7ce1"},
}


def traffic_bytes(name):
    import hashlib
    ent = PMC_TRAFFIC.get(name)
    if ent is None:
        return None
    h = hashlib.sha256()
    for f in ent["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != ent["sha256"]:
        return None
    return int(round((ent["fetch_kib"] * ent["fetch_scale"] + ent["write_kib"] * ent["write_scale"]) * 1024))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# decode workload
# ---------------------------------------------------------------------------
class DecodeBench:
    def __init__(self, wl, torch, bskv, layers=None, B=None, T=None, select_mode="deferred"):
        from workloads import decode_inputs
        self.torch, self.bskv, self.wl = torch, bskv, wl
        self.select_mode = select_mode
        self.dev = torch.device("cuda:0")
        self.L = layers or wl.layers
        self.B = B or wl.B
        self.T = T or wl.T
        t0 = time.time()
        self.layers = decode_inputs(wl, self.dev, layers=self.L, B=self.B, T=self.T)
        torch.cuda.synchronize()
        log(f"[bench] generated {self.L} layers in {time.time() - t0:.1f}s")
        B, H, d, nb = self.B, wl.Hkv, wl.d, self.T // wl.block
        self.nb = nb
        self.kc = [torch.empty(B, H, nb, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        for lay, kc in zip(self.layers, self.kc):
            bskv.kv_block_meanpool(lay["k"], lay["seq_len"], kc)          # cache built at prefill time
        self.f = [torch.empty(B, H, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        self.idx = [torch.empty(B, H, wl.U, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.cnt = [torch.empty(B, H, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.out = [torch.empty(B, wl.Hq, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        # candidate scores of layer l, written by layer l-1's call, read by layer l's
        self.scores = [torch.empty(B, H, nb, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        z = lambda n: torch.zeros(max(int(n), 256), dtype=torch.uint8, device=self.dev)  # noqa: E731
        dt = 1 if wl.dtype == "bf16" else 0
        self.ws_proj = z(bskv.workspace_bytes("proj", B, wl.hidden, H, d, dt))
        self.ws_score = z(bskv.workspace_bytes("score", B, H, 0, nb, d))
        self.ws_attn = z(bskv.workspace_bytes("attn", B, wl.Hq, H, d, wl.U))
        self.ws_layer = z(bskv.workspace_bytes("layer", B, wl.Hq, H, d, wl.hidden, nb, wl.U, dt))
        self.ws_mh = z(bskv.workspace_bytes("multihead", B, H, nb))
        self.side = torch.cuda.Stream(self.dev)
        self.ev_side = {(k, l): torch.cuda.Event() for k in ("start", "sel", "att") for l in range(self.L)}
        torch.cuda.synchronize()

    # the four per-layer launches
    def meanpool(self, l):
        lay = self.layers[l]
        self.bskv.kv_block_meanpool(lay["k"], lay["seq_len"], self.kc[l], 0, self.nb, newest_only=True)

    def proj(self, l):
        lay = self.layers[l]
        self.bskv.forecast_proj(lay["x_sel"], lay["w_sel"], self.wl.Hkv, self.wl.d, out=self.f[l], ws=self.ws_proj)

    def select(self, l):
        wl = self.wl
        self.bskv.forecast_block_score_topk(self.f[l], self.kc[l], wl.topk, wl.n_init, wl.n_local,
                                            seq_len=self.layers[l]["seq_len"], idx=self.idx[l], cnt=self.cnt[l],
                                            ws=self.ws_score)

    def attend(self, l):
        lay = self.layers[l]
        self.bskv.block_sparse_attn_decode(lay["q"], lay["k"], lay["v"], self.idx[l], self.cnt[l], lay["seq_len"],
                                           self.wl.scale, out=self.out[l], ws=self.ws_attn)

    def mh_select(self, l):
        """Baseline selector of layer l from its own queries (comparison only)."""
        wl, lay = self.wl, self.layers[l]
        self.bskv.multihead_block_score_topk(lay["q"], self.kc[l], wl.topk, wl.n_init, wl.n_local, lay["seq_len"],
                                             scale=wl.scale, idx=self.idx[l], cnt=self.cnt[l], ws=self.ws_mh)

    def step_baseline(self):
        """The serial order of a same-layer selector: layer l's blocks are
        chosen from layer l's queries, so selection and attention of a layer
        run one after the other (no lookahead)."""
        for l in range(self.L):
            self.meanpool(l)
            self.mh_select(l)
            self.attend(l)

    def layer(self, l, stages=3):
        """Layer l: newest-block update, attention over B_l, and (lookahead)
        F_l selecting layer l+1; two kernels.  Immediate mode: B_{l+1} is
        complete when the call ends (the top-k runs in its second kernel).
        Deferred mode: the call leaves layer l+1's candidate scores and the
        next call starts with their top-k."""
        wl, lay = self.wl, self.layers[l]
        nxt = l + 1 < self.L
        n = self.layers[l + 1] if nxt else None
        deferred = self.select_mode == "deferred"
        kw = {}
        if nxt and deferred:
            kw["scores_next"] = self.scores[l + 1]
        elif nxt:
            kw["idx_next"], kw["cnt_next"] = self.idx[l + 1], self.cnt[l + 1]
        self.bskv.decode_layer_lookahead(
            lay["q"], lay["k"], lay["v"], lay["seq_len"], self.kc[l], self.idx[l], self.cnt[l], wl.scale,
            out=self.out[l], x=n["x_sel"] if nxt else None, w=n["w_sel"] if nxt else None,
            kc_next=self.kc[l + 1] if nxt else None, scores=self.scores[l] if (deferred and l > 0) else None,
            topk=wl.topk, n_init=wl.n_init, n_local=wl.n_local, stages=stages, ws=self.ws_layer, **kw)

    def step(self):
        # layer 0 is selected by the separate layer-0 projection; then every
        # layer's Forecast selects the next layer while the layer attends
        self.proj(0)
        self.select(0)
        for l in range(self.L):
            self.layer(l)

    def attend_layer(self, l):
        """Layer l's attention over B_l with the merge and the newest-block
        update (the fused layer call without a lookahead: one launch)."""
        wl, lay = self.wl, self.layers[l]
        self.bskv.decode_layer_lookahead(lay["q"], lay["k"], lay["v"], lay["seq_len"], self.kc[l], self.idx[l],
                                         self.cnt[l], wl.scale, out=self.out[l], topk=wl.topk, n_init=wl.n_init,
                                         n_local=wl.n_local, ws=self.ws_layer)

    def step_two_streams(self):
        """One-layer-ahead selection on a side stream: the selection of
        layer l+1 (F_l = x_l W_F, scores against layer l+1's compressed
        keys, top-k + union) runs while layer l attends on the compute
        stream.  It starts once layer l-1 has attended (x_l is computed from
        layer l-1's output in a model); layer l+1 attends once its list is
        complete."""
        torch = self.torch
        main = torch.cuda.current_stream(self.dev)
        side = self.side
        ev_start = self.ev_side[("start", 0)]
        ev_start.record(main)
        side.wait_event(ev_start)
        with torch.cuda.stream(side):
            self.proj(0)
            self.select(0)
        self.ev_side[("sel", 0)].record(side)
        for l in range(self.L):
            if l + 1 < self.L:
                if l >= 1:
                    side.wait_event(self.ev_side[("att", l - 1)])
                with torch.cuda.stream(side):
                    self.proj(l + 1)
                    self.select(l + 1)
                self.ev_side[("sel", l + 1)].record(side)
            main.wait_event(self.ev_side[("sel", l)])
            self.attend_layer(l)
            self.ev_side[("att", l)].record(main)
        main.wait_stream(side)

    def step_per_op(self):
        self.proj(0)
        self.select(0)
        for l in range(self.L):
            self.meanpool(l)
            if l + 1 < self.L:
                self.proj(l + 1)
                self.select(l + 1)
            self.attend(l)

    # algorithmic HBM bytes per launch: what the method must read and write
    # (weights, pooled keys, selected K/V, queries, block lists, outputs);
    # partial results kept in the workspace are not counted
    def bytes_per_launch(self):
        wl, B = self.wl, self.B
        H, d, U = wl.Hkv, wl.d, wl.U
        e = 2 if wl.dtype == "bf16" else 4
        cur = (self.T - 1) // wl.block
        n_cand = max(0, cur - wl.n_local + 1 - wl.n_init)
        proj = wl.hidden * H * d * e + B * wl.hidden * e + B * H * d * 4
        pool = B * H * (wl.block * d * e + d * 4)
        score = B * H * (n_cand * d * 4 + d * 4)
        lists = B * H * (U + 1) * 4
        attn = B * H * (U * wl.block * d * e * 2) + B * wl.Hq * d * e + lists
        out = B * wl.Hq * d * 4
        # the fused kernels are timed over all L layers: K1 of layer 0 has no
        # top-k (its list comes from the separate layer-0 selection) and K1 /
        # K2 of the last layer no projection / scoring; per-launch figures
        # are averages over the timed launches
        nxt = (self.L - 1) / self.L
        res = {"forecast_proj": proj, "kv_block_meanpool": pool, "score_topk": score + lists,
               "attn_decode": attn + out}
        if self.select_mode == "deferred":
            # K1 of every layer but the first runs the top-k, K1 of every
            # layer but the last the projection (timed over all L launches);
            # the candidate scores handed from K2 to the next K1 are an
            # intermediate of this split (0.5 MB each way at B8 x 128K) and
            # are not counted
            res["layer_k1"] = round((proj + lists) * nxt)
            res["layer_k2"] = round(score * nxt + attn + out + pool)
        else:
            # K1 (projection) is launched by every layer but the last and
            # timed over those; K2 of the last layer has no scoring
            res["layer_k1"] = proj
            res["layer_k2"] = round((score + lists) * nxt + attn + out + pool)
        return res

    def step_bytes(self):
        """Algorithmic bytes of one step: L projections (the layer-0 one
        included), L selections (layer 0's by the separate score/top-k call),
        L attentions with their merges, L newest-block updates."""
        b = self.bytes_per_launch()
        return self.L * (b["forecast_proj"] + b["score_topk"] + b["attn_decode"] + b["kv_block_meanpool"])


def time_graph(torch, fn, steps, warmup, use_graph=True):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                                   # one more eager pass on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
    run = g.replay if g is not None else fn
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, g


def kernel_times(torch, bench, reps=3):
    """Average duration per launch of each kernel (or per-op call): the
    launches of one kernel over all layers, repeated `reps` times, are
    captured in a HIP graph and its replay is timed with HIP events on the
    stream it runs on, so host-side launch cost does not enter.  layer_k1/
    k2 are the two kernels of the fused layer, each launched on its own
    (stages 1, 2) after a full pass has filled the workspace they read."""
    res = {}
    for l in range(bench.L):
        bench.layer(l)
    torch.cuda.synchronize()
    for name, fn in (("layer_k1", lambda l: bench.layer(l, 1)), ("layer_k2", lambda l: bench.layer(l, 2)),
                     ("kv_block_meanpool", bench.meanpool), ("forecast_proj", bench.proj),
                     ("score_topk", bench.select), ("attn_decode", bench.attend)):
        # immediate mode: the last layer has no first kernel (no projection)
        layers = range(bench.L - 1) if (name == "layer_k1" and bench.select_mode != "deferred") else range(bench.L)

        def body():
            for _ in range(reps):
                for l in layers:
                    fn(l)
        body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e-3 / (reps * len(layers))
        del g
    return res


def measured_hbm_peaks(torch, gib=2.0):
    """The box's own streaming rate, as context for the 8 TB/s figure: the
    runtime's device copy (read + write bytes per second), HIP events on the
    current stream."""
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    out = {}
    for name, fn, byt in (("copy_GBps", lambda: b.copy_(a), 2 * n),):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(byt * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    return out


def measured_gemm_tflops(torch, n=8192):
    """A plain bf16 GEMM through the vendor BLAS (n x n x n), as context for the
    2.5 PFLOP/s figure."""
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    del a, b, c
    return round(2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)


def per_layer_us(torch, bench, fn, reps=3):
    """Average time of fn(l) over all layers, graph-replayed, HIP events."""
    def body():
        for _ in range(reps):
            for l in range(bench.L):
                fn(l)
    body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st = torch.cuda.current_stream()
    e0.record(st)
    g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * bench.L)


def widened_projection_decode(torch, bench, kt):
    """The layer's projection widened by the Forecast heads for one decode
    token per sequence (Q, the new token's K/V into the cache, F), per layer;
    a GEMV bound by the weight read."""
    wl, B, dev = bench.wl, bench.B, bench.dev
    hid, H, d = wl.hidden, wl.Hkv, wl.d
    N = (wl.Hq + 3 * H) * d
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 600)
    ws = [(torch.randn(N, hid, generator=g, device=dev) * 0.02).to(torch.bfloat16) for _ in range(8)]
    x = torch.randn(B, hid, generator=g, device=dev).to(torch.bfloat16)
    kcache = torch.empty(B, H, 64, d, dtype=torch.bfloat16, device=dev)
    vcache = torch.empty_like(kcache)
    lens = torch.full((B,), 64, dtype=torch.int64, device=dev)
    q = torch.empty(B, wl.Hq, d, dtype=torch.bfloat16, device=dev)
    f = torch.empty(B, H, d, dtype=torch.float32, device=dev)

    class _L:   # eight weight replicas rotated so the 59 MB matrix is not served from the last-level cache
        L = 8

    def fn(l):
        bench.bskv.qkvf_proj_decode(x, ws[l], wl.Hq, H, kcache, vcache, lens, q_out=q, f_out=f)

    t = per_layer_us(torch, _L, fn)
    nbytes = hid * N * 2 + B * hid * 2 + B * (wl.Hq + 2 * H) * d * 2 + B * H * d * 4
    del ws
    torch.cuda.synchronize()
    return {"shape": f"x [{B} x {hid}] @ W [{hid} x {N}]", "us_per_layer": round(t, 3), "bytes": nbytes,
            "GBps": round(nbytes / t / 1e3, 1), "hbm_frac": round(nbytes / t / 1e3 / HBM_PEAK_GBS, 4),
            "forecast_only_proj_us": round(kt["forecast_proj"] * 1e6, 3)}


def window_selection(torch, bench, kt, window=32, stride=16):
    """Selection on the overlapping compression the evaluated models use
    (32-token windows at stride 16, block scores max-pooled from the window
    scores) against the block selector, per layer: the newest-window update
    and the score + top-k launches, on the same Forecast vectors.  The window
    cache holds 4x the block cache's rows, so its scoring streams ~4x the
    bytes."""
    wl, B, H, d = bench.wl, bench.B, bench.wl.Hkv, bench.wl.d
    nw = (bench.T - window) // stride + 1
    kcw = []
    for lay in bench.layers:
        t = torch.empty(B, H, nw, d, dtype=torch.float32, device=bench.dev)
        bench.bskv.kv_window_meanpool(lay["k"], lay["seq_len"], t, window, stride)
        kcw.append(t)
    ws = torch.zeros(max(256, bench.bskv.workspace_bytes("window", B, H, 0, nw)), dtype=torch.uint8, device=bench.dev)
    idx = torch.empty(B, H, wl.U, dtype=torch.int32, device=bench.dev)
    cnt = torch.empty(B, H, dtype=torch.int32, device=bench.dev)

    def sel(l):
        bench.bskv.forecast_window_score_topk(bench.f[l], kcw[l], wl.topk, wl.n_init, wl.n_local,
                                              bench.layers[l]["seq_len"], window, stride, idx=idx, cnt=cnt, ws=ws)

    def pool(l):
        lay = bench.layers[l]
        bench.bskv.kv_window_meanpool(lay["k"], lay["seq_len"], kcw[l], window, stride, newest_only=True)

    sel_us = per_layer_us(torch, bench, sel)
    pool_us = per_layer_us(torch, bench, pool)
    # algorithmic bytes of the window selection: the windows touching the
    # candidate blocks (fp32 rows), the Forecast vectors, the lists
    cur = (bench.T - 1) // wl.block
    c0, c1 = wl.n_init, cur - wl.n_local + 1
    w_lo = max(0, (wl.block * c0 - window) // stride + 1)
    w_hi = min(nw, wl.block * c1 // stride)
    nbytes = B * H * ((w_hi - w_lo) * d * 4 + d * 4 + (wl.U + 1) * 4)
    del kcw, ws
    torch.cuda.synchronize()
    fs_us = kt["score_topk"] * 1e6
    return {"window": window, "stride": stride, "windows": nw, "select_us_per_layer": round(sel_us, 3),
            "select_bytes": nbytes, "select_GBps": round(nbytes / sel_us / 1e3, 1),
            "select_hbm_frac": round(nbytes / sel_us / 1e3 / HBM_PEAK_GBS, 4),
            "newest_window_pool_us_per_layer": round(pool_us, 3),
            "block_select_us_per_layer": round(fs_us, 3), "select_ratio_vs_block": round(sel_us / fs_us, 3)}


def baseline_comparison(torch, bench, step_s, kt, args):
    """Same-GPU comparison with the baseline multi-head selector: its
    selection cost per layer against the Forecast selector's (both as
    separate score + top-k launches over all layers), and a whole step in the
    baseline's serial order against the lookahead step."""
    mh_us = per_layer_us(torch, bench, bench.mh_select)
    serial_s, _ = time_graph(torch, bench.step_baseline, max(5, args.steps // 5), 2, use_graph=not args.no_graph)
    # leave the lookahead lists in place for whoever runs next
    bench.proj(0)
    bench.select(0)
    for l in range(bench.L):
        bench.layer(l)
    torch.cuda.synchronize()
    fs_us = kt["score_topk"] * 1e6
    return {
        "what": "multi-head selector (per-head scores summed, softmax, top-k) from the layer's own queries, "
                "then attention, layer after layer (no lookahead)",
        "select_us_per_layer": round(mh_us, 3), "forecast_select_us_per_layer": round(fs_us, 3),
        "select_ratio": round(mh_us / fs_us, 3),
        "serial_step_ms": round(serial_s * 1e3, 4), "serial_tokens_per_s": round(bench.B / serial_s, 2),
        "step_ratio": round(serial_s / step_s, 3),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def selection_sweep(torch, bench, contexts=(32768, 65536, 131072), reps=3):
    """Selection cost against context length (decode, per layer): score + top-k
    + union of one layer for the whole batch at seq_len = T', on the same
    compressed keys (candidates limited by T').  Graph-replayed launches over
    all layers, HIP events."""
    wl, res = bench.wl, {}
    for tc in contexts:
        if tc > bench.T:
            continue
        lens = torch.full((bench.B,), tc, dtype=torch.int64, device=bench.dev)

        def body():
            for _ in range(reps):
                for l in range(bench.L):
                    bench.bskv.forecast_block_score_topk(bench.f[l], bench.kc[l], wl.topk, wl.n_init, wl.n_local,
                                                         seq_len=lens, idx=bench.idx[l], cnt=bench.cnt[l],
                                                         ws=bench.ws_score)
        body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        res[str(tc)] = round(e0.elapsed_time(e1) * 1e3 / (reps * bench.L), 3)
        del g
    # leave the lists of the full context in place for whoever runs next
    for l in range(bench.L):
        bench.select(l)
    torch.cuda.synchronize()
    return res


def cpu_baseline_decode(bench, budget_s=12.0, layers=None):
    """The fp64 oracle on a bounded sample of the same decode step: layer 0,
    one sequence (batch element 0, all KV heads): the newest-block pooling,
    the Forecast projection, the selection and the attention; repeated until
    the budget is spent, scaled to the full step (x B sequences x L layers).
    Timed twice, with the BLAS/OpenMP thread pools as they come (the host's
    cores) and limited to one thread; the faster leg is the reported value,
    with the thread count it ran on."""
    import numpy as np
    import oracle as orc
    torch, wl = bench.torch, bench.wl
    lay = bench.layers[0]
    n64 = lambda t: t.detach().to(torch.float64).cpu().numpy()  # noqa: E731
    k = n64(lay["k"][0:1])
    v = n64(lay["v"][0:1])
    q = n64(lay["q"][0:1])
    x = n64(lay["x_sel"][0:1])
    w = n64(lay["w_sel"])
    kc = orc.kv_block_meanpool(k, wl.block)                    # the compressed-key cache (not timed)
    lens = np.array([bench.T], dtype=np.int64)

    def sample():
        orc.kv_block_meanpool(k[:, :, bench.T - wl.block:], wl.block)      # incremental update
        f = orc.forecast_proj(x, w, wl.Hkv, wl.d)
        sel = orc.decode_select(f, kc, lens, wl.topk, wl.n_init, wl.n_local, wl.block)
        orc.attend_decode(q, k, v, sel.idx, sel.cnt, lens, wl.scale, wl.block)

    def timed(budget, cap):
        reps, total = 0, 0.0
        while total < budget and reps < cap:
            t0 = time.perf_counter()
            sample()
            total += time.perf_counter() - t0
            reps += 1
        return total / reps, reps, total

    n_layers = bench.L if layers is None else layers
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([int(p.get("num_threads", 1)) for p in info] or [1])
    except Exception:
        pass
    legs = {}
    per, reps, total = timed(budget_s * 2 / 3, 2000)
    legs[threads] = (per, reps, total)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            legs[1] = timed(budget_s / 3, 500)
    except Exception:
        pass
    best = min(legs, key=lambda n: legs[n][0])
    per, reps, total = legs[best]
    step_s = per * bench.B * n_layers
    rate = lambda n: round(bench.B / (legs[n][0] * bench.B * n_layers), 4)  # noqa: E731
    return {"value": bench.B / step_s, "unit": "tokens/s", "cores": best, "kind": "oracle",
            "sample": f"layer 0, batch element 0 (all {wl.Hkv} KV heads): newest-block pooling, projection, "
                      f"selection, attention; {reps} reps in {total:.1f}s on {best} thread(s); per-step time "
                      f"scaled x{bench.B} sequences x{n_layers} layers",
            "sample_seconds": round(per, 4), "value_by_threads": {str(n): rate(n) for n in legs},
            "cpu_model": cpu_model()}


def check_step_outputs(torch, bench):
    """The timed step's outputs (as its last replay left them) against the
    per-op path run afterwards on the same inputs: every layer's block lists
    and counts must be identical and its attention output bit-identical (the
    fused kernels run the same arithmetic in the same order).  Raises on any
    difference, so no throughput is reported for a step that computes
    something else."""
    snap = [(i.clone(), c.clone(), o.clone()) for i, c, o in zip(bench.idx, bench.cnt, bench.out)]
    for o in bench.out:
        o.fill_(float("nan"))
    bench.step_per_op()
    torch.cuda.synchronize()
    bad = [l for l, (i, c, o) in enumerate(snap)
           if not (torch.equal(i, bench.idx[l]) and torch.equal(c, bench.cnt[l]) and torch.equal(o, bench.out[l]))]
    if bad:
        raise RuntimeError(f"timed decode step differs from the per-op path in layers {bad}")
    finite = all(bool(torch.isfinite(o).all()) for _, _, o in snap)
    if not finite:
        raise RuntimeError("timed decode step left non-finite outputs")
    return {"layers_checked": len(snap), "lists_equal": True, "outputs_bit_equal": True}


def decode_select_mode(args, wl):
    """The fused layer's top-k placement for a run: as given, or (auto) in
    the next call's first kernel for 64 or more (b, g) units per layer and
    in this call's second kernel below that (B8 x 128K: 1.47-1.48 vs
    1.55-1.56 ms per step; B4 x 32K: 24.0 vs 26.1 us per layer-step, same
    box)."""
    if args.select_mode != "auto":
        return args.select_mode
    return "deferred" if wl.B * wl.Hkv >= 64 else "immediate"


def run_decode(args, torch, bskv, wl, replicas=None):
    mode = decode_select_mode(args, wl)
    bench = DecodeBench(wl, torch, bskv, layers=replicas, select_mode=mode)
    step_fn = bench.step_per_op if args.per_op else bench.step
    step_s, _ = time_graph(torch, step_fn, args.steps, args.warmup, use_graph=not args.no_graph)
    log(f"[bench] decode step {step_s * 1e3:.3f} ms ({'graph' if not args.no_graph else 'eager'})")
    post_check = check_step_outputs(torch, bench)
    log(f"[bench] timed step outputs match the per-op path: {post_check}")
    kt = kernel_times(torch, bench)
    bpl = bench.bytes_per_launch()
    kernels = {}
    for name, t in kt.items():
        gbs = bpl[name] / t / 1e9
        kernels[name] = {"us": round(t * 1e6, 3), "bytes": bpl[name], "GBps": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    step_bytes = bench.step_bytes()
    dom = "attn_decode" if args.per_op else "layer_k2"
    ach = bpl[dom] / kt[dom] / 1e9
    peaks = measured_hbm_peaks(torch)
    sweep = selection_sweep(torch, bench)
    extra = wl.hidden and not args.core_only
    base_cmp = baseline_comparison(torch, bench, step_s, kt, args) if extra else None
    win_sel = window_selection(torch, bench, kt) if extra else None
    widened = widened_projection_decode(torch, bench, kt) if extra else None
    # replicas: independent copies of one layer's inputs, rotated so that the
    # working set does not sit in the 256 MB cache; the step then covers
    # `replicas` layer-steps of a one-layer model
    per_step_layers = bench.L if replicas is None else 1
    layer_steps = bench.L // per_step_layers
    t_step = step_s / layer_steps
    result = {
        "metric": METRIC, "value": round(bench.B / t_step, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": bench.B, "T": bench.T, "layers": bench.L, "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.d, "hidden": wl.hidden, "block": wl.block, "topk": wl.topk, "n_init": wl.n_init,
                   "n_local": wl.n_local, "hip_graph": not args.no_graph,
                   "path": "per-op" if args.per_op else "fused-layer",
                   "next_layer_topk": None if args.per_op else mode},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_bytes(dom),
                     "bytes_per_launch": bpl[dom], "us_per_launch": round(kt[dom] * 1e6, 3)},
        "step_hbm_frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes": step_bytes,
        "measured_peaks": dict(peaks, roofline_frac_of_copy=round(ach / peaks["copy_GBps"], 4)),
        "select_us_per_layer_vs_T": sweep,
        "baseline_selector": base_cmp,
        "window_selector": win_sel,
        "widened_projection": widened,
        "kernels": kernels,
        "post_timing_check": post_check,
    }
    if replicas is not None:
        result["config"]["layers"] = 1
        result["config"]["replicas"] = replicas
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(bench, args.cpu_budget, layers=per_step_layers)
    return result


# ---------------------------------------------------------------------------
# tiny fp32 decode (a correctness configuration: launch-bound)
# ---------------------------------------------------------------------------
def run_tiny(args, torch, bskv, wl):
    """B1 x 4096, fp32, Forecast vectors given: score + top-k + union, then
    attention (split + merge) with the newest-block pooling, per step (three
    launches).  The work is ~378 KB, so the step is launch-bound; the HBM
    fraction is reported but not meaningful."""
    from workloads import decode_inputs
    dev = torch.device("cuda:0")
    lay = {k: (v.to(dev) if hasattr(v, "to") else v) for k, v in decode_inputs(wl, "cpu")[0].items()}
    nb = wl.T // wl.block
    kc = torch.empty(wl.B, wl.Hkv, nb, wl.d, dtype=torch.float32, device=dev)
    bskv.kv_block_meanpool(lay["k"], lay["seq_len"], kc)
    idx = torch.empty(wl.B, wl.Hkv, wl.U, dtype=torch.int32, device=dev)
    cnt = torch.empty(wl.B, wl.Hkv, dtype=torch.int32, device=dev)
    out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.float32, device=dev)
    ws_s = torch.zeros(max(256, bskv.workspace_bytes("score", wl.B, wl.Hkv, 0, nb, wl.d)), dtype=torch.uint8,
                       device=dev)
    ws_l = torch.zeros(max(256, bskv.workspace_bytes("layer", wl.B, wl.Hq, wl.Hkv, wl.d, 0, nb, wl.U, 0)),
                       dtype=torch.uint8, device=dev)

    def step():
        # selection from the given Forecast (scores, then top-k + union), then
        # the fused layer's second kernel alone (no lookahead): attention
        # splits, their merge and the newest-block pooling in one launch (the
        # newest block is local, so the selection never reads its row)
        bskv.forecast_block_score_topk(lay["f"], kc, wl.topk, wl.n_init, wl.n_local, seq_len=lay["seq_len"],
                                       idx=idx, cnt=cnt, ws=ws_s)
        bskv.decode_layer_lookahead(lay["q"], lay["k"], lay["v"], lay["seq_len"], kc, idx, cnt, wl.scale, out=out,
                                    topk=wl.topk, n_init=wl.n_init, n_local=wl.n_local, ws=ws_l)

    step_s, _ = time_graph(torch, step, args.steps, args.warmup, use_graph=not args.no_graph)
    e = 4
    n_cand = (wl.T - 1) // wl.block - wl.n_local + 1 - wl.n_init
    byt = (wl.B * wl.Hkv * (n_cand * wl.d * 4 + wl.U * wl.block * wl.d * e * 2 + wl.block * wl.d * e)
           + 2 * wl.B * wl.Hq * wl.d * 4)
    ach = byt / step_s / 1e9
    return {
        "metric": "decode step time, tiny fp32 correctness configuration", "value": round(step_s * 1e6, 3),
        "unit": "us/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.d,
                   "topk": wl.topk, "n_init": wl.n_init, "n_local": wl.n_local, "hip_graph": not args.no_graph},
        "roofline": {"bound": "hbm", "kernel": "whole step (launch-bound)", "achieved": round(ach, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 6), "traffic": None,
                     "bytes_per_step": byt},
    }


# ---------------------------------------------------------------------------
# chunked-prefill workload
# ---------------------------------------------------------------------------
class PrefillBench:
    """B x T prefill in chunks: per chunk, pool the chunk's new key blocks,
    select per 64-token query block (pooled Forecast scores, top-k + union),
    then block-sparse causal attention (bf16 MFMA)."""

    def __init__(self, wl, torch, bskv, B=None, T=None):
        from workloads import prefill_inputs
        self.torch, self.bskv, self.wl = torch, bskv, wl
        self.dev = torch.device("cuda:0")
        self.B = B or wl.B
        self.T = T or wl.T
        self.C = wl.chunk
        t0 = time.time()
        inp = prefill_inputs(wl, self.dev, B=self.B, T=self.T)
        self.k, self.v = inp["k"], inp["v"]
        n_chunks = self.T // self.C
        # each chunk's queries and Forecast vectors come out of that chunk's
        # projection: contiguous per chunk
        self.q = [inp["q"][:, :, c * self.C:(c + 1) * self.C].contiguous() for c in range(n_chunks)]
        self.f = [inp["f"][:, :, c * self.C:(c + 1) * self.C].contiguous() for c in range(n_chunks)]
        del inp
        self.n_chunks = n_chunks
        nb = self.T // wl.block
        self.kc = torch.empty(self.B, wl.Hkv, nb, wl.d, dtype=torch.float32, device=self.dev)
        n_qb = self.C // wl.block
        self.idx = [torch.empty(self.B, wl.Hkv, n_qb, wl.U, dtype=torch.int32, device=self.dev) for _ in range(n_chunks)]
        self.cnt = [torch.empty(self.B, wl.Hkv, n_qb, dtype=torch.int32, device=self.dev) for _ in range(n_chunks)]
        self.out = [torch.empty_like(self.q[0]) for _ in range(n_chunks)]
        self.seq_len = torch.full((self.B,), self.T, dtype=torch.int64, device=self.dev)
        self.ws_sel = torch.zeros(max(256, bskv.workspace_bytes("score", self.B, wl.Hkv, self.C, nb, wl.d)),
                                  dtype=torch.uint8, device=self.dev)
        # overlapping compression (32-token windows at stride 16) for the
        # variant's selection
        self.win, self.wst = 32, 16
        self.nw = (self.T - self.win) // self.wst + 1
        self.kcw = torch.empty(self.B, wl.Hkv, self.nw, wl.d, dtype=torch.float32, device=self.dev)
        torch.cuda.synchronize()
        log(f"[bench] prefill inputs in {time.time() - t0:.1f}s")

    def pool(self, c):
        nbc = self.C // self.wl.block
        self.bskv.kv_block_meanpool(self.k, self.seq_len, self.kc, c * nbc, (c + 1) * nbc)

    def select(self, c):
        wl = self.wl
        self.bskv.forecast_block_score_topk(self.f[c], self.kc, wl.topk, wl.n_init, wl.n_local, q_start=c * self.C,
                                            prefill=True, idx=self.idx[c], cnt=self.cnt[c], ws=self.ws_sel)

    def window_pool(self, c):
        """The windows completed inside chunk c."""
        w0 = max(0, (c * self.C - self.win) // self.wst + 1)
        w1 = min(self.nw, ((c + 1) * self.C - self.win) // self.wst + 1)
        self.bskv.kv_window_meanpool(self.k, self.seq_len, self.kcw, self.win, self.wst, w0, w1)

    def window_select(self, c):
        wl = self.wl
        self.bskv.forecast_window_score_topk(self.f[c], self.kcw, wl.topk, wl.n_init, wl.n_local, None, self.win,
                                             self.wst, q_start=c * self.C, idx=self.idx[c], cnt=self.cnt[c])

    def step_window(self):
        for c in range(self.n_chunks):
            self.window_pool(c)
            self.window_select(c)
            self.attend(c)

    def attend(self, c):
        self.bskv.block_sparse_attn_prefill(self.q[c], self.k, self.v, self.idx[c], self.cnt[c], c * self.C,
                                            self.wl.scale, out=self.out[c])

    def step(self):
        for c in range(self.n_chunks):
            self.pool(c)
            self.select(c)
            self.attend(c)

    def min_attention_bytes(self):
        """Least HBM bytes the attention kernel can move per chunk on average:
        the chunk's queries and outputs (bf16), its lists, and every K/V block
        that some query block of the chunk lists, once per (sequence, KV head)."""
        wl = self.wl
        e = 2
        qo = 2 * self.B * wl.Hq * self.C * wl.d * e
        import numpy as np
        tot = 0.0
        for c in range(self.n_chunks):
            idx = self.idx[c].cpu().numpy()
            cnt = self.cnt[c].cpu().numpy()
            used = np.arange(idx.shape[3])[None, None, None, :] < cnt[..., None]
            blocks = sum(np.unique(idx[b, g][used[b, g]]).size for b in range(self.B) for g in range(wl.Hkv))
            tot += qo + blocks * 2 * wl.block * wl.d * e + idx.size * 4 + cnt.size * 4
        return tot / self.n_chunks

    def attention_flops(self):
        """2*d flops for q.k and 2*d for p.v per (query head, token, attended key):
        a listed block contributes 64 keys to each token of the query block,
        except the diagonal block, whose token r sees r + 1 of them."""
        wl = self.wl
        tot = 0.0
        for c in range(self.n_chunks):
            cnt = self.cnt[c].to(self.torch.float64)
            keys_per_qb = (cnt - 1) * 64 * 64 + 64 * 65 / 2          # summed over the 64 tokens
            tot += float(keys_per_qb.sum()) * wl.G * 4 * wl.d
        return tot


def widened_projection_prefill(torch, bench, kt, args):
    """The layer's projection widened by the Forecast heads, per 2048-token
    chunk: (Q, K, V, F) = X [W_Q | W_K | W_V | W_F] with K/V written into the
    cache and only each query block's Forecast sum kept; against the same
    GEMM through the vendor BLAS; the selection from the sums; and the whole
    chunked prefill with the projection in front (projection, pooling,
    selection, attention)."""
    wl, B, C, dev = bench.wl, bench.B, bench.C, bench.dev
    hid, H, d = 4096, wl.Hkv, wl.d
    N = (wl.Hq + 3 * H) * d
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 500)
    x = torch.randn(B, C, hid, generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn(N, hid, generator=g, device=dev) * 0.02).to(torch.bfloat16)      # W^T: one row per column
    kc2 = torch.empty_like(bench.k)
    vc2 = torch.empty_like(bench.v)
    n_qb = C // wl.block
    q = torch.empty(B, wl.Hq, C, d, dtype=torch.bfloat16, device=dev)
    fp = torch.empty(B, H, n_qb, d, dtype=torch.float32, device=dev)
    kcmp = torch.empty_like(bench.kc)
    out = torch.empty_like(q)
    ws_sel = torch.zeros(max(256, bench.bskv.workspace_bytes("pooled", B, H, n_qb, kcmp.shape[2], d)),
                         dtype=torch.uint8, device=dev)

    def proj(c):
        bench.bskv.qkvf_proj_prefill(x, w, wl.Hq, H, kc2, vc2, q_start=c * C, q_out=q, f_pooled=fp)

    def select(c):
        bench.bskv.forecast_block_score_topk_pooled(fp, kcmp, wl.topk, wl.n_init, wl.n_local, q_start=c * C,
                                                    idx=bench.idx[c], cnt=bench.cnt[c], ws=ws_sel)

    def blas(c):
        return x.view(-1, hid) @ w.t()

    def step():
        for c in range(bench.n_chunks):
            proj(c)
            bench.bskv.kv_block_meanpool(kc2, bench.seq_len, kcmp, c * n_qb, (c + 1) * n_qb)
            select(c)
            bench.bskv.block_sparse_attn_prefill(q, kc2, vc2, bench.idx[c], bench.cnt[c], c * C, wl.scale, out=out)

    def per_call(fn, reps=8):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(r % bench.n_chunks)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    step()                                   # fills the caches and compressed keys of every chunk
    torch.cuda.synchronize()
    t_proj, t_blas, t_sel = per_call(proj), per_call(blas), per_call(select)
    flops = 2.0 * B * C * hid * N
    step_s, _ = time_graph(torch, step, max(1, args.steps // 10), 1, use_graph=not args.no_graph)
    del kc2, vc2, x, w
    torch.cuda.synchronize()
    return {
        "shape": f"X [{B * C} x {hid}] @ W [{hid} x {N}] per chunk (Q {wl.Hq}, K/V/F {H} heads of {d}); "
                 f"W stored as W^T [{N} x {hid}]",
        "qkvf_proj_prefill_us": round(t_proj * 1e6, 2), "TFLOPs": round(flops / t_proj / 1e12, 1),
        "mfma_frac": round(flops / t_proj / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "vendor_blas_same_gemm_us": round(t_blas * 1e6, 2),
        "vendor_blas_TFLOPs": round(flops / t_blas / 1e12, 1),
        "pooled_select_us": round(t_sel * 1e6, 2),
        "per_token_select_us": round(kt["score_topk_prefill"] * 1e6, 2),
        "step_with_projection_ms": round(step_s * 1e3, 3),
        "tokens_per_s_with_projection": round(B * bench.T / step_s, 1),
    }


def run_prefill(args, torch, bskv, wl):
    bench = PrefillBench(wl, torch, bskv)
    step_s, _ = time_graph(torch, bench.step, max(1, args.steps // 10), max(1, args.warmup // 5),
                           use_graph=not args.no_graph)
    flops = bench.attention_flops()
    # per-kernel: each kernel over all chunks, graph-replayed, HIP events
    kt = {}
    # attention runs on the block selector's lists; the window selector's
    # launches come last (they overwrite the lists, which are then restored)
    timed = [("kv_block_meanpool", bench.pool), ("score_topk_prefill", bench.select), ("attn_prefill", bench.attend)]
    if not args.core_only:
        timed += [("kv_window_meanpool", bench.window_pool), ("window_select_prefill", bench.window_select)]
    for name, fn in timed:
        def body():
            for c in range(bench.n_chunks):
                fn(c)
        body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        kt[name] = e0.elapsed_time(e1) * 1e-3 / bench.n_chunks
        del g
    for c in range(bench.n_chunks):
        bench.select(c)
    torch.cuda.synchronize()
    B, T, H, d, C = bench.B, bench.T, wl.Hkv, wl.d, bench.C
    f_bytes = B * H * C * d * 2                                   # Forecast vectors of a chunk (bf16)
    kc_read = B * H * sum(max(0, qb - wl.n_local + 1 - wl.n_init) for qb in range(T // 64)) * d * 4 / bench.n_chunks
    per_chunk_flops = flops / bench.n_chunks
    gemm_tf = measured_gemm_tflops(torch)
    att_tf = per_chunk_flops / kt["attn_prefill"] / 1e12
    kernels = {
        "kv_block_meanpool": {"us": round(kt["kv_block_meanpool"] * 1e6, 2),
                              "GBps": round(B * H * C * d * 2 / kt["kv_block_meanpool"] / 1e9, 1)},
        "score_topk_prefill": {"us": round(kt["score_topk_prefill"] * 1e6, 2),
                               "GBps_forecast_read": round(f_bytes / kt["score_topk_prefill"] / 1e9, 1),
                               "pooled_key_rows_read_per_chunk_MB": round(kc_read / 1e6, 1)},
        "attn_prefill": {"us": round(kt["attn_prefill"] * 1e6, 2), "TFLOPs": round(att_tf, 1),
                         "mfma_frac": round(att_tf / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    # least bytes of the attention, from the block selector's lists (the
    # variants below overwrite them)
    min_bytes = bench.min_attention_bytes()
    widened = window_variant = None
    if not args.core_only:
        widened = widened_projection_prefill(torch, bench, kt, args)
        # the overlapping-compression variant (32/16 windows, block scores
        # max-pooled): its pooling and selection per chunk, and its whole step
        # (the window selection leaves the lists of the block selector's place)
        win_step_s, _ = time_graph(torch, bench.step_window, max(1, args.steps // 10), 1,
                                   use_graph=not args.no_graph)
        window_variant = {
            "window": bench.win, "stride": bench.wst,
            "kv_window_meanpool_us": round(kt["kv_window_meanpool"] * 1e6, 2),
            "window_select_prefill_us": round(kt["window_select_prefill"] * 1e6, 2),
            "select_ratio_vs_block": round(kt["window_select_prefill"] / kt["score_topk_prefill"], 3),
            "step_ms": round(win_step_s * 1e3, 3), "tokens_per_s": round(B * T / win_step_s, 1),
        }
    return {
        "metric": "prefill tokens/s at B×T (chunked, block-sparse); % bf16 MFMA peak", "value": round(B * T / step_s, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": max(1, args.steps // 10), "warmup": max(1, args.warmup // 5),
        "ms_per_step": round(step_s * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "chunk": C, "Hq": wl.Hq, "Hkv": H, "head_dim": d,
                   "block": wl.block, "topk": wl.topk, "n_init": wl.n_init, "n_local": wl.n_local,
                   "hip_graph": not args.no_graph},
        "roofline": {"bound": "mfma", "kernel": "attn_prefill", "achieved": round(att_tf, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(att_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_bytes("attn_prefill"), "flops_per_launch": per_chunk_flops,
                     "min_bytes_per_launch": round(min_bytes),
                     "us_per_launch": round(kt["attn_prefill"] * 1e6, 2)},
        "attention_tflop_total": round(flops / 1e12, 2),
        "measured_gemm_bf16_TFLOPs": gemm_tf,
        "roofline_frac_of_measured_gemm": round(att_tf / gemm_tf, 4),
        "kernels": kernels,
        "window_variant": window_variant,
        "widened_projection": widened,
    }


# ---------------------------------------------------------------------------
# offloaded lookahead decode workload
# ---------------------------------------------------------------------------
class OffloadBench:
    """Decode with the whole bf16 KV cache in host-pinned memory.  The GPU
    holds every layer's compressed keys and a 2-slot ring of selected blocks.
    Layer l: F_l selects layer l+1 (projection + score/top-k on the compute
    stream), the side stream gathers layer l+1's blocks from the host pool
    into ring slot (l+1) % 2, and layer l attends from slot l % 2 once its own
    gather (issued one layer earlier) has completed."""

    def __init__(self, wl, torch, bskv, B=None, T=None, layers=None, host_layers=None):
        from workloads import decode_inputs
        self.torch, self.bskv, self.wl = torch, bskv, wl
        self.dev = torch.device("cuda:0")
        self.B = B or wl.B
        self.T = T or wl.T
        self.L = layers or wl.layers
        self.HL = host_layers or wl.host_layers
        t0 = time.time()
        gen = decode_inputs(wl, self.dev, layers=self.HL, B=self.B, T=self.T)
        nb = self.T // wl.block
        self.nb = nb
        self.kc, self.host_k, self.host_v, self.dk, self.dv = [], [], [], [], []
        self.x, self.w, self.q, self.seq_len = [], [], [], gen[0]["seq_len"]
        for lay in gen:
            kc = torch.empty(self.B, wl.Hkv, nb, wl.d, dtype=torch.float32, device=self.dev)
            bskv.kv_block_meanpool(lay["k"], lay["seq_len"], kc)      # built when the cache was written
            hk = torch.empty(lay["k"].shape, dtype=torch.bfloat16, pin_memory=True)
            hv = torch.empty(lay["v"].shape, dtype=torch.bfloat16, pin_memory=True)
            hk.copy_(lay["k"])
            hv.copy_(lay["v"])
            self.kc.append(kc)
            self.host_k.append(hk)
            self.host_v.append(hv)
            self.dk.append(bskv.host_device_pointer(hk))
            self.dv.append(bskv.host_device_pointer(hv))
            self.x.append(lay["x_sel"])
            self.w.append(lay["w_sel"])
            self.q.append(lay["q"])
            del lay["k"], lay["v"]
        del gen
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        U, H, d = wl.U, wl.Hkv, wl.d
        from block_sparse_long_kv_amd.offload import LookaheadRing, OffloadLayer
        self.f = [torch.empty(self.B, H, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        self.idx = [torch.empty(self.B, H, U, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.cnt = [torch.empty(self.B, H, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.out = [torch.empty(self.B, wl.Hq, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        # layer l reads host layer l mod host_layers (the pinned pool holds host_layers distinct layers)
        self.layers = [OffloadLayer(self.host_k[self.h(l)], self.host_v[self.h(l)], self.kc[self.h(l)],
                                    self.x[self.h(l)], self.w[self.h(l)], self.q[self.h(l)], self.seq_len,
                                    self.f[l], self.idx[l], self.cnt[l], self.out[l],
                                    host_k_dev=self.dk[self.h(l)], host_v_dev=self.dv[self.h(l)])
                       for l in range(self.L)]
        z = lambda n: torch.zeros(max(int(n), 256), dtype=torch.uint8, device=self.dev)  # noqa: E731
        self.ws_proj = z(bskv.workspace_bytes("proj", self.B, wl.hidden, H, d, 1))
        self.ws_score = z(bskv.workspace_bytes("score", self.B, H, 0, nb, d))
        self.ws_attn = z(bskv.workspace_bytes("attn", self.B, wl.Hq, H, d, U))
        self.ring = LookaheadRing(self.B, H, U, d, device=self.dev, n_workgroups=256)
        torch.cuda.synchronize()
        log(f"[bench] offload set-up ({self.HL} host layers, {2 * self.HL * hk.numel() * 2 / 2**30:.0f} GiB pinned) "
            f"in {time.time() - t0:.1f}s")

    @property
    def n_wg(self):
        return self.ring.n_workgroups

    @n_wg.setter
    def n_wg(self, v):
        self.ring.n_workgroups = v

    def h(self, l):
        return l % self.HL

    def prefetch(self, l, stream=None):
        self.ring.prefetch(self.layers[l], l % 2, stream=stream)

    def step(self, with_copy=True):
        wl = self.wl
        self.ring.step(self.layers, wl.topk, wl.n_init, wl.n_local, wl.scale, ws_proj=self.ws_proj,
                       ws_score=self.ws_score, ws_attn=self.ws_attn, with_copy=with_copy)

    def copy_only(self):
        for l in range(self.L):
            self.prefetch(l)


def run_offload(args, torch, bskv, wl):
    bench = OffloadBench(wl, torch, bskv)
    # the pages tune the copy kernel's thread-block count to the batch: pick it here
    bench.step(with_copy=False)
    torch.cuda.synchronize()
    sweep = {}
    for nwg in (64, 128, 256, 512, 1024):
        bench.n_wg = nwg
        bench.prefetch(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(4):
            bench.prefetch(l)
        torch.cuda.synchronize()
        sweep[nwg] = (time.perf_counter() - t0) / 4
    bench.n_wg = min(sweep, key=sweep.get)
    log(f"[bench] prefetch workgroups sweep (s per layer): {sweep} -> {bench.n_wg}")

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    # the host link itself: one contiguous pinned -> device copy (DMA engine)
    src = bench.host_k[0].view(-1)[: 1 << 29]
    dst = torch.empty(src.shape, dtype=src.dtype, device=bench.dev)
    t_h2d = timed(lambda: dst.copy_(src, non_blocking=True), 3)
    h2d_gbps = src.numel() * 2 / t_h2d / 1e9
    del dst
    n = max(1, args.steps // 25)
    t_total = timed(bench.step, n)
    t_compute = timed(lambda: bench.step(with_copy=False), n)
    t_copy = timed(bench.copy_only, n)
    hidden = max(0.0, min(1.0, (t_compute + t_copy - t_total) / t_copy))
    U, H, d = wl.U, wl.Hkv, wl.d
    cnt_total = sum(int(c.sum()) for c in bench.cnt)
    copy_bytes = cnt_total * wl.block * d * 2 * 2
    return {
        "metric": "offloaded lookahead decode tokens/s at B×T (KV in host-pinned memory); % copy hidden",
        "value": round(bench.B / t_total, 2), "unit": "tokens/s", "n_gpus": 1, "steps": n, "warmup": 1,
        "ms_per_step": round(t_total * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": bench.B, "T": bench.T, "layers": bench.L, "host_layers": bench.HL,
                   "Hq": wl.Hq, "Hkv": H, "head_dim": d, "topk": wl.topk, "n_init": wl.n_init,
                   "n_local": wl.n_local, "prefetch_workgroups": bench.n_wg},
        "roofline": {"bound": "host-link", "kernel": "prefetch_selected_blocks",
                     "achieved": round(copy_bytes / t_copy / 1e9, 2), "peak": 64.0, "unit": "GB/s",
                     "frac": round(copy_bytes / t_copy / 1e9 / 64.0, 4), "traffic": None,
                     "bytes_per_step": copy_bytes},
        "copy_hidden_frac": round(hidden, 4),
        "h2d_memcpy_GBps": round(h2d_gbps, 2),
        "ms_compute_only": round(t_compute * 1e3, 3), "ms_copy_only": round(t_copy * 1e3, 3),
        "prefetch_sweep_ms_per_layer": {str(k): round(v * 1e3, 3) for k, v in sweep.items()},
    }


# ---------------------------------------------------------------------------
# steady-state offloaded decode: resident block cache + model stand-in
# ---------------------------------------------------------------------------
class SteadyOffloadBench:
    """Decode steps with the whole bf16 KV cache in host-pinned memory and,
    per layer, a GPU-resident cache of S blocks per (b, g) (least recently
    used).  Per layer l of a step, on the compute stream: the layer's Q/K/V
    projection GEMM (stand-in), the selection of layer l+1 from F_l
    (projection + score/top-k), the cache lookup of layer l+1; on the copy
    stream: the copy of layer l+1's missing blocks from host memory; back on
    the compute stream, once layer l's copy is done: attention of layer l from
    its cache, then the output projection and FFN GEMMs of an 8B-class layer
    (stand-ins: random bf16 weights, hipBLASLt through torch).  The Forecast
    input of every layer drifts by a random walk from step to step, which
    sets how many selected blocks change per step."""

    def __init__(self, wl, torch, bskv, n_steps, S=128, drift=None, fused_fill=True):
        from workloads import decode_inputs, drift_walk
        self.torch, self.bskv, self.wl = torch, bskv, wl
        self.dev = torch.device("cuda:0")
        self.B, self.T, self.L, self.HL, self.S = wl.B, wl.T, wl.layers, wl.host_layers, S
        self.drift = wl.drift if drift is None else drift
        t0 = time.time()
        gen = decode_inputs(wl, self.dev, layers=self.HL)
        nb = self.T // wl.block
        H, d, U = wl.Hkv, wl.d, wl.U
        self.kc, self.host_k, self.host_v, self.dk, self.dv, self.w, self.q = [], [], [], [], [], [], []
        x0 = []
        self.seq_len = gen[0]["seq_len"]
        for lay in gen:
            kc = torch.empty(self.B, H, nb, d, dtype=torch.float32, device=self.dev)
            bskv.kv_block_meanpool(lay["k"], lay["seq_len"], kc)
            hk = torch.empty(lay["k"].shape, dtype=torch.bfloat16, pin_memory=True)
            hv = torch.empty(lay["v"].shape, dtype=torch.bfloat16, pin_memory=True)
            hk.copy_(lay["k"])
            hv.copy_(lay["v"])
            self.kc.append(kc)
            self.host_k.append(hk)
            self.host_v.append(hv)
            self.dk.append(bskv.host_device_pointer(hk))
            self.dv.append(bskv.host_device_pointer(hv))
            self.w.append(lay["w_sel"])
            self.q.append(lay["q"])
            x0.append(lay["x_sel"])
            del lay["k"], lay["v"]
        del gen
        # per-layer Forecast inputs of every step: independent random walks
        x0 = torch.stack([x0[l % self.HL] for l in range(self.L)])            # [L, B, hidden]
        self.xs = drift_walk(x0, n_steps, self.drift, wl.seed + 1000)         # [steps, L, B, hidden]
        # stand-in weights of an 8B-class layer: Q/K/V projection, output
        # projection, gate+up and down projections of the FFN
        hid, ffn = wl.hidden, 14336
        g = torch.Generator(device=self.dev)
        g.manual_seed(wl.seed + 2000)
        rnd = lambda *sh: (torch.randn(*sh, generator=g, device=self.dev) * 0.02).to(torch.bfloat16)  # noqa: E731
        self.w_qkv = [rnd(hid, wl.Hq * d + 2 * H * d) for _ in range(self.L)]
        self.w_o = [rnd(wl.Hq * d, hid) for _ in range(self.L)]
        self.w_gu = [rnd(hid, 2 * ffn) for _ in range(self.L)]
        self.w_down = [rnd(ffn, hid) for _ in range(self.L)]
        self.standin_bytes = sum(t.numel() * 2 for t in (self.w_qkv[0], self.w_o[0], self.w_gu[0], self.w_down[0]))
        self.ffn = ffn
        self.caches = [bskv.BlockCache(self.B, H, S, d, device=self.dev) for _ in range(self.L)]
        self.f = [torch.empty(self.B, H, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        self.idx = [torch.empty(self.B, H, U, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.cnt = [torch.empty(self.B, H, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.slot = [torch.empty(self.B, H, U, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.fill = [torch.empty(self.B, H, U, dtype=torch.int32, device=self.dev) for _ in range(self.L)]
        self.n_fill = torch.zeros(self.L, self.B, H, dtype=torch.int32, device=self.dev)
        self.fills = torch.zeros((), dtype=torch.int64, device=self.dev)      # blocks copied, summed over steps
        self.xbuf = torch.empty_like(self.xs[0])                              # this step's Forecast inputs
        self.out = [torch.empty(self.B, wl.Hq, d, dtype=torch.float32, device=self.dev) for _ in range(self.L)]
        z = lambda n: torch.zeros(max(int(n), 256), dtype=torch.uint8, device=self.dev)  # noqa: E731
        self.ws_proj = z(bskv.workspace_bytes("proj", self.B, hid, H, d, 1))
        self.ws_score = z(bskv.workspace_bytes("score", self.B, H, 0, nb, d))
        self.ws_attn = z(bskv.workspace_bytes("attn", self.B, wl.Hq, H, d, U))
        from block_sparse_long_kv_amd.offload import CachedLookahead, OffloadLayer
        self.layers = [OffloadLayer(self.host_k[l % self.HL], self.host_v[l % self.HL], self.kc[l % self.HL],
                                    self.xbuf[l], self.w[l % self.HL], self.q[l % self.HL], self.seq_len,
                                    self.f[l], self.idx[l], self.cnt[l], self.out[l],
                                    host_k_dev=self.dk[l % self.HL], host_v_dev=self.dv[l % self.HL])
                       for l in range(self.L)]
        self.sched = CachedLookahead(self.caches, self.slot, self.fill, [self.n_fill[l] for l in range(self.L)],
                                     device=self.dev, n_workgroups=self.B * H, fused_fill=fused_fill)
        torch.cuda.synchronize()
        log(f"[bench] steady offload set-up ({self.HL} host layers pinned, {self.L} caches of {S} slots, "
            f"{self.L * self.standin_bytes / 1e9:.1f} GB stand-in weights) in {time.time() - t0:.1f}s")

    @property
    def n_wg(self):
        return self.sched.n_workgroups

    @n_wg.setter
    def n_wg(self, v):
        self.sched.n_workgroups = v

    def fill_cache(self, l, stream=None):
        self.sched.fill_cache(self.layers[l], l, stream=stream)

    def standin_pre(self, l):
        return self.xbuf[l] @ self.w_qkv[l]

    def standin_post(self, l):
        torch = self.torch
        a = self.out[l].view(self.B, -1).to(torch.bfloat16)
        h = a @ self.w_o[l]
        gu = h @ self.w_gu[l]
        act = torch.nn.functional.silu(gu[:, : self.ffn]) * gu[:, self.ffn:]
        return act @ self.w_down[l]

    def body(self, with_copy=True, standin=True):
        """One decode step on the Forecast inputs in xbuf (graph-capturable)."""
        wl = self.wl
        self.sched.step(self.layers, wl.topk, wl.n_init, wl.n_local, wl.scale, ws_proj=self.ws_proj,
                        ws_score=self.ws_score, ws_attn=self.ws_attn, with_copy=with_copy,
                        before_layer=self.standin_pre if standin else None,
                        after_layer=self.standin_post if standin else None)

    def copy_only(self):
        for l in range(self.L):
            self.fill_cache(l)


def run_offload_steady(args, torch, bskv, wl):
    warm, n = max(3, args.warmup), max(5, args.steps // 5)
    n_comp = max(3, n // 2)
    wg_sweep, n_sweep = (16, 32, 64, 128), 4
    total = warm + len(wg_sweep) * n_sweep + n + 2 * n_comp
    bench = SteadyOffloadBench(wl, torch, bskv, total, drift=args.drift, fused_fill=args.offload_fill == "fused")
    sync = torch.cuda.synchronize
    graphs = {}

    def graph(with_copy=True, standin=True):
        key = (with_copy, standin, bench.n_wg)
        if args.no_graph:
            return None
        if key not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                bench.body(with_copy=with_copy, standin=standin)
            graphs[key] = g
        return graphs[key]

    def run(t0, t1, **kw):
        g = graph(**kw)
        sync()
        a = time.perf_counter()
        for t in range(t0, t1):
            bench.xbuf.copy_(bench.xs[t])
            if g is None:
                bench.body(**kw)
            else:
                g.replay()
            bench.fills += bench.n_fill.sum()       # outside the graph
        sync()
        return (time.perf_counter() - a) / (t1 - t0)

    # warm-up: eager steps fill the caches, then the graphs are captured
    # (capture itself runs nothing) and replayed
    for t in range(warm):
        bench.xbuf.copy_(bench.xs[t])
        bench.body()
    sync()
    # the copy kernel shares the GPU with the layer's compute: pick its
    # workgroup count (the pages tune it to the batch) on whole steps
    t = warm
    sweep = {}
    for nwg in wg_sweep:
        bench.n_wg = nwg
        run(t, t + 1)
        sweep[nwg] = run(t + 1, t + n_sweep)
        t += n_sweep
    bench.n_wg = min(sweep, key=sweep.get)
    for kw in ({}, {"with_copy": False}, {"with_copy": False, "standin": False}):
        graph(**kw)
    sync()
    bench.fills.zero_()
    t_total = run(t, t + n)
    t += n
    fills_per_step = float(bench.fills) / n
    last_fill = float(bench.n_fill.to(torch.int64).sum())
    sync()
    a = time.perf_counter()
    bench.copy_only()                                                # the last step's copies, alone
    sync()
    t_copy_last = time.perf_counter() - a
    # same steps without the copies (lists and lookups still run), with and
    # without the model stand-in
    t_comp = run(t, t + n_comp, with_copy=False)
    t_path = run(t + n_comp, t + 2 * n_comp, with_copy=False, standin=False)
    blk = wl.block * wl.d * 2 * 2                                    # one block's K and V (bf16)
    copy_bytes = fills_per_step * blk
    copy_gbps = last_fill * blk / t_copy_last / 1e9 if t_copy_last > 0 else None
    t_copy = copy_bytes / (copy_gbps * 1e9) if copy_gbps else 0.0
    hidden = max(0.0, min(1.0, (t_comp + t_copy - t_total) / t_copy)) if t_copy > 0 else 1.0
    nbg = bench.B * wl.Hkv
    return {
        "metric": "steady-state offloaded decode tokens/s at B×T (KV in host-pinned memory, resident block cache); "
                  "% copy hidden",
        "value": round(bench.B / t_total, 2), "unit": "tokens/s", "n_gpus": 1, "steps": n, "warmup": warm,
        "ms_per_step": round(t_total * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": bench.B, "T": bench.T, "layers": bench.L, "host_layers": bench.HL,
                   "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.d, "topk": wl.topk, "n_init": wl.n_init,
                   "n_local": wl.n_local, "planted": wl.plant, "cache_slots": bench.S, "drift": bench.drift,
                   "standin": "per layer x@W_qkv (4096x6144), o-proj (4096x4096), FFN gate+up (4096x28672), "
                              "down (14336x4096), bf16",
                   "prefetch_workgroups": bench.n_wg, "hip_graph": not args.no_graph,
                   "fill": args.offload_fill},
        "roofline": {"bound": "host-link", "kernel": "prefetch_cache_fill", "achieved": round(copy_gbps, 2)
                     if copy_gbps else None, "peak": 64.0, "unit": "GB/s",
                     "frac": round(copy_gbps / 64.0, 4) if copy_gbps else None, "traffic": None,
                     "bytes_per_step": round(copy_bytes)},
        "blocks_fetched_per_bg_layer_step": round(fills_per_step / (nbg * bench.L), 3),
        "fetched_frac_of_union": round(fills_per_step / (nbg * bench.L * wl.U), 4),
        "copy_hidden_frac": round(hidden, 4),
        "ms_compute_only": round(t_comp * 1e3, 3), "ms_path_only": round(t_path * 1e3, 3),
        "ms_copy_only": round(t_copy * 1e3, 3),
        "standin_GB_per_step": round(bench.L * bench.standin_bytes / 1e9, 2),
        "fill_workgroups_sweep_ms_per_step": {str(k): round(v * 1e3, 3) for k, v in sweep.items()},
    }


def _core_args(args, steps=None):
    import copy
    a = copy.copy(args)
    a.core_only, a.no_cpu_baseline, a.per_op = True, True, False
    if steps is not None:
        a.steps = steps
    return a


def side_decode_b4(args, torch, bskv, wl):
    """The B4 x 32K decode workload (one layer, eight replicas rotated so the
    45 MB working set is not served from the last-level cache), compactly."""
    r = run_decode(_core_args(args), torch, bskv, wl, replicas=8)
    k2 = r["kernels"]["layer_k2"]
    return {"workload": wl.name, "tokens_per_s": r["value"], "us_per_layer_step": round(r["ms_per_step"] * 1e3 / 8, 3),
            "step_hbm_frac": r["step_hbm_frac"], "layer_k2_us": k2["us"], "layer_k2_hbm_frac": k2["hbm_frac"],
            "layer_k1_us": r["kernels"]["layer_k1"]["us"], "next_layer_topk": r["config"]["next_layer_topk"],
            "outputs_checked": r["post_timing_check"]}


def side_prefill(args, torch, bskv, wl):
    """The B4 x 128K chunked prefill (pool + select + attend per 2048-token
    chunk), compactly; its parity is covered by the full-size GPU test."""
    r = run_prefill(_core_args(args), torch, bskv, wl)
    at = r["kernels"]["attn_prefill"]
    return {"workload": wl.name, "tokens_per_s": r["value"], "ms_per_step": r["ms_per_step"],
            "attn_ms_per_chunk": round(at["us"] / 1e3, 4), "attn_TFLOPs": at["TFLOPs"], "attn_mfma_frac": at["mfma_frac"],
            "score_topk_us_per_chunk": r["kernels"]["score_topk_prefill"]["us"],
            # the same box's dense bf16 GEMM through torch (hipBLASLt, 8192^3):
            # what the matrix cores deliver to a library kernel here
            "measured_gemm_bf16_TFLOPs": r["measured_gemm_bf16_TFLOPs"],
            "attn_frac_of_measured_gemm": r["roofline_frac_of_measured_gemm"],
            "parity": "tests/test_gpu_fullsize.py::test_prefill_B4_128K_chunks_sampled (10,752 rows vs the oracle)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode-b4", "decode-tiny", "prefill", "offload", "offload-steady"])
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--drift", type=float, default=None,
                    help="offload-steady: random-walk step of the Forecast input per decode step")
    ap.add_argument("--per-op", action="store_true", help="time the per-operation calls instead of the fused layer")
    ap.add_argument("--select-mode", default="auto", choices=["auto", "deferred", "immediate"],
                    help="fused layer: the next layer's top-k in the next call's first kernel (deferred) or in this "
                         "call's second kernel (immediate); auto: deferred from 64 (b, g) units per layer up")
    ap.add_argument("--offload-fill", default="fused", choices=["fused", "stream"],
                    help="offload-steady: copy layer l+1's missing blocks inside layer l's attention launch (fused) "
                         "or on a copy stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--core-only", action="store_true",
                    help="only the workload's own path: no comparison selectors, variants or widened projection "
                         "(for kernel traces and counters)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="also run one device copy of this many GiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path has no multi-GPU leg.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_kv_amd as bskv
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_gib > 0:
        # counter calibration: two copies of known size, the runtime's device
        # copy (nontemporal loads) and an elementwise kernel (plain loads)
        n = int(args.copy_probe_gib * (1 << 30))
        a = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.neg(a.view(torch.bfloat16), out=b.view(torch.bfloat16))
        torch.cuda.synchronize()
        log(f"[bench] copy probes: {n} bytes read, {n} bytes written, each")
        del a, b
    if args.workload == "decode" and not args.core_only and not args.per_op:
        result = run_decode(args, torch, bskv, WORKLOADS["decode-B8-128K-32L"])
        # the other two main workloads, compactly, on the same run
        torch.cuda.empty_cache()
        result["decode_b4"] = side_decode_b4(args, torch, bskv, WORKLOADS["decode-B4-32K"])
        torch.cuda.empty_cache()
        result["prefill"] = side_prefill(args, torch, bskv, WORKLOADS["prefill-B4-128K"])
        print(json.dumps(result), flush=True)
        return
    if args.workload == "decode-tiny":
        result = run_tiny(args, torch, bskv, WORKLOADS["tiny-decode-fp32"])
    elif args.workload == "prefill":
        result = run_prefill(args, torch, bskv, WORKLOADS["prefill-B4-128K"])
    elif args.workload == "offload":
        result = run_offload(args, torch, bskv, WORKLOADS["offload-decode-B16-128K-32L"])
    elif args.workload == "offload-steady":
        result = run_offload_steady(args, torch, bskv, WORKLOADS["offload-steady-B16-128K-32L"])
    else:
        if args.workload == "decode":
            result = run_decode(args, torch, bskv, WORKLOADS["decode-B8-128K-32L"])
        else:
            result = run_decode(args, torch, bskv, WORKLOADS["decode-B4-32K"], replicas=8)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
