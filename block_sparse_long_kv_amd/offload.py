"""Stream ordering of offloaded decode: which library call runs on which
stream, and which event each stream waits on.  No arithmetic happens here:
every step is a call of the C ABI (through the binding), and the ordering is
the caller's part of the contract (include/bskv.h: the library records no
events).

Two schedules of one decode step over a model's layers, both with
one-layer-ahead selection ("SparDA: a fourth projection that lets sparse
attention prefetch its own KV cache", "The fourth projection", Alg. 2: the
Forecast of layer l picks layer l+1's blocks, whose copy from host-pinned
memory runs on a prefetch stream while layer l computes; the compute stream
waits for that copy before layer l+1 attends; Chinese SparDA overview,
系统实现: the GPU reads the pinned host pool directly):

``LookaheadRing``   the whole union of layer l+1 is copied into ring slot
                    (l+1) mod 2; before the copy may overwrite that slot, the
                    copy stream waits until layer l-1, its previous reader,
                    has attended.
``CachedLookahead`` each layer keeps a resident cache of blocks per (b, g);
                    the lookup of layer l+1's list names the missing blocks,
                    and only those are copied (steady state): on the copy
                    stream, or (fused_fill) by extra workgroups of layer l's
                    attention launch on the compute stream.

Both take per-layer inputs as ``OffloadLayer`` records and run eagerly or
under HIP-graph capture (all ordering is by events on the two streams).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import torch

from . import _lib


@dataclass
class OffloadLayer:
    """One layer's tensors for an offloaded decode step.

    host_k, host_v  [B, Hkv, T, d] bf16, pinned host memory (the KV pool)
    host_k_dev, host_v_dev  their device addresses (bskv_host_device_pointer);
                    looked up once when left None
    kc              [B, Hkv, NB, d] fp32 compressed keys (on the GPU)
    x_sel, w_sel    the Forecast input and weights that select this layer
                    (the previous layer's input and Forecast head; for layer
                    0 the separate layer-0 projection)
    q               [B, Hq, d] this layer's query
    seq_len         [B] int64
    f, idx, cnt, out  outputs: Forecast [B, Hkv, d] fp32, block list
                    [B, Hkv, U] int32, count [B, Hkv] int32, attention
                    output [B, Hq, d] fp32
    """
    host_k: torch.Tensor
    host_v: torch.Tensor
    kc: torch.Tensor
    x_sel: torch.Tensor
    w_sel: torch.Tensor
    q: torch.Tensor
    seq_len: torch.Tensor
    f: torch.Tensor
    idx: torch.Tensor
    cnt: torch.Tensor
    out: torch.Tensor
    host_k_dev: Optional[int] = None
    host_v_dev: Optional[int] = None

    def device_pointers(self):
        """Device addresses of the K/V source (its own for device tensors)."""
        if self.host_k_dev is None:
            self.host_k_dev = (self.host_k.data_ptr() if self.host_k.is_cuda
                               else _lib.host_device_pointer(self.host_k))
        if self.host_v_dev is None:
            self.host_v_dev = (self.host_v.data_ptr() if self.host_v.is_cuda
                               else _lib.host_device_pointer(self.host_v))
        return self.host_k_dev, self.host_v_dev


def _select(lay: OffloadLayer, topk, n_init, n_local, n_kv_heads, head_dim, ws_proj, ws_score):
    """F = x_sel @ w_sel, then the top-k + union of this layer's blocks."""
    _lib.forecast_proj(lay.x_sel, lay.w_sel, n_kv_heads, head_dim, out=lay.f, ws=ws_proj)
    _lib.forecast_block_score_topk(lay.f, lay.kc, topk, n_init, n_local, seq_len=lay.seq_len, idx=lay.idx,
                                   cnt=lay.cnt, ws=ws_score)


class LookaheadRing:
    """Two device ring slots of selected blocks and the copy stream that
    fills them (the literal one-layer-ahead prefetch).

    B, n_kv_heads, U, head_dim size the slots: [B, Hkv, U, 64, d] bf16 each
    for K and V.  n_workgroups: the copy kernel's workgroup count (the pages
    tune the prefetch kernel's thread-block count to the batch).
    """

    def __init__(self, B: int, n_kv_heads: int, U: int, head_dim: int, device="cuda", n_workgroups: int = 256,
                 copy_stream: Optional[torch.cuda.Stream] = None):
        dev = torch.device(device)
        self.device = dev
        self.ring_k = [torch.empty(B, n_kv_heads, U, 64, head_dim, dtype=torch.bfloat16, device=dev)
                       for _ in range(2)]
        self.ring_v = [torch.empty_like(self.ring_k[0]) for _ in range(2)]
        self.copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream(dev)
        self.n_workgroups = n_workgroups
        self._events = {}

    def _ev(self, kind: str, l: int) -> torch.cuda.Event:
        key = (kind, l)
        if key not in self._events:
            self._events[key] = torch.cuda.Event()
        return self._events[key]

    def prefetch(self, lay: OffloadLayer, slot: int, stream=None):
        """Copy the listed blocks of one layer into ring slot `slot`."""
        dk, dv = lay.device_pointers()
        _lib.prefetch_selected_blocks(lay.host_k, lay.host_v, lay.idx, lay.cnt, self.ring_k[slot],
                                      self.ring_v[slot], n_workgroups=self.n_workgroups, stream=stream,
                                      src_k_dev=dk, src_v_dev=dv)

    def attend(self, lay: OffloadLayer, slot: int, scale: float, ws_attn=None):
        _lib.block_sparse_attn_decode(lay.q, self.ring_k[slot], self.ring_v[slot], lay.idx, lay.cnt, lay.seq_len,
                                      scale, ring=True, out=lay.out, ws=ws_attn)

    def step(self, layers: Sequence[OffloadLayer], topk: int, n_init: int, n_local: int, scale: float,
             ws_proj=None, ws_score=None, ws_attn=None, with_copy: bool = True,
             on_refill: Optional[Callable[[int, int, torch.cuda.Stream], None]] = None):
        """One decode step over `layers` on the current (compute) stream.

        Per layer l, on the compute stream: the selection of layer l+1 (its
        Forecast input and weights, against its compressed keys); then,
        once layer l's own copy has landed, layer l's attention from ring
        slot l mod 2.  On the copy stream: after layer l+1's list exists and
        after layer l-1 has read slot (l+1) mod 2, the copy of layer l+1's
        blocks into that slot.  with_copy=False leaves the copies and the
        waits out (the slots then hold whatever they held).

        on_refill(l, slot, copy_stream), when given, runs right before the
        copy of layer l into `slot` is issued, with the copy stream current
        and every wait of that copy already in place (so work it issues
        there is ordered like the copy itself).
        """
        comp = torch.cuda.current_stream(self.device)
        cs = self.copy_stream
        H, d = layers[0].kc.shape[1], layers[0].kc.shape[3]
        L = len(layers)

        def issue_copy(l):
            slot = l % 2
            ev_sel = self._ev("sel", l)
            ev_sel.record(comp)
            cs.wait_event(ev_sel)                    # layer l's list exists
            if l >= 2:
                cs.wait_event(self._ev("att", l - 2))   # the slot's previous reader is done
            with torch.cuda.stream(cs):
                if on_refill is not None:
                    on_refill(l, slot, cs)
                self.prefetch(layers[l], slot, stream=cs)
            self._ev("pf", l).record(cs)

        _select(layers[0], topk, n_init, n_local, H, d, ws_proj, ws_score)
        if with_copy:
            issue_copy(0)
        for l in range(L):
            if l + 1 < L:
                _select(layers[l + 1], topk, n_init, n_local, H, d, ws_proj, ws_score)   # F_l picks layer l+1
                if with_copy:
                    issue_copy(l + 1)                # ... and its copy starts while layer l computes
            if with_copy:
                comp.wait_event(self._ev("pf", l))   # layer l's blocks, copied one layer earlier
            self.attend(layers[l], l % 2, scale, ws_attn)
            if with_copy:
                self._ev("att", l).record(comp)
        if with_copy:
            comp.wait_stream(cs)                     # the copy stream joins the compute stream


class CachedLookahead:
    """Offloaded decode with a resident block cache per layer (steady
    state): layer l+1's lookup names its missing blocks, and only those are
    copied from the host pool into the layer's cache on the copy stream
    while layer l computes.

    caches: one BlockCache per layer.  slot, fill, n_fill: per-layer lookup
    outputs ([B, Hkv, U] int32 twice, [B, Hkv] int32).
    fused_fill: the copy of layer l+1's missing blocks runs inside layer l's
    attention launch (bskv_block_sparse_attn_decode_cached_fill: its first
    n_workgroups workgroups copy while the rest attend), all on the compute
    stream: no copy stream and no cross-stream waits; layer 0's copy runs on
    its own ahead of the layers.
    """

    def __init__(self, caches: Sequence["_lib.BlockCache"], slot, fill, n_fill, device="cuda",
                 n_workgroups: int = 128, copy_stream: Optional[torch.cuda.Stream] = None, fused_fill: bool = False):
        self.device = torch.device(device)
        self.caches, self.slot, self.fill, self.n_fill = list(caches), list(slot), list(fill), list(n_fill)
        self.fused_fill = fused_fill
        self.copy_stream = None if fused_fill else (copy_stream if copy_stream is not None
                                                    else torch.cuda.Stream(self.device))
        self.n_workgroups = n_workgroups
        self._events = {}

    def _ev(self, kind: str, l: int) -> torch.cuda.Event:
        key = (kind, l)
        if key not in self._events:
            self._events[key] = torch.cuda.Event()
        return self._events[key]

    def plan(self, lay: OffloadLayer, l: int, topk, n_init, n_local, ws_proj, ws_score):
        H, d = lay.kc.shape[1], lay.kc.shape[3]
        _select(lay, topk, n_init, n_local, H, d, ws_proj, ws_score)
        _lib.block_cache_plan(self.caches[l], lay.idx, lay.cnt, slot=self.slot[l], fill=self.fill[l],
                              n_fill=self.n_fill[l])

    def fill_cache(self, lay: OffloadLayer, l: int, stream=None):
        dk, dv = lay.device_pointers()
        _lib.prefetch_cache_fill(lay.host_k, lay.host_v, lay.idx, self.slot[l], self.fill[l], self.n_fill[l],
                                 self.caches[l], n_workgroups=self.n_workgroups, stream=stream, src_k_dev=dk,
                                 src_v_dev=dv)

    def attend(self, lay: OffloadLayer, l: int, scale: float, ws_attn=None):
        _lib.block_sparse_attn_decode_cached(lay.q, self.caches[l], self.slot[l], lay.idx, lay.cnt, lay.seq_len,
                                             scale, out=lay.out, ws=ws_attn)

    def attend_and_fill(self, lay: OffloadLayer, l: int, nxt: OffloadLayer, scale: float, ws_attn=None):
        """Attention of layer l with the copy of layer l+1's missing blocks in the same launch."""
        dk, dv = nxt.device_pointers()
        _lib.block_sparse_attn_decode_cached_fill(
            lay.q, self.caches[l], self.slot[l], lay.idx, lay.cnt, lay.seq_len, nxt.host_k, nxt.host_v, nxt.idx,
            self.slot[l + 1], self.fill[l + 1], self.n_fill[l + 1], self.caches[l + 1], scale=scale, out=lay.out,
            ws=ws_attn, n_fill_workgroups=self.n_workgroups, src_k_dev=dk, src_v_dev=dv)

    def step(self, layers: Sequence[OffloadLayer], topk: int, n_init: int, n_local: int, scale: float,
             ws_proj=None, ws_score=None, ws_attn=None, with_copy: bool = True,
             before_layer: Optional[Callable[[int], None]] = None,
             after_layer: Optional[Callable[[int], None]] = None,
             on_fill: Optional[Callable[[int, torch.cuda.Stream], None]] = None):
        """One decode step.  Per layer l, on the compute stream:
        before_layer(l) (the caller's own work ahead of the layer's
        attention), the lookup of layer l+1 and, on the copy stream once that
        lookup exists, the copy of its missing blocks; then, once layer l's
        copy has landed, layer l's attention from its cache and
        after_layer(l).  on_fill(l, copy_stream) runs right before the copy
        of layer l is issued, with the copy stream current (fused_fill: the
        compute stream, before the launch that carries the copy)."""
        L = len(layers)
        if self.fused_fill:
            self.plan(layers[0], 0, topk, n_init, n_local, ws_proj, ws_score)
            if with_copy:
                if on_fill is not None:
                    on_fill(0, torch.cuda.current_stream(self.device))
                self.fill_cache(layers[0], 0)
            for l in range(L):
                if before_layer is not None:
                    before_layer(l)
                if l + 1 < L:
                    self.plan(layers[l + 1], l + 1, topk, n_init, n_local, ws_proj, ws_score)
                if with_copy and l + 1 < L:
                    if on_fill is not None:
                        on_fill(l + 1, torch.cuda.current_stream(self.device))
                    self.attend_and_fill(layers[l], l, layers[l + 1], scale, ws_attn)
                else:
                    self.attend(layers[l], l, scale, ws_attn)
                if after_layer is not None:
                    after_layer(l)
            return
        comp = torch.cuda.current_stream(self.device)
        cs = self.copy_stream

        def issue(l):
            self.plan(layers[l], l, topk, n_init, n_local, ws_proj, ws_score)
            if with_copy:
                ev = self._ev("plan", l)
                ev.record(comp)
                cs.wait_event(ev)
                with torch.cuda.stream(cs):
                    if on_fill is not None:
                        on_fill(l, cs)
                    self.fill_cache(layers[l], l, stream=cs)
                self._ev("fill", l).record(cs)

        issue(0)
        for l in range(L):
            if before_layer is not None:
                before_layer(l)
            if l + 1 < L:
                issue(l + 1)                         # F_l selects layer l+1; its missing blocks start copying
            if with_copy:
                comp.wait_event(self._ev("fill", l))
            self.attend(layers[l], l, scale, ws_attn)
            if after_layer is not None:
                after_layer(l)
        if with_copy:
            comp.wait_stream(cs)
