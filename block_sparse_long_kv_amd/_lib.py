"""ctypes marshalling for libbskv.so (see include/bskv.h for the contract)."""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbskv.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python block_sparse_long_kv_amd/build.py`")
lib = ctypes.CDLL(_LIB_PATH)

_p, _i, _i64, _sz, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_I64x3 = ctypes.c_int64 * 3


def _proto(name, res, *args):
    fn = getattr(lib, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_proto("bskv_version", _i)
_proto("bskv_strerror", ctypes.c_char_p, _i)
_proto("bskv_last_error", ctypes.c_char_p)
_proto("bskv_forecast_proj_workspace", _sz, _i, _i, _i, _i, _i)
_proto("bskv_forecast_proj", _i, _p, _p, _i, _i, _i, _i, _i, _p, _p, _sz, _p)
_proto("bskv_kv_block_meanpool", _i, _p, _i, ctypes.POINTER(_i64), _i64, _i, _i, _i, _i, _p, _i64, _i64, _i, _p, _i64,
       _p)
_proto("bskv_score_topk_workspace", _sz, _i, _i, _i, _i64, _i)
_proto("bskv_forecast_block_score_topk", _i, _p, _i, _i, _i64, _p, _i64, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p,
       _p, _sz, _p)
_proto("bskv_kv_window_meanpool", _i, _p, _i, ctypes.POINTER(_i64), _i64, _i, _i, _i, _i, _i, _p, _i64, _i64, _i, _p,
       _i64, _p)
_proto("bskv_window_score_topk_workspace", _sz, _i, _i, _i, _i64)
_proto("bskv_forecast_window_score_topk", _i, _p, _i, _i, _i64, _p, _i64, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p,
       _p, _p, _p, _sz, _p)
_proto("bskv_multihead_score_topk_workspace", _sz, _i, _i, _i64)
_proto("bskv_multihead_block_score_topk", _i, _p, _i, _p, _i64, _p, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p,
       _p, _sz, _p)
_proto("bskv_attn_decode_workspace", _sz, _i, _i, _i, _i, _i)
_proto("bskv_block_sparse_attn_decode", _i, _p, _p, _p, _i, ctypes.POINTER(_i64), _i64, _i, _p, _p, _p, _i, _i, _i,
       _i, _i, _i, _f, _p, _p, _sz, _p)
_proto("bskv_block_sparse_attn_prefill", _i, _p, _p, _p, _i, ctypes.POINTER(_i64), _i64, _p, _p, _i64, _i, _i, _i,
       _i, _i, _i, _i, _f, _p, _p)
_proto("bskv_prefetch_selected_blocks", _i, _p, _p, _i, ctypes.POINTER(_i64), _i64, _p, _p, _p, _p, _i, _i, _i, _i,
       _i, _i, _p)
_proto("bskv_host_device_pointer", _i, _p, ctypes.POINTER(_p))
_proto("bskv_qkvf_proj_decode", _i, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, ctypes.POINTER(_i64), _i64, _p, _p, _p)
_proto("bskv_qkvf_proj_prefill", _i, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _p, _p, _p, ctypes.POINTER(_i64), _i64, _p,
       _p)
_proto("bskv_score_topk_pooled_workspace", _sz, _i, _i, _i, _i64, _i)
_proto("bskv_forecast_block_score_topk_pooled", _i, _p, _i, _i64, _p, _i64, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p,
       _sz, _p)
_proto("bskv_block_cache_reset", _i, _p, _p, _p, _i, _i, _i, _p)
_proto("bskv_block_cache_plan", _i, _p, _p, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p)
_proto("bskv_prefetch_cache_fill", _i, _p, _p, _i, ctypes.POINTER(_i64), _i64, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i,
       _i, _i, _i, _p)
_proto("bskv_block_sparse_attn_decode_cached", _i, _p, _p, _p, _i, _i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _p,
       _p, _sz, _p)
_proto("bskv_block_sparse_attn_decode_cached_fill", _i, _p, _p, _p, _i, _i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f,
       _p, _p, _sz, _p, _p, ctypes.POINTER(_i64), _i64, _p, _p, _p, _p, _p, _p, _i, _i, _p)
_proto("bskv_decode_layer_lookahead_workspace", _sz, _i, _i, _i, _i, _i, _i64, _i, _i)
_proto("bskv_decode_layer_lookahead", _i, _p, _p, _p, _i, ctypes.POINTER(_i64), _i64, _p, _p, _p, _p, _p, _f, _p, _p,
       _p, _i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i64, _i, _i, _i, _i, _p, _sz, _p)

_proto("bskv_decode_layer_lookahead_noalloc_capacity", _sz)
_proto("bskv_decode_layer_lookahead_noalloc", _i, _p, _p, _p, _i, ctypes.POINTER(_i64), _i64, _p, _p, _p, _p, _p, _f,
       _p, _p, _p, _i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i64, _i, _i, _i, _i, _p)

BSKV_F32, BSKV_BF16 = 0, 1
_DT = {torch.float32: BSKV_F32, torch.bfloat16: BSKV_BF16}


class BskvError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.bskv_strerror(status).decode()
        extra = lib.bskv_last_error().decode() if status == -5 else ""
        super().__init__(f"{where}: status {status} ({msg}){': ' + extra if extra else ''}")
        self.status = status


def _check(rc: int, where: str):
    if rc != 0:
        raise BskvError(rc, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _stream(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _whole_blocks(k: torch.Tensor, where: str):
    if k.shape[2] % 64:
        raise ValueError(f"{where}: the K/V buffers must hold whole 64-token blocks (token axis {k.shape[2]}); "
                         "allocate the cache in whole blocks, tokens past seq_len are masked")


def _strides3(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("K/V must be 4-D [B, Hkv, T, d] with a contiguous last dimension")
    return _I64x3(t.stride(0), t.stride(1), t.stride(2))


# Workspaces: one buffer per (device, stream, call kind, layout), allocated
# zero-filled on first use (the decode layer's arrival counters start at
# zero) and reused by later calls of the same kind and layout.
_WS: dict = {}


def workspace_bytes(kind: str, *args) -> int:
    fn = {"proj": lib.bskv_forecast_proj_workspace, "score": lib.bskv_score_topk_workspace,
          "attn": lib.bskv_attn_decode_workspace, "layer": lib.bskv_decode_layer_lookahead_workspace,
          "multihead": lib.bskv_multihead_score_topk_workspace,
          "window": lib.bskv_window_score_topk_workspace,
          "pooled": lib.bskv_score_topk_pooled_workspace}[kind]
    return int(fn(*args))


def _workspace(device, nbytes: int, stream_handle: int, kind: str, layout: tuple) -> torch.Tensor:
    key = (device.index, stream_handle, kind, layout)
    buf = _WS.get(key)
    if buf is None:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def forecast_proj(x, w, n_kv_heads: int, head_dim: int, out=None, ws=None, stream=None):
    """F[b, g, :] = x[b] @ w[:, g*d:(g+1)*d] -> fp32 [B, Hkv, d]."""
    B, hidden = x.shape
    if w.dtype != x.dtype or not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x, w: same dtype, contiguous")
    if out is None:
        out = torch.empty(B, n_kv_heads, head_dim, dtype=torch.float32, device=x.device)
    sh = _stream(stream, x.device)
    lay = (B, hidden, n_kv_heads, head_dim, _dt(x))
    nbytes = workspace_bytes("proj", *lay)
    ws = ws if ws is not None else _workspace(x.device, nbytes, sh, "proj", lay)
    _check(lib.bskv_forecast_proj(_ptr(x), _ptr(w), _dt(x), B, hidden, n_kv_heads, head_dim, _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), sh), "forecast_proj")
    return out


def kv_block_meanpool(k, seq_len, kc, blk_begin: int = 0, blk_end: int | None = None, newest_only: bool = False,
                      stream=None):
    """Write kc[b, g, j] = mean of block j's keys for complete blocks j in [blk_begin, blk_end)."""
    B, H, _, d = k.shape
    nb_cap = kc.shape[2]
    if blk_end is None:
        blk_end = nb_cap
    if kc.dtype != torch.float32 or not kc.is_contiguous() or tuple(kc.shape) != (B, H, nb_cap, d):
        raise ValueError("kc must be contiguous fp32 [B, Hkv, nb_cap, d]")
    sh = _stream(stream, k.device)
    _check(lib.bskv_kv_block_meanpool(_ptr(k), _dt(k), _strides3(k), k.shape[2], B, H, d, 64, _ptr(seq_len),
                                      blk_begin, blk_end,
                                      int(bool(newest_only)), _ptr(kc), nb_cap, sh), "kv_block_meanpool")
    return kc


def forecast_block_score_topk(f, kc, topk: int, n_init: int, n_local: int, seq_len=None, q_start: int = 0,
                              prefill: bool = False, return_scores: bool = False, idx=None, cnt=None, ws=None,
                              stream=None):
    """Block selection: (idx int32 [..., U], cnt int32 [...]) [, scores]."""
    B, H, nb_cap, d = kc.shape
    U = topk + n_init + n_local
    if not f.is_contiguous():
        raise ValueError("f must be contiguous")
    sh = _stream(stream, f.device)
    scores = None
    if prefill:
        Tq = f.shape[2]
        n_qb = math.ceil(Tq / 64)
        idx = idx if idx is not None else torch.empty(B, H, n_qb, U, dtype=torch.int32, device=f.device)
        cnt = cnt if cnt is not None else torch.empty(B, H, n_qb, dtype=torch.int32, device=f.device)
    else:
        Tq = 0
        idx = idx if idx is not None else torch.empty(B, H, U, dtype=torch.int32, device=f.device)
        cnt = cnt if cnt is not None else torch.empty(B, H, dtype=torch.int32, device=f.device)
        if return_scores:
            scores = torch.full((B, H, nb_cap), float("nan"), dtype=torch.float32, device=f.device)
    lay = (B, H, Tq, nb_cap, d)
    nbytes = workspace_bytes("score", *lay)
    ws = ws if ws is not None else _workspace(f.device, nbytes, sh, "score", lay)
    ws_ptr, ws_n = _ptr(ws), ws.numel() * ws.element_size()
    _check(lib.bskv_forecast_block_score_topk(_ptr(f), _dt(f), Tq, q_start, _ptr(kc), nb_cap, _ptr(seq_len), B, H, d,
                                              64, topk, n_init, n_local, _ptr(idx), _ptr(cnt), _ptr(scores), ws_ptr,
                                              ws_n, sh), "forecast_block_score_topk")
    return (idx, cnt, scores) if return_scores else (idx, cnt)


def kv_window_meanpool(k, seq_len, kcw, window: int = 32, stride: int = 16, w_begin: int = 0,
                       w_end: int | None = None, newest_only: bool = False, stream=None):
    """Write kcw[b, g, w] = mean of the keys of window w (positions stride*w
    .. stride*w+window-1) for the complete windows w in [w_begin, w_end)."""
    B, H, _, d = k.shape
    nw_cap = kcw.shape[2]
    if w_end is None:
        w_end = nw_cap
    if kcw.dtype != torch.float32 or not kcw.is_contiguous() or tuple(kcw.shape) != (B, H, nw_cap, d):
        raise ValueError("kcw must be contiguous fp32 [B, Hkv, nw_cap, d]")
    sh = _stream(stream, k.device)
    _check(lib.bskv_kv_window_meanpool(_ptr(k), _dt(k), _strides3(k), k.shape[2], B, H, d, window, stride,
                                       _ptr(seq_len), w_begin, w_end, int(bool(newest_only)), _ptr(kcw), nw_cap, sh),
           "kv_window_meanpool")
    return kcw


def forecast_window_score_topk(f, kcw, topk: int, n_init: int, n_local: int, seq_len=None, window: int = 32,
                               stride: int = 16, q_start: int = 0, return_scores: bool = False, idx=None, cnt=None,
                               ws=None, stream=None):
    """Selection on window-compressed keys (block score = max over the
    block's visible windows).  Decode: f fp32 [B, Hkv, d] -> (idx [B, Hkv, U],
    cnt [B, Hkv]) [, block scores].  Prefill: f [B, Hkv, Tq, d] (fp32 or
    bf16) for the chunk at q_start -> (idx [B, Hkv, n_qb, U], cnt [B, Hkv, n_qb])."""
    B, H, nw_cap, d = kcw.shape
    U = topk + n_init + n_local
    nb = ((nw_cap - 1) * stride + window) // 64
    if not f.is_contiguous():
        raise ValueError("f must be contiguous")
    sh = _stream(stream, f.device)
    prefill = f.dim() == 4
    n_q = f.shape[2] if prefill else 0
    if prefill and return_scores:
        raise ValueError("block scores are returned for decode only")
    lead = (B, H, -(-n_q // 64)) if prefill else (B, H)
    idx = idx if idx is not None else torch.empty(*lead, U, dtype=torch.int32, device=f.device)
    cnt = cnt if cnt is not None else torch.empty(*lead, dtype=torch.int32, device=f.device)
    scores = torch.full((B, H, nb), float("nan"), dtype=torch.float32, device=f.device) if return_scores else None
    lay = (B, H, n_q, nw_cap)
    nbytes = workspace_bytes("window", *lay)
    if ws is None and nbytes > 0:
        ws = _workspace(f.device, nbytes, sh, "window", lay)
    _check(lib.bskv_forecast_window_score_topk(_ptr(f), _dt(f), n_q, q_start, _ptr(kcw), nw_cap, _ptr(seq_len), B, H,
                                               d, 64, window, stride, topk, n_init, n_local, _ptr(idx), _ptr(cnt),
                                               _ptr(scores), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                               sh), "forecast_window_score_topk")
    return (idx, cnt, scores) if return_scores else (idx, cnt)


def multihead_block_score_topk(q, kc, topk: int, n_init: int, n_local: int, seq_len, scale: float | None = None,
                               return_weights: bool = False, idx=None, cnt=None, ws=None, stream=None):
    """Baseline multi-head selection (decode) from the layer's own queries q
    [B, Hq, d]: (idx int32 [B, Hkv, U], cnt int32 [B, Hkv]) [, weights]."""
    B, H, nb_cap, d = kc.shape
    U = topk + n_init + n_local
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    sh = _stream(stream, q.device)
    idx = idx if idx is not None else torch.empty(B, H, U, dtype=torch.int32, device=q.device)
    cnt = cnt if cnt is not None else torch.empty(B, H, dtype=torch.int32, device=q.device)
    weights = None
    if return_weights:
        weights = torch.full((B, H, nb_cap), float("nan"), dtype=torch.float32, device=q.device)
    lay = (B, H, nb_cap)
    nbytes = workspace_bytes("multihead", *lay)
    ws = ws if ws is not None else _workspace(q.device, nbytes, sh, "multihead", lay)
    _check(lib.bskv_multihead_block_score_topk(_ptr(q), _dt(q), _ptr(kc), nb_cap, _ptr(seq_len), B, q.shape[1], H, d,
                                               64, topk, n_init, n_local, scale, _ptr(idx), _ptr(cnt),
                                               _ptr(weights), _ptr(ws), ws.numel() * ws.element_size(), sh),
           "multihead_block_score_topk")
    return (idx, cnt, weights) if return_weights else (idx, cnt)


def block_sparse_attn_decode(q, k, v, idx, cnt, seq_len, scale: float | None = None, ring: bool = False, out=None,
                             ws=None, stream=None):
    """Decode attention over the listed blocks -> fp32 [B, Hq, d].

    k, v: cache [B, Hkv, T, d] (any strides with a contiguous last dim), or,
    with ring=True, a ring [B, Hkv, U, 64, d] filled by prefetch_selected_blocks.
    """
    if ring and k.dim() == 5:
        k = k.flatten(2, 3)
        v = v.flatten(2, 3)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    U = idx.shape[-1]
    if k.stride() != v.stride() or k.dtype != v.dtype or q.dtype != k.dtype or not q.is_contiguous():
        raise ValueError("q contiguous; k, v with identical strides; one dtype")
    scale = (1.0 / math.sqrt(d)) if scale is None else scale
    out = out if out is not None else torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    sh = _stream(stream, q.device)
    lay = (B, Hq, Hkv, d, U)
    nbytes = workspace_bytes("attn", *lay)
    ws = ws if ws is not None else _workspace(q.device, nbytes, sh, "attn", lay)
    _whole_blocks(k, "block_sparse_attn_decode")
    _check(lib.bskv_block_sparse_attn_decode(_ptr(q), _ptr(k), _ptr(v), _dt(k), _strides3(k), k.shape[2], int(bool(ring)),
                                             _ptr(idx), _ptr(cnt), _ptr(seq_len), B, Hq, Hkv, d, 64, U, scale, _ptr(out),
                                             _ptr(ws), ws.numel() * ws.element_size(), sh), "block_sparse_attn_decode")
    return out


def block_sparse_attn_prefill(q, k, v, idx, cnt, q_start: int, scale: float | None = None, out=None, stream=None):
    """Causal block-sparse attention for a prefill chunk -> bf16 [B, Hq, Tq, d]."""
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    U = idx.shape[-1]
    if k.stride() != v.stride() or not q.is_contiguous():
        raise ValueError("q contiguous; k, v with identical strides")
    scale = (1.0 / math.sqrt(d)) if scale is None else scale
    out = out if out is not None else torch.empty_like(q)
    sh = _stream(stream, q.device)
    _whole_blocks(k, "block_sparse_attn_prefill")
    _check(lib.bskv_block_sparse_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _dt(q), _strides3(k), k.shape[2], _ptr(idx),
                                              _ptr(cnt),
                                              q_start, Tq, B, Hq, Hkv, d, 64, U, scale, _ptr(out), sh),
           "block_sparse_attn_prefill")
    return out


def host_device_pointer(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor."""
    dev = _p()
    _check(lib.bskv_host_device_pointer(_p(t.data_ptr()), ctypes.byref(dev)), "host_device_pointer")
    return dev.value


def prefetch_selected_blocks(src_k, src_v, idx, cnt, ring_k, ring_v, n_workgroups: int | None = None, stream=None,
                             src_k_dev: int | None = None, src_v_dev: int | None = None):
    """ring[b, g, u] = src[b, g, block idx[b,g,u]] for u < cnt (K and V).

    src_k/src_v: device tensors, or pinned host tensors (their device address
    is looked up unless passed in src_k_dev/src_v_dev).
    """
    B, H, U = idx.shape
    d = src_k.shape[-1]
    if src_k.stride() != src_v.stride() or not ring_k.is_contiguous() or not ring_v.is_contiguous():
        raise ValueError("src_k/src_v: identical strides; rings contiguous")
    if src_k.is_cuda:
        pk, pv = src_k.data_ptr(), src_v.data_ptr()
    else:
        if not (src_k.is_pinned() and src_v.is_pinned()):
            raise ValueError("host sources must be pinned")
        pk = src_k_dev if src_k_dev is not None else host_device_pointer(src_k)
        pv = src_v_dev if src_v_dev is not None else host_device_pointer(src_v)
    nwg = n_workgroups if n_workgroups is not None else max(1, min(B * H * U, 512))
    sh = _stream(stream, ring_k.device)
    _check(lib.bskv_prefetch_selected_blocks(pk, pv, _dt(ring_k), _strides3(src_k), src_k.shape[2], _ptr(idx), _ptr(cnt),
                                             _ptr(ring_k), _ptr(ring_v), B, H, d, 64, U, nwg, sh),
           "prefetch_selected_blocks")
    return ring_k, ring_v


def qkvf_proj_decode(x, w_t, n_q_heads: int, n_kv_heads: int, k_cache, v_cache, seq_len, q_out=None, f_out=None,
                     stream=None):
    """Widened projection of one token per sequence (w_t [N, hidden], one row
    per output column): returns (q bf16 [B, Hq, d], f fp32 [B, Hkv, d]); the
    token's K/V go into the caches at position seq_len - 1."""
    B, hidden = x.shape
    d = k_cache.shape[-1]
    if x.dtype != torch.bfloat16 or w_t.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16:
        raise TypeError("bf16 only")
    if k_cache.stride() != v_cache.stride() or not x.is_contiguous() or not w_t.is_contiguous():
        raise ValueError("x, w_t contiguous; k/v caches with identical strides")
    q_out = q_out if q_out is not None else torch.empty(B, n_q_heads, d, dtype=torch.bfloat16, device=x.device)
    f_out = f_out if f_out is not None else torch.empty(B, n_kv_heads, d, dtype=torch.float32, device=x.device)
    sh = _stream(stream, x.device)
    _check(lib.bskv_qkvf_proj_decode(_ptr(x), _ptr(w_t), B, hidden, n_q_heads, n_kv_heads, d, _ptr(q_out),
                                     _ptr(k_cache), _ptr(v_cache), _strides3(k_cache), k_cache.shape[2], _ptr(seq_len),
                                     _ptr(f_out), sh), "qkvf_proj_decode")
    return q_out, f_out


def qkvf_proj_prefill(x, w_t, n_q_heads: int, n_kv_heads: int, k_cache, v_cache, q_start: int = 0, q_out=None,
                      f_pooled=None, stream=None):
    """Widened projection of a prefill chunk x [B, Tq, hidden] (w_t [N,
    hidden]): returns (q bf16 [B, Hq, Tq, d], f_pooled fp32 [B, Hkv,
    ceil(Tq/64), d]); K/V go into the caches at positions q_start + t."""
    B, Tq, hidden = x.shape
    d = k_cache.shape[-1]
    w = w_t
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16:
        raise TypeError("bf16 only")
    if k_cache.stride() != v_cache.stride() or not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x, w_t contiguous; k/v caches with identical strides")
    n_qb = -(-Tq // 64)
    q_out = q_out if q_out is not None else torch.empty(B, n_q_heads, Tq, d, dtype=torch.bfloat16, device=x.device)
    f_pooled = f_pooled if f_pooled is not None else torch.empty(B, n_kv_heads, n_qb, d, dtype=torch.float32,
                                                                 device=x.device)
    sh = _stream(stream, x.device)
    _check(lib.bskv_qkvf_proj_prefill(_ptr(x), _ptr(w), B, Tq, hidden, n_q_heads, n_kv_heads, d, q_start, _ptr(q_out),
                                      _ptr(k_cache), _ptr(v_cache), _strides3(k_cache), k_cache.shape[2],
                                      _ptr(f_pooled), sh), "qkvf_proj_prefill")
    return q_out, f_pooled


def forecast_block_score_topk_pooled(f_pooled, kc, topk: int, n_init: int, n_local: int, q_start: int = 0, idx=None,
                                     cnt=None, ws=None, stream=None):
    """Prefill selection from each query block's summed Forecast
    f_pooled [B, Hkv, n_qb, d] fp32: (idx [B, Hkv, n_qb, U], cnt [B, Hkv, n_qb])."""
    B, H, n_qb, d = f_pooled.shape
    U = topk + n_init + n_local
    if f_pooled.dtype != torch.float32 or not f_pooled.is_contiguous():
        raise ValueError("f_pooled must be contiguous fp32")
    idx = idx if idx is not None else torch.empty(B, H, n_qb, U, dtype=torch.int32, device=f_pooled.device)
    cnt = cnt if cnt is not None else torch.empty(B, H, n_qb, dtype=torch.int32, device=f_pooled.device)
    sh = _stream(stream, f_pooled.device)
    lay = (B, H, n_qb, kc.shape[2], d)
    nbytes = workspace_bytes("pooled", *lay)
    ws = ws if ws is not None else _workspace(f_pooled.device, nbytes, sh, "pooled", lay)
    _check(lib.bskv_forecast_block_score_topk_pooled(_ptr(f_pooled), n_qb, q_start, _ptr(kc), kc.shape[2], B, H, d, 64,
                                                     topk, n_init, n_local, _ptr(idx), _ptr(cnt), _ptr(ws),
                                                     ws.numel() * ws.element_size(), sh),
           "forecast_block_score_topk_pooled")
    return idx, cnt


class BlockCache:
    """A resident block cache of one layer: n_slots K/V block slots per
    (b, g) on the device and their slot table (least recently used)."""

    def __init__(self, B: int, n_kv_heads: int, n_slots: int, head_dim: int, dtype=torch.bfloat16, device="cuda",
                 stream=None):
        dev = torch.device(device)
        self.B, self.H, self.S, self.d = B, n_kv_heads, n_slots, head_dim
        self.k = torch.empty(B, n_kv_heads, n_slots, 64, head_dim, dtype=dtype, device=dev)
        self.v = torch.empty_like(self.k)
        self.tags = torch.empty(B, n_kv_heads, n_slots, dtype=torch.int32, device=dev)
        self.stamps = torch.empty(B, n_kv_heads, n_slots, dtype=torch.int64, device=dev)
        self.clock = torch.empty(B, n_kv_heads, dtype=torch.int64, device=dev)
        self.reset(stream)

    def reset(self, stream=None):
        sh = _stream(stream, self.k.device)
        _check(lib.bskv_block_cache_reset(_ptr(self.tags), _ptr(self.stamps), _ptr(self.clock), self.B, self.H, self.S,
                                          sh), "block_cache_reset")


def block_cache_plan(cache: "BlockCache", idx, cnt, slot=None, fill=None, n_fill=None, stream=None):
    """Look one layer's lists up in the cache: (slot, fill, n_fill) int32;
    fill[:n_fill] are the list positions of the blocks to copy."""
    B, H, U = idx.shape
    slot = slot if slot is not None else torch.empty(B, H, U, dtype=torch.int32, device=idx.device)
    fill = fill if fill is not None else torch.empty(B, H, U, dtype=torch.int32, device=idx.device)
    n_fill = n_fill if n_fill is not None else torch.empty(B, H, dtype=torch.int32, device=idx.device)
    sh = _stream(stream, idx.device)
    _check(lib.bskv_block_cache_plan(_ptr(idx), _ptr(cnt), B, H, U, _ptr(cache.tags), _ptr(cache.stamps),
                                     _ptr(cache.clock), cache.S, _ptr(slot), _ptr(fill), _ptr(n_fill), sh),
           "block_cache_plan")
    return slot, fill, n_fill


def prefetch_cache_fill(src_k, src_v, idx, slot, fill, n_fill, cache: "BlockCache", n_workgroups: int | None = None,
                        stream=None, src_k_dev: int | None = None, src_v_dev: int | None = None):
    """Copy the blocks a cache lookup found missing (block idx[u] for the
    list positions u in fill[:n_fill]) from src (device or pinned host) into
    their cache slots slot[u]."""
    B, H, U = fill.shape
    d = src_k.shape[-1]
    if src_k.stride() != src_v.stride():
        raise ValueError("src_k/src_v: identical strides")
    if src_k.is_cuda:
        pk, pv = src_k.data_ptr(), src_v.data_ptr()
    else:
        if not (src_k.is_pinned() and src_v.is_pinned()):
            raise ValueError("host sources must be pinned")
        pk = src_k_dev if src_k_dev is not None else host_device_pointer(src_k)
        pv = src_v_dev if src_v_dev is not None else host_device_pointer(src_v)
    nwg = n_workgroups if n_workgroups is not None else B * H
    sh = _stream(stream, cache.k.device)
    _check(lib.bskv_prefetch_cache_fill(pk, pv, _dt(cache.k), _strides3(src_k), src_k.shape[2], _ptr(idx), _ptr(slot),
                                        _ptr(fill), _ptr(n_fill), _ptr(cache.k), _ptr(cache.v), B, H, d, 64, U, cache.S,
                                        nwg, sh), "prefetch_cache_fill")


def block_sparse_attn_decode_cached(q, cache: "BlockCache", slot, idx, cnt, seq_len, scale: float | None = None,
                                    out=None, ws=None, stream=None):
    """Decode attention over the listed blocks read from a block cache -> fp32 [B, Hq, d]."""
    B, Hq, d = q.shape
    Hkv = cache.H
    U = idx.shape[-1]
    if q.dtype != cache.k.dtype or not q.is_contiguous():
        raise ValueError("q contiguous, of the cache's dtype")
    scale = (1.0 / math.sqrt(d)) if scale is None else scale
    out = out if out is not None else torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    sh = _stream(stream, q.device)
    lay = (B, Hq, Hkv, d, U)
    nbytes = workspace_bytes("attn", *lay)
    ws = ws if ws is not None else _workspace(q.device, nbytes, sh, "attn", lay)
    _check(lib.bskv_block_sparse_attn_decode_cached(_ptr(q), _ptr(cache.k), _ptr(cache.v), _dt(q), cache.S, _ptr(slot),
                                                    _ptr(idx), _ptr(cnt), _ptr(seq_len), B, Hq, Hkv, d, 64, U, scale,
                                                    _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), sh),
           "block_sparse_attn_decode_cached")
    return out


def block_sparse_attn_decode_cached_fill(q, cache: "BlockCache", slot, idx, cnt, seq_len, src_k, src_v, fill_idx,
                                         fill_slot, fill, n_fill, fill_cache: "BlockCache", scale: float | None = None,
                                         out=None, ws=None, n_fill_workgroups: int | None = None, stream=None,
                                         src_k_dev: int | None = None, src_v_dev: int | None = None):
    """block_sparse_attn_decode_cached of one layer, with the copy of another
    layer's missing blocks (prefetch_cache_fill's arguments: its source K/V,
    list fill_idx, plan outputs fill_slot / fill / n_fill, cache fill_cache)
    in the same launch -> fp32 [B, Hq, d]."""
    B, Hq, d = q.shape
    Hkv = cache.H
    U = idx.shape[-1]
    if q.dtype != cache.k.dtype or not q.is_contiguous():
        raise ValueError("q contiguous, of the cache's dtype")
    if fill_idx.shape[-1] != U:
        raise ValueError("fill_idx: the same list length U")
    if src_k.stride() != src_v.stride():
        raise ValueError("src_k/src_v: identical strides")
    if src_k.is_cuda:
        pk, pv = src_k.data_ptr(), src_v.data_ptr()
    else:
        if not (src_k.is_pinned() and src_v.is_pinned()):
            raise ValueError("host sources must be pinned")
        pk = src_k_dev if src_k_dev is not None else host_device_pointer(src_k)
        pv = src_v_dev if src_v_dev is not None else host_device_pointer(src_v)
    scale = (1.0 / math.sqrt(d)) if scale is None else scale
    out = out if out is not None else torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    sh = _stream(stream, q.device)
    lay = (B, Hq, Hkv, d, U)
    nbytes = workspace_bytes("attn", *lay)
    ws = ws if ws is not None else _workspace(q.device, nbytes, sh, "attn", lay)
    nwg = n_fill_workgroups if n_fill_workgroups is not None else B * Hkv
    _check(lib.bskv_block_sparse_attn_decode_cached_fill(
        _ptr(q), _ptr(cache.k), _ptr(cache.v), _dt(q), cache.S, _ptr(slot), _ptr(idx), _ptr(cnt), _ptr(seq_len), B, Hq,
        Hkv, d, 64, U, scale, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), pk, pv, _strides3(src_k),
        src_k.shape[2], _ptr(fill_idx), _ptr(fill_slot), _ptr(fill), _ptr(n_fill), _ptr(fill_cache.k),
        _ptr(fill_cache.v), fill_cache.S, nwg, sh), "block_sparse_attn_decode_cached_fill")
    return out


def decode_layer_lookahead(q, k, v, seq_len, kc, idx, cnt, scale: float | None = None, out=None, x=None, w=None,
                           kc_next=None, scores=None, scores_next=None, idx_next=None, cnt_next=None, topk: int = 0,
                           n_init: int = 1, n_local: int = 1, stages: int = 3, ws=None, stream=None):
    """One decode layer: (when `scores` is given) this layer's top-k + union
    from the candidate scores the previous layer's call wrote, into idx/cnt;
    the newest-block update of kc; this layer's attention over (idx, cnt);
    and (when x is given) the next layer's selection from the Forecast
    x @ w against kc_next: its lists into idx_next / cnt_next when those are
    given (immediate mode), else the raw scores of its candidates into
    scores_next (deferred mode; allocated when not given).
    stages: bit mask of the two launches (3 = both, in order).
    Returns (out, scores_next) (scores_next None without a lookahead or in
    immediate mode)."""
    B, Hq, d = q.shape
    Hkv, nb_cap = kc.shape[1], kc.shape[2]
    U = idx.shape[-1]
    if U != topk + n_init + n_local:
        raise ValueError("idx capacity must equal topk + n_init + n_local")
    sel = x is not None
    immediate = idx_next is not None or cnt_next is not None
    if sel:
        hidden = x.shape[1]
        if immediate and (idx_next is None or cnt_next is None or scores_next is not None):
            raise ValueError("immediate mode takes idx_next and cnt_next (and no scores_next)")
        if not immediate and scores_next is None:
            scores_next = torch.empty(B, Hkv, nb_cap, dtype=torch.float32, device=q.device)
    else:
        hidden = 0
    if k.stride() != v.stride() or not q.is_contiguous():
        raise ValueError("q contiguous; k, v with identical strides")
    for t in (scores, scores_next):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.shape != (B, Hkv, nb_cap)):
            raise ValueError("scores / scores_next: contiguous fp32 [B, Hkv, kc_nb_cap]")
    scale = (1.0 / math.sqrt(d)) if scale is None else scale
    out = out if out is not None else torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    sh = _stream(stream, q.device)
    lay = (B, Hq, Hkv, d, hidden, nb_cap, U, _dt(k))
    nbytes = workspace_bytes("layer", *lay)
    ws = ws if ws is not None else _workspace(q.device, nbytes, sh, "layer", lay)
    _whole_blocks(k, "decode_layer_lookahead")
    _check(lib.bskv_decode_layer_lookahead(_ptr(q), _ptr(k), _ptr(v), _dt(k), _strides3(k), k.shape[2],
                                           _ptr(seq_len), _ptr(kc), _ptr(scores), _ptr(idx), _ptr(cnt), scale,
                                           _ptr(out), _ptr(x), _ptr(w), hidden, _ptr(kc_next), _ptr(scores_next),
                                           _ptr(idx_next), _ptr(cnt_next), B, Hq, Hkv, d, 64, nb_cap, topk, n_init,
                                           n_local, stages, _ptr(ws), ws.numel() * ws.element_size(), sh),
           "decode_layer_lookahead")
    return out, (scores_next if sel else None)


def decode_layer_lookahead_noalloc(q, k, v, seq_len, kc, idx, cnt, scale: float | None = None, out=None, x=None,
                                   w=None, kc_next=None, scores=None, scores_next=None, idx_next=None, cnt_next=None,
                                   topk: int = 0, n_init: int = 1, n_local: int = 1, stages: int = 3, stream=None):
    """decode_layer_lookahead with its workspace in the library's static
    device array (no workspace argument, nothing allocated by the library;
    `out` / `scores_next` are allocated here when not given).  Raises
    BskvError (BSKV_ENOSPC) when the layer's workspace exceeds the array."""
    B, Hq, d = q.shape
    Hkv, nb_cap = kc.shape[1], kc.shape[2]
    U = idx.shape[-1]
    if U != topk + n_init + n_local:
        raise ValueError("idx capacity must equal topk + n_init + n_local")
    sel = x is not None
    immediate = idx_next is not None or cnt_next is not None
    if sel:
        hidden = x.shape[1]
        if immediate and (idx_next is None or cnt_next is None or scores_next is not None):
            raise ValueError("immediate mode takes idx_next and cnt_next (and no scores_next)")
        if not immediate and scores_next is None:
            scores_next = torch.empty(B, Hkv, nb_cap, dtype=torch.float32, device=q.device)
    else:
        hidden = 0
    if k.stride() != v.stride() or not q.is_contiguous():
        raise ValueError("q contiguous; k, v with identical strides")
    for t in (scores, scores_next):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.shape != (B, Hkv, nb_cap)):
            raise ValueError("scores / scores_next: contiguous fp32 [B, Hkv, kc_nb_cap]")
    scale = (1.0 / math.sqrt(d)) if scale is None else scale
    out = out if out is not None else torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    sh = _stream(stream, q.device)
    _whole_blocks(k, "decode_layer_lookahead_noalloc")
    _check(lib.bskv_decode_layer_lookahead_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _dt(k), _strides3(k), k.shape[2], _ptr(seq_len), _ptr(kc), _ptr(scores), _ptr(idx),
        _ptr(cnt), scale, _ptr(out), _ptr(x), _ptr(w), hidden, _ptr(kc_next), _ptr(scores_next), _ptr(idx_next),
        _ptr(cnt_next), B, Hq, Hkv, d, 64, nb_cap, topk, n_init, n_local, stages, sh),
        "decode_layer_lookahead_noalloc")
    return out, (scores_next if sel else None)
