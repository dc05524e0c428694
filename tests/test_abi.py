"""The C ABI loads, exports every symbol declared in include/bskv.h, and
rejects bad arguments on the host before launching anything.  CPU only: every
call here fails validation, so no kernel is launched and no GPU is needed."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bskv.h")

# a missing build is a failure, not a skip: these checks are the boundary's contract
import block_sparse_long_kv_amd as bskv  # noqa: E402
lib = bskv.lib

OK, EINVAL, EDTYPE, EUNSUP, ENOSPC, EHIP = 0, -1, -2, -3, -4, -5
P = 0x10000          # a 16-byte aligned fake address: never dereferenced (validation fails first)
MIS = 0x10008        # misaligned fake address
S3 = (ctypes.c_int64 * 3)(8 * 131072 * 128, 131072 * 128, 128)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bskv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_six_hot_path_calls():
    names = declared_functions()
    for n in ("bskv_forecast_proj", "bskv_kv_block_meanpool", "bskv_forecast_block_score_topk",
              "bskv_block_sparse_attn_decode", "bskv_block_sparse_attn_prefill", "bskv_prefetch_selected_blocks",
              "bskv_decode_layer_lookahead"):
        assert n in names


def test_library_exports_every_declared_symbol():
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_strerror_and_version():
    assert lib.bskv_version() >= 1
    for code in (OK, EINVAL, EDTYPE, EUNSUP, ENOSPC, EHIP):
        assert lib.bskv_strerror(code)
    assert lib.bskv_strerror(-99) == b"unknown status"


def test_workspace_queries_are_pure_host_arithmetic():
    assert lib.bskv_forecast_proj_workspace(8, 4096, 8, 128, 1) >= 16 * 8 * 1024 * 4
    assert lib.bskv_score_topk_workspace(8, 8, 0, 2048, 128) >= 64 * 2048 * 4
    assert lib.bskv_score_topk_workspace(4, 8, 2048, 2048, 128) >= 32 * 32 * 2048 * 4     # prefill score rows
    assert lib.bskv_attn_decode_workspace(8, 32, 8, 128, 69) > 0
    assert lib.bskv_attn_decode_workspace(8, 24, 8, 128, 69) == 0     # group size 3 unsupported
    assert lib.bskv_forecast_proj_workspace(0, 4096, 8, 128, 1) == 0


def test_forecast_proj_validation():
    f = lib.bskv_forecast_proj
    ws = lib.bskv_forecast_proj_workspace(4, 4096, 8, 128, 1)
    assert f(P, P, 7, 4, 4096, 8, 128, P, P, ws, None) == EDTYPE
    assert f(P, P, 1, 0, 4096, 8, 128, P, P, ws, None) == EINVAL
    assert f(None, P, 1, 4, 4096, 8, 128, P, P, ws, None) == EINVAL
    assert f(MIS, P, 1, 4, 4096, 8, 128, P, P, ws, None) == EINVAL
    assert f(P, P, 1, 4, 4000, 8, 128, P, P, ws, None) == EUNSUP
    assert f(P, P, 1, 4, 4096, 8, 128, P, P, ws - 1, None) == ENOSPC


def test_meanpool_validation():
    f = lib.bskv_kv_block_meanpool
    T = 131072
    assert f(P, 3, S3, T, 8, 8, 128, 64, P, 0, 10, 0, P, 2048, None) == EDTYPE
    assert f(P, 1, S3, T, 8, 8, 96, 64, P, 0, 10, 0, P, 2048, None) == EUNSUP
    assert f(P, 1, S3, T, 8, 8, 128, 32, P, 0, 10, 0, P, 2048, None) == EUNSUP
    assert f(P, 1, S3, T, 8, 8, 128, 64, None, 0, 10, 0, P, 2048, None) == EINVAL
    assert f(P, 1, S3, T, 8, 8, 128, 64, P, 5, 2049, 0, P, 2048, None) == EINVAL
    assert f(P, 1, S3, -1, 8, 8, 128, 64, P, 0, 10, 0, P, 2048, None) == EINVAL
    bad = (ctypes.c_int64 * 3)(8 * 131072 * 128, 131072 * 128, 100)   # token stride not 16-byte aligned
    assert f(P, 1, bad, T, 8, 8, 128, 64, P, 0, 10, 0, P, 2048, None) == EINVAL


def test_score_topk_validation():
    f = lib.bskv_forecast_block_score_topk
    ws = lib.bskv_score_topk_workspace(8, 8, 0, 2048, 128)
    args = dict(f=P, dt=0, nq=0, q0=0, kc=P, cap=2048, sl=P, B=8, H=8, d=128, blk=64, k=64, ni=1, nl=4,
                idx=P, cnt=P, sc=None, ws=P, wsb=ws)

    def call(**kw):
        a = {**args, **kw}
        return f(a["f"], a["dt"], a["nq"], a["q0"], a["kc"], a["cap"], a["sl"], a["B"], a["H"], a["d"], a["blk"],
                 a["k"], a["ni"], a["nl"], a["idx"], a["cnt"], a["sc"], a["ws"], a["wsb"], None)
    assert call(nl=0) == EINVAL                 # the current block must stay reachable
    assert call(ni=0) == EINVAL
    assert call(k=-1) == EINVAL
    assert call(dt=1) == EDTYPE                 # decode Forecast must be fp32
    assert call(cap=20000) == EUNSUP
    assert call(d=96) == EUNSUP
    assert call(wsb=ws - 4) == ENOSPC
    assert call(sl=None) == EINVAL
    assert call(nq=2048, q0=100) == EINVAL      # prefill chunk must start on a block boundary
    assert call(nq=2048, sc=P) == EINVAL        # no debug scores in prefill


def test_multihead_select_validation():
    f = lib.bskv_multihead_block_score_topk
    ws = lib.bskv_multihead_score_topk_workspace(8, 8, 2048)
    assert ws >= 64 * 2048 * 4
    assert lib.bskv_multihead_score_topk_workspace(0, 8, 2048) == 0
    args = dict(q=P, dt=1, kc=P, cap=2048, sl=P, B=8, Hq=32, H=8, d=128, blk=64, k=64, ni=1, nl=4, sc=0.088,
                idx=P, cnt=P, w=None, ws=P, wsb=ws)

    def call(**kw):
        a = {**args, **kw}
        return f(a["q"], a["dt"], a["kc"], a["cap"], a["sl"], a["B"], a["Hq"], a["H"], a["d"], a["blk"], a["k"],
                 a["ni"], a["nl"], a["sc"], a["idx"], a["cnt"], a["w"], a["ws"], a["wsb"], None)
    assert call(dt=5) == EDTYPE
    assert call(q=None) == EINVAL
    assert call(sl=None) == EINVAL
    assert call(kc=MIS) == EINVAL
    assert call(nl=0) == EINVAL
    assert call(ni=0) == EINVAL
    assert call(k=-1) == EINVAL
    assert call(sc=0.0) == EINVAL
    assert call(sc=float("nan")) == EINVAL
    assert call(Hq=24) == EUNSUP                # group size 3
    assert call(d=96) == EUNSUP
    assert call(blk=32) == EUNSUP
    assert call(cap=20000) == EUNSUP
    assert call(wsb=ws - 4) == ENOSPC


def test_window_select_validation():
    mp = lib.bskv_kv_window_meanpool
    assert mp(P, 5, S3, 131072, 8, 8, 128, 32, 16, P, 0, 10, 0, P, 8191, None) == EDTYPE
    assert mp(None, 1, S3, 131072, 8, 8, 128, 32, 16, P, 0, 10, 0, P, 8191, None) == EINVAL
    assert mp(P, 1, S3, 131072, 8, 8, 128, 48, 16, P, 0, 10, 0, P, 8191, None) == EUNSUP   # window 48
    assert mp(P, 1, S3, 131072, 8, 8, 128, 32, 64, P, 0, 10, 0, P, 8191, None) == EUNSUP   # stride > window
    assert mp(P, 1, S3, 131072, 8, 8, 128, 64, 24, P, 0, 10, 0, P, 8191, None) == EUNSUP   # stride 24
    assert mp(P, 1, S3, 131072, 8, 8, 96, 32, 16, P, 0, 10, 0, P, 8191, None) == EUNSUP
    assert mp(P, 1, S3, 131072, 8, 8, 128, 32, 16, P, 5, 4, 0, P, 8191, None) == EINVAL    # w_end < w_begin
    assert mp(P, 1, S3, 131072, 8, 8, 128, 32, 16, P, 0, 8192, 0, P, 8191, None) == EINVAL  # past the cap
    f = lib.bskv_forecast_window_score_topk
    ws = lib.bskv_window_score_topk_workspace(8, 8, 0, 8191)
    assert ws >= 64 * 8191 * 4
    assert lib.bskv_window_score_topk_workspace(8, 0, 0, 8191) == 0
    assert lib.bskv_window_score_topk_workspace(8, 8, 2048, 8191) == 0      # prefill needs none
    args = dict(f=P, fdt=0, nq=0, q0=0, kcw=P, cap=8191, sl=P, B=8, H=8, d=128, blk=64, win=32, st=16, k=64, ni=1,
                nl=4, idx=P, cnt=P, sc=None, ws=P, wsb=ws)

    def call(**kw):
        a = {**args, **kw}
        return f(a["f"], a["fdt"], a["nq"], a["q0"], a["kcw"], a["cap"], a["sl"], a["B"], a["H"], a["d"], a["blk"],
                 a["win"], a["st"], a["k"], a["ni"], a["nl"], a["idx"], a["cnt"], a["sc"], a["ws"], a["wsb"], None)
    assert call(fdt=5) == EDTYPE
    assert call(fdt=1) == EDTYPE                      # decode Forecast must be fp32
    assert call(f=None) == EINVAL
    assert call(kcw=MIS) == EINVAL
    assert call(sl=None) == EINVAL
    assert call(ni=0) == EINVAL
    assert call(nl=0) == EINVAL
    assert call(k=-1) == EINVAL
    assert call(cap=0) == EINVAL
    assert call(nq=-1) == EINVAL
    assert call(d=96) == EUNSUP
    assert call(blk=32) == EUNSUP
    assert call(win=16, st=16) == EUNSUP
    assert call(win=32, st=64) == EUNSUP
    assert call(cap=8 * 12288) == EUNSUP             # more than 12288 blocks
    assert call(wsb=ws - 4) == ENOSPC
    assert call(nq=2048, q0=100, fdt=1) == EINVAL    # prefill chunk start not a multiple of the block
    assert call(nq=2048, sc=P, fdt=1) == EINVAL      # no scores in prefill


def test_block_cache_validation():
    assert lib.bskv_block_cache_reset(None, P, P, 2, 8, 128, None) == EINVAL
    assert lib.bskv_block_cache_reset(P, P, P, 2, 8, 0, None) == EINVAL
    assert lib.bskv_block_cache_reset(P, P, P, 2, 8, 2048, None) == EUNSUP
    plan = lib.bskv_block_cache_plan
    assert plan(P, P, 2, 8, 69, P, P, P, 128, None, P, P, None) == EINVAL      # no slot output
    assert plan(P, P, 2, 8, 69, P, P, P, 128, P, P, None, None) == EINVAL      # no copy count
    assert plan(P, P, 2, 8, 129, P, P, P, 128, P, P, P, None) == EINVAL       # more list entries than slots
    assert plan(P, P, 0, 8, 69, P, P, P, 128, P, P, P, None) == EINVAL
    assert plan(P, P, 2, 8, 69, P, P, P, 4096, P, P, P, None) == EUNSUP
    fillf = lib.bskv_prefetch_cache_fill

    def fcall(src=P, dt=1, fill=P, nf=P, d=128, S=128, nwg=64):
        return fillf(src, P, dt, S3, 131072, P, P, fill, nf, P, P, 2, 8, d, 64, 69, S, nwg, None)
    assert fcall(dt=5) == EDTYPE
    assert fcall(fill=None) == EINVAL
    assert fcall(nf=None) == EINVAL
    assert fcall(src=MIS) == EINVAL
    assert fcall(nwg=0) == EINVAL
    assert fcall(d=96) == EUNSUP
    assert fcall(S=2048) == EUNSUP
    att = lib.bskv_block_sparse_attn_decode_cached
    ws = lib.bskv_attn_decode_workspace(2, 32, 8, 128, 69)

    def call(dt=1, hq=32, d=128, S=128, slot=P, sc=0.088, wsb=ws):
        return att(P, P, P, dt, S, slot, P, P, P, 2, hq, 8, d, 64, 69, sc, P, P, wsb, None)
    assert call(dt=5) == EDTYPE
    assert call(slot=None) == EINVAL
    assert call(hq=24) == EUNSUP
    assert call(d=96) == EUNSUP
    assert call(S=2048) == EUNSUP
    assert call(sc=0.0) == EINVAL
    assert call(wsb=ws - 4) == ENOSPC
    # attention of one layer with another layer's cache fill in the same launch
    af = lib.bskv_block_sparse_attn_decode_cached_fill
    P2 = 0x20000

    def fcall2(dt=1, d=128, S=128, fS=128, slot=P, fill=P, fck=P2, fcv=P2 + 0x100, src=P, nwg=64, sc=0.088, wsb=ws):
        return af(P, P, P + 0x100, dt, S, slot, P, P, P, 2, 32, 8, d, 64, 69, sc, P, P, wsb, src, P, S3, 131072, P, P,
                  fill, P, fck, fcv, fS, nwg, None)
    assert fcall2(dt=5) == EDTYPE
    assert fcall2(slot=None) == EINVAL
    assert fcall2(fill=None) == EINVAL
    assert fcall2(src=MIS) == EINVAL
    assert fcall2(fck=P) == EINVAL            # fills the cache this call reads
    assert fcall2(fcv=P + 0x100) == EINVAL
    assert fcall2(nwg=0) == EINVAL
    assert fcall2(fS=0) == EINVAL
    assert fcall2(d=96) == EUNSUP
    assert fcall2(fS=2048) == EUNSUP
    assert fcall2(sc=0.0) == EINVAL
    assert fcall2(wsb=ws - 4) == ENOSPC


def test_qkvf_proj_validation():
    dec = lib.bskv_qkvf_proj_decode

    def dcall(x=P, B=8, hidden=4096, hq=32, hkv=8, d=128, sl=P):
        return dec(x, P, B, hidden, hq, hkv, d, P, P, P, S3, 131072, sl, P, None)
    assert dcall(x=None) == EINVAL
    assert dcall(x=MIS) == EINVAL
    assert dcall(sl=None) == EINVAL
    assert dcall(B=0) == EINVAL
    assert dcall(d=96) == EUNSUP
    assert dcall(hidden=3584) == EUNSUP               # not a multiple of 1024
    assert dcall(B=65) == EUNSUP
    pre = lib.bskv_qkvf_proj_prefill

    def pcall(B=4, tq=2048, hidden=4096, hq=32, hkv=8, d=128, q0=0, kv_len=131072, fp=P):
        return pre(P, P, B, tq, hidden, hq, hkv, d, q0, P, P, P, S3, kv_len, fp, None)
    assert pcall(fp=None) == EINVAL
    assert pcall(fp=MIS) == EINVAL
    assert pcall(q0=32) == EINVAL                     # chunk start off the block grid
    assert pcall(q0=131072 - 1024) == EINVAL          # chunk past the cache
    assert pcall(tq=0) == EINVAL
    assert pcall(d=96) == EUNSUP
    assert pcall(hidden=4000) == EUNSUP
    assert pcall(hkv=1, d=64) == EUNSUP               # a 64-column head group would straddle a tile
    pooled = lib.bskv_forecast_block_score_topk_pooled
    pws = lib.bskv_score_topk_pooled_workspace(4, 8, 32, 2048, 128)
    assert pws >= 32 * 32 * 2048 * 4

    def scall(fp=P, nqb=32, q0=0, d=128, blk=64, ni=1, nl=4, cap=2048, ws=P, wsb=pws):
        return pooled(fp, nqb, q0, P, cap, 4, 8, d, blk, 64, ni, nl, P, P, ws, wsb, None)
    assert scall(ws=None) == EINVAL
    assert scall(wsb=pws - 4) == ENOSPC
    assert scall(fp=None) == EINVAL
    assert scall(nqb=0) == EINVAL
    assert scall(q0=32) == EINVAL
    assert scall(ni=0) == EINVAL
    assert scall(d=96) == EUNSUP
    assert scall(blk=128) == EUNSUP
    assert scall(cap=20000) == EUNSUP


def test_attn_decode_validation():
    f = lib.bskv_block_sparse_attn_decode
    ws = lib.bskv_attn_decode_workspace(8, 32, 8, 128, 69)

    def call(q=P, dt=1, hq=32, hkv=8, d=128, blk=64, U=69, scale=0.088, wsb=ws, strides=S3, kv_len=131072):
        return f(q, P, P, dt, strides, kv_len, 0, P, P, P, 8, hq, hkv, d, blk, U, scale, P, P, wsb, None)
    assert call(dt=5) == EDTYPE
    assert call(hq=30) == EUNSUP
    assert call(hq=24) == EUNSUP
    assert call(d=256) == EUNSUP
    assert call(blk=128) == EUNSUP
    assert call(q=MIS) == EINVAL
    assert call(q=None) == EINVAL
    assert call(scale=0.0) == EINVAL
    assert call(scale=float("nan")) == EINVAL
    assert call(wsb=ws - 1) == ENOSPC
    assert call(kv_len=-64) == EINVAL
    assert call(kv_len=131072 - 5) == EINVAL     # K/V buffers hold whole blocks
    assert call(kv_len=300) == EINVAL
    # one (b, g)'s K/V must span less than 2 GiB (32-bit load offsets) ...
    big = (ctypes.c_int64 * 3)(1 << 40, 1 << 30, 1 << 14)
    assert call(strides=big, kv_len=1 << 16) == EUNSUP
    # ... and 64 token strides of any call less than 2 GiB
    huge = (ctypes.c_int64 * 3)(1 << 40, 1 << 30, 1 << 24)
    assert call(strides=huge, kv_len=64) == EINVAL


def test_attn_prefill_validation():
    f = lib.bskv_block_sparse_attn_prefill

    def call(dt=1, q0=0, tq=2048, hq=32, hkv=8, d=128, kv_len=131072):
        return f(P, P, P, dt, S3, kv_len, P, P, q0, tq, 4, hq, hkv, d, 64, 97, 0.088, P, None)
    assert call(dt=0) == EDTYPE
    assert call(kv_len=300, tq=300) == EINVAL    # K/V buffers hold whole blocks
    assert call(q0=32) == EINVAL
    assert call(tq=0) == EINVAL
    assert call(hq=12) == EUNSUP
    assert call(d=80) == EUNSUP


def test_prefetch_validation():
    f = lib.bskv_prefetch_selected_blocks
    T = 131072
    assert f(P, P, 1, S3, T, P, P, P, P, 16, 8, 128, 64, 69, 0, None) == EINVAL
    assert f(P, P, 4, S3, T, P, P, P, P, 16, 8, 128, 64, 69, 64, None) == EDTYPE
    assert f(P, None, 1, S3, T, P, P, P, P, 16, 8, 128, 64, 69, 64, None) == EINVAL
    assert f(P, P, 1, S3, T, P, P, P, P, 16, 8, 128, 32, 69, 64, None) == EUNSUP
    assert f(P, P, 1, S3, -1, P, P, P, P, 16, 8, 128, 64, 69, 64, None) == EINVAL


def test_host_device_pointer_rejects_null():
    out = ctypes.c_void_p()
    assert lib.bskv_host_device_pointer(None, ctypes.byref(out)) == EINVAL


def test_decode_layer_validation():
    f = lib.bskv_decode_layer_lookahead
    ws = lib.bskv_decode_layer_lookahead_workspace(8, 32, 8, 128, 4096, 2048, 69, 1)
    assert ws > lib.bskv_decode_layer_lookahead_workspace(8, 32, 8, 128, 0, 2048, 69, 1)

    def call(x=P, w=P, kcn=P, scn=P, sc=P, hidden=4096, stages=3, dt=1, hq=32, nl=4, wsb=ws, kv_len=131072,
             idx=P, idn=None, cnn=None):
        return f(P, P, P, dt, S3, kv_len, P, P, sc, idx, P, 0.088, P, x, w, hidden, kcn, scn, idn, cnn, 8, hq, 8, 128,
                 64, 2048, 64, 1, nl, stages, P, wsb, None)
    assert call(kv_len=131072 - 1) == EINVAL     # K/V buffers hold whole blocks
    assert call(x=None) == EINVAL            # lookahead arguments: all or none
    assert call(scn=None) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(idn=P, cnn=P) == EINVAL           # both forms of the next selection
    assert call(scn=None, idn=P) == EINVAL        # immediate mode needs both lists
    assert call(stages=0) == EINVAL
    assert call(stages=4) == EINVAL
    assert call(dt=3) == EDTYPE
    assert call(hq=24) == EUNSUP
    assert call(hidden=1000) == EUNSUP
    assert call(nl=0) == EINVAL
    assert call(wsb=ws - 16) == ENOSPC


def test_noalloc_layer_rejects_oversized_workspace_on_the_host():
    """The allocation-free layer refuses, before touching any device, a
    layer whose workspace exceeds its static array (and bad sizes)."""
    cap = lib.bskv_decode_layer_lookahead_noalloc_capacity()
    assert cap == 16 << 20
    f = lib.bskv_decode_layer_lookahead_noalloc

    def call(B=8, hq=32, hkv=8, nb=2048):
        return f(P, P, P, 1, S3, 131072, P, P, None, P, P, 0.088, P, P, P, 4096, P, P, None, None, B, hq, hkv, 128, 64,
                 nb, 64, 1, 4, 3, None)
    assert lib.bskv_decode_layer_lookahead_workspace(512, 32, 8, 128, 4096, 2048, 69, 1) > cap
    assert call(B=512) == ENOSPC
    assert b"16 MiB" in lib.bskv_last_error()
    assert call(hq=24) == EINVAL


def test_largest_unit_counts_are_rejected_on_the_host():
    """B * n_kv_heads above 65535 (the decode calls' per-(b, g) grid and the
    fused layer's counter region) is BSKV_EUNSUPPORTED, found before any
    workspace check or launch; 65535 itself passes that check (and then
    fails only on the deliberately small workspace)."""
    att = lib.bskv_block_sparse_attn_decode
    lay = lib.bskv_decode_layer_lookahead

    def call_att(B, hkv):
        return att(P, P, P, 1, S3, 131072, 0, P, P, P, B, 4 * hkv, hkv, 128, 64, 69, 0.088, P, P, 256, None)

    def call_lay(B, hkv):
        return lay(P, P, P, 1, S3, 131072, P, P, None, P, P, 0.088, P, None, None, 0, None, None, None, None, B,
                   4 * hkv, hkv, 128, 64, 2048, 64, 1, 4, 3, P, 256, None)
    for fn in (call_att, call_lay):
        assert fn(8192, 8) == EUNSUP          # 65536 units
        assert fn(65536, 1) == EUNSUP
        assert fn(65535, 1) == ENOSPC         # at the limit: only the workspace is short
