"""Seeded input generators.

One torch.Generator per workload, seeded with the workload's seed, on the
device the tensors are drawn on (small cases on the CPU, large ones on the
GPU).  The draw order is fixed and documented per function, so a workload is
reproduced exactly from (seed, device).  N(m, s^2) below means variance s^2.

Planted blocks make the top-k well separated: k candidate blocks per
(batch, KV head) get an offset o = |g| * F_hat added to all of their keys
before rounding, with g ~ N(0, 4 I_d) and F_hat the unit direction of the
Forecast that selects that layer.  Building F_hat needs x @ W (one float32
torch matmul); that product only shapes the input -- the oracle and the
library each compute the Forecast themselves from x and W.
"""
from __future__ import annotations

import torch

from .configs import Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, std=1.0):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * std


def _plant(k32, fdir, planted, gvec, block):
    """Add |g| * F_hat to every key of each planted block (in place, fp32)."""
    B, H, T, d = k32.shape
    kb = k32.view(B, H, T // block, block, d)
    norm = gvec.norm(dim=-1)                                   # [B, H, P]
    off = norm[..., None] * fdir[:, :, None, :]                # [B, H, P, d]
    bi = torch.arange(B, device=k32.device)[:, None, None]
    hi = torch.arange(H, device=k32.device)[None, :, None]
    kb[bi, hi, planted] += off[:, :, :, None, :]


def _unit(v):
    return v / v.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def decode_inputs(wl: Workload, device="cpu", layers: int | None = None, B: int | None = None,
                  T: int | None = None):
    """Per-layer decode inputs of a decode/offload workload.

    Draw order per layer: [F (if the Forecast is given) | W_sel, x_sel], K, V,
    q, plant choice (argsort of uniform draws over the candidates), g.
      W_sel [hidden, Hkv*d] ~ N(0, 0.02^2)  Forecast weights selecting this layer
      x_sel [B, hidden]     ~ N(0, 1)       hidden state fed to W_sel
      F     [B, Hkv, d]     ~ N(0, 1)       (fp32, when hidden is None)
      K, V  [B, Hkv, T, d]  ~ N(0, 1);  q [B, Hq, d] ~ N(0, 1)
    All rounded to the workload dtype after planting.  seq_len = T for all b.
    """
    B = B or wl.B
    T = T or wl.T
    L = layers or wl.layers
    dt = _DT[wl.dtype]
    gen = _gen(wl.seed, device)
    cur = (T - 1) // wl.block
    n_cand = cur - wl.n_local - wl.n_init + 1
    n_plant = min(wl.topk if wl.plant is None else wl.plant, max(n_cand, 0))
    out = []
    for _ in range(L):
        lay = {}
        if wl.hidden is None:
            f = _randn((B, wl.Hkv, wl.d), gen, device)
            lay["f"] = f
            fdir = _unit(f)
        else:
            w = _randn((wl.hidden, wl.Hkv * wl.d), gen, device, 0.02).to(dt)
            x = _randn((B, wl.hidden), gen, device).to(dt)
            lay["w_sel"], lay["x_sel"] = w, x
            fdir = _unit((x.float() @ w.float()).view(B, wl.Hkv, wl.d))
        k = _randn((B, wl.Hkv, T, wl.d), gen, device)
        v = _randn((B, wl.Hkv, T, wl.d), gen, device).to(dt)
        q = _randn((B, wl.Hq, wl.d), gen, device).to(dt)
        if n_plant > 0:
            u = torch.rand(B, wl.Hkv, n_cand, generator=gen, device=device)
            planted = torch.argsort(u, dim=-1)[..., :n_plant] + wl.n_init
            gvec = _randn((B, wl.Hkv, n_plant, wl.d), gen, device, 2.0)
            _plant(k, fdir, planted, gvec, wl.block)
        else:
            planted = torch.zeros(B, wl.Hkv, 0, dtype=torch.int64, device=device)
        lay["k"] = k.to(dt)
        del k
        lay["v"], lay["q"] = v, q
        lay["planted"] = planted
        lay["seq_len"] = torch.full((B,), T, dtype=torch.int64, device=device)
        out.append(lay)
    return out


def drift_walk(x0, n_steps: int, step: float, seed: int):
    """Forecast inputs of successive decode steps: a random walk from x0,
    x_t = (x_{t-1} + step * e_t) / sqrt(1 + step^2) with e_t ~ N(0, I), which
    keeps the entries' variance.  x0: [..., hidden]; returns
    [n_steps, ..., hidden] of x0's dtype (x_0 itself excluded)."""
    gen = _gen(seed, x0.device)
    x = x0.float()
    out = torch.empty((n_steps,) + tuple(x0.shape), dtype=x0.dtype, device=x0.device)
    norm = (1.0 + step * step) ** 0.5
    for t in range(n_steps):
        x = (x + step * torch.randn(x.shape, generator=gen, device=x.device)) / norm
        out[t] = x.to(x0.dtype)
    return out


def prefill_inputs(wl: Workload, device="cpu", B: int | None = None, T: int | None = None):
    """Inputs of the chunked-prefill workload.

    Draw order: Q [B, Hq, T, d], K, V [B, Hkv, T, d], F [B, Hkv, T, d] (one
    Forecast vector per token and KV head), all N(0, 1); then the planted
    blocks (round(plant_frac * NB) per (b, g), drawn without replacement from
    [1, NB)) and their offsets g ~ N(0, 4 I_d) (a random direction each),
    added to the keys before rounding to bf16.
    """
    B = B or wl.B
    T = T or wl.T
    dt = _DT[wl.dtype]
    gen = _gen(wl.seed, device)
    NB = T // wl.block
    q = _randn((B, wl.Hq, T, wl.d), gen, device).to(dt)
    k = _randn((B, wl.Hkv, T, wl.d), gen, device)
    v = _randn((B, wl.Hkv, T, wl.d), gen, device).to(dt)
    f = _randn((B, wl.Hkv, T, wl.d), gen, device).to(dt)
    n_plant = int(round((wl.plant_frac or 0.0) * NB))
    if n_plant > 0 and NB > 1:
        n_plant = min(n_plant, NB - 1)
        u = torch.rand(B, wl.Hkv, NB - 1, generator=gen, device=device)
        planted = torch.argsort(u, dim=-1)[..., :n_plant] + 1
        gvec = _randn((B, wl.Hkv, n_plant, wl.d), gen, device, 2.0)
        kb = k.view(B, wl.Hkv, NB, wl.block, wl.d)
        bi = torch.arange(B, device=device)[:, None, None]
        hi = torch.arange(wl.Hkv, device=device)[None, :, None]
        kb[bi, hi, planted] += gvec[:, :, :, None, :]
    else:
        planted = torch.zeros(B, wl.Hkv, 0, dtype=torch.int64, device=device)
    return {"q": q, "k": k.to(dt), "v": v, "f": f, "planted": planted}


def random_decode_case(seed: int, B: int, Hq: int, Hkv: int, d: int, T: int, block: int = 64,
                       dtype: str = "f32", hidden: int | None = None, seq_len=None,
                       plant: int = 0, topk: int = 0, n_init: int = 1, n_local: int = 1,
                       device="cpu"):
    """A small decode case for parity tests (ragged lengths allowed).

    Draw order: [F | W_sel, x_sel], K, V, q, then (plant > 0) plant choice and
    g as in decode_inputs, for the batch's shortest length.  seq_len: list of
    per-batch lengths (default T for all), each in [1, T].
    """
    dt = _DT[dtype]
    gen = _gen(seed, device)
    case = {}
    if hidden is None:
        f = _randn((B, Hkv, d), gen, device)
        case["f"] = f
        fdir = _unit(f)
    else:
        w = _randn((hidden, Hkv * d), gen, device, 0.02).to(dt)
        x = _randn((B, hidden), gen, device).to(dt)
        case["w_sel"], case["x_sel"] = w, x
        fdir = _unit((x.float() @ w.float()).view(B, Hkv, d))
    k = _randn((B, Hkv, T, d), gen, device)
    v = _randn((B, Hkv, T, d), gen, device).to(dt)
    q = _randn((B, Hq, d), gen, device).to(dt)
    lens = [T] * B if seq_len is None else [int(s) for s in seq_len]
    if plant > 0:
        cur = (min(lens) - 1) // block
        n_cand = cur - n_local - n_init + 1
        n_plant = min(plant, n_cand)
        if n_plant > 0:
            u = torch.rand(B, Hkv, n_cand, generator=gen, device=device)
            planted = torch.argsort(u, dim=-1)[..., :n_plant] + n_init
            gvec = _randn((B, Hkv, n_plant, d), gen, device, 2.0)
            _plant(k, fdir, planted, gvec, block)
    case["k"] = k.to(dt)
    case["v"], case["q"] = v, q
    case["seq_len"] = torch.tensor(lens, dtype=torch.int64, device=device)
    return case


def random_prefill_case(seed: int, B: int, Hq: int, Hkv: int, d: int, T: int, block: int = 64,
                        n_plant: int = 0, device="cpu"):
    """A small bf16 prefill case: Q, K, V, F ~ N(0, 1), plus n_plant random
    N(0, 4 I_d) key offsets per (b, g) on blocks drawn from [1, NB)."""
    gen = _gen(seed, device)
    NB = T // block
    q = _randn((B, Hq, T, d), gen, device).to(torch.bfloat16)
    k = _randn((B, Hkv, T, d), gen, device)
    v = _randn((B, Hkv, T, d), gen, device).to(torch.bfloat16)
    f = _randn((B, Hkv, T, d), gen, device).to(torch.bfloat16)
    n_plant = min(n_plant, max(NB - 1, 0))
    if n_plant > 0:
        u = torch.rand(B, Hkv, NB - 1, generator=gen, device=device)
        planted = torch.argsort(u, dim=-1)[..., :n_plant] + 1
        gvec = _randn((B, Hkv, n_plant, d), gen, device, 2.0)
        kb = k[:, :, : NB * block].reshape(B, Hkv, NB, block, d)
        bi = torch.arange(B, device=device)[:, None, None]
        hi = torch.arange(Hkv, device=device)[None, :, None]
        kb[bi, hi, planted] += gvec[:, :, :, None, :]
        k[:, :, : NB * block] = kb.reshape(B, Hkv, NB * block, d)
    return {"q": q, "k": k.to(torch.bfloat16), "v": v, "f": f}
