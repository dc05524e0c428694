"""Comparison helpers for the GPU parity tests (not a test module)."""
import numpy as np
import torch

import oracle as orc


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def check_selection(gpu_idx, gpu_cnt, sel, topk, rel=1e-3):
    """Selected ids must equal the oracle's wherever the k-th / (k+1)-th fp64
    score gap exceeds `rel` (relative); inside that band the GPU's set may swap
    only blocks whose fp64 scores lie within the band around the k-th score.
    Returns the number of problems that differed inside a near-tie band."""
    U = sel.idx.shape[-1]
    gi = gpu_idx.detach().cpu().numpy().reshape(-1, U)
    gc = gpu_cnt.detach().cpu().numpy().reshape(-1)
    oi = sel.idx.reshape(-1, U)
    oc = sel.cnt.reshape(-1)
    assert gi.shape == oi.shape
    tie_swaps = 0
    for p in range(gi.shape[0]):
        c = int(oc[p])
        assert int(gc[p]) == c, f"problem {p}: count {gc[p]} != {c}"
        assert (gi[p, c:] == -1).all(), f"problem {p}: padding"
        if (gi[p, :c] == oi[p, :c]).all():
            continue
        scores = sel.scores[p]
        gap = orc.kth_gap(scores, topk)
        assert gap <= rel, f"problem {p}: selection differs although the k-th gap is {gap:.3g}"
        vals = sorted(scores.values(), reverse=True)
        s_k = vals[topk - 1]
        band = rel * max(abs(s_k), 1e-30)
        g_set, o_set = set(gi[p, :c].tolist()), set(oi[p, :c].tolist())
        assert list(gi[p, :c]) == sorted(g_set)
        for j in g_set ^ o_set:
            assert j in scores and abs(scores[j] - s_k) <= band, f"problem {p}: block {j} outside the tie band"
        tie_swaps += 1
    return tie_swaps


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def fp32_sum_tol(abs_terms_sum, n_terms):
    """Error bound of an fp32 sum of n products (inputs rounded to bf16 or
    fp32 once, products formed and added in fp32), against the exact sum:
    each product within 2^-24 relative, the sum's rounding errors a random
    walk of n steps bounded at 4 standard deviations, all scaled by the sum
    of the products' magnitudes: (4 sqrt(n) + 1) 2^-24 sum |x_i w_i|, plus
    the smallest normal so an all-zero sum still compares.  abs_terms_sum is
    sum |x_i w_i| per output (e.g. |x| @ |w|)."""
    u = 2.0 ** -24
    return (4.0 * np.sqrt(n_terms) + 1.0) * u * np.asarray(abs_terms_sum, dtype=np.float64) + 1.2e-38


def fp32_sum_close(got, want, abs_terms_sum, n_terms):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return bool(np.all(np.abs(got - want) <= fp32_sum_tol(abs_terms_sum, n_terms)))
