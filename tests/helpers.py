"""Shared helpers for the GPU parity tests: seeded inputs (bit-identical on the
CPU and the GPU through ``synthetic``) and comparison utilities."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synthetic as syn

BF16_TOL = 2e-2   # max-abs, bf16 storage with fp32 accumulation
F32_TOL = 1e-4    # max-abs, fp32 storage


def gen(shape, seed, name, *, dtype, device, scale=1.0, kind="normal", layer=0, grid=8):
    return syn.make(shape, seed, syn.TID[name], dtype=dtype, device=device, scale=scale, kind=kind,
                    layer=layer, grid=grid)


def both(shape, seed, name, *, dtype, scale=1.0, kind="normal", layer=0, grid=8):
    """The same seeded tensor on the GPU and (as float64 numpy) on the CPU.

    Each side is generated on its own device; the CPU copy never comes from the GPU."""
    g = gen(shape, seed, name, dtype=dtype, device="cuda", scale=scale, kind=kind, layer=layer, grid=grid)
    c = gen(shape, seed, name, dtype=dtype, device="cpu", scale=scale, kind=kind, layer=layer, grid=grid)
    if dtype == torch.float8_e4m3fn:  # decoded by the oracle's own E4M3 decoder
        return g, oracle.fp8_decode(c.view(torch.uint8).numpy())
    return g, c.double().numpy()


def to_np(t):
    if t.dtype == torch.float8_e4m3fn:
        return oracle.fp8_decode(t.detach().cpu().view(torch.uint8).numpy())
    return t.detach().float().cpu().double().numpy()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def round_to(x, dtype):
    """Round a float64 numpy array to the storage dtype (RNE), back to float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(dtype).double().numpy()


def near_tie_check(gpu_row, oracle_row, oracle_scores, nvis, k, eps):
    """Compare one GPU top-k row with the oracle's row (fp64 scores).

    The GPU row must be ascending, unique and -1 padded to min(k, nvis) kept
    entries.  Entries on which the two disagree must all be near-ties: their
    oracle score within eps (scalar or per entry) plus the largest eps of the
    k-th score.  Returns the number of such disagreements (0 expected)."""
    gpu_row = np.asarray(gpu_row)
    keep = min(k, nvis)
    g = gpu_row[:keep].tolist()
    assert np.all(gpu_row[keep:] == -1), "padding is not -1"
    assert all(0 <= x < nvis for x in g), "index outside the visible range"
    assert g == sorted(g) and len(set(g)) == keep, "indices not ascending/unique"
    o = [int(x) for x in oracle_row if x >= 0]
    diff = set(g) ^ set(o)
    if not diff:
        return 0
    v = oracle_scores[:nvis]
    kth = np.sort(v)[::-1][keep - 1]
    e = np.broadcast_to(np.asarray(eps, dtype=np.float64), v.shape)
    bound = e + e.max()
    bad = [s for s in diff if abs(v[s] - kth) > bound[s]]
    assert not bad, "non-tie disagreement at %s (kth=%r)" % ([(s, v[s]) for s in bad[:5]], kth)
    return len(diff) // 2


def index_eps(q, w, k):
    """Per-query fp32 accumulation bound for the indexer score of every entry.

    q [H, dI], w [H] (or None), k [L, dI] float64.  The bound is
    2 * (dI + H) * 2^-24 * sum_h |w_h| * sum_c |q_hc k_sc| (a standard
    recursive-summation bound with margin), returned per entry."""
    H, dI = q.shape
    wa = np.ones(H) if w is None else np.abs(w)
    mag = np.abs(k) @ (np.abs(q).T * 1.0)  # [L, H]
    return 2.0 * (dI + H) * 2.0 ** -24 * (mag @ wa)


def index_eps_fp8(q, w, k):
    """Per-entry bound for FP8 (E4M3) indexer scores on the GPU.

    The products of two E4M3 values are exact in fp32, but gfx950's fp8
    MFMA (v_mfma_f32_16x16x32_fp8_fp8) does not sum them at fp32 precision:
    on 2000 random 16x128 x 128x16 products per input scale the error of one
    instruction (32 products) reached ~1150 x 2^-24 of the sum of |products|,
    and ~440 x 2^-24 for four chained ones (a 128-dim dot product).  The
    bound takes 2^-12 (4096 x 2^-24) of sum_c |q_hc k_sc| per head, weighted
    by |w_h|, plus the fp32 bound of the epilogue (ReLU, weights, head sum)."""
    H, dI = q.shape
    wa = np.ones(H) if w is None else np.abs(w)
    mag = (np.abs(k) @ np.abs(q).T) @ wa
    return 2.0 ** -12 * mag + index_eps(q, w, k)


def fp8_ulp(x):
    """Spacing of E4M3 values at |x| (2^-9 in the subnormal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


def default_scale(d):
    return 1.0 / math.sqrt(d)
