"""Seeded synthetic inputs, bit-identical on the CPU and on the GPU.

This module holds none of the attention method's arithmetic.  It only turns
(seed, tensor id, element index) into numbers, so that the oracle (CPU) and the
HIP path (GPU) can be fed the very same values without copying multi-GB inputs
across PCIe: any element, row range or row subset can be regenerated on either
device.

Generator:
  * counter: the flat element index i (int64) of a tensor of a given id;
  * hash: two rounds of Chris Wellons' "lowbias32" 32-bit integer hash
    (x ^= x>>16; x *= 0x7feb352d; x ^= x>>15; x *= 0x846ca68b; x ^= x>>16),
    keyed by (seed, tensor id).  All products are formed from 16-bit halves in
    int64 so that nothing overflows on either device;
  * normal values: the top 16 hash bits index a 65536-entry table of standard
    normal quantiles at (j + 1/2) / 65536 (computed once on the host in fp64
    by Python's statistics.NormalDist and rounded to fp32), then one fp32
    multiply by the scale and a round-to-nearest-even cast to the storage
    dtype.  Every step is exact or a single IEEE rounding, so CPU and GPU agree
    bit for bit;
  * uniform values: the top 24 hash bits times 2**-24 (exact in fp32);
  * integer grids: hash mod (2G+1) - G, times a power of two (exact).
"""
from __future__ import annotations

import statistics

import torch

_MASK32 = 0xFFFFFFFF

# Tensor ids: fixed per role so every consumer regenerates the same values.
TID = {
    "q": 1, "q_idx": 2, "w_idx": 3, "k": 4, "v": 5, "k_idx": 6,
    "z_k": 7, "z_v": 8, "z_idx": 9,
    "xb_k": 10, "xb_v": 11, "xb_idx": 12, "zb_k": 13, "zb_v": 14, "zb_idx": 15,
    "sink": 16, "kr": 17, "vr": 18, "kc": 19, "vc": 20, "bias": 21, "idx": 22,
    "scores": 23, "kic": 24,
}


def tensor_key(seed: int, tid: int, layer: int = 0) -> tuple[int, int]:
    """Two 32-bit keys for (seed, tensor id, layer), computed with Python ints."""
    def h(x):
        x &= _MASK32
        x ^= x >> 16
        x = (x * 0x7FEB352D) & _MASK32
        x ^= x >> 15
        x = (x * 0x846CA68B) & _MASK32
        x ^= x >> 16
        return x
    k1 = h((seed * 0x9E3779B9) ^ (tid * 0x85EBCA6B) ^ (layer * 0xC2B2AE35))
    k2 = h(k1 ^ 0x27D4EB2F)
    return k1, k2


def _mul32(x: torch.Tensor, mult: int) -> torch.Tensor:
    lo = mult & 0xFFFF
    hi = mult >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _MASK32


def _hash32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def hash_bits(index: torch.Tensor, key: tuple[int, int]) -> torch.Tensor:
    """32 pseudo-random bits (int64 in [0, 2^32)) per int64 element index."""
    k1, k2 = key
    lo = index & _MASK32
    hi = (index >> 32) & _MASK32
    return _hash32(_hash32(lo ^ k1) ^ (hi ^ k2))


_TABLES: dict = {}


def _normal_table(device) -> torch.Tensor:
    dev = torch.device(device)
    key = str(dev)
    if key not in _TABLES:
        if "cpu" not in _TABLES:
            nd = statistics.NormalDist()
            vals = [nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)]
            _TABLES["cpu"] = torch.tensor(vals, dtype=torch.float64).to(torch.float32)
        _TABLES[key] = _TABLES["cpu"].to(dev)
    return _TABLES[key]


def _values(kind: str, bits: torch.Tensor, scale: float, grid: int, device) -> torch.Tensor:
    if kind == "normal":
        v = _normal_table(device)[bits >> 16]
        return v * torch.tensor(scale, dtype=torch.float32, device=v.device)
    if kind == "uniform":  # [0, 1) * scale
        v = (bits >> 8).to(torch.float32) * (2.0 ** -24)
        return v * torch.tensor(scale, dtype=torch.float32, device=v.device)
    if kind == "grid":  # integers in [-grid, grid] times scale (a power of two)
        v = ((bits % (2 * grid + 1)) - grid).to(torch.float32)
        return v * torch.tensor(scale, dtype=torch.float32, device=v.device)
    raise ValueError(kind)


def fill_(out: torch.Tensor, seed: int, tid: int, *, kind: str = "normal",
          scale: float = 1.0, grid: int = 8, layer: int = 0,
          chunk: int = 1 << 25) -> torch.Tensor:
    """Fill a contiguous tensor in place, element i taking value(i)."""
    assert out.is_contiguous()
    flat = out.view(-1)
    key = tensor_key(seed, tid, layer)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(s, e, dtype=torch.int64, device=out.device)
        flat[s:e] = _values(kind, hash_bits(idx, key), scale, grid, out.device).to(out.dtype)
    return out


def mxfp4_(out: torch.Tensor, seed: int, tid: int, n: int, *, scale_lo: int = 127, scale_hi: int = 127,
           layer: int = 0) -> torch.Tensor:
    """Fill a uint8 buffer holding an MXFP4 tensor of n elements: n/2 bytes of
    uniformly random E2M1 code pairs, then n/32 E8M0 scale bytes uniform in
    [scale_lo, scale_hi].  Random codes, not a quantisation of values."""
    assert out.dtype == torch.uint8 and out.numel() == n // 2 + n // 32
    key = tensor_key(seed, tid, layer)
    idx = torch.arange(out.numel(), dtype=torch.int64, device=out.device)
    bits = hash_bits(idx, key)
    span = scale_hi - scale_lo + 1
    codes = bits & 0xFF
    scales = scale_lo + (bits >> 8) % span
    out.copy_(torch.where(idx < n // 2, codes, scales).to(torch.uint8))
    return out


def make(shape, seed: int, tid: int, *, dtype=torch.float32, device="cpu",
         kind: str = "normal", scale: float = 1.0, grid: int = 8, layer: int = 0) -> torch.Tensor:
    out = torch.empty(tuple(shape), dtype=dtype, device=device)
    return fill_(out, seed, tid, kind=kind, scale=scale, grid=grid, layer=layer)


def rows(full_shape, row_ids, seed: int, tid: int, *, dtype=torch.float32,
         device="cpu", kind: str = "normal", scale: float = 1.0, grid: int = 8,
         layer: int = 0) -> torch.Tensor:
    """Regenerate a subset of rows of a tensor of shape [..., D], addressed by
    flat row number (the product of the leading indices); returns [len, D]."""
    D = int(full_shape[-1])
    r = torch.as_tensor(row_ids, dtype=torch.int64, device=device).reshape(-1, 1)
    idx = r * D + torch.arange(D, dtype=torch.int64, device=device).reshape(1, -1)
    key = tensor_key(seed, tid, layer)
    return _values(kind, hash_bits(idx, key), scale, grid, device).to(dtype)


def sample_indices(seed: int, tid: int, n_rows: int, k: int, nvis, *, layer: int = 0):
    """Per row, k distinct indices drawn without replacement from [0, nvis),
    sorted ascending and padded with -1 when nvis < k (int32 [n_rows, k], CPU).
    A random ordering of hash values stands in for a shuffle."""
    nvis = torch.as_tensor(nvis, dtype=torch.int64).expand(n_rows)
    out = torch.full((n_rows, k), -1, dtype=torch.int32)
    key = tensor_key(seed, tid, layer)
    for r in range(n_rows):
        nv = int(nvis[r])
        if nv <= 0:
            continue
        ii = torch.arange(nv, dtype=torch.int64) + r * (1 << 32) // max(n_rows, 1)
        order = torch.argsort(hash_bits(ii, key), stable=True)
        take = order[: min(k, nv)]
        out[r, : take.numel()] = torch.sort(take).values.to(torch.int32)
    return out
