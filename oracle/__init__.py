"""CPU oracle for the CSA / HCA hybrid compressed attention path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code with
the HIP library and never imports it.

The arithmetic lives in ``csa_oracle.c`` (plain loops, fp64 accumulation);
this module builds it with gcc, loads it with ctypes and marshals numpy
arrays.  Every input is converted to float64 first, which is exact for bf16 and
fp32 values.

Pinning status (what checks each function against the pages or mathematics,
see tests/test_oracle_*.py):
  num_entries / num_visible   pinned (counts from the pages, the Block-24 example)
  compress                    pinned (mean pooling, identity, convexity, shift
                              invariance, scipy softmax brute force, two-path
                              causality); the two-path bias row layout is a
                              convention: parity unpinned for the bias layout
  index_scores                pinned (the 8 / -7 ReLU example, brute force via
                              numpy einsum); absence of a scale: parity unpinned
  topk                        pinned (O(L^2) rank-count brute force, ties, +-0)
  sparse_attn / dense_attn    pinned (torch SDPA textbook MQA incl. sink as an
                              extra logit, one-hot probability mass, sink limits,
                              the 0.15 / 0.85 example, order invariance)
  fp8_decode / fp8_encode     pinned (all 256 codes against torch's float8_e4m3fn,
                              named values, ties to even, round trips); the
                              choice of E4M3 itself is a reading of the pages
                              (they name FP8 without an encoding)
  minifloat_decode            pinned (E4M3 and E5M2 against torch's float8 types
                              on every finite code)
  e2m1_decode / e8m0_decode / pinned (E2M1 is the decoder above with 2 exponent
  mxfp4_decode                bits, bias 1, and its values are E4M3 values that
                              round-trip through fp8_encode; E8M0 against torch's
                              float8_e8m0fnu on all 256 codes; block layout by
                              single-element and single-scale buffers); the
                              MXFP4 reading of "FP4" and the buffer layout are
                              conventions: parity unpinned for the layout
  mxfp4_encode                pinned (round trip of every representable block
                              through mxfp4_decode, the nearest-value property
                              by brute force over all 15 values at the block's
                              scale, named ties to even, 4 <= amax / 2^E < 8,
                              saturation, clamped scales); the scale rule is
                              the OCP conversion, a reading (the pages name no
                              encoding)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "libcsa_oracle.so")
_lock = threading.Lock()
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, IEEE fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            lib.oracle_num_entries.restype = _i64
            lib.oracle_num_entries.argtypes = [_i64, _i64]
            lib.oracle_num_visible.restype = _i64
            lib.oracle_num_visible.argtypes = [_i64, _i64]
            lib.oracle_compress.restype = ctypes.c_int
            lib.oracle_compress.argtypes = [_d, _d, _d, _d, _d] + [_i64] * 8 + [_d]
            lib.oracle_index_scores.restype = None
            lib.oracle_index_scores.argtypes = [_d, _d, _d, _i64, _i64,
                                                ctypes.POINTER(_i64), _i64, _i64,
                                                _i64, _i64, _d]
            lib.oracle_topk.restype = None
            lib.oracle_topk.argtypes = [_d, ctypes.POINTER(_i64), _i64, _i64, _i64,
                                        ctypes.POINTER(ctypes.c_int32)]
            lib.oracle_sparse_attn.restype = ctypes.c_int
            lib.oracle_sparse_attn.argtypes = [
                _d, _d, _d, _i64, ctypes.POINTER(ctypes.c_int32), _i64, _d, _d, _i64,
                _i64, _d, ctypes.c_double, _i64, _i64, ctypes.POINTER(_i64), _i64,
                _i64, _i64, _d, _d]
            lib.oracle_dense_attn.restype = ctypes.c_int
            lib.oracle_dense_attn.argtypes = [
                _d, _d, _d, _i64, _i64, _d, _d, _i64, _i64, _d, ctypes.c_double,
                _i64, _i64, ctypes.POINTER(_i64), _i64, _i64, _i64, _d, _d]
            _lib = lib
    return _lib


# ---- FP8 storage (OCP 8-bit floating point, E4M3 flavour) -----------------
# The pages let the indexer's q.k path run in low precision (FP8 / FP4) and the
# main KV in FP8, without naming an encoding.  The reading taken here is the
# OCP E4M3 format (the one gfx950's converters and fp8 MFMAs use): 1 sign bit,
# 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds subnormals
# m * 2**-9; exponent 15 with mantissa 7 is NaN; there are no infinities, so
# the largest finite value is 1.75 * 2**8 = 448.


def minifloat_decode(codes, ebits: int, mbits: int, bias: int) -> np.ndarray:
    """Codes of a binary float with one sign bit (the top bit), `ebits`
    exponent bits and `mbits` fraction bits -> float64, by the fields:
    exponent 0 is subnormal (f * 2^(1 - bias - mbits)), otherwise
    (1 + f / 2^mbits) * 2^(e - bias).  Special codes (NaN, infinities) are the
    caller's to apply."""
    c = np.asarray(codes).astype(np.int64)
    nb = 1 + ebits + mbits
    sign = np.where((c >> (nb - 1)) & 1, -1.0, 1.0)
    e = (c >> mbits) & ((1 << ebits) - 1)
    f = (c & ((1 << mbits) - 1)).astype(np.float64)
    mag = np.where(e == 0, f * 2.0 ** (1 - bias - mbits),
                   (1.0 + f / 2.0 ** mbits) * np.exp2(e.astype(np.float64) - bias))
    return sign * mag


def fp8_decode(codes) -> np.ndarray:
    """E4M3 byte codes (any integer array) -> float64 values, from the format's
    definition (bias 7; the all-ones exponent and fraction is NaN)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    v = minifloat_decode(c, 4, 3, 7)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e2m1_decode(codes) -> np.ndarray:
    """FP4 E2M1 nibble codes -> float64 (bias 1, no special codes)."""
    return minifloat_decode(np.asarray(codes).astype(np.int64) & 0xF, 2, 1, 1)


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale bytes -> 2^(e - 127); 255 is NaN."""
    e = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def mxfp4_decode(buf, shape) -> np.ndarray:
    """An MXFP4 buffer of logical shape `shape` -> float64 array of that shape.

    Layout: prod(shape)/2 code bytes, element 2i in the low nibble of byte i
    and 2i+1 in the high nibble, then prod(shape)/32 E8M0 scale bytes, scale
    j of a row multiplying its elements 32j .. 32j+31 (OCP microscaling: a
    block of 32 elements shares one power-of-two scale)."""
    b = np.asarray(buf).astype(np.int64).reshape(-1)
    shape = tuple(int(x) for x in shape)
    n = int(np.prod(shape))
    d = shape[-1]
    assert d % 32 == 0 and b.size == n // 2 + n // 32
    codes = b[: n // 2]
    el = np.empty(n, dtype=np.int64)
    el[0::2] = codes & 0xF
    el[1::2] = codes >> 4
    vals = e2m1_decode(el).reshape(n // d, d // 32, 32)
    sc = e8m0_decode(b[n // 2:]).reshape(n // d, d // 32, 1)
    return (vals * sc).reshape(shape)


def mxfp4_encode(x) -> np.ndarray:
    """float values of shape (..., d), d a multiple of 32 -> an MXFP4 buffer
    (uint8, the layout mxfp4_decode reads), by the OCP microscaling
    conversion: a block of 32 consecutive elements of a row shares the scale
    2^E, E = floor(log2(largest magnitude in the block)) - 2 (2 being the
    exponent of E2M1's largest magnitude, 6 = 1.5 * 2^2), E clamped to E8M0's
    range [-127, 127] and an all-zero block taking -127; each element is the
    E2M1 magnitude nearest to |x| / 2^E (of two equally near, the one with
    the even code; beyond 6 the nearest is 6, so large values saturate) with
    x's own sign bit (a negative value that rounds to 0 keeps code 8).
    NaN and infinities are rejected."""
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("mxfp4_encode: NaN or infinity has no MXFP4 code")
    d = x.shape[-1]
    assert d % 32 == 0
    blk = x.reshape(-1, 32)
    amax = np.abs(blk).max(axis=1)
    _, ex = np.frexp(amax)  # amax = f * 2^ex, 0.5 <= f < 1: floor(log2 amax) = ex - 1
    E = np.where(amax > 0, ex - 1 - 2, -127)
    E = np.clip(E, -127, 127)
    y = np.abs(blk) / np.exp2(E.astype(np.float64))[:, None]  # exact: a power-of-two scaling
    grid = e2m1_decode(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6
    dist = np.abs(y[..., None] - grid)
    best = dist.min(axis=-1, keepdims=True)
    near = dist == best
    # of the nearest codes (one, or two on a tie) take the even one
    code = np.where(near[..., 0::2].any(axis=-1), np.argmax(near[..., 0::2], axis=-1) * 2,
                    np.argmax(near, axis=-1))
    code = code + np.where(np.signbit(blk), 8, 0)
    flat = code.reshape(-1)
    out = np.empty(flat.size // 2 + flat.size // 32, dtype=np.uint8)
    out[: flat.size // 2] = (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)
    out[flat.size // 2:] = (E + 127).astype(np.uint8)
    return out


def fp8_encode(x) -> np.ndarray:
    """float values -> E4M3 byte codes, rounding to nearest with ties to the
    even code.  Magnitudes of 464 and above (past the midpoint above 448) and
    NaN are rejected: the format has no infinities."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) >= 464.0).any():
        raise ValueError("fp8_encode: NaN or magnitude >= 464 has no E4M3 code")
    # All finite non-negative values, ascending with the code (0x00 .. 0x7E).
    grid = fp8_decode(np.arange(0x7F))
    a = np.abs(x).reshape(-1)
    hi = np.searchsorted(grid, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == grid[hi], hi, np.where(pick_hi, hi, lo))
    neg = np.signbit(x.reshape(-1))
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8).reshape(x.shape)


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor on the CPU
        a = a.detach().to("cpu")
        if str(a.dtype) == "torch.float8_e4m3fn":  # decoded here, not by torch
            return np.ascontiguousarray(fp8_decode(a.view(dtype=__import__("torch").uint8).numpy()))
        a = a.double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_d)


def num_entries(n: int, m: int) -> int:
    return int(_load().oracle_num_entries(n, m))


def num_visible(t: int, m: int) -> int:
    return int(_load().oracle_num_visible(t, m))


def compress(x_a, z_a, m, *, x_b=None, z_b=None, bias=None, n=None, p0=0,
             e0=0, e1=None):
    """Block-weighted compression; arrays [B][n_raw][D] for positions p0...

    Returns float64 [B][e1-e0][D]."""
    x_a, z_a, x_b, z_b, bias = map(_f64, (x_a, z_a, x_b, z_b, bias))
    B, n_raw, D = x_a.shape
    if n is None:
        n = p0 + n_raw
    if e1 is None:
        e1 = num_entries(n, m)
    if (x_b is None) != (z_b is None):
        raise ValueError("x_b and z_b go together")
    out = np.zeros((B, e1 - e0, D), dtype=np.float64)
    rc = _load().oracle_compress(_p(x_a), _p(z_a), _p(x_b), _p(z_b), _p(bias), B, n,
                                 D, m, p0, n_raw, e0, e1, _p(out))
    if rc != 0:
        raise ValueError("oracle_compress: raw rows do not cover the entries (%d)" % rc)
    return out


def _tpos(T, n_ctx, tpos):
    if tpos is None:
        tpos = np.arange(n_ctx - T, n_ctx, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(tpos, dtype=np.int64))


def index_scores(q_idx, k_idx, m, *, w=None, n_ctx=None, tpos=None):
    """Indexer scores float64 [B][T][L]; invisible entries are -inf."""
    q_idx, k_idx, w = map(_f64, (q_idx, k_idx, w))
    B, T, HI, dI = q_idx.shape
    L = k_idx.shape[1]
    tp = _tpos(T, n_ctx, tpos)
    out = np.empty((B, T, L), dtype=np.float64)
    _load().oracle_index_scores(_p(q_idx), _p(w), _p(k_idx), B, T,
                                tp.ctypes.data_as(ctypes.POINTER(_i64)), L, HI, dI, m,
                                _p(out))
    return out


def topk(scores, nvis, k):
    """Top-k per row of scores [..., L] over the first nvis entries.

    Returns int32 [..., k], ascending indices, -1 padded."""
    s = _f64(scores)
    lead = s.shape[:-1]
    L = s.shape[-1]
    R = int(np.prod(lead)) if lead else 1
    nv = np.ascontiguousarray(np.broadcast_to(np.asarray(nvis, dtype=np.int64), lead).reshape(-1))
    if np.isnan(s).any():
        raise ValueError("scores contain NaN")
    out = np.empty((R, k), dtype=np.int32)
    _load().oracle_topk(_p(s.reshape(R, L)), nv.ctypes.data_as(ctypes.POINTER(_i64)), R, L,
                        k, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return out.reshape(lead + (k,))


def index_topk(q_idx, k_idx, m, k, *, w=None, n_ctx=None, tpos=None):
    """Scores then selection; returns (idx int32 [B][T][k], scores float64 [B][T][L])."""
    q = _f64(q_idx)
    T = q.shape[1]
    tp = _tpos(T, n_ctx, tpos)
    sc = index_scores(q, k_idx, m, w=w, n_ctx=n_ctx, tpos=tp)
    L = sc.shape[-1]
    nv = np.minimum(tp // m, L)
    idx = topk(sc, np.broadcast_to(nv, sc.shape[:-1]), k)
    return idx, sc


def sparse_attn(q, kc, vc, idx, kr, vr, W, *, sink=None, scale=None, n_ctx=None,
                tpos=None):
    """CSA attention; returns (out float64 [B][T][H][d], lse float64 [B][T][H])."""
    q, kc, vc, kr, vr, sink = map(_f64, (q, kc, vc, kr, vr, sink))
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    B, T, H, d = q.shape
    L = kc.shape[1]
    R = 0 if kr is None else kr.shape[1]
    if kr is None:
        kr = vr = np.zeros((B, 1, d))
    k = idx.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if n_ctx is None:
        raise ValueError("n_ctx is required")
    tp = _tpos(T, n_ctx, tpos)
    out = np.zeros((B, T, H, d))
    lse = np.zeros((B, T, H))
    rc = _load().oracle_sparse_attn(_p(q), _p(kc), _p(vc), L,
                                    idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), k,
                                    _p(kr), _p(vr), R, W, _p(sink), float(scale), B, T,
                                    tp.ctypes.data_as(ctypes.POINTER(_i64)), n_ctx, H, d,
                                    _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_sparse_attn: bad index or window position")
    return out, lse


def dense_attn(q, kc, vc, m, kr, vr, W, *, sink=None, scale=None, n_ctx=None,
               tpos=None):
    """HCA attention; returns (out float64 [B][T][H][d], lse float64 [B][T][H])."""
    q, kc, vc, kr, vr, sink = map(_f64, (q, kc, vc, kr, vr, sink))
    B, T, H, d = q.shape
    L = kc.shape[1]
    R = 0 if kr is None else kr.shape[1]
    if kr is None:
        kr = vr = np.zeros((B, 1, d))
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if n_ctx is None:
        raise ValueError("n_ctx is required")
    tp = _tpos(T, n_ctx, tpos)
    out = np.zeros((B, T, H, d))
    lse = np.zeros((B, T, H))
    rc = _load().oracle_dense_attn(_p(q), _p(kc), _p(vc), L, m, _p(kr), _p(vr), R, W,
                                   _p(sink), float(scale), B, T,
                                   tp.ctypes.data_as(ctypes.POINTER(_i64)), n_ctx, H, d,
                                   _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_dense_attn: bad window position")
    return out, lse
