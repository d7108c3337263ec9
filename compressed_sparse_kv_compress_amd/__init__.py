"""MI355X (gfx950) hybrid compressed attention: CSA and HCA hot path.

A thin Python binding over the C ABI in ``include/csa.h`` (libcsa.so): it only
marshals arguments.  Tensors are torch device tensors used as memory; every
step of the computation runs in the HIP kernels.  If libcsa.so has not been
built, importing this package raises: there is no fallback.

Functions mirror the C entry points: csa_compress, hca_compress,
csa_index_score, csa_topk_select, csa_index_topk, csa_sparse_attn and
hca_dense_attn.  Outputs and workspaces are allocated with torch on the
inputs' device unless passed in; work is enqueued on the current stream.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libcsa.so is not built: run `python compressed_sparse_kv_compress_amd/build.py` "
        "(the HIP library is the only implementation)")

_lib = ctypes.CDLL(LIB_PATH)

CSA_F32, CSA_BF16, CSA_FP8, CSA_MXFP4 = 0, 1, 2, 3
_STATUS = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_UNSUPPORTED",
           3: "CSA_ERR_WORKSPACE", 4: "CSA_ERR_HIP"}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_i32 = ctypes.c_int
_f32 = ctypes.c_float


class Layout(ctypes.Structure):
    """csa_layout_t: per-sequence lengths (device int64 [B]), a block table of
    paged compressed caches (device int32 [B][bt_stride], `page` entries per
    page, `num_pages` pages per pool) and ring-mode raw windows.  Build it
    with layout(); keep the tensors alive while calls use it."""
    _fields_ = [("seq_len", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int64),
                ("page", ctypes.c_int64), ("num_pages", ctypes.c_int64), ("window_ring", ctypes.c_int32)]


def layout(seq_len=None, block_table=None, page=0, num_pages=0, ring=False):
    """A Layout from torch tensors (seq_len int64 [B], block_table int32 [B][bt_stride])."""
    for t, dt in ((seq_len, torch.int64), (block_table, torch.int32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise TypeError("seq_len must be contiguous int64 and block_table contiguous int32")
    return Layout(None if seq_len is None else seq_len.data_ptr(),
                  None if block_table is None else block_table.data_ptr(),
                  0 if block_table is None else block_table.shape[1], page, num_pages, 1 if ring else 0)


def _lay(lay):
    return None if lay is None else ctypes.byref(lay)


def _sig(name, args, res=_i32):
    fn = getattr(_lib, name)
    fn.argtypes = args
    fn.restype = res
    return fn


_csa_compress = _sig("csa_compress", [_vp] * 6 + [_i64] * 9 + [_i32, _vp])
_hca_compress = _sig("hca_compress", [_vp] * 4 + [_i64] * 9 + [_i32, _vp])
_csa_index_score = _sig("csa_index_score", [_vp] * 3 + [_i64] * 7 + [_vp, _i32, _vp])
_csa_topk_select_workspace = _sig("csa_topk_select_workspace", [_i64] * 4, _sz)
_csa_topk_select = _sig("csa_topk_select", [_vp] + [_i64] * 6 + [_vp, _vp, _vp, _sz, _vp])
_csa_index_topk_workspace = _sig("csa_index_topk_workspace", [_i64] * 5, _sz)
_csa_index_topk = _sig("csa_index_topk", [_vp] * 3 + [_i64] * 8 + [_vp, _vp, _vp, _sz, _i32, _vp])
_LP = ctypes.POINTER(Layout)
_csa_index_topk_ex = _sig("csa_index_topk_ex", [_LP] + [_vp] * 3 + [_i64] * 8 + [_vp, _vp, _vp, _sz, _i32, _vp])
_csa_sparse_attn_ex = _sig("csa_sparse_attn_ex", [_LP] + [_vp] * 3 + [_i64, _vp, _i64, _vp, _vp, _i64, _i64, _vp,
                                                                        _f32] + [_i64] * 5 + [_vp, _vp, _vp, _sz, _i32, _vp])
_hca_dense_attn_ex = _sig("hca_dense_attn_ex", [_LP] + [_vp] * 3 + [_i64, _i64, _vp, _vp, _i64, _i64, _vp, _f32]
                          + [_i64] * 5 + [_vp, _vp, _vp, _sz, _i32, _vp])
_csa_compress_append = _sig("csa_compress_append", [_LP] + [_vp] * 9 + [_i64, _vp, _vp] + [_i64] * 4 + [_i32, _vp])
_csa_window_append = _sig("csa_window_append", [_vp] * 5 + [_i64] * 3 + [_i32, _vp])
_csa_index_topk_noalloc = _sig("csa_index_topk_noalloc", [_vp] * 3 + [_i64] * 8 + [_vp, _vp, _i32, _vp])
_csa_index_topk_noalloc_max_bytes = _sig("csa_index_topk_noalloc_max_bytes", [], _sz)
_csa_attn_workspace = _sig("csa_attn_workspace", [_i64] * 5, _sz)
_csa_sparse_attn_workspace = _sig("csa_sparse_attn_workspace", [_i64] * 6 + [_i32], _sz)
_csa_sparse_attn = _sig("csa_sparse_attn", [_vp] * 3 + [_i64, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _f32]
                        + [_i64] * 5 + [_vp, _vp, _vp, _sz, _i32, _vp])
_hca_dense_attn_workspace = _sig("hca_dense_attn_workspace", [_i64] * 8 + [_i32], _sz)
_hca_dense_attn = _sig("hca_dense_attn", [_vp] * 3 + [_i64, _i64, _vp, _vp, _i64, _i64, _vp, _f32]
                       + [_i64] * 5 + [_vp, _vp, _vp, _sz, _i32, _vp])
_csa_status_string = _sig("csa_status_string", [_i32], ctypes.c_char_p)
_csa_last_error = _sig("csa_last_error", [], ctypes.c_char_p)
_csa_time_next_scan = _sig("csa_time_next_scan", [_vp, _vp])


class CsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _csa_last_error().decode(errors="replace")
        super().__init__("%s: %s (%s)" % (where, _STATUS.get(status, status), detail))


def _check(st, where):
    if st != 0:
        raise CsaError(st, where)


class MXFP4:
    """An OCP MXFP4 tensor of logical shape `shape` (last dimension d, a
    multiple of 32) held in one uint8 buffer `data`: prod(shape)/2 bytes of
    E2M1 codes (element 2i in the low nibble of byte i), then prod(shape)/32
    E8M0 scale bytes, one per 32 consecutive elements of a row."""

    def __init__(self, data: torch.Tensor, shape):
        shape = tuple(int(x) for x in shape)
        n = 1
        for x in shape:
            n *= x
        if data.dtype != torch.uint8 or not data.is_contiguous():
            raise TypeError("MXFP4 data must be a contiguous uint8 tensor")
        if shape[-1] % 32 or data.numel() != n // 2 + n // 32:
            raise ValueError("MXFP4 buffer of %d bytes does not hold shape %s" % (data.numel(), shape))
        self.data, self.shape = data, shape

    @property
    def device(self):
        return self.data.device

    def data_ptr(self):
        return self.data.data_ptr()

    def is_contiguous(self):
        return True


def _dt(t) -> int:
    if isinstance(t, MXFP4):
        return CSA_MXFP4
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.float8_e4m3fn:  # OCP FP8 E4M3
        return CSA_FP8
    raise TypeError("storage dtype must be bfloat16, float32 or float8_e4m3fn, got %s" % t.dtype)


def _attn_dt(q, kc) -> int:
    """Attention's dtype code: the K/V storage type.  FP8 K/V comes with a
    bf16 query (and output); otherwise q and the cache share one type."""
    if kc.dtype == torch.float8_e4m3fn:
        if q.dtype != torch.bfloat16:
            raise TypeError("FP8 K/V attention takes a bfloat16 query, got %s" % q.dtype)
        return CSA_FP8
    if q.dtype != kc.dtype:
        raise TypeError("q (%s) and the K/V cache (%s) differ" % (q.dtype, kc.dtype))
    return _dt(q)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(dev=None):
    return torch.cuda.current_stream(dev).cuda_stream


def status_string(st: int) -> str:
    return _csa_status_string(st).decode()


# ---------------------------------------------------------------------------
# compression
# ---------------------------------------------------------------------------

def _compress_out(x, B, ne, D, out, out_ld, mxfp4):
    """The output of a bulk compression and its dtype code: bf16 rows in and
    MXFP4 entries out when `mxfp4` is set or `out` is an MXFP4 tensor."""
    mx = mxfp4 or isinstance(out, MXFP4)
    if mx and x.dtype != torch.bfloat16:
        raise TypeError("MXFP4 entries are compressed from bfloat16 rows, got %s" % x.dtype)
    if mx and out is not None and not isinstance(out, MXFP4):
        raise TypeError("MXFP4 entries need an MXFP4 output tensor")
    if out is None:
        if mx:
            nel = B * ne * D
            out = MXFP4(torch.empty(nel // 2 + nel // 32, dtype=torch.uint8, device=x.device), (B, ne, D))
        else:
            out = torch.empty((B, ne, D), dtype=x.dtype, device=x.device)
        out_ld = ne
    elif out_ld is None:
        out_ld = out.shape[1]
    return out, out_ld, (CSA_MXFP4 if mx else _dt(x))


def csa_compress(x_a, z_a, m, *, x_b=None, z_b=None, bias=None, n=None, p0=0, e0=0, e1=None,
                 out=None, out_ld=None, mxfp4=False):
    """Block-weighted compression of [B][n_raw][D] raw rows (positions p0..).

    Returns out [B][e1-e0][D] (or writes into ``out`` with row stride out_ld);
    with ``mxfp4`` (bf16 rows) the entries come back as an MXFP4 tensor."""
    B, n_raw, D = x_a.shape
    n = p0 + n_raw if n is None else n
    e1 = -(-n // m) if e1 is None else e1
    out, out_ld, dt = _compress_out(x_a, B, e1 - e0, D, out, out_ld, mxfp4)
    st = _csa_compress(_ptr(x_a), _ptr(z_a), _ptr(x_b), _ptr(z_b), _ptr(bias), out.data_ptr(), B, n, D,
                       m, p0, n_raw, e0, e1, out_ld, dt, _stream(x_a.device))
    _check(st, "csa_compress")
    return out


def hca_compress(x, z, m=128, *, bias=None, n=None, p0=0, e0=0, e1=None, out=None, out_ld=None,
                 mxfp4=False):
    B, n_raw, D = x.shape
    n = p0 + n_raw if n is None else n
    e1 = -(-n // m) if e1 is None else e1
    out, out_ld, dt = _compress_out(x, B, e1 - e0, D, out, out_ld, mxfp4)
    st = _hca_compress(_ptr(x), _ptr(z), _ptr(bias), out.data_ptr(), B, n, D, m, p0, n_raw, e0, e1,
                       out_ld, dt, _stream(x.device))
    _check(st, "hca_compress")
    return out


def csa_compress_append(x_a, z_a, m, rings, pos, cache, *, x_b=None, z_b=None, bias=None, layout=None, L=None):
    """One new raw token per sequence (x_a, z_a [B][D]; x_b, z_b in two-path
    mode): staged into `rings` (ring_xa, ring_za[, ring_xb, ring_zb], each
    [B][S][D]) at slot pos % S; the entry pos // m is written to `cache` when
    the token completes its block.  pos: device int64 [B].  An MXFP4 `cache`
    (bf16 rows and rings) receives MXFP4 entries."""
    B, D = x_a.shape
    S = rings[0].shape[1]
    rx_b = rings[2] if len(rings) > 2 else None
    rz_b = rings[3] if len(rings) > 2 else None
    L = cache.shape[1] if L is None else L
    if isinstance(cache, MXFP4):
        if x_a.dtype != torch.bfloat16:
            raise TypeError("MXFP4 entries are compressed from bfloat16 rows, got %s" % x_a.dtype)
        dt = CSA_MXFP4
    else:
        dt = _dt(x_a)
    st = _csa_compress_append(_lay(layout), _ptr(x_a), _ptr(z_a), _ptr(x_b), _ptr(z_b), _ptr(bias), _ptr(rings[0]),
                              _ptr(rings[1]), _ptr(rx_b), _ptr(rz_b), S, _ptr(pos), _ptr(cache), L, B, D, m,
                              dt, _stream(x_a.device))
    _check(st, "csa_compress_append")
    return cache


def csa_window_append(k_new, v_new, kr, vr, pos):
    """Raw window rows of one new token per sequence into ring slot pos % R."""
    B, d = k_new.shape
    R = kr.shape[1]
    st = _csa_window_append(_ptr(k_new), _ptr(v_new), _ptr(kr), _ptr(vr), _ptr(pos), B, R, d, _dt(k_new),
                            _stream(k_new.device))
    _check(st, "csa_window_append")


# ---------------------------------------------------------------------------
# indexer and top-k
# ---------------------------------------------------------------------------

def csa_index_score(q_idx, k_idx, m, *, w_idx=None, n_ctx, out=None):
    B, T, HI, dI = q_idx.shape
    L = k_idx.shape[1]
    if out is None:
        out = torch.empty((B, T, L), dtype=torch.float32, device=q_idx.device)
    st = _csa_index_score(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, T, n_ctx, L, HI, dI, m,
                          out.data_ptr(), _dt(q_idx), _stream(q_idx.device))
    _check(st, "csa_index_score")
    return out


def csa_topk_select_workspace(B, T, L, k) -> int:
    return int(_csa_topk_select_workspace(B, T, L, k))


def csa_topk_select(score, m, k, *, n_ctx, idx=None, out_score=None, want_scores=False, ws=None):
    B, T, L = score.shape
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=score.device)
    if want_scores and out_score is None:
        out_score = torch.empty((B, T, k), dtype=torch.float32, device=score.device)
    if ws is None:
        ws = torch.empty(max(16, csa_topk_select_workspace(B, T, L, k)), dtype=torch.uint8,
                         device=score.device)
    st = _csa_topk_select(_ptr(score), B, T, n_ctx, L, m, k, idx.data_ptr(), _ptr(out_score),
                          ws.data_ptr(), ws.numel() * ws.element_size(), _stream(score.device))
    _check(st, "csa_topk_select")
    return (idx, out_score) if want_scores else idx


def csa_index_topk_workspace(B, T, L, H_I, k) -> int:
    return int(_csa_index_topk_workspace(B, T, L, H_I, k))


def csa_index_topk(q_idx, k_idx, m, k, *, w_idx=None, n_ctx, ws=None, idx=None, out_score=None,
                   want_scores=False, layout=None, L=None):
    """Index + top-k.  layout (a Layout) selects csa_index_topk_ex: then
    k_idx may be a paged pool and L (the longest sequence's capacity in
    entries) must be given."""
    B, T, HI, dI = q_idx.shape
    L = k_idx.shape[1] if L is None else L
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=q_idx.device)
    if want_scores and out_score is None:
        out_score = torch.empty((B, T, k), dtype=torch.float32, device=q_idx.device)
    if ws is None:
        nb = max(16, csa_index_topk_workspace(B, T, L, HI, k))
        ws = torch.zeros(nb, dtype=torch.uint8, device=q_idx.device)
    args = (_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, T, n_ctx, L, HI, dI, m, k, idx.data_ptr(), _ptr(out_score),
            ws.data_ptr(), ws.numel() * ws.element_size(), _dt(q_idx), _stream(q_idx.device))
    if layout is None:
        _check(_csa_index_topk(*args), "csa_index_topk")
    else:
        _check(_csa_index_topk_ex(_lay(layout), *args), "csa_index_topk_ex")
    return (idx, out_score) if want_scores else idx


def csa_index_topk_noalloc_max_bytes() -> int:
    return int(_csa_index_topk_noalloc_max_bytes())


def csa_index_topk_noalloc(q_idx, k_idx, m, k, *, w_idx, n_ctx, idx, out_score=None):
    """csa_index_topk through the library's static scratch: no workspace, and
    the caller passes the outputs (nothing is allocated by this call)."""
    B, T, HI, dI = q_idx.shape
    L = k_idx.shape[1]
    st = _csa_index_topk_noalloc(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), B, T, n_ctx, L, HI, dI, m, k,
                                 idx.data_ptr(), _ptr(out_score), _dt(q_idx), _stream(q_idx.device))
    _check(st, "csa_index_topk_noalloc")
    return idx


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _attn_out(q, out, lse, want_lse):
    B, T, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    return out, lse


def csa_attn_workspace(B, T, H, d, n_rows) -> int:
    return int(_csa_attn_workspace(B, T, H, d, n_rows))


def csa_sparse_attn_workspace(B, T, H, d, k, W, dtype) -> int:
    return int(_csa_sparse_attn_workspace(B, T, H, d, k, W, dtype))


def hca_dense_attn_workspace(B, T, H, d, L, m, n_ctx, W, dtype) -> int:
    return int(_hca_dense_attn_workspace(B, T, H, d, L, m, n_ctx, W, dtype))


def _ws(nbytes, dev, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def csa_sparse_attn(q, kc, vc, idx, *, kr=None, vr=None, W=0, sink=None, scale=None, n_ctx,
                    out=None, lse=None, want_lse=False, ws=None, layout=None, L=None):
    """CSA attention.  layout selects csa_sparse_attn_ex (paged kc / vc pools
    need L, the capacity in entries)."""
    B, T, H, d = q.shape
    L = kc.shape[1] if L is None else L
    k = idx.shape[-1]
    R = 0 if kr is None else kr.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out, lse = _attn_out(q, out, lse, want_lse)
    dt = _attn_dt(q, kc)
    need = csa_sparse_attn_workspace(B, T, H, d, k, W, dt) if layout is None else csa_attn_workspace(B, T, H, d,
                                                                                                     k + W)
    wp, wn = _ws(need, q.device, ws)
    args = (_ptr(q), _ptr(kc), _ptr(vc), L, _ptr(idx), k, _ptr(kr), _ptr(vr), R, W, _ptr(sink), scale, B, T,
            n_ctx, H, d, out.data_ptr(), _ptr(lse), wp, wn, dt, _stream(q.device))
    if layout is None:
        _check(_csa_sparse_attn(*args), "csa_sparse_attn")
    else:
        _check(_csa_sparse_attn_ex(_lay(layout), *args), "csa_sparse_attn_ex")
    return (out, lse) if want_lse else out


def hca_dense_attn(q, kc, vc, m, *, kr=None, vr=None, W=0, sink=None, scale=None, n_ctx, out=None,
                   lse=None, want_lse=False, ws=None, layout=None, L=None):
    """HCA attention.  layout selects hca_dense_attn_ex (paged pools need L)."""
    B, T, H, d = q.shape
    L = kc.shape[1] if L is None else L
    R = 0 if kr is None else kr.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out, lse = _attn_out(q, out, lse, want_lse)
    dt = _attn_dt(q, kc)
    if layout is None:
        need = hca_dense_attn_workspace(B, T, H, d, L, m, n_ctx, W, dt)
    else:
        need = csa_attn_workspace(B, T, H, d, min(L, (n_ctx - 1) // m) + W)
    wp, wn = _ws(need, q.device, ws)
    args = (_ptr(q), _ptr(kc), _ptr(vc), L, m, _ptr(kr), _ptr(vr), R, W, _ptr(sink), scale, B, T, n_ctx, H, d,
            out.data_ptr(), _ptr(lse), wp, wn, dt, _stream(q.device))
    if layout is None:
        _check(_hca_dense_attn(*args), "hca_dense_attn")
    else:
        _check(_hca_dense_attn_ex(_lay(layout), *args), "hca_dense_attn_ex")
    return (out, lse) if want_lse else out


def time_next_scan(start, stop):
    """The next indexer scan kernel launched from this thread records the
    torch.cuda.Event pair `start` / `stop` (created with enable_timing=True)
    as it starts and ends; start.elapsed_time(stop) is then that kernel's
    duration.  None, None clears a pending request."""
    if start is None and stop is None:
        _check(_csa_time_next_scan(None, None), "csa_time_next_scan")
        return
    for e in (start, stop):
        if e.cuda_event == 0:  # torch creates the event on its first record
            e.record()
    _check(_csa_time_next_scan(start.cuda_event, stop.cuda_event), "csa_time_next_scan")
