"""Host-side checks of the C ABI: the library loads and exports every entry
point declared in include/csa.h, and argument validation rejects bad calls
before anything reaches the GPU (these calls enqueue no work)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "compressed_sparse_kv_compress_amd", "libcsa.so")
HDR = os.path.join(ROOT, "include", "csa.h")


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?:csa_status_t|size_t|const char\*)\s+(\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libcsa.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_hot_path_calls():
    names = _declared()
    for n in ("csa_compress", "hca_compress", "csa_index_topk", "csa_sparse_attn", "hca_dense_attn",
              "csa_index_score", "csa_topk_select", "csa_attn_workspace", "csa_index_topk_workspace"):
        assert n in names


def _params(name):
    """Parameter names of a function declared in the header."""
    src = re.sub(r"/\*.*?\*/", "", open(HDR).read(), flags=re.S)
    m = re.search(r"\b%s\s*\(([^)]*)\)\s*;" % name, src)
    assert m, name
    return [re.findall(r"(\w+)\s*$", p.strip())[0] for p in m.group(1).split(",") if p.strip() != "void"]


# The boundary the hot path is built to: every call, in argument order.  The
# stream is `stream` (a void* holding a hipStream_t) and the dtype `dtype`
# everywhere.  csa_compress / hca_compress add (p0, n_raw, e0, e1, out_ld)
# after m, so the same call writes a decode-time entry into a cache slot.
CONTRACT = {
    "csa_compress": ["x_a", "z_a", "x_b", "z_b", "bias", "out", "B", "n", "D", "m",
                     "p0", "n_raw", "e0", "e1", "out_ld", "dtype", "stream"],
    "hca_compress": ["x", "z", "bias", "out", "B", "n", "D", "m", "p0", "n_raw", "e0", "e1", "out_ld",
                     "dtype", "stream"],
    "csa_index_topk_workspace": ["B", "T", "L", "H_I", "k"],
    "csa_index_topk": ["q_idx", "w_idx", "k_idx", "B", "T", "n_ctx", "L", "H_I", "d_I", "m", "k", "idx",
                       "out_score", "ws", "ws_bytes", "dtype", "stream"],
    "csa_attn_workspace": ["B", "T", "H", "d", "n_rows"],
    "csa_sparse_attn": ["q", "kc", "vc", "L", "idx", "k", "kr", "vr", "R", "W", "sink", "scale", "B", "T",
                        "n_ctx", "H", "d", "out", "lse", "ws", "ws_bytes", "dtype", "stream"],
    "hca_dense_attn": ["q", "kc", "vc", "L", "m", "kr", "vr", "R", "W", "sink", "scale", "B", "T", "n_ctx",
                       "H", "d", "out", "lse", "ws", "ws_bytes", "dtype", "stream"],
    "csa_status_string": ["status"],
}


def test_header_matches_the_boundary_contract(lib):
    names = _declared()
    for name, params in CONTRACT.items():
        assert name in names, name
        assert hasattr(lib, name), name
        assert _params(name) == params, (name, _params(name))


def test_attn_workspace_covers_both_attention_calls(lib):
    aw = lib.csa_attn_workspace
    aw.argtypes, aw.restype = [I] * 5, Z
    sw = lib.csa_sparse_attn_workspace
    sw.argtypes, sw.restype = [I] * 6 + [ctypes.c_int], Z
    dw = lib.hca_dense_attn_workspace
    dw.argtypes, dw.restype = [I] * 8 + [ctypes.c_int], Z
    for B, T in ((1, 1), (16, 1), (4, 1), (1, 300)):
        # sparse: k + W rows; dense at 1M tokens, m = 128: 7812 visible + W
        assert aw(B, T, 64, 512, 1024 + 128) >= sw(B, T, 64, 512, 1024, 128, 1)
        assert aw(B, T, 64, 512, 7812 + 128) >= dw(B, T, 64, 512, 7813, 128, 1000000, 128, 1)
        assert aw(B, T, 64, 512, 7812) >= dw(B, T, 64, 512, 7813, 128, 1000000, 0, 2)
    assert aw(0, 1, 64, 512, 100) == 0
    # fewer heads than one MFMA head group (the fp32 kernel's shapes): no split workspace, no fault
    assert aw(3, 1, 8, 64, 440) == 0


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def _call(lib, name, argtypes, *args):
    fn = getattr(lib, name)
    fn.argtypes = argtypes
    fn.restype = ctypes.c_int
    return fn(*args)


V, I, Z, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def test_status_strings(lib):
    lib.csa_status_string.restype = ctypes.c_char_p
    lib.csa_status_string.argtypes = [ctypes.c_int]
    assert lib.csa_status_string(0) == b"CSA_OK"
    assert lib.csa_status_string(3) == b"CSA_ERR_WORKSPACE"


def test_compress_rejects_bad_arguments(lib):
    args = [V] * 6 + [I] * 9 + [ctypes.c_int, V]
    # D not a multiple of 8
    assert _call(lib, "csa_compress", args, FAKE, FAKE, None, None, None, FAKE,
                 1, 16, 12, 4, 0, 16, 0, 4, 4, 1, None) == 1
    # entry range beyond ceil(n/m)
    assert _call(lib, "csa_compress", args, FAKE, FAKE, None, None, None, FAKE,
                 1, 16, 16, 4, 0, 16, 0, 5, 5, 1, None) == 1
    # two-path needs the previous block: raw rows starting at 8 cannot serve entry 2
    assert _call(lib, "csa_compress", args, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                 1, 16, 16, 4, 8, 8, 2, 4, 2, 1, None) == 1
    # misaligned pointer
    assert _call(lib, "csa_compress", args, FAKE + 2, FAKE, None, None, None, FAKE,
                 1, 16, 16, 4, 0, 16, 0, 4, 4, 1, None) == 1
    # unknown dtype
    assert _call(lib, "csa_compress", args, FAKE, FAKE, None, None, None, FAKE,
                 1, 16, 16, 4, 0, 16, 0, 4, 4, 7, None) == 1
    # nothing to do is fine and enqueues nothing
    assert _call(lib, "csa_compress", args, None, None, None, None, None, None,
                 1, 16, 16, 4, 0, 16, 2, 2, 0, 1, None) == 0


def test_index_and_attention_reject_bad_arguments(lib):
    idx_args = [V] * 3 + [I] * 8 + [V, V, V, Z, ctypes.c_int, V]
    # unsupported indexer shape for bf16 (H_I = 48)
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 48, 128, 4, 8,
                 FAKE, None, FAKE, 1 << 20, 1, None) == 2
    # workspace below one row of scores
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 128, 4, 8,
                 FAKE, None, FAKE, 16, 1, None) == 3
    # k = 0
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 128, 4, 0,
                 FAKE, None, FAKE, 1 << 20, 1, None) == 1
    attn = [V] * 3 + [I, V, I, V, V, I, I, V, F] + [I] * 5 + [V, V, V, Z, ctypes.c_int, V]
    # window without enough raw rows
    assert _call(lib, "csa_sparse_attn", attn, FAKE, FAKE, FAKE, 10, FAKE, 4, FAKE, FAKE, 8, 128,
                 None, 0.1, 1, 1, 400, 64, 512, FAKE, None, FAKE, 1 << 30, 1, None) == 1
    # unsupported head count for the bf16 MFMA kernel
    assert _call(lib, "csa_sparse_attn", attn, FAKE, FAKE, FAKE, 10, FAKE, 4, None, None, 0, 0,
                 None, 0.1, 1, 1, 40, 8, 512, FAKE, None, None, 0, 1, None) == 2
    dense = [V] * 3 + [I, I, V, V, I, I, V, F] + [I] * 5 + [V, V, V, Z, ctypes.c_int, V]
    # missing split workspace for a decode-shaped dense call
    assert _call(lib, "hca_dense_attn", dense, FAKE, FAKE, FAKE, 7813, 128, None, None, 0, 0, None,
                 0.04, 4, 1, 1000000, 64, 512, FAKE, None, None, 0, 1, None) == 3
    # non-finite scale
    assert _call(lib, "hca_dense_attn", dense, FAKE, FAKE, FAKE, 7813, 128, None, None, 0, 0, None,
                 float("inf"), 4, 1, 1000000, 64, 512, FAKE, None, None, 0, 1, None) == 1


def test_fp8_storage_is_validated(lib):
    """CSA_FP8 (2) is a known dtype: accepted by compression, the indexer
    (d_I = 128, H_I a multiple of 16 up to 128) and attention over an FP8 K/V
    cache (d = 512 only); 4 is unknown."""
    idx_args = [V] * 3 + [I] * 8 + [V, V, V, Z, ctypes.c_int, V]
    # FP8 indexer with d_I = 64: no kernel
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 64, 4, 8,
                 FAKE, None, FAKE, 1 << 20, 2, None) == 2
    # FP8 indexer with H_I = 48: no kernel
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 48, 128, 4, 8,
                 FAKE, None, FAKE, 1 << 20, 2, None) == 2
    # FP8 indexer, supported shape, but k = 0: an argument error, so the dtype itself passed
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 128, 4, 0,
                 FAKE, None, FAKE, 1 << 20, 2, None) == 1
    # unknown dtype 4
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 128, 4, 8,
                 FAKE, None, FAKE, 1 << 20, 4, None) == 1
    attn = [V] * 3 + [I, V, I, V, V, I, I, V, F] + [I] * 5 + [V, V, V, Z, ctypes.c_int, V]
    # FP8 K/V attention with d = 256: no kernel
    assert _call(lib, "csa_sparse_attn", attn, FAKE, FAKE, FAKE, 10, FAKE, 4, None, None, 0, 0,
                 None, 0.1, 1, 1, 40, 64, 256, FAKE, None, None, 0, 2, None) == 2
    dense = [V] * 3 + [I, I, V, V, I, I, V, F] + [I] * 5 + [V, V, V, Z, ctypes.c_int, V]
    assert _call(lib, "hca_dense_attn", dense, FAKE, FAKE, FAKE, 7813, 128, None, None, 0, 0, None,
                 0.04, 4, 1, 1000000, 64, 256, FAKE, None, None, 0, 2, None) == 2
    # d = 512 with H = 48: no kernel either
    assert _call(lib, "hca_dense_attn", dense, FAKE, FAKE, FAKE, 7813, 128, None, None, 0, 0, None,
                 0.04, 4, 1, 1000000, 48, 512, FAKE, None, None, 0, 2, None) == 2
    # ... and with a supported shape, a missing workspace is the error (nothing is launched)
    assert _call(lib, "hca_dense_attn", dense, FAKE, FAKE, FAKE, 7813, 128, None, None, 0, 0, None,
                 0.04, 4, 1, 1000000, 64, 512, FAKE, None, None, 0, 2, None) == 3
    # FP8 compression: nothing to do is fine (no launch), D not a multiple of 8 is an error
    args = [V] * 6 + [I] * 9 + [ctypes.c_int, V]
    assert _call(lib, "csa_compress", args, None, None, None, None, None, None,
                 1, 16, 16, 4, 0, 16, 2, 2, 0, 2, None) == 0
    assert _call(lib, "csa_compress", args, FAKE, FAKE, None, None, None, FAKE,
                 1, 16, 12, 4, 0, 16, 0, 4, 4, 2, None) == 1


def test_mxfp4_storage_is_validated(lib):
    """CSA_MXFP4 (3): the indexer (d_I = 128, H_I a multiple of 16 up to 128)
    and the output of compression (D a multiple of 32); attention rejects it
    as unsupported."""
    idx_args = [V] * 3 + [I] * 8 + [V, V, V, Z, ctypes.c_int, V]
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 64, 4, 8,
                 FAKE, None, FAKE, 1 << 20, 3, None) == 2
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 48, 128, 4, 8,
                 FAKE, None, FAKE, 1 << 20, 3, None) == 2
    # supported shape, k = 0: an argument error, so the dtype itself passed
    assert _call(lib, "csa_index_topk", idx_args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 128, 4, 0,
                 FAKE, None, FAKE, 1 << 20, 3, None) == 1
    args = [V] * 6 + [I] * 9 + [ctypes.c_int, V]
    # D = 16 holds no 32-element block
    assert _call(lib, "csa_compress", args, FAKE, FAKE, None, None, None, FAKE,
                 1, 16, 16, 4, 0, 16, 0, 4, 4, 3, None) == 1
    # D = 32, empty entry range: accepted, nothing to do
    assert _call(lib, "csa_compress", args, FAKE, FAKE, None, None, None, FAKE,
                 1, 16, 32, 4, 0, 16, 2, 2, 4, 3, None) == 0
    attn = [V] * 3 + [I, V, I, V, V, I, I, V, F] + [I] * 5 + [V, V, V, Z, ctypes.c_int, V]
    assert _call(lib, "csa_sparse_attn", attn, FAKE, FAKE, FAKE, 10, FAKE, 4, None, None, 0, 0,
                 None, 0.1, 1, 1, 40, 64, 512, FAKE, None, None, 0, 3, None) == 2


def test_noalloc_rejects_rows_beyond_its_scratch(lib):
    """The allocation-free index + top-k refuses, before enqueuing anything, a
    query row whose scores and selection state exceed its static scratch."""
    lib.csa_index_topk_noalloc_max_bytes.restype = Z
    assert lib.csa_index_topk_noalloc_max_bytes() == 32 << 20
    args = [V] * 3 + [I] * 8 + [V, V, ctypes.c_int, V]
    # L = 10M entries: 40 MB of scores for one row
    assert _call(lib, "csa_index_topk_noalloc", args, FAKE, None, FAKE, 1, 1, 40_000_000, 10_000_000, 64, 128,
                 4, 1024, FAKE, None, 1, None) == 2
    # invalid arguments are still reported as such
    assert _call(lib, "csa_index_topk_noalloc", args, FAKE, None, FAKE, 1, 1, 100, 25, 64, 128, 4, 0,
                 FAKE, None, 1, None) == 1
    # batch 0: nothing to do
    assert _call(lib, "csa_index_topk_noalloc", args, None, None, None, 0, 1, 100, 25, 64, 128, 4, 8,
                 None, None, 1, None) == 0


def test_time_next_scan_takes_both_events_or_neither(lib):
    """The scan-timing request needs an event pair; NULL, NULL clears it and
    enqueues nothing (no GPU needed)."""
    args = [V, V]
    assert _call(lib, "csa_time_next_scan", args, FAKE, None) == 1
    assert _call(lib, "csa_time_next_scan", args, None, FAKE) == 1
    assert _call(lib, "csa_time_next_scan", args, None, None) == 0
