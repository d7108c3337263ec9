"""Empty and degenerate inputs on the GPU, against the oracle where it has
values: batch 0, rows that see no compressed entry, an empty cache, k above
the visible count, attention over no selected row (-1 indices only, no
window) with and without a sink, and dense attention with nothing visible but
the window."""
import numpy as np
import pytest
import torch

import oracle
from helpers import BF16_TOL, both, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:  # collected on the CPU, skipped by the marker selection
    csa = None

BF = torch.bfloat16


def test_batch_zero_is_a_no_op_everywhere():
    q = torch.zeros((0, 1, 64, 128), dtype=BF, device="cuda")
    k = torch.zeros((0, 50, 128), dtype=BF, device="cuda")
    idx = csa.csa_index_topk(q, k, 4, 16, n_ctx=200)
    assert idx.shape == (0, 1, 16)
    sc = csa.csa_index_score(q, k, 4, n_ctx=200)
    assert sc.shape == (0, 1, 50)
    qa = torch.zeros((0, 1, 64, 512), dtype=BF, device="cuda")
    kc = torch.zeros((0, 50, 512), dtype=BF, device="cuda")
    ii = torch.zeros((0, 1, 8), dtype=torch.int32, device="cuda")
    assert csa.csa_sparse_attn(qa, kc, kc, ii, n_ctx=200).shape == (0, 1, 64, 512)
    assert csa.hca_dense_attn(qa, kc, kc, 4, n_ctx=200).shape == (0, 1, 64, 512)
    torch.cuda.synchronize()


@pytest.mark.parametrize("L", [0, 300])
def test_index_rows_with_nothing_visible_and_k_above_visible(L):
    """Queries at t < m see no entry (all -1, scores -inf); later ones see
    fewer than k entries (all of them, ascending, then -1)."""
    B, T, HI, dI, m, k = 1, 12, 64, 128, 4, 64
    n_ctx = 12
    q, q_c = both((B, T, HI, dI), 5, "q_idx", dtype=BF, scale=dI ** -0.5)
    Lr = max(L, 1)
    kk, k_c = both((B, Lr, dI), 5, "k_idx", dtype=BF, scale=dI ** -0.5)
    kk, k_c = kk[:, :L].contiguous(), k_c[:, :L]
    got = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    sc = to_np(csa.csa_index_score(q, kk, m, n_ctx=n_ctx))
    for t in range(T):
        nv = min(L, t // m)
        want = np.full(k, -1)
        want[:nv] = np.arange(nv)
        assert np.array_equal(got[0, t], want), t
        assert np.all(np.isneginf(sc[0, t, nv:]))
    if L:
        w_idx, _ = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
        assert np.array_equal(got, w_idx)


@pytest.mark.parametrize("use_sink", [True, False])
def test_sparse_attn_over_no_row(use_sink):
    """Only -1 indices and no window: with a sink the output is 0 and lse the
    sink logit; without one the output is 0 and lse -inf (no mass at all)."""
    B, T, H, d, L, k = 1, 2, 64, 512, 40, 32
    n_ctx = 4 * L
    q, q_c = both((B, T, H, d), 6, "q", dtype=BF, scale=d ** -0.5)
    kc, kc_c = both((B, L, d), 6, "kc", dtype=BF, scale=d ** -0.5)
    vc, vc_c = both((B, L, d), 6, "vc", dtype=BF, scale=d ** -0.5)
    sk, sk_c = both((H,), 6, "sink", dtype=torch.float32)
    idx = torch.full((B, T, k), -1, dtype=torch.int32, device="cuda")
    out, lse = csa.csa_sparse_attn(q, kc, vc, idx, W=0, sink=sk if use_sink else None, n_ctx=n_ctx,
                                   want_lse=True)
    torch.cuda.synchronize()
    o_w, l_w = oracle.sparse_attn(q_c, kc_c, vc_c, np.full((B, T, k), -1), None, None, 0,
                                  sink=sk_c if use_sink else None, n_ctx=n_ctx)
    assert np.all(to_np(out) == 0.0) and np.all(o_w == 0.0)
    lg = to_np(lse)
    if use_sink:
        assert np.max(np.abs(lg - l_w)) <= 1e-5 and np.max(np.abs(lg[0, 0] - sk_c)) <= 1e-5
    else:
        assert np.all(np.isneginf(lg)) and np.all(np.isneginf(l_w))


def test_dense_attn_with_only_the_window_visible():
    """n_ctx < m: no compressed entry is visible, the raw window carries all
    the mass (equals the oracle, and the sparse kernel with no index)."""
    B, T, H, d, m, W = 2, 1, 64, 512, 128, 64
    n_ctx = 100
    L = 1
    R = T + W - 1
    q, q_c = both((B, T, H, d), 8, "q", dtype=BF, scale=d ** -0.5)
    kc, kc_c = both((B, L, d), 8, "kc", dtype=BF, scale=d ** -0.5)
    vc, vc_c = both((B, L, d), 8, "vc", dtype=BF, scale=d ** -0.5)
    kr, kr_c = both((B, R, d), 8, "kr", dtype=BF, scale=d ** -0.5)
    vr, vr_c = both((B, R, d), 8, "vr", dtype=BF, scale=d ** -0.5)
    sk, sk_c = both((H,), 8, "sink", dtype=torch.float32)
    out = csa.hca_dense_attn(q, kc, vc, m, kr=kr, vr=vr, W=W, sink=sk, n_ctx=n_ctx)
    idx = torch.full((B, T, 8), -1, dtype=torch.int32, device="cuda")
    out2 = csa.csa_sparse_attn(q, kc, vc, idx, kr=kr, vr=vr, W=W, sink=sk, n_ctx=n_ctx)
    torch.cuda.synchronize()
    o_w, _ = oracle.dense_attn(q_c, kc_c, vc_c, m, kr_c, vr_c, W, sink=sk_c, n_ctx=n_ctx)
    assert np.max(np.abs(to_np(out) - o_w)) <= BF16_TOL
    assert np.max(np.abs(to_np(out2) - to_np(out))) <= 4e-3
