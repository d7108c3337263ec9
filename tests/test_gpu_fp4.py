"""GPU parity of the MXFP4 indexer (q^I and k^I as OCP MXFP4) against the oracle.

The pages run the indexer's q.k in FP4 (shareware.cn Hybrid Attention
article, its list of what is compressed); MXFP4 is the reading taken: E2M1
codes with one E8M0 scale per 32 elements.  Inputs are random codes and
scales drawn by ``synthetic`` on each device and decoded for the oracle by its
own MXFP4 decoder.  With unit scales every product is a multiple of 1/4 below
37, so per-head sums, their ReLU and the head sum stay exact in fp32 (at most
21 significant bits): scores and top-k are then compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from helpers import both, index_eps, near_tie_check, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:  # collected on the CPU, skipped by the marker selection
    csa = None


def mx_both(shape, seed, name, lo=127, hi=127):
    """The same MXFP4 tensor generated on the GPU (as the binding's MXFP4) and
    on the CPU (decoded by the oracle to float64)."""
    import synthetic as syn
    n = int(np.prod(shape))
    nb = n // 2 + n // 32
    g = syn.mxfp4_(torch.empty(nb, dtype=torch.uint8, device="cuda"), seed, syn.TID[name], n,
                   scale_lo=lo, scale_hi=hi)
    c = syn.mxfp4_(torch.empty(nb, dtype=torch.uint8), seed, syn.TID[name], n, scale_lo=lo, scale_hi=hi)
    return csa.MXFP4(g, shape), oracle.mxfp4_decode(c.numpy(), shape)


def test_mxfp4_generator_is_bit_identical_on_both_devices():
    import synthetic as syn
    n = 37 * 128
    a = syn.mxfp4_(torch.empty(n // 2 + n // 32, dtype=torch.uint8, device="cuda"), 5, 6, n, scale_lo=120,
                   scale_hi=133)
    b = syn.mxfp4_(torch.empty(n // 2 + n // 32, dtype=torch.uint8), 5, 6, n, scale_lo=120, scale_hi=133)
    assert torch.equal(a.cpu(), b)


@pytest.mark.parametrize("HI", [64, 16, 128])
def test_index_scores_mxfp4_exact_with_unit_scales(HI):
    B, T, m, dI = 2, 3, 4, 128
    n_ctx = 4 * 3001 + 2
    L = -(-n_ctx // m)
    q, q_c = mx_both((B, T, HI, dI), 700 + HI, "q_idx")
    k, k_c = mx_both((B, L, dI), 700 + HI, "k_idx")
    got = to_np(csa.csa_index_score(q, k, m, n_ctx=n_ctx))
    want = oracle.index_scores(q_c, k_c, m, n_ctx=n_ctx)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("HI", [64, 32])
def test_index_scores_mxfp4_scaled_and_weighted_match_oracle(HI):
    """Scales 2^-2 .. 2^2 and fp32 head weights: within the fp32 accumulation
    bound of the head sum."""
    B, T, m, dI = 2, 2, 4, 128
    n_ctx = 4 * 2500 + 3
    L = -(-n_ctx // m)
    q, q_c = mx_both((B, T, HI, dI), 800 + HI, "q_idx", 125, 129)
    k, k_c = mx_both((B, L, dI), 800 + HI, "k_idx", 125, 129)
    w, w_c = both((B, T, HI), 800 + HI, "w_idx", dtype=torch.float32, kind="uniform")
    got = to_np(csa.csa_index_score(q, k, m, w_idx=w, n_ctx=n_ctx))
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    for b in range(B):
        for t in range(T):
            eps = index_eps(q_c[b, t], w_c[b, t], k_c[b])
            f = fin[b, t]
            assert np.all(np.abs(got[b, t][f] - want[b, t][f]) <= eps[f] + 1e-30)


def test_index_topk_mxfp4_exact_with_unit_scales():
    B, T, HI, dI, m, k = 2, 2, 64, 128, 4, 256
    n_ctx = 4 * 6000 + 3
    L = -(-n_ctx // m)
    q, q_c = mx_both((B, T, HI, dI), 31, "q_idx")
    kk, k_c = mx_both((B, L, dI), 31, "k_idx")
    idx = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    widx, _ = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    assert np.array_equal(idx, widx)


@pytest.mark.parametrize("B,T,L,HI,k,lo,hi", [(16, 1, 250000, 64, 1024, 125, 129), (4, 3, 9000, 32, 512, 127, 127),
                                              (2, 2, 700, 64, 1024, 120, 133), (4, 4, 60000, 128, 2048, 125, 129),
                                              (1, 1, 250000, 64, 1024, 125, 129), (4, 1, 250000, 64, 1024, 125, 129)])
def test_index_topk_mxfp4_single_pass_equals_score_then_select(B, T, L, HI, k, lo, hi):
    """Fused scan-and-select on MXFP4 keys == scores written out and selected
    by the stand-alone top-k, bit for bit; one row against the oracle (exact
    up to certified near ties)."""
    dI, m = 128, 4
    n_ctx = m * L
    q, q_c = mx_both((B, T, HI, dI), 900 + L, "q_idx", lo, hi)
    kk, k_c = mx_both((B, L, dI), 900 + L, "k_idx", lo, hi)
    idx1, s1 = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx, want_scores=True)
    sc = csa.csa_index_score(q, kk, m, n_ctx=n_ctx)
    idx2, s2 = csa.csa_topk_select(sc, m, k, n_ctx=n_ctx, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    b, t = B - 1, T - 1
    nv = min(L, (n_ctx - T + t) // m)
    want, osc = oracle.index_topk(q_c[b:b + 1, t:t + 1], k_c[b:b + 1], m, k, n_ctx=n_ctx,
                                  tpos=np.array([n_ctx - T + t]))
    eps = index_eps(q_c[b, t], None, k_c[b])[:nv]
    assert near_tie_check(idx1[b, t].cpu().numpy(), want[0, 0], osc[0, 0], nv, k, eps) <= 2


@pytest.mark.parametrize("scaled", [False, True])
def test_index_mxfp4_prefill_rows_equal_single_rows_and_oracle(scaled):
    """64 query rows of one sequence (the 16-row prefill kernel) give, row by
    row, the bits of the same query scored alone (the streaming scan); with
    unit scales they equal the oracle exactly, with scales 2^-2 .. 2^2 and fp32
    head weights within the summation bound; csa_index_topk keeps the oracle's
    selection of those scores."""
    B, T, HI, dI, m, k = 1, 64, 64, 128, 4, 256
    n_ctx = 4 * 5000 + 1  # three 1920-key parts; the rows' visible counts differ
    L = -(-n_ctx // m)
    lo, hi = (125, 129) if scaled else (127, 127)
    q, q_c = mx_both((B, T, HI, dI), 900 + scaled, "q_idx", lo, hi)
    kk, k_c = mx_both((B, L, dI), 900 + scaled, "k_idx", lo, hi)
    w = w_c = None
    if scaled:
        w, w_c = both((B, T, HI), 900, "w_idx", dtype=torch.float32, kind="uniform")
    got = to_np(csa.csa_index_score(q, kk, m, w_idx=w, n_ctx=n_ctx))
    ncode = T * HI * dI // 2
    for t in range(T):  # row t as its own one-query MXFP4 tensor: its codes, then its scales
        codes = q.data[t * HI * dI // 2:(t + 1) * HI * dI // 2]
        scales = q.data[ncode + t * HI * dI // 32:ncode + (t + 1) * HI * dI // 32]
        qt = csa.MXFP4(torch.cat([codes, scales]).contiguous(), (1, 1, HI, dI))
        one = csa.csa_index_score(qt, kk, m, w_idx=None if w is None else w[:, t:t + 1].contiguous(),
                                  n_ctx=n_ctx - T + 1 + t)
        assert np.array_equal(got[:, t], to_np(one)[:, 0]), t
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    if not scaled:
        assert np.array_equal(got, want)
    else:
        for t in range(T):
            eps = index_eps(q_c[0, t], w_c[0, t], k_c[0])
            f = fin[0, t]
            assert np.all(np.abs(got[0, t][f] - want[0, t][f]) <= eps[f] + 1e-30), t
    idx = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_ctx).cpu().numpy()
    nv = np.minimum((n_ctx - T + np.arange(T)) // m, L)
    assert np.array_equal(idx, oracle.topk(got.astype(np.float64), np.broadcast_to(nv, (B, T)), k))
