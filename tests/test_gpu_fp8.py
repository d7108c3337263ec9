"""GPU parity of the FP8 (OCP E4M3) storage paths against the oracle.

The pages let the indexer's q.k path and the main KV run in low precision
(shareware.cn Hybrid Attention article, its list of what is compressed);
CSA_FP8 is the E4M3 reading of that.  Inputs are generated on each device by
``synthetic`` (E4M3 by round-to-nearest-even from the same fp32 values) and
decoded for the oracle by the oracle's own E4M3 decoder."""
import numpy as np
import pytest
import torch

import oracle
from helpers import BF16_TOL, both, fp8_ulp, gen, index_eps_fp8, near_tie_check, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:  # collected on the CPU, skipped by the marker selection
    csa = None

F8 = torch.float8_e4m3fn


def test_generator_is_bit_identical_on_both_devices_fp8():
    import synthetic as syn
    for kind, scale in (("normal", 128 ** -0.5), ("normal", 3.0), ("uniform", 1.0), ("grid", 2.0 ** -4)):
        a = syn.make((3, 1000, 72), 9, 4, dtype=F8, device="cuda", kind=kind, scale=scale)
        b = syn.make((3, 1000, 72), 9, 4, dtype=F8, device="cpu", kind=kind, scale=scale)
        assert torch.equal(a.cpu().view(torch.uint8), b.view(torch.uint8))


# ---------------------------------------------------------------------------
# compression with FP8 storage: fp32 arithmetic, output rounded to E4M3
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m,D,two", [(1003, 4, 128, True), (1003, 4, 512, False), (1000, 128, 512, False),
                                       (77, 128, 64, False), (40, 4, 32, True)])
def test_compress_fp8_within_one_ulp_of_oracle(n, m, D, two):
    """The exact (fp64) compressed value and the GPU's E4M3 output differ by
    at most one E4M3 step: the GPU rounds its fp32 result to nearest, and the
    fp32 arithmetic may move a value across a rounding midpoint."""
    seed = 300 + n + D
    B = 2
    xa, xa_c = both((B, n, D), seed, "k_idx", dtype=F8, scale=D ** -0.5)
    za, za_c = both((B, n, D), seed, "z_idx", dtype=F8, scale=0.5)
    kw, kw_c = {}, {}
    if two:
        xb, xb_c = both((B, n, D), seed, "xb_idx", dtype=F8, scale=D ** -0.5)
        zb, zb_c = both((B, n, D), seed, "zb_idx", dtype=F8, scale=0.5)
        kw, kw_c = dict(x_b=xb, z_b=zb), dict(x_b=xb_c, z_b=zb_c)
    got = csa.csa_compress(xa, za, m, **kw)
    torch.cuda.synchronize()
    assert got.dtype == F8
    want = oracle.compress(xa_c, za_c, m, **kw_c)
    g = to_np(got)
    assert g.shape == want.shape
    assert np.all(np.abs(g - want) <= fp8_ulp(want) * (1 + 1e-9))
    # and most outputs are the nearest E4M3 value of the exact result
    assert np.mean(g == oracle.fp8_decode(oracle.fp8_encode(want))) > 0.97


def test_compress_fp8_decode_refresh_equals_bulk():
    B, n, D, m = 2, 128 * 40, 128, 128
    x = gen((B, n, D), 5, "k_idx", dtype=F8, device="cuda", scale=D ** -0.5)
    z = gen((B, n, D), 5, "z_idx", dtype=F8, device="cuda", scale=0.5)
    bulk = csa.hca_compress(x, z, m)
    L = n // m
    slot = torch.zeros((B, 1, D), dtype=F8, device="cuda")
    p0 = n - m
    csa.hca_compress(x[:, p0:].contiguous(), z[:, p0:].contiguous(), m, n=n, p0=p0, e0=L - 1, e1=L, out=slot,
                     out_ld=1)
    torch.cuda.synchronize()
    # the single-entry launch slices each block over 16 lanes: same value within one E4M3 step
    a, b = to_np(slot[:, 0]), to_np(bulk[:, L - 1])
    assert np.all(np.abs(a - b) <= fp8_ulp(b) * (1 + 1e-9))


# ---------------------------------------------------------------------------
# indexer scores and top-k with FP8 q and k
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("HI", [64, 32, 16, 128])
def test_index_scores_fp8_match_oracle(HI):
    B, T, m, dI = 2, 3, 4, 128
    n_ctx = 4 * 3001 + 2
    L = -(-n_ctx // m)
    seed = 500 + HI
    q, q_c = both((B, T, HI, dI), seed, "q_idx", dtype=F8, scale=dI ** -0.5)
    k, k_c = both((B, L, dI), seed, "k_idx", dtype=F8, scale=dI ** -0.5)
    w, w_c = both((B, T, HI), seed, "w_idx", dtype=torch.float32, kind="uniform")
    got = to_np(csa.csa_index_score(q, k, m, w_idx=w, n_ctx=n_ctx))
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.all(np.isneginf(got[~fin]))
    for b in range(B):
        for t in range(T):
            eps = index_eps_fp8(q_c[b, t], w_c[b, t], k_c[b])
            f = fin[b, t]
            assert np.all(np.abs(got[b, t][f] - want[b, t][f]) <= eps[f] + 1e-30)


def test_index_fp8_exact_on_grid_inputs():
    """Grid values k/16 (|k| <= 8, exact in E4M3) and weights in {1, 2}: every
    partial sum has at most 11 significant bits, so the scores and the top-k
    are exact, whatever the MFMA's internal summation precision."""
    B, T, HI, dI, m, k = 2, 2, 64, 128, 4, 256
    n_ctx = 4 * 6000 + 3
    L = -(-n_ctx // m)
    q, q_c = both((B, T, HI, dI), 19, "q_idx", dtype=F8, kind="grid", scale=2.0 ** -4)
    kk, k_c = both((B, L, dI), 19, "k_idx", dtype=F8, kind="grid", scale=2.0 ** -4)
    w = gen((B, T, HI), 19, "w_idx", dtype=torch.float32, device="cuda", kind="grid", grid=1).abs() + 1.0
    w_c = (gen((B, T, HI), 19, "w_idx", dtype=torch.float32, device="cpu", kind="grid", grid=1).abs()
           + 1.0).double().numpy()
    got = to_np(csa.csa_index_score(q, kk, m, w_idx=w, n_ctx=n_ctx))
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    assert np.array_equal(got, want)
    idx = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_ctx).cpu().numpy()
    widx, _ = oracle.index_topk(q_c, k_c, m, k, w=w_c, n_ctx=n_ctx)
    assert np.array_equal(idx, widx)


@pytest.mark.parametrize("HI,grid", [(64, False), (32, False), (64, True)])
def test_index_fp8_prefill_rows_equal_single_rows_and_oracle(HI, grid):
    """64 query rows of one sequence (the 16-row prefill kernel) give, row by
    row, the bits of the same query scored alone (the streaming scan), match
    the oracle within the fp8 summation bound (exactly on grid inputs), and
    csa_index_topk keeps the oracle's selection of those scores."""
    B, T, dI, m, k = 1, 64, 128, 4, 256
    n_ctx = 4 * 5000 + 1  # three 1920-key parts; the rows' visible counts differ
    L = -(-n_ctx // m)
    seed = 700 + HI
    kw = dict(kind="grid", scale=2.0 ** -4) if grid else dict(scale=dI ** -0.5)
    q, q_c = both((B, T, HI, dI), seed, "q_idx", dtype=F8, **kw)
    kk, k_c = both((B, L, dI), seed, "k_idx", dtype=F8, **kw)
    if grid:
        w = gen((B, T, HI), seed, "w_idx", dtype=torch.float32, device="cuda", kind="grid", grid=1).abs() + 1.0
        w_c = (gen((B, T, HI), seed, "w_idx", dtype=torch.float32, device="cpu", kind="grid", grid=1).abs()
               + 1.0).double().numpy()
    else:
        w, w_c = both((B, T, HI), seed, "w_idx", dtype=torch.float32, scale=HI ** -0.5)
    got = to_np(csa.csa_index_score(q, kk, m, w_idx=w, n_ctx=n_ctx))
    for t in range(T):
        one = csa.csa_index_score(q[:, t:t + 1].contiguous(), kk, m, w_idx=w[:, t:t + 1].contiguous(),
                                  n_ctx=n_ctx - T + 1 + t)
        assert np.array_equal(got[:, t], to_np(one)[:, 0]), t
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    if grid:
        assert np.array_equal(got, want)
    else:
        for t in range(T):
            eps = index_eps_fp8(q_c[0, t], w_c[0, t], k_c[0])
            f = fin[0, t]
            assert np.all(np.abs(got[0, t][f] - want[0, t][f]) <= eps[f] + 1e-30), t
    idx = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_ctx).cpu().numpy()
    nv = np.minimum((n_ctx - T + np.arange(T)) // m, L)
    assert np.array_equal(idx, oracle.topk(got.astype(np.float64), np.broadcast_to(nv, (B, T)), k))


@pytest.mark.parametrize("B,T,L,HI,k,wts", [(16, 1, 250000, 64, 1024, True), (4, 3, 9000, 32, 512, False),
                                             (2, 2, 700, 64, 1024, True), (2, 8, 30000, 16, 256, False),
                                             (4, 4, 60000, 128, 2048, True), (1, 1, 250000, 64, 1024, True),
                                             (8, 1, 32768, 64, 1024, False), (4, 1, 250000, 64, 1024, True),
                                             (2, 1, 250000, 32, 1024, False)])
def test_index_topk_fp8_single_pass_equals_score_then_select(B, T, L, HI, k, wts):
    """The fused scan-and-select path on FP8 keys gives the same indices and
    scores, bit for bit, as the scores written out and selected by the
    stand-alone top-k; one row is also checked against the oracle (exact up
    to certified near ties)."""
    dI, m = 128, 4
    n_ctx = m * L
    seed = 600 + L
    q, q_c = both((B, T, HI, dI), seed, "q_idx", dtype=F8, scale=dI ** -0.5)
    kk, k_c = both((B, L, dI), seed, "k_idx", dtype=F8, scale=dI ** -0.5)
    w = w_c = None
    if wts:
        w, w_c = both((B, T, HI), seed, "w_idx", dtype=torch.float32, scale=HI ** -0.5)
    idx1, s1 = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_ctx, want_scores=True)
    sc = csa.csa_index_score(q, kk, m, w_idx=w, n_ctx=n_ctx)
    idx2, s2 = csa.csa_topk_select(sc, m, k, n_ctx=n_ctx, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    b, t = B - 1, T - 1
    nv = min(L, (n_ctx - T + t) // m)
    want, osc = oracle.index_topk(q_c[b:b + 1, t:t + 1], k_c[b:b + 1], m, k, n_ctx=n_ctx,
                                  tpos=np.array([n_ctx - T + t]), w=None if w_c is None else w_c[b:b + 1, t:t + 1])
    eps = index_eps_fp8(q_c[b, t], None if w_c is None else w_c[b, t], k_c[b])[:nv]
    assert near_tie_check(idx1[b, t].cpu().numpy(), want[0, 0], osc[0, 0], nv, k, eps) <= 4


def test_index_topk_fp8_gaussian_exact_up_to_near_ties():
    B, T, m, HI, dI, k = 2, 3, 4, 64, 128, 1024
    n_ctx = 4 * 20000 + 1
    L = -(-n_ctx // m)
    q, q_c = both((B, T, HI, dI), 23, "q_idx", dtype=F8, scale=dI ** -0.5)
    kk, k_c = both((B, L, dI), 23, "k_idx", dtype=F8, scale=dI ** -0.5)
    got = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    want, sc = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    ties = 0
    for b in range(B):
        for t in range(T):
            nv = min(L, (n_ctx - T + t) // m)
            ties += near_tie_check(got[b, t], want[b, t], sc[b, t], nv, k,
                                   index_eps_fp8(q_c[b, t], None, k_c[b])[:nv])
    assert ties <= 6


# ---------------------------------------------------------------------------
# attention over an FP8 K/V cache (bf16 query and output)
# ---------------------------------------------------------------------------

def _attn_fp8_inputs(B, T, H, d, L, R, seed, kv_scale):
    q, q_c = both((B, T, H, d), seed, "q", dtype=torch.bfloat16, scale=d ** -0.5)
    kc, kc_c = both((B, L, d), seed, "kc", dtype=F8, scale=kv_scale)
    vc, vc_c = both((B, L, d), seed, "vc", dtype=F8, scale=kv_scale)
    kr, kr_c = both((B, R, d), seed, "kr", dtype=F8, scale=kv_scale)
    vr, vr_c = both((B, R, d), seed, "vr", dtype=F8, scale=kv_scale)
    sk, sk_c = both((H,), seed, "sink", dtype=torch.float32)
    return (q, kc, vc, kr, vr, sk), (q_c, kc_c, vc_c, kr_c, vr_c, sk_c)


# kv_scale 1/sqrt(d): K/V values as stored by the bf16 workloads (many E4M3
# subnormals); kv_scale 1: unit-scale codes with the K scale folded into the
# softmax scale (scale = 1/d), the way a per-tensor FP8 scale is applied.
@pytest.mark.parametrize("B,T,L,k,W,kv_scale,use_sink", [
    (2, 1, 4000, 1024, 128, 512 ** -0.5, True),
    (1, 3, 300, 100, 7, 1.0, False),
    (2, 2, 900, 64, 0, 1.0, True),
    (1, 40, 500, 64, 16, 512 ** -0.5, True),
    (1, 520, 300, 64, 16, 1.0, True),
])
def test_sparse_attn_fp8_matches_oracle(B, T, L, k, W, kv_scale, use_sink):
    import synthetic as syn
    H, d, m = 64, 512, 4
    n_ctx = L * m
    R = T + max(W, 1) - 1
    g, c = _attn_fp8_inputs(B, T, H, d, L, R, 53 + T, kv_scale)
    q, kc, vc, kr, vr, sk = g
    q_c, kc_c, vc_c, kr_c, vr_c, sk_c = c
    scale = d ** -0.5 if kv_scale != 1.0 else 1.0 / d
    tpos = np.arange(n_ctx - T, n_ctx)
    nv = np.minimum(tpos // m, L)
    idx_c = syn.sample_indices(9, syn.TID["idx"], B * T, k, np.tile(nv, B) - 3).reshape(B, T, k)
    idx = idx_c.cuda()
    out, lse = csa.csa_sparse_attn(q, kc, vc, idx, kr=kr if W else None, vr=vr if W else None, W=W,
                                   sink=sk if use_sink else None, scale=scale, n_ctx=n_ctx, want_lse=True)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    o_w, l_w = oracle.sparse_attn(q_c, kc_c, vc_c, idx_c.numpy(), kr_c, vr_c, W,
                                  sink=sk_c if use_sink else None, scale=scale, n_ctx=n_ctx)
    assert np.max(np.abs(to_np(out) - o_w)) <= BF16_TOL
    assert np.max(np.abs(to_np(lse) - l_w)) <= 1e-3


@pytest.mark.parametrize("B,T,L,m,W,kv_scale", [
    (2, 1, 3000, 128, 0, 512 ** -0.5),
    (1, 2, 700, 4, 128, 1.0),
    (1, 40, 100, 4, 16, 512 ** -0.5),
    (1, 1, 7813, 128, 128, 1.0),
])
def test_dense_attn_fp8_matches_oracle(B, T, L, m, W, kv_scale):
    H, d = 64, 512
    n_ctx = L * m - (m // 2)
    R = T + max(W, 1) - 1
    g, c = _attn_fp8_inputs(B, T, H, d, L, R, 61 + L, kv_scale)
    q, kc, vc, kr, vr, sk = g
    q_c, kc_c, vc_c, kr_c, vr_c, sk_c = c
    scale = d ** -0.5 if kv_scale != 1.0 else 1.0 / d
    out, lse = csa.hca_dense_attn(q, kc, vc, m, kr=kr if W else None, vr=vr if W else None, W=W, sink=sk,
                                  scale=scale, n_ctx=n_ctx, want_lse=True)
    torch.cuda.synchronize()
    o_w, l_w = oracle.dense_attn(q_c, kc_c, vc_c, m, kr_c, vr_c, W, sink=sk_c, scale=scale, n_ctx=n_ctx)
    assert np.max(np.abs(to_np(out) - o_w)) <= BF16_TOL
    assert np.max(np.abs(to_np(lse) - l_w)) <= 1e-3


@pytest.mark.parametrize("sparse,T", [(True, 1), (True, 24), (False, 1), (False, 24)])
def test_attn_fp8_equals_bf16_path_on_the_same_values(sparse, T):
    """Every E4M3 code is a bf16 value, and the FP8 kernels convert before the
    same MFMA sequence: on the bf16 copy of the same cache the bf16 kernels
    must give bit-identical outputs and lse."""
    import synthetic as syn
    B, H, d, L, m, k, W = 2, 64, 512, 1200, 4, 256, 128
    n_ctx = L * m
    R = T + W - 1
    g, _ = _attn_fp8_inputs(B, T, H, d, L, R, 71, 1.0)
    q, kc, vc, kr, vr, sk = g
    up = [x.to(torch.bfloat16) for x in (kc, vc, kr, vr)]
    nv = np.minimum(np.arange(n_ctx - T, n_ctx) // m, L)
    idx = syn.sample_indices(5, syn.TID["idx"], B * T, k, np.tile(nv, B)).reshape(B, T, k).cuda()
    if sparse:
        f = lambda kc_, vc_, kr_, vr_: csa.csa_sparse_attn(q, kc_, vc_, idx, kr=kr_, vr=vr_, W=W, sink=sk,
                                                           scale=1.0 / d, n_ctx=n_ctx, want_lse=True)
    else:
        f = lambda kc_, vc_, kr_, vr_: csa.hca_dense_attn(q, kc_, vc_, m, kr=kr_, vr=vr_, W=W, sink=sk,
                                                          scale=1.0 / d, n_ctx=n_ctx, want_lse=True)
    o8, l8 = f(kc, vc, kr, vr)
    o16, l16 = f(*up)
    torch.cuda.synchronize()
    assert torch.equal(o8.view(torch.int16), o16.view(torch.int16))
    assert torch.equal(l8, l16)


def test_attn_fp8_shape_and_query_checks():
    B, T, H, d, L, k, W = 1, 1, 64, 256, 100, 8, 4
    q = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, L, d), dtype=F8, device="cuda")
    idx = torch.zeros((B, T, k), dtype=torch.int32, device="cuda")
    kr = torch.zeros((B, W, d), dtype=F8, device="cuda")
    with pytest.raises(csa.CsaError, match="UNSUPPORTED"):  # FP8 K/V needs d = 512
        csa.csa_sparse_attn(q, kc, kc, idx, kr=kr, vr=kr, W=W, n_ctx=4 * L)
    with pytest.raises(TypeError):  # an FP8 cache takes a bf16 query
        csa.csa_sparse_attn(q.to(F8), kc, kc, idx, kr=kr, vr=kr, W=W, n_ctx=4 * L)
