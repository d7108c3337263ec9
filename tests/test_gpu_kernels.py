"""GPU parity of each kernel against the fp64 oracle on small seeded inputs
that span several tiles and a ragged tail, plus edge cases.

Inputs are generated independently on each device by ``synthetic`` (bit-
identical), never copied from the GPU to the oracle."""
import numpy as np
import pytest
import torch

import oracle
from helpers import BF16_TOL, F32_TOL, both, gen, index_eps, max_abs, near_tie_check, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:  # collected on the CPU, skipped by the marker selection
    csa = None

DT = {"bf16": torch.bfloat16, "f32": torch.float32}
TOL = {"bf16": BF16_TOL, "f32": F32_TOL}


# ---------------------------------------------------------------------------
# compression
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n,m,D,two", [(1003, 4, 512, True), (1003, 4, 128, False),
                                       (1000, 128, 512, False), (77, 128, 64, False),
                                       (4096, 4, 64, False), (40, 4, 32, True)])
def test_compress_matches_oracle(dt, n, m, D, two):
    seed = 100 + n + D
    B = 2
    xa, xa_c = both((B, n, D), seed, "k", dtype=DT[dt], scale=D ** -0.5)
    za, za_c = both((B, n, D), seed, "z_k", dtype=DT[dt], scale=0.5)
    bias = bias_c = None
    kw, kw_c = {}, {}
    if two:
        xb, xb_c = both((B, n, D), seed, "xb_k", dtype=DT[dt], scale=D ** -0.5)
        zb, zb_c = both((B, n, D), seed, "zb_k", dtype=DT[dt], scale=0.5)
        kw, kw_c = dict(x_b=xb, z_b=zb), dict(x_b=xb_c, z_b=zb_c)
        bias, bias_c = both((2 * m, D), seed, "bias", dtype=torch.float32, scale=0.3)
    got = csa.csa_compress(xa, za, m, bias=bias, **kw)
    torch.cuda.synchronize()
    want = oracle.compress(xa_c, za_c, m, bias=bias_c, **kw_c)
    assert got.shape == want.shape
    assert max_abs(to_np(got), want) <= TOL[dt]


def test_compress_decode_slot_equals_bulk():
    # one new entry written into a cache slot from the last raw tokens only
    B, n, D, m = 3, 4096 + 8, 512, 4
    xa = gen((B, n, D), 7, "k", dtype=torch.bfloat16, device="cuda", scale=D ** -0.5)
    za = gen((B, n, D), 7, "z_k", dtype=torch.bfloat16, device="cuda", scale=0.5)
    xb = gen((B, n, D), 7, "xb_k", dtype=torch.bfloat16, device="cuda", scale=D ** -0.5)
    zb = gen((B, n, D), 7, "zb_k", dtype=torch.bfloat16, device="cuda", scale=0.5)
    bulk = csa.csa_compress(xa, za, m, x_b=xb, z_b=zb)
    L = n // m
    cache = torch.zeros((B, L + 5, D), dtype=torch.bfloat16, device="cuda")
    p0 = n - 2 * m
    tail = lambda t: t[:, p0:].contiguous()
    csa.csa_compress(tail(xa), tail(za), m, x_b=tail(xb), z_b=tail(zb), n=n, p0=p0, e0=L - 1, e1=L,
                     out=cache[:, L - 1:], out_ld=L + 5)
    torch.cuda.synchronize()
    assert torch.equal(cache[:, L - 1], bulk[:, L - 1])
    assert torch.count_nonzero(cache[:, : L - 1]) == 0 and torch.count_nonzero(cache[:, L:]) == 0


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,D,m,n", [(16, 512, 128, 1_000_000), (3, 128, 128, 5000), (2, 64, 64, 130)])
def test_compress_single_entry_decode_refresh(dt, B, D, m, n):
    # few entries with long blocks take the token-sliced path; raw rows cover
    # only the newest complete block
    e = n // m - 1
    p0 = e * m
    xs, xs_c = both((B, m, D), 3 + D, "k", dtype=DT[dt], scale=D ** -0.5)
    zs, zs_c = both((B, m, D), 3 + D, "z_k", dtype=DT[dt], scale=0.5)
    bias, bias_c = both((m, D), 3 + D, "bias", dtype=torch.float32, scale=0.3)
    got = csa.hca_compress(xs, zs, m, bias=bias, n=n, p0=p0, e0=e, e1=e + 1)
    torch.cuda.synchronize()
    want = oracle.compress(xs_c, zs_c, m, bias=bias_c, n=n, p0=p0, e0=e, e1=e + 1)
    assert max_abs(to_np(got), want) <= TOL[dt]


# ---------------------------------------------------------------------------
# indexer scores and top-k
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt,HI,dI", [("bf16", 64, 128), ("bf16", 32, 128), ("bf16", 64, 64),
                                      ("f32", 4, 32)])
def test_index_scores_match_oracle(dt, HI, dI):
    B, T, m = 2, 3, 4
    n_ctx = 4 * 3001 + 2
    L = -(-n_ctx // m)
    seed = 11 + HI + dI
    q, q_c = both((B, T, HI, dI), seed, "q_idx", dtype=DT[dt], scale=dI ** -0.5)
    k, k_c = both((B, L, dI), seed, "k_idx", dtype=DT[dt], scale=dI ** -0.5)
    w, w_c = both((B, T, HI), seed, "w_idx", dtype=torch.float32, kind="uniform")
    got = to_np(csa.csa_index_score(q, k, m, w_idx=w, n_ctx=n_ctx))
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.all(np.isneginf(got[~fin]))
    for b in range(B):
        for t in range(T):
            eps = index_eps(q_c[b, t], w_c[b, t], k_c[b])
            f = fin[b, t]
            assert np.all(np.abs(got[b, t][f] - want[b, t][f]) <= eps[f] + 1e-30)


def test_index_scores_exact_on_grid_inputs():
    # grid values k/16 (|k| <= 8) and w in {1, 2}: every fp32 partial sum is exact
    B, T, HI, dI, m = 2, 2, 64, 128, 4
    n_ctx = 4 * 2050
    L = n_ctx // m
    q, q_c = both((B, T, HI, dI), 3, "q_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    k, k_c = both((B, L, dI), 3, "k_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    w = gen((B, T, HI), 3, "w_idx", dtype=torch.float32, device="cuda", kind="grid", grid=1).abs() + 1.0
    w_c = (gen((B, T, HI), 3, "w_idx", dtype=torch.float32, device="cpu", kind="grid", grid=1).abs()
           + 1.0).double().numpy()
    got = to_np(csa.csa_index_score(q, k, m, w_idx=w, n_ctx=n_ctx))
    want = oracle.index_scores(q_c, k_c, m, w=w_c, n_ctx=n_ctx)
    assert np.array_equal(got, want)


def _seeded_scores(B, T, L, seed, device):
    """Scores with many exact ties, signed zeros and negatives."""
    s = gen((B, T, L), seed, "scores", dtype=torch.float32, device=device, kind="grid", grid=40,
            scale=0.25)
    z = gen((B, T, L), seed + 1, "scores", dtype=torch.float32, device=device, kind="uniform")
    s = torch.where((s == 0) & (z < 0.5), torch.tensor(-0.0, device=device), s)
    return s


@pytest.mark.parametrize("B,T,L,m,k", [(2, 3, 5000, 1, 64), (1, 4, 250000, 4, 1024),
                                      (3, 1, 33000, 4, 1024), (2, 5, 700, 1, 1024), (1, 2, 9000, 1, 1),
                                      # general merge (parts x min(k, 16384) > 16384 slots), staged parts
                                      (1, 2, 250000, 1, 2048),
                                      # general merge with parts and merge emitting straight to memory
                                      (1, 2, 250000, 1, 4096),
                                      # k above one part: every part kept whole, general merge
                                      (1, 2, 250000, 1, 20000),
                                      # one part, k above the LDS staging size: direct emit in both kernels
                                      (2, 2, 10000, 1, 4096),
                                      # the edges of the 8192-score parts: k = a quarter of a part (taken),
                                      # k one above (16384-score parts), 16 half parts filling the merge
                                      # tile exactly (taken), and one more (16384-score parts)
                                      (2, 2, 16384, 1, 2048), (2, 2, 16385, 1, 2049),
                                      (1, 2, 131072, 1, 1024), (1, 2, 131073, 1, 1024)])
def test_topk_select_bit_exact_on_seeded_scores(B, T, L, m, k):
    n_ctx = L * m
    sg = _seeded_scores(B, T, L, 5 + L, "cuda")
    sc = _seeded_scores(B, T, L, 5 + L, "cpu").double().numpy()
    idx, osc = csa.csa_topk_select(sg, m, k, n_ctx=n_ctx, want_scores=True)
    torch.cuda.synchronize()
    tpos = np.arange(n_ctx - T, n_ctx)
    nv = np.minimum(tpos // m, L)
    want = oracle.topk(sc, np.broadcast_to(nv, (B, T)), k)
    got = idx.cpu().numpy()
    assert np.array_equal(got, want)
    gs = osc.cpu().double().numpy()
    for b in range(B):
        for t in range(T):
            sel = want[b, t] >= 0
            assert np.array_equal(gs[b, t][sel], sc[b, t][want[b, t][sel]])
            assert np.all(np.isneginf(gs[b, t][~sel]))


def _structured(s, pattern):
    """Periodic structure that defeats a sampled threshold estimate (the
    samples sit at fixed offsets of each thread's entries), so the exact
    selection has to fall back to all keys, or sees a skewed survivor set."""
    pos = torch.arange(s.shape[-1], device=s.device)
    if pattern == "boost32":    # every 32nd entry far above the rest
        return s + 8.0 * (pos % 32 == 0).to(s.dtype)
    if pattern == "sink16":     # every 16th entry far below the rest
        return s - 8.0 * (pos % 16 == 0).to(s.dtype)
    if pattern == "steps":      # a handful of levels, long runs of exact ties
        return torch.floor(s * 2.0) + (pos % 3 == 0).to(s.dtype)
    if pattern == "ramp":       # increasing with the index, tiny noise
        return pos.to(s.dtype) * 1e-3 + s * 1e-6
    raise ValueError(pattern)


@pytest.mark.parametrize("pattern", ["boost32", "sink16", "steps", "ramp"])
@pytest.mark.parametrize("L,k", [(250000, 1024), (40000, 2048), (20000, 64), (250000, 2048), (10000, 4096)])
def test_topk_select_exact_on_structured_scores(pattern, L, k):
    B, T, m = 2, 2, 1
    n_ctx = L * m
    sg = _structured(gen((B, T, L), 70 + L, "scores", dtype=torch.float32, device="cuda"), pattern)
    sc = _structured(gen((B, T, L), 70 + L, "scores", dtype=torch.float32, device="cpu"), pattern)
    idx, osc = csa.csa_topk_select(sg, m, k, n_ctx=n_ctx, want_scores=True)
    torch.cuda.synchronize()
    nv = np.minimum(np.arange(n_ctx - T, n_ctx) // m, L)
    want = oracle.topk(sc.double().numpy(), np.broadcast_to(nv, (B, T)), k)
    assert np.array_equal(idx.cpu().numpy(), want)
    gs, sv = osc.cpu().numpy(), sc.numpy()
    for b in range(B):
        for t in range(T):
            assert np.array_equal(gs[b, t], sv[b, t][want[b, t]])


def test_index_topk_bit_exact_on_grid_inputs():
    B, T, HI, dI, m, k = 2, 2, 64, 128, 4, 256
    n_ctx = 4 * 6000 + 3
    L = -(-n_ctx // m)
    q, q_c = both((B, T, HI, dI), 9, "q_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    kk, k_c = both((B, L, dI), 9, "k_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    got = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    want, _ = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    assert np.array_equal(got, want)
    # a workspace holding one row at a time gives the same result
    ws = torch.zeros(csa.csa_index_topk_workspace(1, 1, L, HI, k), dtype=torch.uint8, device="cuda")
    got2 = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx, ws=ws).cpu().numpy()
    assert np.array_equal(got2, want)


@pytest.mark.parametrize("k", [2048, 4096])
def test_index_topk_one_row_workspace_general_merge(k):
    """csa_index_topk with a workspace of one query row at k = 2048 / 4096
    over 250,000 entries: each row is scored, then selected by the part
    kernel and the general merge (16 parts x k slots).  Grid inputs make every
    fp32 score exact, so the indices must equal the oracle's bit for bit."""
    B, T, HI, dI, m = 1, 2, 16, 128, 4
    L = 250000
    n_ctx = m * L
    q, q_c = both((B, T, HI, dI), 17, "q_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    kk, k_c = both((B, L, dI), 17, "k_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    ws = torch.zeros(csa.csa_index_topk_workspace(1, 1, L, HI, k), dtype=torch.uint8, device="cuda")
    got = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx, ws=ws).cpu().numpy()
    full = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    want, _ = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    assert np.array_equal(got, want)
    assert np.array_equal(full, want)


@pytest.mark.parametrize("B,T,L,HI,k,wts,boost", [(16, 1, 250000, 64, 1024, True, 1), (4, 3, 9000, 32, 512, False, 1),
                                                   (2, 2, 700, 64, 1024, True, 1), (4, 16, 60000, 128, 2048, True, 1),
                                                   (2, 8, 30000, 16, 256, False, 1), (4, 1, 250000, 64, 1024, True, 32),
                                                   (4, 1, 250000, 64, 1024, False, 16), (4, 1, 250000, 64, 1024, True, -1),
                                                   (3, 2, 120000, 64, 512, True, -1),
                                                   (1, 1, 250000, 64, 1024, True, 1), (1, 1, 250000, 64, 1024, False, -1),
                                                   (1, 1, 250000, 64, 1024, True, 16), (8, 1, 32768, 64, 1024, True, 1),
                                                   (8, 1, 32768, 64, 1024, True, -1), (1, 2, 200000, 32, 512, False, 1)])
def test_index_topk_single_pass_equals_score_then_select(B, T, L, HI, k, wts, boost):
    """Shapes where the indexer selects its parts' candidates itself (no score
    matrix) give the same indices and scores, bit for bit, as the scores
    written out and selected by the stand-alone top-k (rows with fewer
    visible entries than k are padded alike).  boost > 1: every boost-th key
    row is scaled by 4 (exact in bf16), a periodic structure that misleads a
    sampled threshold; boost = -1: the last sixteenth of the key rows is
    scaled by 4, so the row's top-k sits in one part (the merge cannot use the
    parts' short lists and reads the full ones).  Batch 1 and 8 rows of
    32768 have too many parts for the single-pass plan: csa_index_topk writes
    the scores with exact per-part lists and merges those (boost = 1), or,
    when the lists do not settle a row (boost = -1, 16), runs the stand-alone
    top-k on the written scores; they are checked against the oracle row."""
    dI, m = 128, 4
    n_ctx = m * L
    seed = 40 + L
    q, q_c = both((B, T, HI, dI), seed, "q_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    kk, k_c = both((B, L, dI), seed, "k_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    if boost > 1:
        kk[:, ::boost] *= 4
        k_c[:, ::boost] *= 4
    elif boost == -1:
        kk[:, L - L // 16:] *= 4
        k_c[:, L - L // 16:] *= 4
    w = w_c = None
    if wts:
        w, w_c = both((B, T, HI), seed, "w_idx", dtype=torch.float32, scale=HI ** -0.5)
    idx1, s1 = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_ctx, want_scores=True)
    sc = csa.csa_index_score(q, kk, m, w_idx=w, n_ctx=n_ctx)
    idx2, s2 = csa.csa_topk_select(sc, m, k, n_ctx=n_ctx, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    # every row: the selection over the GPU's own fp32 scores is the stable
    # sort of those scores (no near-tie allowance), and the kept scores are
    # those scores
    sc_np = sc.cpu().double().numpy()
    nv_all = np.minimum((n_ctx - T + np.arange(T)) // m, L)
    want_all = oracle.topk(sc_np, np.broadcast_to(nv_all, (B, T)), k)
    assert np.array_equal(idx1.cpu().numpy(), want_all)
    s1_np = s1.cpu().double().numpy()
    for bb in range(B):
        for tt in range(T):
            sel = want_all[bb, tt] >= 0
            assert np.array_equal(s1_np[bb, tt][sel], sc_np[bb, tt][want_all[bb, tt][sel]])
    # one row against the oracle (exact up to certified near ties)
    b, t = B - 1, T - 1
    nv = min(L, (n_ctx - T + t) // m)
    want, osc = oracle.index_topk(q_c[b:b + 1, t:t + 1], k_c[b:b + 1], m, k, n_ctx=n_ctx,
                                  tpos=np.array([n_ctx - T + t]), w=None if w_c is None else w_c[b:b + 1, t:t + 1])
    eps = index_eps(q_c[b, t], None if w_c is None else w_c[b, t], k_c[b])[:nv]
    assert near_tie_check(idx1[b, t].cpu().numpy(), want[0, 0], osc[0, 0], nv, k, eps) <= 1


@pytest.mark.parametrize("dt,HI,dI,k", [("bf16", 64, 128, 1024), ("f32", 4, 32, 64)])
def test_index_topk_gaussian_exact_up_to_near_ties(dt, HI, dI, k):
    B, T, m = 2, 3, 4
    n_ctx = 4 * 20000 + 1
    L = -(-n_ctx // m)
    q, q_c = both((B, T, HI, dI), 21, "q_idx", dtype=DT[dt], scale=dI ** -0.5)
    kk, k_c = both((B, L, dI), 21, "k_idx", dtype=DT[dt], scale=dI ** -0.5)
    got = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    sc_gpu = csa.csa_index_score(q, kk, m, n_ctx=n_ctx).cpu().double().numpy()
    want, sc = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    ties = 0
    for b in range(B):
        for t in range(T):
            nv = min(L, (n_ctx - T + t) // m)
            ties += near_tie_check(got[b, t], want[b, t], sc[b, t], nv, k,
                                   index_eps(q_c[b, t], None, k_c[b])[:nv])
    assert ties <= 1
    # the selection on the GPU's own scores is exactly their stable sort
    nv_all = np.minimum((n_ctx - T + np.arange(T)) // m, L)
    assert np.array_equal(got, oracle.topk(sc_gpu, np.broadcast_to(nv_all, (B, T)), k))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _attn_inputs(dt, B, T, H, d, L, R, seed):
    q, q_c = both((B, T, H, d), seed, "q", dtype=DT[dt], scale=d ** -0.5)
    kc, kc_c = both((B, L, d), seed, "kc", dtype=DT[dt], scale=d ** -0.5)
    vc, vc_c = both((B, L, d), seed, "vc", dtype=DT[dt], scale=d ** -0.5)
    kr, kr_c = both((B, R, d), seed, "kr", dtype=DT[dt], scale=d ** -0.5)
    vr, vr_c = both((B, R, d), seed, "vr", dtype=DT[dt], scale=d ** -0.5)
    sk, sk_c = both((H,), seed, "sink", dtype=torch.float32)
    return (q, kc, vc, kr, vr, sk), (q_c, kc_c, vc_c, kr_c, vr_c, sk_c)


@pytest.mark.parametrize("dt,B,T,H,d,L,k,W,use_sink", [
    ("bf16", 2, 1, 64, 512, 4000, 1024, 128, True),
    ("bf16", 1, 3, 64, 256, 300, 100, 7, False),
    ("bf16", 2, 2, 128, 128, 900, 64, 0, True),
    ("bf16", 1, 2, 64, 128, 50, 64, 16, True),
    ("bf16", 1, 520, 64, 128, 300, 64, 16, True),
    ("bf16", 4, 4, 64, 256, 500, 128, 32, True),  # 1024 (query, head) pairs at d = 256: two lane groups per row
    ("f32", 1, 16, 8, 64, 1024, 64, 128, True),
])
def test_sparse_attn_matches_oracle(dt, B, T, H, d, L, k, W, use_sink):
    import synthetic as syn
    m = 4
    n_ctx = L * m
    R = T + max(W, 1) - 1
    g, c = _attn_inputs(dt, B, T, H, d, L, R, 31 + d)
    q, kc, vc, kr, vr, sk = g
    q_c, kc_c, vc_c, kr_c, vr_c, sk_c = c
    tpos = np.arange(n_ctx - T, n_ctx)
    nv = np.minimum(tpos // m, L)
    idx_c = syn.sample_indices(7, syn.TID["idx"], B * T, k, np.tile(nv, B) - 3).reshape(B, T, k)
    idx = idx_c.cuda()
    out, lse = csa.csa_sparse_attn(q, kc, vc, idx, kr=kr if W else None, vr=vr if W else None, W=W,
                                   sink=sk if use_sink else None, n_ctx=n_ctx, want_lse=True)
    torch.cuda.synchronize()
    o_w, l_w = oracle.sparse_attn(q_c, kc_c, vc_c, idx_c.numpy(), kr_c, vr_c, W,
                                  sink=sk_c if use_sink else None, n_ctx=n_ctx)
    assert max_abs(to_np(out), o_w) <= TOL[dt]
    assert max_abs(to_np(lse), l_w) <= 1e-3


@pytest.mark.parametrize("dt,B,T,H,d,L,m,W", [
    ("bf16", 2, 1, 64, 512, 3000, 128, 0),
    ("bf16", 1, 2, 64, 512, 700, 4, 128),
    ("bf16", 1, 40, 64, 128, 100, 4, 16),
    ("bf16", 1, 520, 64, 128, 200, 4, 16),
    ("bf16", 1, 1, 64, 512, 9000, 4, 128),  # one query, 9127 rows: 143 splits, merged in two round trips
    ("f32", 1, 2, 8, 64, 500, 4, 128),
])
def test_dense_attn_matches_oracle(dt, B, T, H, d, L, m, W):
    n_ctx = L * m - (m // 2)
    R = T + max(W, 1) - 1
    g, c = _attn_inputs(dt, B, T, H, d, L, R, 41 + L)
    q, kc, vc, kr, vr, sk = g
    q_c, kc_c, vc_c, kr_c, vr_c, sk_c = c
    out, lse = csa.hca_dense_attn(q, kc, vc, m, kr=kr if W else None, vr=vr if W else None, W=W, sink=sk,
                                  n_ctx=n_ctx, want_lse=True)
    torch.cuda.synchronize()
    o_w, l_w = oracle.dense_attn(q_c, kc_c, vc_c, m, kr_c, vr_c, W, sink=sk_c, n_ctx=n_ctx)
    assert max_abs(to_np(out), o_w) <= TOL[dt]
    assert max_abs(to_np(lse), l_w) <= 1e-3


def test_sparse_with_all_entries_equals_dense_on_gpu():
    B, T, H, d, L, m, W = 2, 1, 64, 512, 600, 4, 128
    n_ctx = L * m
    R = T + W - 1
    g, _ = _attn_inputs("bf16", B, T, H, d, L, R, 77)
    q, kc, vc, kr, vr, sk = g
    nv = (n_ctx - 1) // m
    idx = torch.full((B, T, 640), -1, dtype=torch.int32, device="cuda")
    idx[..., :nv] = torch.arange(nv, dtype=torch.int32, device="cuda")
    a = csa.csa_sparse_attn(q, kc, vc, idx, kr=kr, vr=vr, W=W, sink=sk, n_ctx=n_ctx)
    b = csa.hca_dense_attn(q, kc, vc, m, kr=kr, vr=vr, W=W, sink=sk, n_ctx=n_ctx)
    torch.cuda.synchronize()
    assert max_abs(to_np(a), to_np(b)) <= 4e-3


def test_generator_is_bit_identical_on_both_devices():
    import synthetic as syn
    for kind in ("normal", "uniform", "grid"):
        a = syn.make((3, 1000, 72), 9, 4, dtype=torch.bfloat16, device="cuda", kind=kind, scale=0.25)
        b = syn.make((3, 1000, 72), 9, 4, dtype=torch.bfloat16, device="cpu", kind=kind, scale=0.25)
        assert torch.equal(a.cpu(), b)


@pytest.mark.parametrize("B,T,L,HI,wts", [(2, 64, 9000, 64, True), (1, 128, 30000, 32, False),
                                          (1, 64, 5000, 16, True), (1, 72, 4100, 128, False), (1, 64, 3000, 128, True)])
def test_index_scores_prefill_rows_equal_single_query_scan(B, T, L, HI, wts):
    """Many queries per sequence take the 8-row prefill scoring kernel; every
    row must equal, bit for bit, the same query scored alone (one query per
    call takes the streaming scan), over all L entries incl. the -inf ones."""
    dI, m = 128, 4
    n_ctx = m * L - 3
    seed = 70 + T
    q, _ = both((B, T, HI, dI), seed, "q_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    kk, _ = both((B, L, dI), seed, "k_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    w = both((B, T, HI), seed, "w_idx", dtype=torch.float32, scale=HI ** -0.5)[0] if wts else None
    full = csa.csa_index_score(q, kk, m, w_idx=w, n_ctx=n_ctx)
    for b in {0, B - 1}:
        for t in (0, 7, 8, T - 9, T - 1):
            one = csa.csa_index_score(q[b:b + 1, t:t + 1].contiguous(), kk[b:b + 1].contiguous(), m,
                                      w_idx=None if w is None else w[b:b + 1, t:t + 1].contiguous(),
                                      n_ctx=n_ctx - T + t + 1)
            torch.cuda.synchronize()
            assert torch.equal(full[b, t].view(torch.int32), one[0, 0].view(torch.int32)), (b, t)


def test_index_topk_prefill_rows_match_oracle():
    """Index + top-k for 64 queries of one sequence (8-row scoring, then the
    stand-alone top-k): exact on grid inputs, near-tie certified on Gaussian."""
    B, T, HI, dI, m, k = 1, 64, 64, 128, 4, 512
    n_ctx = 4 * 7000 + 1
    L = -(-n_ctx // m)
    q, q_c = both((B, T, HI, dI), 91, "q_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    kk, k_c = both((B, L, dI), 91, "k_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    idx = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    want, _ = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    assert np.array_equal(idx, want)
    q, q_c = both((B, T, HI, dI), 92, "q_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    kk, k_c = both((B, L, dI), 92, "k_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    got = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx).cpu().numpy()
    want, sc = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    ties = 0
    for t in range(0, T, 9):
        nv = min(L, (n_ctx - T + t) // m)
        ties += near_tie_check(got[0, t], want[0, t], sc[0, t], nv, k, index_eps(q_c[0, t], None, k_c[0])[:nv])
    assert ties <= 1


def test_timed_scan_launch_gives_the_same_selection():
    """A scan launched with csa_time_next_scan's event pair (hipExtLaunchKernel)
    selects exactly what the ordinary launch selects, and its events time it."""
    B, T, L, HI, dI, m, k = 16, 1, 250000, 64, 128, 4, 1024
    n_ctx = m * L
    q, _ = both((B, T, HI, dI), 91, "q_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    kk, _ = both((B, L, dI), 91, "k_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    idx1 = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    csa.time_next_scan(start, stop)
    idx2 = csa.csa_index_topk(q, kk, m, k, n_ctx=n_ctx)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    ms = start.elapsed_time(stop)
    assert 0.0 < ms < 100.0
    csa.time_next_scan(None, None)  # nothing pending afterwards
