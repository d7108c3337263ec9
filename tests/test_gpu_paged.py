"""Serving layouts on the GPU: per-sequence lengths and paged compressed
caches (a block table mapping each sequence's logical pages to pages of a
shared pool, as in trdm.cn section 3's Paged Attention paragraph).

The same logical caches are laid out densely ([B][L][d]) and as pools with
shuffled pages.  Paged calls must give bit for bit what the dense calls with
the same lengths give; the selection must equal per-sequence calls on the
dense caches bit for bit (the score of an entry does not depend on the
batch); attention must match the fp64 oracle per sequence."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from helpers import BF16_TOL, F32_TOL, max_abs, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:
    csa = None

SEED = 14
PAGE = 64


def make(shape, name, scale, device, dtype=torch.bfloat16, layer=0, kind="normal"):
    return syn.make(shape, SEED, syn.TID[name], dtype=dtype, device=device, scale=scale, layer=layer, kind=kind)


def paged(dense, npages_extra, seed):
    """A pool holding dense [B][L][D]'s pages at shuffled places, plus unused
    pages of garbage; returns (pool [npages * PAGE][D], block table [B][P])."""
    B, L, D = dense.shape
    P = -(-L // PAGE)
    npages = B * P + npages_extra
    perm = torch.randperm(npages, generator=torch.Generator().manual_seed(seed))[:B * P].reshape(B, P)
    pool = torch.full((npages * PAGE, D), 7.0, dtype=dense.dtype, device=dense.device)
    padded = torch.zeros((B, P * PAGE, D), dtype=dense.dtype, device=dense.device)
    padded[:, :L] = dense
    rows = (perm.to(dense.device).reshape(B, P, 1) * PAGE + torch.arange(PAGE, device=dense.device)).reshape(B, -1)
    for b in range(B):
        pool[rows[b]] = padded[b]
    return pool, perm.to(torch.int32).to(dense.device), npages


LENS = (40000, 27003, 33337)
# eight sequences of up to 131,072 tokens, k = 1024: more key ranges per row
# than the single-pass scan takes, so index + top-k runs the listed path
LENS8 = (131072, 118003, 99999, 131000, 64001, 120000, 100003, 77777)


@pytest.mark.parametrize("dt,lens,k", [("bf16", LENS, 512), ("fp8", LENS, 512), ("bf16", LENS8, 1024),
                                       ("fp8", LENS8, 1024)])
def test_paged_varlen_index_topk(dt, lens, k):
    LENS = lens
    B, HI, dI, m = len(LENS), 64, 128, 4
    n_max = max(LENS)
    L = n_max // m + 3  # capacity in entries
    sto = torch.bfloat16 if dt == "bf16" else torch.float8_e4m3fn
    q = make((B, 1, HI, dI), "q_idx", dI ** -0.5, "cuda", dtype=sto)
    kk = make((B, L, dI), "kic", dI ** -0.5, "cuda", dtype=sto)
    w = make((B, 1, HI), "w_idx", HI ** -0.5, "cuda", dtype=torch.float32)
    lens = torch.tensor(LENS, dtype=torch.int64, device="cuda")
    pool, bt, npages = paged(kk.view(torch.uint8) if dt == "fp8" else kk, 5, 1)
    if dt == "fp8":
        pool = pool.view(torch.float8_e4m3fn)
    lay_d = csa.layout(seq_len=lens)
    lay_p = csa.layout(seq_len=lens, block_table=bt, page=PAGE, num_pages=npages)
    i_d, s_d = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_max, layout=lay_d, want_scores=True)
    i_p, s_p = csa.csa_index_topk(q, pool, m, k, w_idx=w, n_ctx=n_max, layout=lay_p, L=L, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(i_d, i_p)
    assert torch.equal(s_d.view(torch.int32), s_p.view(torch.int32))
    for b, n in enumerate(LENS):
        one, s1 = csa.csa_index_topk(q[b:b + 1].contiguous(), kk[b:b + 1].contiguous(), m, k,
                                     w_idx=w[b:b + 1].contiguous(), n_ctx=n, want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(one[0], i_p[b]), b
        assert torch.equal(s1[0].view(torch.int32), s_p[b].view(torch.int32)), b
    # the oracle on one sequence, on exact grid inputs (bf16 only)
    if dt == "bf16":
        qg = make((B, 1, HI, dI), "q_idx", 2.0 ** -4, "cuda", kind="grid")
        kg = make((B, L, dI), "kic", 2.0 ** -4, "cuda", kind="grid")
        poolg, _, _ = paged(kg, 5, 1)
        got = csa.csa_index_topk(qg, poolg, m, k, n_ctx=n_max, layout=lay_p, L=L).cpu().numpy()
        for b, n in enumerate(LENS):
            qc = make((B, 1, HI, dI), "q_idx", 2.0 ** -4, "cpu", kind="grid").double().numpy()[b:b + 1]
            kc = make((B, L, dI), "kic", 2.0 ** -4, "cpu", kind="grid").double().numpy()[b:b + 1]
            want, _ = oracle.index_topk(qc, kc, m, k, n_ctx=n)
            assert np.array_equal(got[b], want[0]), b


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_paged_varlen_attention(dt):
    sto = torch.bfloat16 if dt == "bf16" else torch.float32
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    H, d = (64, 512) if dt == "bf16" else (8, 64)
    B, m_c, m_h, k, W = len(LENS), 4, 128, 256, 128
    n_max = max(LENS)
    Lc, Lh = n_max // m_c + 1, n_max // m_h + 1
    R = W
    q = make((B, 1, H, d), "q", d ** -0.5, "cuda", dtype=sto)
    kc = make((B, Lc, d), "kc", d ** -0.5, "cuda", dtype=sto)
    vc = make((B, Lc, d), "vc", d ** -0.5, "cuda", dtype=sto)
    kh = make((B, Lh, d), "kc", d ** -0.5, "cuda", dtype=sto, layer=1)
    vh = make((B, Lh, d), "vc", d ** -0.5, "cuda", dtype=sto, layer=1)
    kr = make((B, R, d), "kr", d ** -0.5, "cuda", dtype=sto)
    vr = make((B, R, d), "vr", d ** -0.5, "cuda", dtype=sto)
    sink = make((H,), "sink", 1.0, "cuda", dtype=torch.float32)
    nv = [min((n - 1) // m_c, Lc) for n in LENS]
    idx_c = np.stack([syn.sample_indices(3, syn.TID["idx"], 1, k, np.array([v])).reshape(k) for v in nv])
    idx_c[1, 7] = -1  # an empty slot
    idx = torch.from_numpy(idx_c.astype(np.int32)).reshape(B, 1, k).cuda()
    lens = torch.tensor(LENS, dtype=torch.int64, device="cuda")
    pkc, bt_c, np_c = paged(kc, 3, 2)
    pvc, _, _ = paged(vc, 3, 2)
    pkh, bt_h, np_h = paged(kh, 2, 3)
    pvh, _, _ = paged(vh, 2, 3)
    lay_d = csa.layout(seq_len=lens)
    lay_pc = csa.layout(seq_len=lens, block_table=bt_c, page=PAGE, num_pages=np_c)
    lay_ph = csa.layout(seq_len=lens, block_table=bt_h, page=PAGE, num_pages=np_h)
    o_d = csa.csa_sparse_attn(q, kc, vc, idx, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_max, layout=lay_d)
    o_p = csa.csa_sparse_attn(q, pkc, pvc, idx, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_max, layout=lay_pc, L=Lc)
    h_p = csa.hca_dense_attn(q, pkh, pvh, m_h, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_max, layout=lay_ph, L=Lh)
    h_d = csa.hca_dense_attn(q, kh, vh, m_h, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_max, layout=lay_d)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_p)  # same plan, same rows: the pool only moves them
    cpu = lambda t, name, layer=0: make(t.shape, name, d ** -0.5, "cpu", dtype=sto, layer=layer).double().numpy()  # noqa: E731
    q_c, kc_c, vc_c = cpu(q, "q"), cpu(kc, "kc"), cpu(vc, "vc")
    kh_c, vh_c = cpu(kh, "kc", 1), cpu(vh, "vc", 1)
    kr_c, vr_c = cpu(kr, "kr"), cpu(vr, "vr")
    sink_c = make((H,), "sink", 1.0, "cpu", dtype=torch.float32).double().numpy()
    for b, n in enumerate(LENS):
        sl = slice(b, b + 1)
        o_c, _ = oracle.sparse_attn(q_c[sl], kc_c[sl], vc_c[sl], idx_c[sl].reshape(1, 1, k), kr_c[sl], vr_c[sl], W,
                                    sink=sink_c, n_ctx=n)
        assert max_abs(to_np(o_p[sl]), o_c) <= tol, b
        oh_c, _ = oracle.dense_attn(q_c[sl], kh_c[sl], vh_c[sl], m_h, kr_c[sl], vr_c[sl], W, sink=sink_c, n_ctx=n)
        assert max_abs(to_np(h_p[sl]), oh_c) <= tol, b
        assert max_abs(to_np(h_d[sl]), oh_c) <= tol, b


def test_paged_append_writes_the_pool_row():
    """csa_compress_append into a paged cache: the entry a token completes
    lands in the pool row its block table names, equal to bulk compression."""
    B, D, m, n = 2, 512, 4, 4096
    x = make((B, n, D), "k", D ** -0.5, "cuda")
    z = make((B, n, D), "z_k", 0.5, "cuda")
    xb = make((B, n, D), "xb_k", D ** -0.5, "cuda")
    zb = make((B, n, D), "zb_k", 0.5, "cuda")
    bulk = csa.csa_compress(x, z, m, x_b=xb, z_b=zb)
    L = n // m
    pool, bt, npages = paged(torch.zeros((B, L, D), dtype=torch.bfloat16, device="cuda"), 4, 9)
    lay = csa.layout(block_table=bt, page=PAGE, num_pages=npages)
    S = 2 * m
    p = n - 1  # completes entry L - 1
    rings = [torch.zeros((B, S, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    slots = torch.arange(p - S + 1, p, device="cuda") % S
    for r, src in zip(rings, (x, z, xb, zb)):
        r[:, slots] = src[:, p - S + 1:p]
    pos = torch.full((B,), p, dtype=torch.int64, device="cuda")
    csa.csa_compress_append(x[:, p].contiguous(), z[:, p].contiguous(), m, rings, pos, pool, x_b=xb[:, p].contiguous(),
                            z_b=zb[:, p].contiguous(), layout=lay, L=L)
    torch.cuda.synchronize()
    for b in range(B):
        row = int(bt[b, (L - 1) // PAGE]) * PAGE + (L - 1) % PAGE
        assert torch.equal(pool[row], bulk[b, L - 1]), b
