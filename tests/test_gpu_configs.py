"""GPU parity at the full sizes of the five workload configurations, in the
launch configurations the benchmark uses, checked against the fp64 oracle on
sampled outputs (the oracle regenerates the same seeded inputs on the CPU).

  1. CSA layer, fp32, n = 4096, 16 decode queries (end to end from raw tokens)
  2. CSA decode, bf16, B = 8, n = 131072 (compress -> indexer/top-k -> attention)
  3. HCA decode, bf16, B = 4, n = 1,000,000 (bulk compression, dense attention)
  4. CSA prefill chunk, bf16, 65536 queries over a 262144-token prefix (query
     subsets at both ends of the chunk)
  5. the 8-layer CSA/HCA decode step of bench.py at n = 1,000,000, B = 16
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from helpers import BF16_TOL, F32_TOL, index_eps, max_abs, near_tie_check, round_to, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:
    csa = None

BF = torch.bfloat16


def g_make(shape, seed, name, dtype, scale, device, layer=0, kind="normal"):
    return syn.make(shape, seed, syn.TID[name], dtype=dtype, device=device, scale=scale, layer=layer, kind=kind)


def c_rows(full_shape, rows, seed, name, dtype, scale, layer=0):
    """Rows of a seeded tensor regenerated on the CPU as float64 [len, D]."""
    return syn.rows(full_shape, rows, seed, syn.TID[name], dtype=dtype, scale=scale,
                    layer=layer).double().numpy()


def seq_rows(b, n, lo=0, hi=None):
    hi = n if hi is None else hi
    return np.arange(b * n + lo, b * n + hi)


def check_topk_rows(got, want, scores, q_c, k_c, nvis, k, w_c=None):
    ties = 0
    for r in range(got.shape[0]):
        eps = index_eps(q_c[r], None if w_c is None else w_c[r], k_c)[: nvis[r]]
        ties += near_tie_check(got[r], want[r], scores[r], int(nvis[r]), k, eps)
    return ties


# ---------------------------------------------------------------------------
# config 1: fp32 CSA layer end to end
# ---------------------------------------------------------------------------

def test_config1_csa_fp32_end_to_end():
    seed, B, n, T, H, d, HI, dI, m, k, W = 1, 1, 4096, 16, 8, 64, 4, 32, 4, 64, 128
    f32 = torch.float32
    sd, si = d ** -0.5, dI ** -0.5
    dev = "cuda"
    xk, xv = g_make((B, n, d), seed, "k", f32, sd, dev), g_make((B, n, d), seed, "v", f32, sd, dev)
    zk, zv = g_make((B, n, d), seed, "z_k", f32, 0.5, dev), g_make((B, n, d), seed, "z_v", f32, 0.5, dev)
    xi, zi = g_make((B, n, dI), seed, "k_idx", f32, si, dev), g_make((B, n, dI), seed, "z_idx", f32, 0.5, dev)
    q = g_make((B, T, H, d), seed, "q", f32, sd, dev)
    qi = g_make((B, T, HI, dI), seed, "q_idx", f32, si, dev)
    wi = g_make((B, T, HI), seed, "w_idx", f32, HI ** -0.5, dev)
    sink = g_make((H,), seed, "sink", f32, 1.0, dev)
    kc, vc, ki = csa.csa_compress(xk, zk, m), csa.csa_compress(xv, zv, m), csa.csa_compress(xi, zi, m)
    idx = csa.csa_index_topk(qi, ki, m, k, w_idx=wi, n_ctx=n)
    R = T + W - 1
    out, lse = csa.csa_sparse_attn(q, kc, vc, idx, kr=xk[:, n - R:].contiguous(), vr=xv[:, n - R:].contiguous(),
                                   W=W, sink=sink, n_ctx=n, want_lse=True)
    torch.cuda.synchronize()

    cpu = lambda t: t.cpu().double().numpy()  # noqa: E731  (regenerate on the CPU)
    C = {nm: g_make(t.shape, seed, nm, f32, sc, "cpu").double().numpy()
         for nm, t, sc in (("k", xk, sd), ("v", xv, sd), ("z_k", zk, 0.5), ("z_v", zv, 0.5),
                           ("k_idx", xi, si), ("z_idx", zi, 0.5), ("q", q, sd), ("q_idx", qi, si),
                           ("w_idx", wi, HI ** -0.5))}
    sink_c = g_make((H,), seed, "sink", f32, 1.0, "cpu").double().numpy()
    kc_c = round_to(oracle.compress(C["k"], C["z_k"], m), f32)
    vc_c = round_to(oracle.compress(C["v"], C["z_v"], m), f32)
    ki_c = round_to(oracle.compress(C["k_idx"], C["z_idx"], m), f32)
    assert max_abs(cpu(kc), kc_c) <= F32_TOL and max_abs(cpu(ki), ki_c) <= F32_TOL
    idx_c, sc = oracle.index_topk(C["q_idx"], ki_c, m, k, w=C["w_idx"], n_ctx=n)
    nvis = np.array([(n - T + i) // m for i in range(T)])
    ties = check_topk_rows(idx.cpu().numpy()[0], idx_c[0], sc[0], C["q_idx"][0], ki_c[0], nvis, k,
                           w_c=C["w_idx"][0])
    assert ties == 0, "near-tie disagreements: %d" % ties
    o_c, l_c = oracle.sparse_attn(C["q"], kc_c, vc_c, idx_c, C["k"][:, n - R:], C["v"][:, n - R:], W,
                                  sink=sink_c, n_ctx=n)
    assert max_abs(cpu(out), o_c) <= F32_TOL
    assert max_abs(cpu(lse), l_c) <= F32_TOL


# ---------------------------------------------------------------------------
# config 2: CSA decode at 128K, B = 8
# ---------------------------------------------------------------------------

def test_config2_csa_decode_128k():
    seed, B, n, H, d, HI, dI, m, k, W = 2, 8, 131072, 64, 512, 64, 128, 4, 1024, 128
    sd, si = d ** -0.5, dI ** -0.5
    L = n // m
    dev = "cuda"
    # raw streams on the GPU; bulk compression exactly as a prefill would do it
    caches = {}
    for nm, zn, D, sc in (("k", "z_k", d, sd), ("v", "z_v", d, sd), ("k_idx", "z_idx", dI, si)):
        x = g_make((B, n, D), seed, nm, BF, sc, dev)
        z = g_make((B, n, D), seed, zn, BF, 0.5, dev)
        caches[nm] = csa.csa_compress(x, z, m)
        del x, z
    q = g_make((B, 1, H, d), seed, "q", BF, sd, dev)
    qi = g_make((B, 1, HI, dI), seed, "q_idx", BF, si, dev)
    wi = g_make((B, 1, HI), seed, "w_idx", torch.float32, HI ** -0.5, dev)
    sink = g_make((H,), seed, "sink", torch.float32, 1.0, dev)
    kr = syn.rows((B, n, d), np.concatenate([seq_rows(b, n, n - W) for b in range(B)]), seed, syn.TID["k"],
                  dtype=BF, device=dev, scale=sd).reshape(B, W, d)
    vr = syn.rows((B, n, d), np.concatenate([seq_rows(b, n, n - W) for b in range(B)]), seed, syn.TID["v"],
                  dtype=BF, device=dev, scale=sd).reshape(B, W, d)
    idx = csa.csa_index_topk(qi, caches["k_idx"], m, k, w_idx=wi, n_ctx=n)
    out, lse = csa.csa_sparse_attn(q, caches["k"], caches["v"], idx, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n,
                                   want_lse=True)
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy()

    for b in (5,):  # sampled sequence: everything for it is recomputed by the oracle
        ki_c = round_to(oracle.compress(c_rows((B, n, dI), seq_rows(b, n), seed, "k_idx", BF, si).reshape(1, n, dI),
                                        c_rows((B, n, dI), seq_rows(b, n), seed, "z_idx", BF, 0.5).reshape(1, n, dI),
                                        m), BF)
        assert max_abs(to_np(caches["k_idx"][b:b + 1]), ki_c) <= BF16_TOL
        qi_c = c_rows((B, 1, HI, dI), np.arange(b * HI, (b + 1) * HI), seed, "q_idx", BF, si).reshape(1, 1, HI, dI)
        wi_c = c_rows((B, 1, HI), np.arange(b, b + 1), seed, "w_idx", torch.float32, HI ** -0.5).reshape(1, 1, HI)
        idx_c, sc = oracle.index_topk(qi_c, ki_c, m, k, w=wi_c, n_ctx=n)
        ties = check_topk_rows(idx_g[b], idx_c[0], sc[0], qi_c[0], ki_c[0], np.array([(n - 1) // m]), k,
                               w_c=wi_c[0])
        assert ties <= 1
        kc_c = round_to(oracle.compress(c_rows((B, n, d), seq_rows(b, n), seed, "k", BF, sd).reshape(1, n, d),
                                        c_rows((B, n, d), seq_rows(b, n), seed, "z_k", BF, 0.5).reshape(1, n, d),
                                        m), BF)
        vc_c = round_to(oracle.compress(c_rows((B, n, d), seq_rows(b, n), seed, "v", BF, sd).reshape(1, n, d),
                                        c_rows((B, n, d), seq_rows(b, n), seed, "z_v", BF, 0.5).reshape(1, n, d),
                                        m), BF)
        assert max_abs(to_np(caches["k"][b:b + 1]), kc_c) <= BF16_TOL
        q_c = c_rows((B, 1, H, d), np.arange(b * H, (b + 1) * H), seed, "q", BF, sd).reshape(1, 1, H, d)
        kr_c = c_rows((B, n, d), seq_rows(b, n, n - W), seed, "k", BF, sd).reshape(1, W, d)
        vr_c = c_rows((B, n, d), seq_rows(b, n, n - W), seed, "v", BF, sd).reshape(1, W, d)
        sink_c = g_make((H,), seed, "sink", torch.float32, 1.0, "cpu").double().numpy()
        # attention checked twice: the oracle fed the GPU's own selection, and
        # end to end (the oracle's own selection)
        o_g, l_g = oracle.sparse_attn(q_c, kc_c, vc_c, idx_g[b:b + 1], kr_c, vr_c, W, sink=sink_c, n_ctx=n)
        assert max_abs(to_np(out[b:b + 1]), o_g) <= BF16_TOL
        assert max_abs(to_np(lse[b:b + 1]), l_g) <= 1e-2
        o_c, l_c = oracle.sparse_attn(q_c, kc_c, vc_c, idx_c, kr_c, vr_c, W, sink=sink_c, n_ctx=n)
        assert max_abs(to_np(out[b:b + 1]), o_c) <= BF16_TOL
        assert max_abs(to_np(lse[b:b + 1]), l_c) <= 1e-2


# ---------------------------------------------------------------------------
# config 3: HCA at 1M, B = 4
# ---------------------------------------------------------------------------

def test_config3_hca_compress_1m_sampled_entries():
    seed, B, n, d, m = 3, 4, 1_000_000, 512, 128
    sd = d ** -0.5
    L = -(-n // m)
    assert L == 7813
    out = {}
    for nm, zn in (("k", "z_k"),):
        x = g_make((B, n, d), seed, nm, BF, sd, "cuda")
        z = g_make((B, n, d), seed, zn, BF, 0.5, "cuda")
        out[nm] = csa.hca_compress(x, z, m)
        del x, z
    torch.cuda.synchronize()
    got = to_np(out["k"])
    rng = np.random.default_rng(0)
    for b in (0, 3):
        ents = sorted(set(rng.integers(0, L - 1, 6).tolist()) | {0, L - 2, L - 1})  # includes the partial block
        for j in ents:
            lo, hi = j * m, min(n, (j + 1) * m)
            xr = c_rows((B, n, d), seq_rows(b, n, lo, hi), seed, "k", BF, sd).reshape(1, hi - lo, d)
            zr = c_rows((B, n, d), seq_rows(b, n, lo, hi), seed, "z_k", BF, 0.5).reshape(1, hi - lo, d)
            want = oracle.compress(xr, zr, m, n=n, p0=lo, e0=j, e1=j + 1)
            assert max_abs(got[b:b + 1, j:j + 1], want) <= BF16_TOL, (b, j)


def test_config3_hca_dense_decode_1m():
    seed, B, n, H, d, m = 3, 4, 1_000_000, 64, 512, 128
    sd = d ** -0.5
    L = -(-n // m)
    kc = g_make((B, L, d), seed, "kc", BF, sd, "cuda")
    vc = g_make((B, L, d), seed, "vc", BF, sd, "cuda")
    q = g_make((B, 1, H, d), seed, "q", BF, sd, "cuda")
    sink = g_make((H,), seed, "sink", torch.float32, 1.0, "cuda")
    out, lse = csa.hca_dense_attn(q, kc, vc, m, sink=sink, n_ctx=n, want_lse=True)
    torch.cuda.synchronize()
    kc_c = g_make((B, L, d), seed, "kc", BF, sd, "cpu").double().numpy()
    vc_c = g_make((B, L, d), seed, "vc", BF, sd, "cpu").double().numpy()
    q_c = g_make((B, 1, H, d), seed, "q", BF, sd, "cpu").double().numpy()
    sink_c = g_make((H,), seed, "sink", torch.float32, 1.0, "cpu").double().numpy()
    o_c, l_c = oracle.dense_attn(q_c, kc_c, vc_c, m, None, None, 0, sink=sink_c, n_ctx=n)
    assert max_abs(to_np(out), o_c) <= BF16_TOL
    assert max_abs(to_np(lse), l_c) <= 1e-2


# ---------------------------------------------------------------------------
# config 4: CSA prefill chunk (query subsets at both ends of the 64K chunk)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("where", ["first", "last"])
def test_config4_csa_prefill_chunk(where):
    seed, H, d, HI, dI, m, k, W = 4, 64, 512, 64, 128, 4, 1024, 128
    sd, si = d ** -0.5, dI ** -0.5
    prefix, chunk, Tq = 262144, 65536, 256
    n_full = prefix + chunk
    L = n_full // m
    n_ctx = prefix + Tq if where == "first" else n_full  # queries n_ctx-Tq .. n_ctx-1
    dev = "cuda"
    kc = g_make((1, L, d), seed, "kc", BF, sd, dev)
    vc = g_make((1, L, d), seed, "vc", BF, sd, dev)
    ki = g_make((1, L, dI), seed, "kic", BF, si, dev)
    # per-query tensors of the whole chunk; this launch takes Tq of them
    q0 = (n_ctx - Tq) - prefix
    q = syn.rows((1, chunk, H, d), np.arange(q0 * H, (q0 + Tq) * H), seed, syn.TID["q"], dtype=BF,
                 device=dev, scale=sd).reshape(1, Tq, H, d)
    qi = syn.rows((1, chunk, HI, dI), np.arange(q0 * HI, (q0 + Tq) * HI), seed, syn.TID["q_idx"], dtype=BF,
                  device=dev, scale=si).reshape(1, Tq, HI, dI)
    wi = syn.rows((1, chunk, HI), np.arange(q0, q0 + Tq), seed, syn.TID["w_idx"], dtype=torch.float32,
                  device=dev, scale=HI ** -0.5).reshape(1, Tq, HI)
    R = Tq + W - 1
    raw = np.arange(n_ctx - R, n_ctx)
    kr = syn.rows((1, n_full, d), raw, seed, syn.TID["kr"], dtype=BF, device=dev, scale=sd).reshape(1, R, d)
    vr = syn.rows((1, n_full, d), raw, seed, syn.TID["vr"], dtype=BF, device=dev, scale=sd).reshape(1, R, d)
    sink = g_make((H,), seed, "sink", torch.float32, 1.0, dev)
    idx = csa.csa_index_topk(qi, ki, m, k, w_idx=wi, n_ctx=n_ctx)
    out = csa.csa_sparse_attn(q, kc, vc, idx, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_ctx)
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy()[0]

    sample = [0, 1, 97, Tq - 2, Tq - 1]
    ki_c = g_make((1, L, dI), seed, "kic", BF, si, "cpu").double().numpy()
    qi_c = syn.rows((1, chunk, HI, dI), np.concatenate([np.arange((q0 + s) * HI, (q0 + s + 1) * HI) for s in sample]),
                    seed, syn.TID["q_idx"], dtype=BF, scale=si).double().numpy().reshape(1, len(sample), HI, dI)
    wi_c = syn.rows((1, chunk, HI), np.array([q0 + s for s in sample]), seed, syn.TID["w_idx"],
                    dtype=torch.float32, scale=HI ** -0.5).double().numpy().reshape(1, len(sample), HI)
    tpos = np.array([n_ctx - Tq + s for s in sample])
    idx_c, sc = oracle.index_topk(qi_c, ki_c, m, k, w=wi_c, tpos=tpos)
    ties = check_topk_rows(idx_g[sample], idx_c[0], sc[0], qi_c[0], ki_c[0], np.minimum(tpos // m, L), k,
                           w_c=wi_c[0])
    assert ties <= 1
    same = [i for i, s in enumerate(sample) if np.array_equal(idx_g[s], idx_c[0, i])]
    assert len(same) >= len(sample) - 1  # a near-tie swap may differ in at most one sampled row
    kc_c = g_make((1, L, d), seed, "kc", BF, sd, "cpu").double().numpy()
    vc_c = g_make((1, L, d), seed, "vc", BF, sd, "cpu").double().numpy()
    q_c = syn.rows((1, chunk, H, d), np.concatenate([np.arange((q0 + s) * H, (q0 + s + 1) * H) for s in sample]),
                   seed, syn.TID["q"], dtype=BF, scale=sd).double().numpy().reshape(1, len(sample), H, d)
    kr_c = syn.rows((1, n_full, d), raw, seed, syn.TID["kr"], dtype=BF, scale=sd).double().numpy().reshape(1, R, d)
    vr_c = syn.rows((1, n_full, d), raw, seed, syn.TID["vr"], dtype=BF, scale=sd).double().numpy().reshape(1, R, d)
    sink_c = g_make((H,), seed, "sink", torch.float32, 1.0, "cpu").double().numpy()
    got = to_np(out)[0][sample]
    # attention checked twice on every sampled query: the oracle fed the GPU's
    # own selection, and end to end (the oracle's selection; a near-tie swap
    # moves one row of weight ~1/1152, far inside the bound)
    o_g, _ = oracle.sparse_attn(q_c, kc_c, vc_c, idx_g[sample][None], kr_c, vr_c, W, sink=sink_c, n_ctx=n_ctx,
                                tpos=tpos)
    assert max_abs(got, o_g[0]) <= BF16_TOL
    o_c, _ = oracle.sparse_attn(q_c, kc_c, vc_c, idx_c, kr_c, vr_c, W, sink=sink_c, n_ctx=n_ctx, tpos=tpos)
    assert max_abs(got, o_c[0]) <= BF16_TOL


# ---------------------------------------------------------------------------
# config 5: the benchmark's 8-layer decode step (n = 1M, B = 16)
# ---------------------------------------------------------------------------

def _check_stack_layers(st, state, b, layers):
    """The given layers of a decode step of sequence b against the oracle: the
    entry the decoded token completes (when it does) and each layer's output,
    with the CSA attention checked twice (the GPU's selection, end to end)."""
    import bench
    SEED, bf = bench.SEED, BF
    sd, si = st.d ** -0.5, st.dI ** -0.5
    sub = bench.Stack(B=b + 1, n_ctx=st.n_ctx)  # row numbering of sequences 0..b is the same as in the full batch
    t = st.t
    for li in layers:
        lay = state.layers[li]
        kind = lay["kind"]
        q_c = c_rows((st.B, 1, st.H, st.d), np.arange(b * st.H, (b + 1) * st.H), SEED, "q", bf, sd,
                     layer=li).reshape(1, 1, st.H, st.d)
        sink_c = syn.make((st.H,), SEED, syn.TID["sink"], layer=li).double().numpy()
        kr_c = bench.raw_rows(sub, "kr", li, st.n_ctx - st.W, st.W, st.d, "cpu", sd)[b:].double().numpy()
        vr_c = bench.raw_rows(sub, "vr", li, st.n_ctx - st.W, st.W, st.d, "cpu", sd)[b:].double().numpy()
        got_out = to_np(lay["out"][b:b + 1])
        if kind == "csa":
            m = st.m_csa
            L = lay["kc"].shape[1]
            e = t // m
            assert st.emits(m)
            # the entry completed by the decoded token (two-path), for K, V and the index keys
            new = {}
            for s, cache, D, sc in (("k", "kc", st.d, sd), ("v", "vc", st.d, sd), ("idx", "ki", st.dI, si)):
                arrs = [bench.raw_rows(sub, nm, li, (e - 1) * m, 2 * m, D, "cpu", scl)[b:].double().numpy()
                        for nm, scl in zip(bench.STREAMS[s], (sc, 0.5, sc, 0.5))]
                want = oracle.compress(arrs[0], arrs[1], m, x_b=arrs[2], z_b=arrs[3], n=st.n_ctx, p0=(e - 1) * m,
                                       e0=e, e1=e + 1)
                assert max_abs(to_np(lay[cache][b:b + 1, e:e + 1]), want) <= BF16_TOL
                new[s] = round_to(want[0, 0], bf)
            ki_c = c_rows((st.B, L, st.dI), seq_rows(b, L), SEED, "kic", bf, si, layer=li)
            ki_c[e] = new["idx"]  # rewritten by the step (not visible to the token)
            ki_c = ki_c.reshape(1, L, st.dI)
            qi_c = c_rows((st.B, 1, st.HI, st.dI), np.arange(b * st.HI, (b + 1) * st.HI), SEED, "q_idx", bf, si,
                          layer=li).reshape(1, 1, st.HI, st.dI)
            wi_c = c_rows((st.B, 1, st.HI), np.arange(b, b + 1), SEED, "w_idx", torch.float32, st.HI ** -0.5,
                          layer=li).reshape(1, 1, st.HI)
            idx_c, sc = oracle.index_topk(qi_c, ki_c, m, st.k, w=wi_c, n_ctx=st.n_ctx)
            got_idx = lay["idx"].cpu().numpy()[b]
            ties = check_topk_rows(got_idx, idx_c[0], sc[0], qi_c[0], ki_c[0], np.array([st.nv_csa]), st.k,
                                   w_c=wi_c[0])
            assert ties <= 1
            # the rows either selection reads (the GPU's and the oracle's)
            sel = np.union1d(idx_c[0, 0][idx_c[0, 0] >= 0], got_idx[0][got_idx[0] >= 0])
            kc_c = np.zeros((1, L, st.d))
            vc_c = np.zeros((1, L, st.d))
            kc_c[0, sel] = c_rows((st.B, L, st.d), b * L + sel, SEED, "kc", bf, sd, layer=li)
            vc_c[0, sel] = c_rows((st.B, L, st.d), b * L + sel, SEED, "vc", bf, sd, layer=li)
            o_g, _ = oracle.sparse_attn(q_c, kc_c, vc_c, got_idx[None], kr_c, vr_c, st.W, sink=sink_c,
                                        n_ctx=st.n_ctx)
            assert max_abs(got_out, o_g) <= BF16_TOL
            o_c, _ = oracle.sparse_attn(q_c, kc_c, vc_c, idx_c, kr_c, vr_c, st.W, sink=sink_c, n_ctx=st.n_ctx)
            assert max_abs(got_out, o_c) <= BF16_TOL
        elif kind == "hca":
            m = st.m_hca
            L = lay["kc"].shape[1]
            kc_c = c_rows((st.B, L, st.d), seq_rows(b, L), SEED, "kc", bf, sd, layer=li)
            vc_c = c_rows((st.B, L, st.d), seq_rows(b, L), SEED, "vc", bf, sd, layer=li)
            if st.emits(m):  # the entry the token completes is written (and is not visible to it)
                e = t // m
                for s, arr in (("k", kc_c), ("v", vc_c)):
                    x = bench.raw_rows(sub, s, li, e * m, m, st.d, "cpu", sd)[b:].double().numpy()
                    z = bench.raw_rows(sub, "z_" + s, li, e * m, m, st.d, "cpu", 0.5)[b:].double().numpy()
                    want = oracle.compress(x, z, m, n=st.n_ctx, p0=e * m, e0=e, e1=e + 1)
                    assert max_abs(to_np(lay["kc" if s == "k" else "vc"][b:b + 1, e:e + 1]), want) <= BF16_TOL
                    arr[e] = round_to(want[0, 0], bf)
            o_c, _ = oracle.dense_attn(q_c, kc_c.reshape(1, L, st.d), vc_c.reshape(1, L, st.d), m, kr_c, vr_c,
                                       st.W, sink=sink_c, n_ctx=st.n_ctx)
            assert max_abs(got_out, o_c) <= BF16_TOL
        else:  # window only
            o_c, _ = oracle.dense_attn(q_c, np.zeros((1, 0, st.d)), np.zeros((1, 0, st.d)), st.m_hca, kr_c, vr_c,
                                       st.W, sink=sink_c, n_ctx=st.n_ctx)
            assert max_abs(got_out, o_c) <= BF16_TOL


def test_config5_stack_step_sampled():
    import bench
    st = bench.Stack(B=16)
    state = bench.GpuState(st)
    state.step()
    torch.cuda.synchronize()
    _check_stack_layers(st, state, 11, (0, 1))  # one CSA and one HCA layer, sequence 11
    del state
    torch.cuda.empty_cache()


@pytest.mark.parametrize("schedule", ["alternate", "flash", "pro"])
def test_batch1_step_every_layer_eager_and_graph(schedule):
    """The batch-1 decode step at 1M tokens under each layer schedule: replayed
    as one HIP graph it gives the eager step's outputs bit for bit (every
    replay, with eager work between them), and every layer of it matches the
    oracle."""
    import bench
    st = bench.Stack(B=1, schedule=schedule)
    state = bench.GpuState(st)
    state.step()
    torch.cuda.synchronize()
    eager = [(lay["out"].clone(), lay.get("idx", torch.zeros(1)).clone()) for lay in state.layers]
    replay = state.capture()
    for _ in range(3):
        for lay in state.layers:
            lay["out"].zero_()
            if "idx" in lay:
                lay["idx"].fill_(-5)
        torch.cuda.synchronize()
        replay()
        torch.cuda.synchronize()
        for (o, i), lay in zip(eager, state.layers):
            assert torch.equal(o, lay["out"])
            if "idx" in lay:
                assert torch.equal(i, lay["idx"])
        state.step()  # eager work between the replays
        torch.cuda.synchronize()
    _check_stack_layers(st, state, 0, range(st.layers))
    del state, replay
    torch.cuda.empty_cache()


def test_step_is_deterministic():
    import bench
    st = bench.Stack(B=2, n_ctx=65536)
    state = bench.GpuState(st)
    state.step()
    torch.cuda.synchronize()
    first = [(lay["out"].clone(), lay.get("idx", torch.zeros(1)).clone()) for lay in state.layers]
    for _ in range(2):
        state.step()
    torch.cuda.synchronize()
    for (o, i), lay in zip(first, state.layers):
        assert torch.equal(o, lay["out"])
        if "idx" in lay:
            assert torch.equal(i, lay["idx"])
