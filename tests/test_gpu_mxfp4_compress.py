"""GPU parity of compression that writes MXFP4 entries (the indexer's keys in
FP4: shareware.cn Hybrid Attention article, its list of what is compressed;
MXFP4 with the OCP conversion is the reading taken).

Where floating point decides a code, both sides decide on the same value:
  * grid inputs with zero logits (means of a power-of-two count of grid
    values) make every compressed value the same in fp32 and fp64, so the
    GPU's MXFP4 bytes equal the oracle's encoding of the oracle's fp64
    compression;
  * on Gaussian inputs with logits and biases, the oracle encodes the GPU's
    own fp32 compression (the fp32-output kernel on the same values folds in
    the same order), and the bytes must be equal; the decoded entries are
    checked against the fp64 compression within the format's rounding.
Per-token appends into an MXFP4 cache (dense and paged) equal the bulk MXFP4
compression bit for bit, and the indexer over compressed MXFP4 keys matches
the oracle end to end."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from helpers import both, index_eps, near_tie_check

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:
    csa = None

BF = torch.bfloat16


def mx_bytes(t):
    return t.data.cpu().numpy()


@pytest.mark.parametrize("two,m,B,n", [(False, 4, 2, 4 * 301 + 2), (True, 4, 3, 4 * 257),
                                       (False, 16, 2, 16 * 40 + 8)])
def test_compress_mxfp4_bit_exact_on_grid_mean_pooling(two, m, B, n):
    """Every entry averages a power-of-two count of grid values (a trailing
    block of 2 or 8 tokens; two-path blocks of 8 candidates), so the fp64
    weights and sums are exact as well: a block of 3 would leave the oracle a
    residue of order 1e-17 where fp32 gives 0, and a different sign bit."""
    D = 128
    x, x_c = both((B, n, D), 50 + m, "k_idx", dtype=BF, kind="grid", scale=2.0 ** -3)
    z, z_c = both((B, n, D), 50 + m, "z_idx", dtype=BF, scale=0.0)
    kw, kw_c = {}, {}
    if two:
        xb, xb_c = both((B, n, D), 60 + m, "xb_k", dtype=BF, kind="grid", scale=2.0 ** -3)
        zb, zb_c = both((B, n, D), 60 + m, "zb_k", dtype=BF, scale=0.0)
        kw, kw_c = dict(x_b=xb, z_b=zb), dict(x_b=xb_c, z_b=zb_c)
    got = csa.csa_compress(x, z, m, mxfp4=True, **kw)
    torch.cuda.synchronize()
    want = oracle.mxfp4_encode(oracle.compress(x_c, z_c, m, **kw_c))
    assert np.array_equal(mx_bytes(got), want)


@pytest.mark.parametrize("two,m,B,n,bias", [(True, 4, 2, 4 * 700 + 2, True), (False, 4, 3, 4 * 500, False),
                                            (False, 128, 2, 128 * 520 + 77, True)])
def test_compress_mxfp4_equals_encoded_fp32_compression(two, m, B, n, bias):
    D = 128
    g = lambda shape, seed, name, sc, dt=BF, layer=0: syn.make(shape, seed, syn.TID[name], dtype=dt,
                                                               device="cuda", scale=sc, layer=layer)
    c = lambda shape, seed, name, sc, dt=BF, layer=0: syn.make(shape, seed, syn.TID[name], dtype=dt,
                                                               scale=sc, layer=layer).double().numpy()
    s = D ** -0.5
    x, z = g((B, n, D), 7, "k_idx", s), g((B, n, D), 7, "z_idx", 0.5)
    x_c, z_c = c((B, n, D), 7, "k_idx", s), c((B, n, D), 7, "z_idx", 0.5)
    kw, kw_c = {}, {}
    if two:
        kw = dict(x_b=g((B, n, D), 8, "xb_k", s), z_b=g((B, n, D), 8, "zb_k", 0.5))
        kw_c = dict(x_b=c((B, n, D), 8, "xb_k", s), z_b=c((B, n, D), 8, "zb_k", 0.5))
    if bias:
        span = 2 * m if two else m
        kw["bias"] = g((span, D), 9, "bias", 0.3, torch.float32)
        kw_c["bias"] = c((span, D), 9, "bias", 0.3, torch.float32)
    got = csa.csa_compress(x, z, m, mxfp4=True, **kw)
    # the fp32-output kernel on the same values (bf16 widened exactly)
    f32 = {key: (v.float() if v.dtype == BF else v) for key, v in kw.items()}
    vals = csa.csa_compress(x.float(), z.float(), m, **f32)
    torch.cuda.synchronize()
    assert (B * vals.shape[1] * (D // 4)) >= 32768 or m < 32, "fp32 launch must fold in one lane"
    v = vals.cpu().double().numpy()
    assert np.array_equal(mx_bytes(got), oracle.mxfp4_encode(v))
    # decoded entries against the fp64 compression: the E2M1 rounding error at
    # the block's scale s is at most s / 4 below 1.75 s... 2 s at saturation;
    # the fp32 compression adds its own small error
    want = oracle.compress(x_c, z_c, m, **kw_c)
    dec = oracle.mxfp4_decode(mx_bytes(got), want.shape)
    sc = oracle.e8m0_decode(mx_bytes(got)[want.size // 2:]).reshape(*want.shape[:-1], D // 32)
    bound = np.repeat(2.0 * sc, 32, axis=-1) + 1e-5
    assert np.all(np.abs(dec - want) <= bound)


@pytest.mark.parametrize("paged", [False, True])
def test_compress_mxfp4_appends_equal_bulk(paged):
    """One token per step per sequence, two-path m = 4, prefixes of different
    phase: every entry an append writes equals the bulk MXFP4 entry."""
    B, D, m, S, steps = 2, 128, 4, 8, 61
    prefix = (40, 43)
    N = max(prefix) + steps
    s = D ** -0.5
    mk = lambda name, sc, seed: syn.make((B, N, D), seed, syn.TID[name], dtype=BF, device="cuda", scale=sc)
    xa, za, xb, zb = mk("k_idx", s, 21), mk("z_idx", 0.5, 21), mk("xb_k", s, 22), mk("zb_k", 0.5, 22)
    bias = syn.make((2 * m, D), 23, syn.TID["bias"], device="cuda", scale=0.3)
    ref = csa.csa_compress(xa, za, m, x_b=xb, z_b=zb, bias=bias, mxfp4=True)
    L = N // m + 1
    layout, page = None, 16
    if paged:
        per = -(-L // page)
        npages = B * per + 3
        perm = torch.randperm(npages, generator=torch.Generator().manual_seed(5))[:B * per]
        table = perm.view(B, per).to(torch.int32).cuda()
        layout = csa.layout(block_table=table, page=page, num_pages=npages)
        rows = npages * page
    else:
        rows = B * L
    nel = rows * D
    cache = csa.MXFP4(torch.zeros(nel // 2 + nel // 32, dtype=torch.uint8, device="cuda"),
                      (B, L, D) if not paged else (rows, 1, D))
    rings = [torch.zeros((B, S, D), dtype=BF, device="cuda") for _ in range(4)]
    for b, p in enumerate(prefix):  # the prefix's last 2m raw rows, slot u % S
        for u in range(p - 2 * m, p):
            for r, src in zip(rings, (xa, za, xb, zb)):
                r[b, u % S] = src[b, u]
    written = set()
    for st in range(steps):
        pos = torch.tensor([p + st for p in prefix], dtype=torch.int64, device="cuda")
        sel = lambda t: torch.stack([t[b, prefix[b] + st] for b in range(B)]).contiguous()
        csa.csa_compress_append(sel(xa), sel(za), m, rings, pos, cache, x_b=sel(xb), z_b=sel(zb), bias=bias,
                                layout=layout, L=L)
        for b in range(B):
            p = prefix[b] + st
            if (p + 1) % m == 0:
                written.add((b, p // m))
    torch.cuda.synchronize()
    got, want = mx_bytes(cache), mx_bytes(ref)
    half, want_half = nel // 2, B * ref.shape[1] * D // 2
    assert len(written) >= 2 * (steps // m)
    for b, j in sorted(written):
        row = b * L + j
        if paged:
            row = int(table[b, j // page]) * page + j % page
        wr = b * ref.shape[1] + j
        assert np.array_equal(got[row * D // 2:(row + 1) * D // 2], want[wr * D // 2:(wr + 1) * D // 2]), (b, j)
        assert np.array_equal(got[half + row * D // 32:half + (row + 1) * D // 32],
                              want[want_half + wr * D // 32:want_half + (wr + 1) * D // 32]), (b, j)


def test_index_topk_on_compressed_mxfp4_keys_matches_oracle():
    """Grid keys, zero logits: compression is exact on both sides, so the
    oracle scores the keys the GPU holds (its own compression and encoding);
    the selection must match up to certified near-ties."""
    B, T, m, HI, dI, k = 2, 2, 4, 64, 128, 256
    n = 4 * 3000 + 2
    x, x_c = both((B, n, dI), 71, "k_idx", dtype=BF, kind="grid", scale=2.0 ** -3)
    z, z_c = both((B, n, dI), 71, "z_idx", dtype=BF, scale=0.0)
    keys = csa.csa_compress(x, z, m, mxfp4=True)
    q = syn.mxfp4_(torch.empty(B * T * HI * dI // 2 + B * T * HI * dI // 32, dtype=torch.uint8, device="cuda"),
                   72, syn.TID["q_idx"], B * T * HI * dI)
    q_cpu = syn.mxfp4_(torch.empty(B * T * HI * dI // 2 + B * T * HI * dI // 32, dtype=torch.uint8), 72,
                       syn.TID["q_idx"], B * T * HI * dI)
    qm = csa.MXFP4(q, (B, T, HI, dI))
    q_c = oracle.mxfp4_decode(q_cpu.numpy(), (B, T, HI, dI))
    k_c = oracle.mxfp4_decode(oracle.mxfp4_encode(oracle.compress(x_c, z_c, m)), (B, -(-n // m), dI))
    idx = csa.csa_index_topk(qm, keys, m, k, n_ctx=n).cpu().numpy()
    want, osc = oracle.index_topk(q_c, k_c, m, k, n_ctx=n)
    for b in range(B):
        for t in range(T):
            nv = min(k_c.shape[1], (n - T + t) // m)
            eps = index_eps(q_c[b, t], None, k_c[b])[:nv]
            assert near_tie_check(idx[b, t], want[b, t], osc[b, t], nv, k, eps) <= 2


def test_fp8_kv_mxfp4_index_step_csa_layer_matches_oracle():
    """The decode step with the pages' storage mix (FP8 main KV, MXFP4 indexer
    q and keys, the appends compressing bf16 index-key rows to MXFP4), first
    CSA layer of sequence 1: the index-key entry the token completes equals
    bulk MXFP4 compression of the same raw rows byte for byte and decodes to
    the fp64 compression within the format's rounding; the selection matches
    the oracle on the decoded q and keys up to certified near-ties; the
    attention matches the oracle fed the GPU's selection."""
    import bench
    from helpers import BF16_TOL, max_abs, to_np
    st = bench.Stack(B=2, n_ctx=65536, eb=1, index_fmt="mxfp4")
    state = bench.GpuState(st)
    state.step()
    torch.cuda.synchronize()
    li, b = 0, 1
    lay = state.layers[li]
    assert lay["kind"] == "csa" and st.emits(st.m_csa)
    m, t, L, dI, HI, d, H, W, k = st.m_csa, st.t, st.L_csa, st.dI, st.HI, st.d, st.H, st.W, st.k
    e, si = t // m, dI ** -0.5
    scales = (si, 0.5, si, 0.5)

    # the completed entry: byte for byte the bulk MXFP4 entry of the same rows
    raw = [bench.raw_rows(st, nm, li, (e - 1) * m, 2 * m, dI, "cuda", sc) for nm, sc in zip(bench.STREAMS["idx"], scales)]
    bulk = csa.csa_compress(raw[0], raw[1], m, x_b=raw[2], z_b=raw[3], n=st.n_ctx, p0=(e - 1) * m, e0=e, e1=e + 1,
                            mxfp4=True)
    cache, one = mx_bytes(lay["ki"]), mx_bytes(bulk)
    row, half = b * L + e, st.B * L * dI // 2
    assert np.array_equal(cache[row * dI // 2:(row + 1) * dI // 2], one[b * dI // 2:(b + 1) * dI // 2])
    assert np.array_equal(cache[half + row * dI // 32:half + (row + 1) * dI // 32],
                          one[st.B * dI // 2 + b * dI // 32:st.B * dI // 2 + (b + 1) * dI // 32])
    raw_c = [bench.raw_rows(st, nm, li, (e - 1) * m, 2 * m, dI, "cpu", sc).double().numpy()
             for nm, sc in zip(bench.STREAMS["idx"], scales)]
    want = oracle.compress(raw_c[0], raw_c[1], m, x_b=raw_c[2], z_b=raw_c[3], n=st.n_ctx, p0=(e - 1) * m, e0=e,
                           e1=e + 1)[b, 0]
    dec = oracle.mxfp4_decode(cache[row * dI // 2:(row + 1) * dI // 2].tolist() +
                              cache[half + row * dI // 32:half + (row + 1) * dI // 32].tolist(), (1, dI))[0]
    blk_scale = np.repeat(oracle.e8m0_decode(cache[half + row * dI // 32:half + (row + 1) * dI // 32]), 32)
    assert np.all(np.abs(dec - want) <= 2.0 * blk_scale + 1e-5)

    # the selection over the generated MXFP4 q and keys (the rewritten entry is not visible)
    def mx_cpu(shape, name):
        n = int(np.prod(shape))
        buf = syn.mxfp4_(torch.empty(n // 2 + n // 32, dtype=torch.uint8), bench.SEED, syn.TID[name], n,
                         scale_lo=bench.MX_SCALES[0], scale_hi=bench.MX_SCALES[1], layer=li)
        return oracle.mxfp4_decode(buf.numpy(), shape)
    q_c = mx_cpu((st.B, 1, HI, dI), "q_idx")[b:b + 1]
    k_c = mx_cpu((st.B, L, dI), "kic")[b:b + 1]
    w_c = syn.make((st.B, 1, HI), bench.SEED, syn.TID["w_idx"], scale=HI ** -0.5, layer=li).double().numpy()[b:b + 1]
    idx_c, sc = oracle.index_topk(q_c, k_c, m, k, w=w_c, n_ctx=st.n_ctx)
    got_idx = lay["idx"].cpu().numpy()[b, 0]
    nv = st.nv_csa
    eps = index_eps(q_c[0, 0], w_c[0, 0], k_c[0])[:nv]
    assert near_tie_check(got_idx, idx_c[0, 0], sc[0, 0], nv, k, eps) <= 2

    # attention over the GPU's selection: FP8 K/V rows and window, bf16 query
    f8 = torch.float8_e4m3fn
    sel = got_idx[got_idx >= 0]
    kc_c = np.zeros((1, L, d))
    vc_c = np.zeros((1, L, d))
    for name, arr in (("kc", kc_c), ("vc", vc_c)):
        rows = syn.rows((st.B, L, d), b * L + sel, bench.SEED, syn.TID[name], dtype=f8, scale=1.0, layer=li)
        arr[0, sel] = oracle.fp8_decode(rows.view(torch.uint8).numpy())
    kr_c = oracle.fp8_decode(bench.raw_rows(st, "kr", li, t - W + 1, W, d, "cpu", 1.0, f8)[b:b + 1]
                             .view(torch.uint8).numpy())
    vr_c = oracle.fp8_decode(bench.raw_rows(st, "vr", li, t - W + 1, W, d, "cpu", 1.0, f8)[b:b + 1]
                             .view(torch.uint8).numpy())
    q = syn.make((st.B, 1, H, d), bench.SEED, syn.TID["q"], dtype=BF, scale=d ** -0.5, layer=li).double().numpy()
    sink = syn.make((H,), bench.SEED, syn.TID["sink"], layer=li).double().numpy()
    o_g, _ = oracle.sparse_attn(q[b:b + 1], kc_c, vc_c, got_idx[None, None], kr_c, vr_c, W, sink=sink,
                                scale=state.ascale, n_ctx=st.n_ctx)
    assert max_abs(to_np(lay["out"][b:b + 1]), o_g) <= BF16_TOL
    del state
    torch.cuda.empty_cache()
