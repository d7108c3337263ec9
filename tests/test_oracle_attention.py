"""Pins for the oracle's sparse (CSA) and dense (HCA) attention with a sink.

The textbook pins use torch's scaled_dot_product_attention in float64 on the
CPU: block size 1, k >= n and a window of one token turn CSA into plain causal
MQA attention, and a sink is an extra key with a zero value whose logit is the
sink value.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa_mqa(q, K, V, tpos, sink=None, scale=None):
    """q [B,T,H,d], K/V [B,n,d]; causal over positions 0..t; optional sink."""
    B, T, H, d = q.shape
    n = K.shape[1]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)  # B H T d
    Kt = torch.from_numpy(K)[:, None].expand(B, H, n, d).contiguous()
    Vt = torch.from_numpy(V)[:, None].expand(B, H, n, d).contiguous()
    allowed = torch.tensor([[s <= t for s in range(n)] for t in tpos])
    mask = torch.zeros((H, T, n), dtype=torch.float64).masked_fill(~allowed[None], -torch.inf)
    if sink is not None:
        Kt = torch.cat([Kt, torch.zeros(B, H, 1, d, dtype=torch.float64)], 2)
        Vt = torch.cat([Vt, torch.zeros(B, H, 1, d, dtype=torch.float64)], 2)
        sc = torch.from_numpy(np.asarray(sink, dtype=np.float64))[:, None, None].expand(H, T, 1)
        mask = torch.cat([mask, sc], 2)
    out = F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask[None], scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


def _csa_as_dense_causal(q, K, V, tpos, sink=None):
    """Block size 1, idx = every visible entry, window of 1 (the token itself)."""
    B, T, H, d = q.shape
    n = K.shape[1]
    kc = oracle.compress(K, np.zeros_like(K), 1)
    vc = oracle.compress(V, np.zeros_like(V), 1)
    idx = np.full((B, T, n), -1, dtype=np.int32)
    for i, t in enumerate(tpos):
        idx[:, i, :t] = np.arange(t)
    return oracle.sparse_attn(q, kc, vc, idx, K, V, 1, sink=sink, n_ctx=n, tpos=tpos)


def test_block1_csa_equals_causal_mqa_textbook():
    B, n, H, d, T = 2, 24, 4, 8, 6
    q, K, V = _rand((B, T, H, d), 1), _rand((B, n, d), 2), _rand((B, n, d), 3)
    tpos = list(range(n - T, n))
    out, _ = _csa_as_dense_causal(q, K, V, tpos)
    np.testing.assert_allclose(out, _sdpa_mqa(q, K, V, tpos), atol=1e-13)


def test_sink_is_an_extra_logit_with_no_value():
    B, n, H, d, T = 1, 16, 3, 4, 4
    q, K, V = _rand((B, T, H, d), 4), _rand((B, n, d), 5), _rand((B, n, d), 6)
    sink = _rand((H,), 7)
    tpos = [0, 3, 9, 15]
    out, lse = _csa_as_dense_causal(q, K, V, tpos, sink=sink)
    np.testing.assert_allclose(out, _sdpa_mqa(q, K, V, tpos, sink=sink), atol=1e-13)
    # lse against torch.logsumexp over the causal logits and the sink logit
    for i, t in enumerate(tpos):
        lg = torch.from_numpy(np.einsum("hd,sd->hs", q[0, i], K[0, : t + 1]) / np.sqrt(d))
        ref = torch.logsumexp(torch.cat([lg, torch.from_numpy(sink)[:, None]], 1), 1)
        np.testing.assert_allclose(lse[0, i], ref.numpy(), atol=1e-13)


def _onehot_case(nrows, d, seed):
    """Value rows e_0, e_1, ...: the output of a head is its probability vector."""
    assert nrows <= d
    V = np.zeros((1, nrows, d))
    V[0, np.arange(nrows), np.arange(nrows)] = 1.0
    return V


def test_probability_mass_plus_sink_is_one():
    n, H, d = 12, 4, 16
    K = _rand((1, n, d), 8)
    V = _onehot_case(n, d, 0)
    q = _rand((1, 1, H, d), 9)
    sink = _rand((H,), 10)
    kc, vc = K[:, :8], V[:, :8]  # entries 0..7 stand for compressed rows
    idx = np.array([[[0, 2, 5, 7, -1]]], dtype=np.int32)
    out, lse = oracle.sparse_attn(q, kc, vc, idx, K, V, 3, sink=sink, n_ctx=n, tpos=[11])
    p = out[0, 0]
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1) + np.exp(sink - lse[0, 0]), 1.0, atol=1e-14)


def test_sink_example_from_pages(golden):
    g = golden("sink_mass.json")
    n, H, d = 4, 1, 4
    K = np.zeros((1, n, d))
    V = _onehot_case(n, d, 0)
    q = np.zeros((1, 1, H, d))  # every real logit is 0: sum of exp is the row count
    rows = 2
    sigma = np.log(g["sink_mass"] / g["real_mass"] * rows)
    idx = np.array([[[0, 1]]], dtype=np.int32)
    out, lse = oracle.sparse_attn(q, K, V, idx, K, V, 0, sink=[sigma], n_ctx=n, tpos=[3])
    np.testing.assert_allclose(out[0, 0, 0].sum(), g["real_mass"], atol=1e-15)
    np.testing.assert_allclose(np.exp(sigma - lse[0, 0, 0]), g["sink_mass"], atol=1e-15)


def test_sink_limits():
    n, H, d = 10, 2, 8
    K, V = _rand((1, n, d), 11), _rand((1, n, d), 12)
    q = _rand((1, 1, H, d), 13)
    idx = np.array([[[1, 3, 4]]], dtype=np.int32)
    big, _ = oracle.sparse_attn(q, K, V, idx, K, V, 2, sink=[1e4, 1e4], n_ctx=n, tpos=[9])
    assert np.abs(big).max() < 1e-300
    none, _ = oracle.sparse_attn(q, K, V, idx, K, V, 2, n_ctx=n, tpos=[9])
    small, _ = oracle.sparse_attn(q, K, V, idx, K, V, 2, sink=[-1e4, -1e4], n_ctx=n, tpos=[9])
    np.testing.assert_array_equal(none, small)


def test_output_invariant_to_index_order_and_padding():
    n, H, d, L = 40, 4, 8, 10
    K, V = _rand((1, n, d), 14), _rand((1, n, d), 15)
    kc, vc = _rand((1, L, d), 16), _rand((1, L, d), 17)
    q = _rand((1, 1, H, d), 18)
    a = np.array([[[0, 3, 4, 8, -1, -1]]], dtype=np.int32)
    b = np.array([[[-1, 8, 0, -1, 4, 3]]], dtype=np.int32)
    oa, la = oracle.sparse_attn(q, kc, vc, a, K, V, 5, n_ctx=n, tpos=[39])
    ob, lb = oracle.sparse_attn(q, kc, vc, b, K, V, 5, n_ctx=n, tpos=[39])
    np.testing.assert_allclose(oa, ob, atol=1e-14)
    np.testing.assert_allclose(la, lb, atol=1e-14)


@pytest.mark.parametrize("W", [0, 3, 64])
def test_sparse_with_every_visible_entry_equals_dense(W):
    B, n, m, H, d, T = 2, 64, 4, 4, 8, 5
    L = n // m
    kc, vc = _rand((B, L, d), 19), _rand((B, L, d), 20)
    R = T + max(W, 1) - 1
    kr, vr = _rand((B, R, d), 21), _rand((B, R, d), 22)
    q = _rand((B, T, H, d), 23)
    sink = _rand((H,), 24)
    tpos = np.arange(n - T, n)
    idx = np.full((B, T, L + 3), -1, dtype=np.int32)
    for i, t in enumerate(tpos):
        idx[:, i, : t // m] = np.arange(t // m)
    os_, ls_ = oracle.sparse_attn(q, kc, vc, idx, kr, vr, W, sink=sink, n_ctx=n)
    od, ld = oracle.dense_attn(q, kc, vc, m, kr, vr, W, sink=sink, n_ctx=n)
    np.testing.assert_allclose(os_, od, atol=1e-13)
    np.testing.assert_allclose(ls_, ld, atol=1e-13)


def test_dense_hca_block1_equals_causal_mqa_textbook():
    # block size 1, window of one token: HCA over every earlier entry plus the
    # token itself is causal attention
    B, n, H, d, T = 1, 20, 2, 8, 3
    q, K, V = _rand((B, T, H, d), 25), _rand((B, n, d), 26), _rand((B, n, d), 27)
    sink = _rand((H,), 28)
    tpos = [5, 12, 19]
    out, _ = oracle.dense_attn(q, K, V, 1, K, V, 1, sink=sink, n_ctx=n, tpos=tpos)
    np.testing.assert_allclose(out, _sdpa_mqa(q, K, V, tpos, sink=sink), atol=1e-13)


def test_window_clips_at_sequence_start():
    n, H, d = 8, 1, 4
    K, V = _rand((1, n, d), 29), _rand((1, n, d), 30)
    q = _rand((1, 1, H, d), 31)
    idx = np.full((1, 1, 4), -1, dtype=np.int32)
    out, _ = oracle.sparse_attn(q, K, V, idx, K, V, 128, n_ctx=n, tpos=[2])
    np.testing.assert_allclose(out, _sdpa_mqa(q, K, V, [2]), atol=1e-14)


def test_bad_index_is_rejected():
    K = _rand((1, 4, 2), 32)
    q = _rand((1, 1, 1, 2), 33)
    with pytest.raises(ValueError):
        oracle.sparse_attn(q, K, K, np.array([[[4]]], dtype=np.int32), K, K, 0, n_ctx=4)
