"""Pins for the oracle's entry counts, visibility and block-weighted compression.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden), closed forms, invariants, or scipy's softmax.
"""
import numpy as np
import pytest
import scipy.special

import oracle


def test_entry_counts_match_pages(golden):
    g = golden("counts.json")
    assert oracle.num_entries(g["n_tokens"], g["csa_block"]) == g["csa_entries"]
    assert oracle.num_entries(g["n_tokens"], g["hca_block"]) == g["hca_entries"]


def test_block24_causality_example(golden):
    g = golden("causal_block24.json")
    m, t = g["block"], g["query_position"]
    nv = oracle.num_visible(t, m)
    assert nv == g["visible_blocks"]  # blocks 0..23 readable
    blk = list(range(24 * m, 25 * m))
    assert blk == g["block_24_tokens"]
    assert 24 >= nv  # block 24 (holds the future token 99) is not readable
    # the raw window of 128 tokens ending at t covers the same-block history
    lo = max(0, t - 128 + 1)
    assert all(lo <= u <= t for u in g["window_must_cover"])


def test_visibility_is_strict_at_block_end():
    # a block whose last token is t itself is not strictly before t
    assert oracle.num_visible(99, 4) == 24
    assert oracle.num_visible(100, 4) == 25
    assert oracle.num_visible(0, 4) == 0
    assert oracle.num_visible(127, 128) == 0
    assert oracle.num_visible(128, 128) == 1


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("n,m", [(16, 4), (18, 4), (300, 128), (5, 1)])
def test_uniform_logits_give_mean_pooling(n, m):
    x = _rand((2, n, 6), 1)
    z = np.zeros_like(x)
    out = oracle.compress(x, z, m)
    L = -(-n // m)
    assert out.shape == (2, L, 6)
    for j in range(L):
        ref = x[:, j * m:min(n, (j + 1) * m), :].mean(axis=1)
        np.testing.assert_allclose(out[:, j], ref, rtol=0, atol=1e-13)


def test_block_size_one_is_identity():
    x = _rand((2, 9, 5), 2)
    z = _rand((2, 9, 5), 3)
    np.testing.assert_array_equal(oracle.compress(x, z, 1), x)


def test_constant_block_gives_the_constant_and_convexity():
    x = _rand((1, 32, 8), 4)
    z = 3 * _rand((1, 32, 8), 5)
    out = oracle.compress(x, z, 4)
    blk = x.reshape(1, 8, 4, 8)
    assert np.all(out <= blk.max(axis=2) + 1e-14)
    assert np.all(out >= blk.min(axis=2) - 1e-14)
    c = np.full((1, 8, 3), 0.625)
    np.testing.assert_allclose(oracle.compress(c, _rand((1, 8, 3), 6), 4), 0.625, atol=1e-15)


def test_shift_invariance_per_block_and_channel():
    x = _rand((2, 16, 4), 7)
    z = _rand((2, 16, 4), 8)
    shift = np.repeat(_rand((2, 4, 4), 9) * 10, 4, axis=1)  # constant within a block
    np.testing.assert_allclose(oracle.compress(x, z + shift, 4), oracle.compress(x, z, 4),
                               atol=1e-13)


def test_closed_form_two_tokens():
    # logits (0, ln 3) give weights 1/4, 3/4
    x = np.array([[[2.0], [6.0]]])
    z = np.array([[[0.0], [np.log(3.0)]]])
    np.testing.assert_allclose(oracle.compress(x, z, 2)[0, 0, 0], 2 * 0.25 + 6 * 0.75,
                               atol=1e-14)


def test_single_path_against_scipy_softmax():
    B, n, D, m = 2, 23, 5, 4
    x, z = _rand((B, n, D), 10), _rand((B, n, D), 11)
    bias = _rand((m, D), 12)
    out = oracle.compress(x, z, m, bias=bias)
    for j in range(-(-n // m)):
        lo, hi = j * m, min(n, (j + 1) * m)
        w = scipy.special.softmax(z[:, lo:hi] + bias[: hi - lo][None], axis=1)
        np.testing.assert_allclose(out[:, j], (w * x[:, lo:hi]).sum(axis=1), atol=1e-13)


def test_two_path_against_scipy_softmax(golden):
    g = golden("two_path_blocks.json")
    B, n, D, m = 2, 22, 3, g["block"]
    xa, za, xb, zb = (_rand((B, n, D), s) for s in (20, 21, 22, 23))
    bias = _rand((2 * m, D), 24)
    out = oracle.compress(xa, za, m, x_b=xb, z_b=zb, bias=bias)
    for j in range(-(-n // m)):
        a = list(range(j * m, min(n, (j + 1) * m)))
        b = list(range((j - 1) * m, j * m)) if j >= 1 else []
        if j == g["entry"]:
            assert a == g["a_path_tokens"] and b == g["b_path_tokens"]
        lg = np.concatenate([zb[:, b] + bias[:len(b)][None], za[:, a] + bias[m:m + len(a)][None]], 1)
        val = np.concatenate([xb[:, b], xa[:, a]], axis=1)
        w = scipy.special.softmax(lg, axis=1)
        np.testing.assert_allclose(out[:, j], (w * val).sum(axis=1), atol=1e-13)


def test_two_path_with_silent_b_stream_equals_single_path():
    B, n, D, m = 1, 20, 4, 4
    xa, za, xb = _rand((B, n, D), 30), _rand((B, n, D), 31), _rand((B, n, D), 32)
    zb = np.full((B, n, D), -np.inf)
    np.testing.assert_allclose(oracle.compress(xa, za, m, x_b=xb, z_b=zb),
                               oracle.compress(xa, za, m), atol=1e-15)


def test_two_path_is_causal_and_uses_previous_block():
    B, n, D, m = 1, 24, 4, 4
    xa, za, xb, zb = (_rand((B, n, D), s) for s in (40, 41, 42, 43))
    base = oracle.compress(xa, za, m, x_b=xb, z_b=zb)
    j = 3  # tokens 12..15 (A) and 8..11 (B)
    for arr in (xa, xb):
        pert = arr.copy()
        pert[:, (j + 1) * m:] += 5.0  # future tokens
        args = dict(x_b=pert if arr is xb else xb, z_b=zb)
        got = oracle.compress(pert if arr is xa else xa, za, m, **args)
        np.testing.assert_array_equal(got[:, : j + 1], base[:, : j + 1])
    pert = xb.copy()
    pert[:, (j - 1) * m] += 5.0  # previous block through stream B changes entry j
    got = oracle.compress(xa, za, m, x_b=pert, z_b=zb)
    assert np.abs(got[:, j] - base[:, j]).max() > 1e-6
    np.testing.assert_array_equal(got[:, j - 2], base[:, j - 2])


def test_bias_rows_address_positions():
    # a dominant bias on one position makes the entry equal that token's value
    B, n, D, m = 1, 12, 2, 4
    xa, za, xb, zb = (_rand((B, n, D), s) for s in (50, 51, 52, 53))
    for r in range(2 * m):
        bias = np.zeros((2 * m, D))
        bias[r] = 1e4
        out = oracle.compress(xa, za, m, x_b=xb, z_b=zb, bias=bias)
        j = 2
        src = xb[:, (j - 1) * m + r] if r < m else xa[:, j * m + (r - m)]
        np.testing.assert_allclose(out[:, j], src, atol=1e-12)


def test_subrange_equals_full():
    B, n, D, m = 2, 40, 3, 4
    xa, za, xb, zb = (_rand((B, n, D), s) for s in (60, 61, 62, 63))
    full = oracle.compress(xa, za, m, x_b=xb, z_b=zb)
    p0, e0, e1 = 12, 4, 10  # entry 4 reads tokens 12..19
    sub = oracle.compress(xa[:, p0:], za[:, p0:], m, x_b=xb[:, p0:], z_b=zb[:, p0:],
                          n=n, p0=p0, e0=e0, e1=e1)
    np.testing.assert_array_equal(sub, full[:, e0:e1])
    with pytest.raises(ValueError):
        oracle.compress(xa[:, p0:], za[:, p0:], m, x_b=xb[:, p0:], z_b=zb[:, p0:], n=n,
                        p0=p0, e0=3, e1=10)
