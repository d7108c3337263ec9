"""Pins for the oracle's Lightning Indexer scores and its top-k selection."""
import numpy as np
import pytest

import oracle


def test_relu_example_from_pages(golden):
    g = golden("relu_heads.json")
    h = np.array(g["head_scores"], dtype=np.float64)
    # two heads, d_I = 2, one key e_0: head dots are exactly 8 and -7
    q = np.zeros((1, 1, 2, 2))
    q[0, 0, :, 0] = h
    k = np.array([[[1.0, 0.0]]])
    sc = oracle.index_scores(q, k, 1, n_ctx=2)
    assert sc[0, 0, 0] == g["sum_with_relu"]
    assert sc[0, 0, 0] != g["sum_without_relu"]
    assert h.sum() == g["sum_without_relu"]


def test_single_positive_head_is_a_matrix_product():
    # with one head and non-negative operands, ReLU is inactive and the score
    # is the plain dot product: a numpy matmul
    rng = np.random.default_rng(0)
    q = np.abs(rng.standard_normal((2, 3, 1, 16)))
    k = np.abs(rng.standard_normal((2, 40, 16)))
    sc = oracle.index_scores(q, k, 1, tpos=[40, 40, 40])
    ref = np.matmul(k, q[:, :, 0, :].transpose(0, 2, 1)).transpose(0, 2, 1)
    np.testing.assert_allclose(sc, ref, rtol=1e-14)


def test_all_positive_heads_reduce_to_weighted_query():
    rng = np.random.default_rng(1)
    q = np.abs(rng.standard_normal((1, 2, 4, 8)))
    w = rng.uniform(0, 1, (1, 2, 4))
    k = np.abs(rng.standard_normal((1, 30, 8)))
    sc = oracle.index_scores(q, k, 1, w=w, tpos=[30, 30])
    qe = (w[..., None] * q).sum(axis=2)  # [1, 2, 8]
    np.testing.assert_allclose(sc, np.matmul(qe, k.transpose(0, 2, 1)), rtol=1e-13)


def test_negative_heads_contribute_nothing_and_weights_are_linear():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 6, 8))
    k = rng.standard_normal((1, 50, 8))
    w = rng.uniform(0, 1, (1, 1, 6))
    base = oracle.index_scores(q, k, 1, w=w, n_ctx=51)
    np.testing.assert_allclose(oracle.index_scores(q, k, 1, w=2 * w, n_ctx=51), 2 * base,
                               rtol=1e-15)
    assert np.all(oracle.index_scores(q, k, 1, n_ctx=51) >= 0)
    # a head flipped to all-negative dots against every key adds zero
    q2 = np.concatenate([q, np.zeros((1, 1, 1, 8))], axis=2)
    q2[0, 0, 6, 0] = -1.0
    k2 = k.copy()
    k2[..., 0] = np.abs(k2[..., 0]) + 0.1
    w2 = np.concatenate([w, [[[5.0]]]], axis=2)
    np.testing.assert_allclose(oracle.index_scores(q2, k2, 1, w=w2, n_ctx=51),
                               oracle.index_scores(q, k2, 1, w=w, n_ctx=51), rtol=1e-15)


def test_visibility_masks_future_blocks():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 3, 2, 4))
    k = rng.standard_normal((1, 10, 4))
    sc = oracle.index_scores(q, k, 4, tpos=[3, 4, 39])
    assert np.all(np.isneginf(sc[0, 0]))          # t=3: nothing complete
    assert np.isfinite(sc[0, 1, 0]) and np.all(np.isneginf(sc[0, 1, 1:]))
    assert np.all(np.isfinite(sc[0, 2, :9])) and np.isneginf(sc[0, 2, 9])


def _brute_topk(v, nv, k):
    """Rank counting: entry s is kept iff fewer than k visible entries beat it,
    where s' beats s if v[s'] > v[s], or v[s'] == v[s] and s' < s."""
    keep = []
    for s in range(nv):
        beat = sum(1 for s2 in range(nv) if v[s2] > v[s] or (v[s2] == v[s] and s2 < s))
        if beat < k:
            keep.append(s)
    return keep + [-1] * (k - len(keep))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_count_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, L = 5, 37
    v = rng.integers(-3, 4, (R, L)).astype(np.float64)  # many ties
    v[v == 0] = np.where(rng.random((v == 0).sum()) < 0.5, -0.0, 0.0)  # mixed signed zeros
    nvis = rng.integers(0, L + 1, R)
    for k in (1, 4, 16, 40):
        got = oracle.topk(v, nvis, k)
        for r in range(R):
            assert got[r].tolist() == _brute_topk(v[r], int(nvis[r]), k)


def test_topk_matches_python_stable_sort():
    rng = np.random.default_rng(9)
    v = np.round(rng.standard_normal((4, 200)), 1)
    nv = np.array([200, 150, 3, 0])
    got = oracle.topk(v, nv, 16)
    for r in range(4):
        order = sorted(range(int(nv[r])), key=lambda s: -v[r, s])  # Python's sort is stable
        want = sorted(order[:16]) + [-1] * (16 - min(16, int(nv[r])))
        assert got[r].tolist() == want


def test_signed_zeros_tie_to_lower_index():
    v = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0]])
    assert oracle.topk(v, [5], 2).tolist() == [[0, 1]]
    v = np.array([[0.0, -0.0, -1.0, -0.0]])
    assert oracle.topk(v, [4], 3).tolist() == [[0, 1, 3]]


def test_index_topk_small_k_ge_visible_selects_everything():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 2, 4))
    k = rng.standard_normal((1, 8, 4))
    idx, _ = oracle.index_topk(q, k, 4, 16, tpos=[17, 30])
    assert idx[0, 0].tolist() == [0, 1, 2, 3] + [-1] * 12
    assert idx[0, 1].tolist() == list(range(7)) + [-1] * 9
