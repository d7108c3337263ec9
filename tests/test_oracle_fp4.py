"""Pins of the oracle's MXFP4 decoding (CPU).

The pages run the indexer's q.k in FP4 without naming an encoding
(shareware.cn Hybrid Attention article, its list of what is compressed); the
MXFP4 reading (E2M1 elements, one E8M0 scale per 32) is pinned here through
checks that do not restate the decoder: the generic minifloat decoder against
torch's 8-bit float types, E8M0 against torch's float8_e8m0fnu, E2M1 values
against the independently pinned E4M3 encoder, and the block layout through
buffers with a single non-zero element or a single changed scale."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_decode(dtype):
    return torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


def test_minifloat_decoder_matches_torch_e4m3_on_every_finite_code():
    codes = np.arange(256)
    want = _torch_decode(torch.float8_e4m3fn)
    fin = (codes & 0x7F) != 0x7F
    got = oracle.minifloat_decode(codes, 4, 3, 7)
    assert np.array_equal(got[fin], want[fin])


def test_minifloat_decoder_matches_torch_e5m2_on_every_finite_code():
    codes = np.arange(256)
    want = _torch_decode(torch.float8_e5m2)
    fin = ((codes >> 2) & 0x1F) != 0x1F
    got = oracle.minifloat_decode(codes, 5, 2, 15)
    assert np.array_equal(got[fin], want[fin])


def test_e8m0_matches_torch_on_all_codes():
    want = _torch_decode(torch.float8_e8m0fnu)
    got = oracle.e8m0_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_e2m1_values_are_e4m3_values_and_symmetric():
    v = oracle.e2m1_decode(np.arange(16))
    # every E2M1 value is exactly representable in E4M3 (3 fraction bits >= 1)
    assert np.array_equal(oracle.fp8_decode(oracle.fp8_encode(v)), v)
    assert np.array_equal(v[8:], -v[:8])            # the top bit is the sign
    assert np.all(np.diff(v[:8]) > 0)               # codes ascend with the value
    assert v[0] == 0.0 and v[1] == 0.5 and v[7] == 6.0  # smallest subnormal, largest finite
    assert len(set(np.abs(v).tolist())) == 8


def test_mxfp4_single_element_lands_at_its_position():
    rows, d = 3, 64
    n = rows * d
    for r, e, code, sc in ((0, 0, 0x2, 127), (1, 33, 0x7, 130), (2, 63, 0xB, 120), (2, 2, 0x5, 127)):
        buf = np.zeros(n // 2 + n // 32, dtype=np.uint8)
        buf[n // 2:] = 127
        flat = r * d + e
        buf[flat // 2] = code << (4 * (flat % 2))
        buf[n // 2 + r * (d // 32) + e // 32] = sc
        got = oracle.mxfp4_decode(buf, (rows, d))
        want = np.zeros((rows, d))
        want[r, e] = oracle.e2m1_decode(code) * 2.0 ** (sc - 127)
        assert np.array_equal(got, want)


def test_mxfp4_scale_covers_exactly_its_32_elements():
    rows, d = 2, 128
    n = rows * d
    buf = np.full(n // 2 + n // 32, 0x22, dtype=np.uint8)  # every element 1.0
    buf[n // 2:] = 127
    base = oracle.mxfp4_decode(buf, (rows, d))
    assert np.all(base == 1.0)
    buf[n // 2 + 1 * 4 + 2] = 129  # row 1, block 2
    got = oracle.mxfp4_decode(buf, (rows, d))
    changed = got != base
    assert changed.sum() == 32 and np.all(changed[1, 64:96]) and np.all(got[1, 64:96] == 4.0)


def test_mxfp4_generator_is_deterministic_and_in_range():
    n = 64 * 128
    a = syn.mxfp4_(torch.empty(n // 2 + n // 32, dtype=torch.uint8), 3, syn.TID["k_idx"], n, scale_lo=125,
                   scale_hi=129)
    b = syn.mxfp4_(torch.empty(n // 2 + n // 32, dtype=torch.uint8), 3, syn.TID["k_idx"], n, scale_lo=125,
                   scale_hi=129)
    assert torch.equal(a, b)
    sc = a[n // 2:].numpy()
    assert sc.min() >= 125 and sc.max() <= 129 and len(np.unique(sc)) == 5
    assert len(np.unique(a[: n // 2].numpy())) > 100  # code bytes spread over the range


# ---- the encoder (compression writes MXFP4 index keys) ----------------------
# Pinned against the decoder above and by brute force, never by retyping its
# rule: every representable block survives a round trip, each element is the
# nearest of the 15 values at its block's scale, the named midpoints go to the
# even code, and the scale is the one power of two that puts the block's
# largest magnitude in [4, 8).

def _all_values_at(E):
    return oracle.e2m1_decode(np.arange(16)) * 2.0 ** E


def test_mxfp4_encode_round_trips_every_representable_block():
    rng = np.random.default_rng(3)
    rows, d = 64, 128
    codes = rng.integers(0, 16, size=(rows * d // 32, 32))
    # one element per block of magnitude 4 or 6 (codes 6 / 7, either sign) fixes
    # the block's scale as the one it was drawn with
    codes[np.arange(codes.shape[0]), rng.integers(0, 32, size=codes.shape[0])] = \
        rng.choice([6, 7, 14, 15], size=codes.shape[0])
    flat = codes.reshape(-1)
    scales = rng.integers(1, 250, size=rows * d // 32)
    buf = np.concatenate([(flat[0::2] | (flat[1::2] << 4)), scales]).astype(np.uint8)
    x = oracle.mxfp4_decode(buf, (rows, d))
    assert np.array_equal(oracle.mxfp4_encode(x), buf)


def test_mxfp4_encode_picks_the_nearest_value_at_the_block_scale():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 64)) * np.exp2(rng.integers(-20, 20, size=(40, 1)))
    buf = oracle.mxfp4_encode(x)
    got = oracle.mxfp4_decode(buf, x.shape)
    scale = oracle.e8m0_decode(buf[x.size // 2:]).reshape(40, 2)
    for r in range(40):
        for j in range(2):
            blk = x[r, 32 * j:32 * j + 32]
            s = scale[r, j]
            assert 4.0 <= np.abs(blk).max() / s < 8.0
            vals = _all_values_at(np.log2(s))
            best = np.abs(blk[:, None] - vals[None, :]).min(axis=1)
            assert np.array_equal(np.abs(got[r, 32 * j:32 * j + 32] - blk), best)


def test_mxfp4_encode_named_ties_saturation_and_signs():
    # scale 2^0 (the block holds 4.0); each midpoint goes to the even code
    vals = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.5, -0.3, -0.1, 0.0, -0.0, 6.0, 5.5, 2.75]
    want = [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -0.5, -0.0, 0.0, -0.0, 6.0, 6.0, 3.0]
    x = np.array([vals + [0.0] * 16])
    buf = oracle.mxfp4_encode(x)
    assert buf[-1] == 127
    got = oracle.mxfp4_decode(buf, x.shape)[0, :16]
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(np.array(want)))
    # codes: -0.1 rounds to zero but keeps the sign bit (code 8)
    assert (buf[5] & 0xF) == 8


def test_mxfp4_encode_scale_clamps():
    x = np.zeros((1, 32))
    assert oracle.mxfp4_encode(x)[-1] == 0            # an all-zero block: the smallest scale
    x[0, 3] = 2.0 ** -140                              # below 4 * 2^-127: still the smallest scale
    buf = oracle.mxfp4_encode(x)
    assert buf[-1] == 0 and np.array_equal(oracle.mxfp4_decode(buf, x.shape), np.zeros((1, 32)))
    x[0, 3] = 2.0 ** -120 * 3                          # floor(log2) = -119 -> E = -121
    assert oracle.mxfp4_encode(x)[-1] == 127 - 121
    with pytest.raises(ValueError):
        oracle.mxfp4_encode(np.full((1, 32), np.nan))
