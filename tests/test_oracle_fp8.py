"""Pins for the oracle's FP8 (OCP E4M3) storage helpers.

The pages allow FP8 for the main KV and FP8/FP4 for the indexer's q.k path
(shareware.cn Hybrid Attention article, the low-precision items of its
summary of what is compressed; the Lightning Indexer section of the trdm.cn
attention article) but name no encoding; E4M3 is the reading taken.  The
decoder is written from the format's definition and checked here against an
independent implementation (torch's float8_e4m3fn), named values and the
rounding rule."""
import numpy as np
import pytest
import torch

import oracle


def test_decode_all_codes_match_torch():
    d = oracle.fp8_decode(np.arange(256))
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t))
    ok = ~np.isnan(d)
    assert np.array_equal(d[ok], t[ok])
    assert np.array_equal(np.signbit(d[ok]), np.signbit(t[ok]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0xC0, -2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9), (0x01, 2.0 ** -9), (0x00, 0.0),
    (0x3C, 1.5), (0x34, 0.75),
])
def test_named_values(code, value):
    assert oracle.fp8_decode(code) == value


def test_nan_and_negative_zero():
    assert np.isnan(oracle.fp8_decode(0x7F)) and np.isnan(oracle.fp8_decode(0xFF))
    z = oracle.fp8_decode(0x80)
    assert z == 0.0 and np.signbit(z)
    # no infinities: every other code is finite
    d = oracle.fp8_decode(np.arange(256))
    assert np.isfinite(d[[c for c in range(256) if c not in (0x7F, 0xFF)]]).all()


def test_encode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(oracle.fp8_encode(oracle.fp8_decode(codes)), codes)


def test_encode_ties_to_even():
    # midpoints between neighbours: the even mantissa wins
    assert oracle.fp8_encode(1.0625) == 0x38      # 1.0 (m=0) vs 1.125 (m=1)
    assert oracle.fp8_encode(1.1875) == 0x3A      # 1.125 (m=1) vs 1.25 (m=2)
    assert oracle.fp8_encode(2.0 ** -10) == 0x00  # 0 vs the smallest subnormal
    assert oracle.fp8_encode(3 * 2.0 ** -10) == 0x02
    assert oracle.fp8_encode(-1.0625) == 0xB8
    assert oracle.fp8_encode(463.0) == 0x7E


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(size=20000) * 0.09, rng.normal(size=20000) * 40.0])
    x = x.astype(np.float32).astype(np.float64)  # exactly representable in fp32 for torch
    t = torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_encode(x), t)


def test_encode_rejects_what_has_no_code():
    with pytest.raises(ValueError):
        oracle.fp8_encode(464.0)
    with pytest.raises(ValueError):
        oracle.fp8_encode(np.nan)


def test_oracle_reads_fp8_tensors_with_its_own_decoder():
    codes = torch.tensor([[0x38, 0x40, 0x01, 0xC0]], dtype=torch.uint8)
    got = oracle._f64(codes.view(torch.float8_e4m3fn))
    assert np.array_equal(got, np.array([[1.0, 2.0, 2.0 ** -9, -2.0]]))
