"""Pins of the oracle's number codecs against their format definitions and library routines."""
import numpy as np
import pytest
import torch

from oracle.codecs import (E4M3_VALUES, bf16_bits, bf16_from_bits, bf16_round, e4m3_decode,
                           e4m3_encode)


def _finite_f32_patterns(rng, n):
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_matches_torch_rne_on_all_high_halves():
    # every sign/exponent/top-7-fraction pattern, with low halves below, at and above the tie
    hi = np.arange(2**16, dtype=np.uint32) << 16
    for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
        f = (hi | np.uint32(low)).view(np.float32)
        f = f[np.isfinite(f)]
        ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(bf16_bits(f), ref)


def test_bf16_matches_torch_on_random_patterns():
    f = _finite_f32_patterns(np.random.default_rng(1), 2_000_000)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(f), ref)


def test_bf16_hand_cases():
    one = 1.0
    assert bf16_round(one + 2.0**-8) == 1.0                      # tie, even side is 1.0
    assert bf16_round(one + 3 * 2.0**-8) == one + 2.0**-6        # tie, even side rounds up
    assert bf16_round(one + 2.0**-8 + 2.0**-20) == one + 2.0**-7  # above the tie
    assert bf16_round(-(one + 2.0**-8)) == -1.0
    assert bf16_round(2.0**-133) == 2.0**-133                    # smallest bf16 subnormal
    assert bf16_round(2.0**-134) == 0.0                          # tie to even zero
    assert np.isinf(bf16_round(np.float32(3.4e38)))              # rounds past the largest bf16
    np.testing.assert_array_equal(bf16_from_bits(np.array([0x3F80, 0xC000])), [1.0, -2.0])


def test_e4m3_table_known_codes():
    v = E4M3_VALUES
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0**-9 and v[0x07] == 7 * 2.0**-9     # subnormals
    assert v[0x08] == 2.0**-6                                # smallest normal
    assert v[0x38] == 1.0 and v[0x3A] == 1.25
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                          # codes are monotone in value


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_e4m3_hand_ties_and_saturation():
    cases = {
        1.0625: 0x38,          # between 1.0 (m=0) and 1.125 (m=1): tie to even -> 1.0
        1.1875: 0x3A,          # between 1.125 (m=1) and 1.25 (m=2): tie to even -> 1.25
        1.3125: 0x3A,          # between 1.25 (m=2) and 1.375 (m=3): tie to even -> 1.25
        2.0**-10: 0x00,        # half the smallest subnormal: tie to even zero
        3 * 2.0**-10: 0x02,    # between m=1 and m=2 subnormals: tie to even -> m=2
        500.0: 0x7E, 1e30: 0x7E, np.inf: 0x7E, 448.0: 0x7E, 440.0: 0x7E,
        -500.0: 0xFE, -np.inf: 0xFE,
        -2.0**-11: 0x80,       # rounds to negative zero
    }
    for x, c in cases.items():
        assert int(e4m3_encode(np.float32(x))) == c, (x, hex(int(e4m3_encode(np.float32(x)))), hex(c))
    assert int(e4m3_encode(np.float32(np.nan))) == 0x7F


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(2)
    finite = E4M3_VALUES[np.isfinite(E4M3_VALUES)]
    mids = (np.sort(finite)[1:] + np.sort(finite)[:-1]) / 2
    xs = np.concatenate([
        finite, mids, mids * (1 + 2.0**-20), mids * (1 - 2.0**-20),
        rng.normal(0, 30, 500_000), rng.normal(0, 0.01, 200_000),
        _finite_f32_patterns(rng, 500_000),
    ]).astype(np.float32)
    xs = xs[np.abs(xs) <= 448.0]
    ref = torch.from_numpy(xs.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(xs), ref)
