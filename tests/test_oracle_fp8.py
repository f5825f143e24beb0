"""Pins of the oracle's FP8 E4M3 codes (CPU only).

Facts outside the oracle: torch's own float8_e4m3fn dtype (an independent
implementation of the OCP E4M3 format), values the format definition fixes
(largest finite value, smallest normal and subnormal, named codes, ties to
even), and the round trip over all 256 codes. Each pin also runs against
deliberately broken codecs, each of which must fail at least one pin.
"""

import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_encode(y):
    t = torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _probe_values():
    mags = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    quarters = mags[:-1] + (mags[1:] - mags[:-1]) / 4
    rng = np.random.default_rng(11)
    rand = rng.uniform(-448, 448, 4000)
    tiny = rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000)
    vals = np.concatenate([mags, -mags, mids, -mids, quarters, -quarters, rand, tiny])
    return vals.astype(np.float32)


# ---------------------------------------------------------------- pins ----
def pin_decode_matches_torch(dec, enc):
    codes = np.arange(256, dtype=np.uint8)
    got, want = dec(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def pin_encode_matches_torch(dec, enc):
    y = _probe_values()
    assert np.array_equal(enc(y), _torch_encode(y))


def pin_named_values(dec, enc):
    # (value, code) pairs fixed by the format: bias 7, 3 mantissa bits, max 448
    named = [(1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
             (7 * 2.0 ** -9, 0x07), (240.0, 0x77), (0.0, 0x00), (-0.0, 0x80), (-1.0, 0xB8),
             (1.75, 0x3E), (0.5, 0x30)]
    for v, c in named:
        assert int(enc(np.float32(v))) == c, (v, hex(c))
        assert dec(np.uint8(c)) == v
    assert np.isnan(dec(np.uint8(0x7F))) and np.isnan(dec(np.uint8(0xFF)))


def pin_ties_to_even(dec, enc):
    ties = [(2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (1.0625, 0x38), (1.1875, 0x3A),
            (-1.0625, 0xB8), (432.0, 0x7E), (5 * 2.0 ** -10, 0x02)]
    for v, c in ties:
        assert int(enc(np.float32(v))) == c, (v, hex(c))


def pin_round_trip(dec, enc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(enc(dec(codes).astype(np.float32)), codes)


PINS = [pin_decode_matches_torch, pin_encode_matches_torch, pin_named_values, pin_ties_to_even,
        pin_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_fp8_pins(pin):
    pin(fp8.e4m3_decode, fp8.e4m3_encode)


def test_quantize_scale_and_clamp():
    s = 2.0 ** -6
    assert int(fp8.quantize(np.float32(1.0), s)) == 0x68  # y = 64 = 1.0 * 2^6
    assert int(fp8.quantize(np.float32(10.0), s)) == 0x7E  # 640 clamps to 448
    assert int(fp8.quantize(np.float32(-10.0), s)) == 0xFE
    x = np.random.default_rng(3).standard_normal(10000).astype(np.float32)
    back = fp8.dequantize(fp8.quantize(x, s), s)
    # within half a step of the format: relative 2^-4 for normals, absolute 2^-10 * s below
    err = np.abs(back - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) + 1e-12)
    # division is in fp32: a non-power-of-two scale quantizes x / scale, not x * (1 / scale)
    s2 = np.float32(0.3)
    y = np.float32(0.7) / s2
    assert int(fp8.quantize(np.float32(0.7), float(s2))) == int(fp8.e4m3_encode(y))


def test_quantize_non_finite_and_overflow():
    """Reading for values the format cannot hold: NaN of either sign or any
    payload -> the NaN code 0x7F; +-inf, and finite values whose fp32 quotient
    overflows, saturate to +-448 (0x7E / 0xFE)."""
    bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFBFFFFF], dtype=np.uint32)
    nans = bits.view(np.float32)
    assert np.all(fp8.quantize(nans, 0.5) == 0x7F)
    assert np.all(fp8.quantize(nans, 2.0 ** -6) == 0x7F)
    inf = np.array([np.inf, -np.inf], dtype=np.float32)
    assert list(fp8.quantize(inf, 0.0123)) == [0x7E, 0xFE]
    big = np.array([3.0e38, -3.0e38], dtype=np.float32)  # 3e38 / 1e-3 overflows fp32
    assert list(fp8.quantize(big, 1e-3)) == [0x7E, 0xFE]
    # a NaN among finite values leaves the others alone
    mixed = np.array([1.0, np.nan, -1.0], dtype=np.float32)
    assert list(fp8.quantize(mixed, 2.0 ** -6)) == [0x68, 0x7F, 0xE8]
    # the NaN code decodes to NaN, the saturated codes to +-448
    assert np.isnan(fp8.e4m3_decode(np.uint8(0x7F)))
    assert list(fp8.e4m3_decode(np.array([0x7E, 0xFE], dtype=np.uint8))) == [448.0, -448.0]


# ----------------------------------------------------- planted mistakes ----
def _enc_truncate(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    mags = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    idx = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 126).astype(np.uint8)
    return np.where(np.signbit(y), idx | np.uint8(0x80), idx).astype(np.uint8)


def _enc_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    mags = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    pick_lo = (a - mags[lo]) < (mags[hi] - a)
    idx = np.where(pick_lo, lo, hi).astype(np.uint8)
    return np.where(np.signbit(y), idx | np.uint8(0x80), idx).astype(np.uint8)


def _dec_bias8(codes):
    return fp8.e4m3_decode(codes) / 2.0


def _enc_no_sign_zero(y):
    c = fp8.e4m3_encode(y)
    return np.where(c == 0x80, np.uint8(0), c).astype(np.uint8)


MUTANTS = {
    "truncating encoder": (fp8.e4m3_decode, _enc_truncate),
    "ties away from zero": (fp8.e4m3_decode, _enc_ties_away),
    "exponent bias 8": (_dec_bias8, fp8.e4m3_encode),
    "signed zero lost": (fp8.e4m3_decode, _enc_no_sign_zero),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_codec_mistakes_are_caught(name):
    dec, enc = MUTANTS[name]
    caught = 0
    for pin in PINS:
        try:
            pin(dec, enc)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin catches: {name}"
