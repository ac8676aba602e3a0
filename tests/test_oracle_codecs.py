"""Pins for the oracle's number formats (bf16 and OCP E4M3FN).

The pages only say "FP8" / "8-bit"; the format is OCP E4M3FN (bias 7, max 448, no infinities).
Pins: the spec's closed-form values, torch's own casts (an independent library implementation of the
same formats), exhaustive round trips and the tie/saturation rules.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = []


def _torch_e4m3_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_decode_closed_forms(orc):
    dec = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    # spec values: smallest subnormal, largest subnormal, smallest normal, one, largest finite
    assert dec[0x00] == 0.0 and not math.copysign(1.0, dec[0x00]) < 0
    assert dec[0x01] == 2.0 ** -9
    assert dec[0x07] == 7 * 2.0 ** -9
    assert dec[0x08] == 2.0 ** -6
    assert dec[0x38] == 1.0
    assert dec[0x3C] == 1.5
    assert dec[0x7E] == 448.0
    assert math.isnan(dec[0x7F]) and math.isnan(dec[0xFF])
    assert dec[0x80] == 0.0 and math.copysign(1.0, dec[0x80]) < 0
    assert dec[0xFE] == -448.0
    # sign symmetry and monotonicity of the positive finite codes
    assert np.array_equal(dec[0x80:0xFF], -dec[0x00:0x7F])
    assert np.all(np.diff(dec[0x00:0x7F].astype(np.float64)) > 0)


def test_e4m3_decode_matches_torch_exhaustively(orc):
    dec = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_decode_all()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(dec), ~finite)
    assert np.array_equal(dec[finite].view(np.uint32), ref[finite].view(np.uint32))


def test_e4m3_encode_round_trip_every_code(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = orc.e4m3_decode(codes)
    assert np.array_equal(orc.e4m3_encode(vals), codes)


def test_e4m3_encode_ties_to_even_and_saturation(orc):
    dec = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (dec[:-1] + dec[1:]) / 2  # every midpoint is exactly representable in fp32
    got = orc.e4m3_encode(mids.astype(np.float32))
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    # a hair above / below each midpoint goes up / down
    above = np.nextafter(mids.astype(np.float32), np.float32(np.inf))
    below = np.nextafter(mids.astype(np.float32), np.float32(-np.inf))
    assert np.array_equal(orc.e4m3_encode(above), (lo + 1).astype(np.uint8))
    assert np.array_equal(orc.e4m3_encode(below), lo.astype(np.uint8))
    # satfinite: everything at or beyond 448 becomes +-448; NaN stays NaN
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e6, 3e38], dtype=np.float32)
    assert np.all(orc.e4m3_encode(big) == 0x7E)
    assert np.all(orc.e4m3_encode(-big) == 0xFE)
    assert orc.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F
    # below half the smallest subnormal rounds to signed zero; exactly half ties to zero (even)
    tiny = np.array([2.0 ** -11, 2.0 ** -10, -2.0 ** -11], dtype=np.float32)
    assert list(orc.e4m3_encode(tiny)) == [0x00, 0x00, 0x80]


def test_e4m3_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.uniform(0, 1, 20000) * 448.0,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(x), ref)


def test_bf16_matches_torch(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),  # subnormal range
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32),
    ])
    # exact ties: upper 16 bits odd / even with lower bits 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_from_f32(x)
    assert np.array_equal(got, ref)
    back = orc.bf16_to_f32(got)
    assert np.array_equal(back.view(np.uint32), (got.astype(np.uint32) << 16))
    assert orc.bf16_to_f32(orc.bf16_from_f32(np.array([np.nan], dtype=np.float32)))[0] != orc.bf16_to_f32(
        orc.bf16_from_f32(np.array([np.nan], dtype=np.float32)))[0]
