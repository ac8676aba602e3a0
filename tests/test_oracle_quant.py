"""Pins for the oracle's quantization steps: K mean (smoothing vector), per-block INT8 of Q and K',
per-channel E4M3 of V, the zero guard (all-zero channel -> no division by zero, TMAP I2V write-up,
section "优化算子细节"), and the exact integer scores.

Pins are hand-computed closed forms, error bounds that hold for any correct symmetric quantizer, and
numpy's int64 matmul as an independent computation of the integer scores.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch


def bf(x) -> np.ndarray:
    """fp32 values that are exactly representable in bf16 -> their 16-bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float32), torch.from_numpy(x)), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def rnd_bf(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------------------------------- INT8 blocks
def test_block_quant_hand_values(orc):
    # amax = 127 -> inv = 1 and scale = 1, so codes are x rounded half to even
    x = np.zeros((64, 64), dtype=np.float32)
    vals = [127.0, -127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, -0.5, 7.0, -100.0]
    x[0, :len(vals)] = vals
    codes, scales = orc.quant_q(bf(x), 64)
    assert scales[0] == np.float32(1.0)
    assert list(codes[0, :len(vals)]) == [127, -127, 2, 4, -2, -4, 0, 2, 126, 0, 7, -100]
    assert np.all(codes[1:] == 0)


def test_block_quant_scale_and_error_bound(orc):
    q = rnd_bf((300, 128), 11, 2.0)
    codes, scales = orc.quant_q(q, 128)
    assert codes.shape == (384, 128) and scales.shape == (3,)
    x = f32(q)
    for b in range(3):
        blk = x[b * 128:(b + 1) * 128]
        a = np.max(np.abs(blk))
        # the scale is amax/127 rounded once (fp32)
        assert Fraction(float(scales[b])) - Fraction(float(a)) / 127 <= Fraction(float(scales[b])) * Fraction(1, 2 ** 23)
        c = codes[b * 128:b * 128 + blk.shape[0]].astype(np.float64)
        assert np.max(np.abs(c)) == 127
        assert np.all(np.abs(c) <= 127)
        # round-to-nearest: |x/s - code| <= 1/2 (+ rounding of the reciprocal)
        err = np.abs(blk.astype(np.float64) * (127.0 / a) - c)
        assert np.max(err) <= 0.5 + 1e-4
        # the element holding the amax quantizes to +-127 with its sign
        i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        assert c[i] == 127 * np.sign(blk[i])
    # pad rows of the ragged tail block are zero
    assert np.all(codes[300:] == 0)


def test_zero_guard(orc):
    x = np.zeros((128, 64), dtype=np.float32)
    codes, scales = orc.quant_q(bf(x), 64)
    assert np.all(scales == 0) and np.all(codes == 0)
    # amax below 2^-100 is treated as zero; at 2^-99 it is not
    x[5, 3] = 2.0 ** -110
    x[70, 3] = 2.0 ** -99
    codes, scales = orc.quant_q(bf(x), 64)
    assert scales[0] == 0 and np.all(codes[:64] == 0)
    assert scales[1] > 0 and codes[70, 3] == 127 and np.all(np.isfinite(scales))
    # V: an all-zero channel gives scale 0 and codes 0, other channels unaffected
    v = rnd_bf((100, 16), 5)
    v[:, 7] = 0
    vc, vs = orc.quant_v(v)
    assert vs[7] == 0 and np.all(vc[:, 7] == 0)
    assert np.all(vs[np.arange(16) != 7] > 0)


# ------------------------------------------------------------------------------------------- K mean
def test_k_mean_constant_channel_is_exact(orc):
    k = np.full((256, 8), 0.5, dtype=np.float32)
    k[:, 1] = -3.0
    kb = bf(k)
    mu = orc.k_mean(kb)
    assert mu[0] == 0.5 and mu[1] == -3.0
    codes, scales = orc.quant_k(kb, 64, mu)
    # K' = K - mu is identically zero -> every K block hits the guard
    assert np.all(codes == 0) and np.all(scales == 0)


def test_k_mean_two_level_order(orc):
    # 2^24 followed by 127 ones.  Adding 1 to 2^24 in fp32 is a tie that rounds back to 2^24, so the
    # first 64-token run sums to 2^24 and the second to 64: total 16777280, mean 131072.5.
    # (A flat sequential sum would give 131072, a pairwise sum yet another value, the exact mean 131072.9921875.)
    k = np.ones((128, 1), dtype=np.float32)
    k[0, 0] = 2.0 ** 24
    assert orc.k_mean(bf(k))[0] == np.float32(131072.5)


def test_k_mean_error_bound_random(orc):
    kb = rnd_bf((1000, 32), 9, 3.0)
    x = f32(kb).astype(np.float64)
    mu = orc.k_mean(kb).astype(np.float64)
    exact = np.array([math.fsum(x[:, c]) for c in range(32)]) / 1000
    bound = 1000 * 2.0 ** -24 * np.sum(np.abs(x), axis=0) / 1000 + np.abs(exact) * 2.0 ** -23
    assert np.all(np.abs(mu - exact) <= bound)


def test_smoothing_removes_channel_offsets(orc):
    # integer-valued K (exact in bf16, exact sums): adding a per-channel integer offset moves the mean by
    # exactly that offset, so K' and therefore the codes and scales are unchanged
    rng = np.random.default_rng(1)
    k = rng.integers(-20, 21, size=(256, 16)).astype(np.float32)
    off = rng.integers(-50, 51, size=(1, 16)).astype(np.float32)
    c1, s1 = orc.quant_k(bf(k), 64, orc.k_mean(bf(k)))
    c2, s2 = orc.quant_k(bf(k + off), 64, orc.k_mean(bf(k + off)))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# ------------------------------------------------------------------------------------------- V E4M3
def test_v_quant_exact_codes_when_amax_is_448(orc):
    # a channel whose amax is 448 has inv = 1, so its codes are the E4M3 encodings of the values
    dec = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    vals = np.concatenate([dec[::3], -dec[1::5]]).astype(np.float32)
    vals = vals[np.abs(vals) == np.abs(vals)]
    v = np.zeros((vals.size + 1, 2), dtype=np.float32)
    v[:-1, 0] = vals
    v[-1, 0] = 448.0
    v[:, 1] = 1.0
    vbf = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(vbf.float(), torch.from_numpy(v))
    codes, scales = orc.quant_v(vbf.view(torch.int16).numpy().view(np.uint16))
    assert scales[0] == 1.0 and scales[1] == np.float32(1.0 / 448.0)
    assert np.array_equal(orc.e4m3_decode(codes[:, 0]), v[:, 0])
    assert np.all(codes[:, 1] == 0x7E)  # constant channel: every value is the amax -> 448


def test_v_quant_relative_error_bound(orc):
    v = rnd_bf((500, 32), 4)
    codes, scales = orc.quant_v(v)
    x = f32(v).astype(np.float64)
    s = scales.astype(np.float64)[None, :]
    deq = orc.e4m3_decode(codes).astype(np.float64) * s
    # E4M3 keeps 3 mantissa bits: half an ulp is 2^-4 relative for normals, 2^-10 absolute (in units of
    # the scale) for subnormals; the fp32 roundings of 448/amax and amax/448 add ~1e-7 relative
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)
    # the channel amax maps to the largest code
    assert np.all(np.max(codes.astype(np.int32) & 0x7F, axis=0) == 0x7E)


# ------------------------------------------------------------------------------------------- integer scores
def test_qk_int_matches_numpy_int64(orc):
    rng = np.random.default_rng(2)
    qc = rng.integers(-127, 128, size=(70, 128)).astype(np.int8)
    kc = rng.integers(-127, 128, size=(45, 128)).astype(np.int8)
    s = orc.qk_int(qc, kc)
    assert np.array_equal(s, qc.astype(np.int64) @ kc.astype(np.int64).T)
    # extreme: every code +-127 -> |S| = 128 * 127^2 fits int32
    qc[:] = 127
    kc[:] = -127
    assert np.all(orc.qk_int(qc, kc) == -128 * 127 * 127)
