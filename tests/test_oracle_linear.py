"""Pins of the quantized-linear oracle (TMAP I2V write-up, section "FFN性能优化 / 线性层量化": linear layers with
8-bit weights, per-block 128 x 128 quantization, W8A8 with a W8A16 fallback) against what the mathematics fixes:

* the per-block INT8 rule: the block maximum maps to code +-127, every value is within half a step of its
  reconstruction, an all-zero block gets scale 0, and blocks do not influence each other;
* inputs on the quantization grid (each block's values are integer multiples of a power of two, with 127 times it
  present) are represented exactly, so both W8A8 and W8A16 return the unquantized product x W^T + b exactly;
* scaling x by 2 scales y by exactly 2;
* for any input, |y - x W^T| is within the bound that half a quantization step per operand allows.
"""
import numpy as np
import pytest

import oracle

BLK = oracle.LINEAR_BLK


def bf(x):
    return oracle.bf16_from_f32(np.asarray(x, dtype=np.float32))


def val(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def grid_matrix(rng, rows, cols, exps):
    """Values k * 2^e(block) with integer |k| <= 127 and 127 * 2^e present in every block (exact in bf16)."""
    k = rng.integers(-127, 128, size=(rows, cols)).astype(np.float64)
    e = np.zeros((rows, cols))
    for i in range(0, rows, BLK):
        for j in range(0, cols, BLK):
            k[i, j] = 127 if (i + j) % 2 == 0 else -127
            e[i:i + BLK, j:j + BLK] = exps[(i // BLK) % len(exps), (j // BLK) % exps.shape[1]]
    return k * np.exp2(e)


def block_view(a, i, j):
    return a[i * BLK:(i + 1) * BLK, j * BLK:(j + 1) * BLK]


def test_quant_blocks_rule():
    rng = np.random.default_rng(11)
    # ragged in both directions: the last row block holds 44 rows, the last column block 74 columns
    x = rng.standard_normal((300, 330)).astype(np.float32) * np.exp2(rng.integers(-3, 4, size=(1, 330)))
    x[128:256, 256:330] = 0.0  # one all-zero block
    xb = bf(x)
    codes, scales = oracle.quant_blocks(xb)
    assert codes.shape == (300, 330) and scales.shape == (3, 3)
    xv = val(xb)
    for i in range(3):
        for j in range(3):
            c, v, s = block_view(codes, i, j).astype(np.float64), block_view(xv, i, j), float(scales[i, j])
            if not v.any():
                assert s == 0.0 and not c.any()
                continue
            assert np.abs(c).max() == 127
            at = np.unravel_index(np.argmax(np.abs(v)), v.shape)
            assert abs(c[at]) == 127 and np.sign(c[at]) == np.sign(v[at])
            # half a step, plus the fp32 rounding of 127/a and of x * (127/a) that decides the code near a tie
            # (|x/s| <= 127, two roundings of 2^-24 each: below 2^-16 of a step)
            assert np.all(np.abs(v - c * s) <= s * (0.5 + 2.0 ** -16))
    # blocks are independent: changing block (0, 0) leaves every other block as it was
    x2 = x.copy()
    x2[:128, :128] *= 3.0
    c2, s2 = oracle.quant_blocks(bf(x2))
    keep = np.ones((300, 330), bool)
    keep[:128, :128] = False
    assert np.array_equal(c2[keep], codes[keep])
    assert np.array_equal(np.delete(s2.ravel(), 0), np.delete(scales.ravel(), 0))


@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a8_and_w8a16_are_exact_on_the_grid(with_bias):
    rng = np.random.default_rng(12)
    M, N, K = 300, 200, 384
    x = grid_matrix(rng, M, K, np.array([[-4, -2, 0], [1, -1, -3], [2, 0, -5]]))
    w = grid_matrix(rng, N, K, np.array([[-6, -7, -5], [-8, -4, -6]]))
    xb, wb = bf(x), bf(w)
    assert np.array_equal(val(xb), x) and np.array_equal(val(wb), w)
    bias = bf(rng.integers(-64, 64, size=N) * 0.25) if with_bias else None
    xq, sx = oracle.quant_blocks(xb)
    wq, sw = oracle.quant_blocks(wb)
    assert np.all(np.log2(sx) == np.round(np.log2(sx))) and np.all(np.log2(sw) == np.round(np.log2(sw)))
    exact = x @ w.T + (0.0 if bias is None else val(bias))
    y8, mag8 = oracle.linear_w8a8(xq, sx, wq, sw, bias)
    y16, _ = oracle.linear_w8a16(xb, wq, sw, bias)
    assert np.array_equal(y8, exact)
    assert np.array_equal(y16, exact)
    assert np.all(mag8 >= np.abs(y8))


def test_scaling_x_by_two_scales_y_by_two():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((260, 256)).astype(np.float32)
    w = rng.standard_normal((130, 256)).astype(np.float32)
    wq, sw = oracle.quant_blocks(bf(w))
    y1 = oracle.linear_w8a8(*oracle.quant_blocks(bf(x)), wq, sw)[0]
    y2 = oracle.linear_w8a8(*oracle.quant_blocks(bf(2 * x)), wq, sw)[0]
    assert np.array_equal(y2, 2 * y1)
    z1 = oracle.linear_w8a16(bf(x), wq, sw)[0]
    z2 = oracle.linear_w8a16(bf(2 * x), wq, sw)[0]
    assert np.array_equal(z2, 2 * z1)


def test_error_within_half_a_step_per_operand():
    rng = np.random.default_rng(14)
    M, N, K = 200, 260, 512
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, :7] *= 20.0                       # outlier channels widen the first K block's steps
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb, wb = bf(x), bf(w)
    xv, wv = val(xb), val(wb)
    xq, sx = oracle.quant_blocks(xb)
    wq, sw = oracle.quant_blocks(wb)
    # half a step per element (plus the fp32 slop of the code decision, as in test_quant_blocks_rule)
    ex = np.repeat(np.repeat(sx.astype(np.float64) * (0.5 + 2.0 ** -16), BLK, 0), BLK, 1)[:M, :K]
    ew = np.repeat(np.repeat(sw.astype(np.float64) * (0.5 + 2.0 ** -16), BLK, 0), BLK, 1)[:N, :K]
    exact = xv @ wv.T
    bound8 = np.abs(xv) @ ew.T + ex @ np.abs(wv).T + ex @ ew.T
    y8 = oracle.linear_w8a8(xq, sx, wq, sw)[0]
    assert np.all(np.abs(y8 - exact) <= bound8 * (1 + 1e-9))
    y16 = oracle.linear_w8a16(xb, wq, sw)[0]
    assert np.all(np.abs(y16 - exact) <= (np.abs(xv) @ ew.T) * (1 + 1e-9))
    # and the bound is not vacuous: the quantized product is close to the exact one
    rel = np.linalg.norm(y8 - exact) / np.linalg.norm(exact)
    assert rel < 0.05, rel
