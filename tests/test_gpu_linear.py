"""GPU parity of the quantized linear layer (sattn_quantize_blocks, sattn_linear_quantized, sattn_linear through the
C ABI) with the CPU oracle (TMAP I2V write-up, section "FFN性能优化 / 线性层量化": 8-bit weights in 128 x 128
blocks, W8A8 with a W8A16 fallback).

* Codes and block scales are integer decisions: bit-exact against the oracle.
* Outputs are compared with the oracle's fp64 value y.  The kernels multiply exactly (int32 per K block in W8A8;
  exact bf16 x int8 products in W8A16) and round in fp32: the scale product, one FMA per K block, the partial sums
  inside a K block (W8A16 only), the bias add, then the bf16 rounding of the result.  The bound used is
      |y_gpu - y| <= 2^-8 |y| + (K/128 + 3) 2^-23 mag           (W8A8)
      |y_gpu - y| <= 2^-8 |y| + (K/128 + 3 + 128) 2^-23 mag     (W8A16)
  where mag is the oracle's sum of the magnitudes of the terms (1 bf16 ulp of the result plus the fp32 rounding
  of the accumulation).
* Against the unquantized product x W^T + b (fp64), the GPU output is as close as the oracle's quantized layer
  (cosine within 1e-4 of the oracle's), which itself stays above 0.99 on this input recipe (x with x20 outlier
  channels, which widen the steps of their 128 x 128 blocks).
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

from parity_helpers import say

pytestmark = pytest.mark.gpu

BLK = sattn.SATTN_LINEAR_BLK


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def val(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check(y_gpu_bits, y, mag, K, w8a8, label):
    got = val(y_gpu_bits)
    assert np.all(np.isfinite(got)), label
    slack = (K // BLK + 3 + (0 if w8a8 else 128)) * 2.0 ** -23
    err = np.abs(got - y)
    lim = 2.0 ** -8 * np.abs(y) + slack * mag
    worst = np.max(err / np.maximum(lim, 1e-300))
    say(f"  {label}: max err / bound {worst:.3f}, rel-L2 vs fp64 {np.linalg.norm(got - y) / np.linalg.norm(y):.2e}")
    assert np.all(err <= lim), f"{label}: {np.sum(err > lim)} elements outside the bound (worst ratio {worst:.3f})"


def weight_codes(w_host: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor):
    """The oracle's own codes and block scales of a weight, after checking that the GPU's equal them bit for bit; the
    references below are built from these, never from the GPU's."""
    wq_o, sw_o = oracle.quant_blocks(bits(w_host))
    assert np.array_equal(wq.cpu().numpy(), wq_o), "weight codes differ from the oracle's"
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), sw_o.view(np.uint32)), "weight scales differ"
    return wq_o, sw_o


def cosine(a, b):
    return float(np.sum(a * b) / np.sqrt(np.sum(a * a) * np.sum(b * b)))


def close_to_exact(got, ref, exact, label):
    if not np.any(exact):
        return
    cg, cr = cosine(got, exact), cosine(ref, exact)
    say(f"  {label}: cosine vs unquantized {cg:.6f} (oracle {cr:.6f})")
    assert cr >= 0.99 and cg >= cr - 1e-4, (cg, cr)


SHAPES = [
    ("ragged", 300, 200, 384),   # M, N ragged (3 x 2 tiles), 3 K blocks
    ("tiny", 1, 8, 128),         # a single row, a single K block
    ("edge", 129, 136, 256),     # one row and 8 columns into the second tiles
    ("odd-n", 70, 100, 640),     # N not a multiple of 8 (element-wise tail stores), 5 K blocks
]


@pytest.mark.parametrize("name,M,N,K", SHAPES, ids=[s[0] for s in SHAPES])
def test_quantize_blocks_bit_exact(name, M, N, K):
    x, w, _ = wl.linear_host_inputs(M, N, K, seed=71)
    xh = x.clone()
    xh[:min(M, 128), :128] = 0  # an all-zero block: scale 0, codes 0
    for t in (xh, w):
        codes, scales = sattn.quantize_blocks(t.cuda())
        oc, os_ = oracle.quant_blocks(bits(t))
        assert np.array_equal(codes.cpu().numpy(), oc)
        assert np.array_equal(scales.cpu().numpy(), os_)


@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("name,M,N,K", SHAPES, ids=[s[0] for s in SHAPES])
def test_linear_small(name, M, N, K, with_bias):
    x, w, b = wl.linear_host_inputs(M, N, K, seed=72, with_bias=with_bias)
    xd, wd = x.cuda(), w.cuda()
    bd = None if b is None else b.cuda()
    wq, sw = sattn.quantize_blocks(wd)
    wq_o, sw_o = weight_codes(w, wq, sw)
    bb = None if b is None else bits(b)
    exact = val(bits(x)) @ val(bits(w)).T + (0.0 if b is None else val(bb))
    # W8A8
    y8 = sattn.linear(xd, wq, sw, bd, mode=sattn.SATTN_LINEAR_W8A8)
    xq, sx = oracle.quant_blocks(bits(x))
    ref, mag = oracle.linear_w8a8(xq, sx, wq_o, sw_o, bb)
    check(bits(y8), ref, mag, K, True, f"{name} W8A8")
    close_to_exact(val(bits(y8)), ref, exact, f"{name} W8A8")
    # the same on codes prepared separately
    xq_d, sx_d = sattn.quantize_blocks(xd)
    y8q = sattn.linear_quantized(xq_d, sx_d, wq, sw, bd)
    assert torch.equal(y8q.view(torch.int16), y8.view(torch.int16))
    # W8A16
    y16 = sattn.linear(xd, wq, sw, bd, mode=sattn.SATTN_LINEAR_W8A16)
    ref16, mag16 = oracle.linear_w8a16(bits(x), wq_o, sw_o, bb)
    check(bits(y16), ref16, mag16, K, False, f"{name} W8A16")
    close_to_exact(val(bits(y16)), ref16, exact, f"{name} W8A16")


def test_linear_w8a16_long_k():
    """W8A16 with more K blocks than the 256-row tile keeps scale lists for (2049): the 128-row tile takes over at
    M > 128 (three row tiles, the last one ragged)."""
    M, N, K = 300, 16, 2049 * BLK
    x, w, b = wl.linear_host_inputs(M, N, K, seed=74)
    wq, sw = sattn.quantize_blocks(w.cuda())
    wq_o, sw_o = weight_codes(w, wq, sw)
    y = sattn.linear(x.cuda(), wq, sw, b.cuda(), mode=sattn.SATTN_LINEAR_W8A16)
    ref, mag = oracle.linear_w8a16(bits(x), wq_o, sw_o, bits(b))
    check(bits(y), ref, mag, K, False, "long-K W8A16")


def test_linear_w8a16_wide_row_stride():
    """W8A16 reads bf16 x at the caller's row stride: at 2^22 + 8 elements, 256 rows span more than 2^31 bytes, so
    the 128-row tile takes over at M > 128 (x occupies about 1.1 GB on the device; only K columns are read)."""
    M, N, K = 129, 24, 128
    ldx = (1 << 22) + 8
    x, w, b = wl.linear_host_inputs(M, N, K, seed=75)
    xd = torch.zeros((M, ldx), dtype=torch.bfloat16, device="cuda")
    xd[:, :K] = x.cuda()
    wq, sw = sattn.quantize_blocks(w.cuda())
    wq_o, sw_o = weight_codes(w, wq, sw)
    y = sattn.linear(xd[:, :K], wq, sw, b.cuda(), mode=sattn.SATTN_LINEAR_W8A16)
    ref, mag = oracle.linear_w8a16(bits(x), wq_o, sw_o, bits(b))
    check(bits(y), ref, mag, K, False, "wide-stride W8A16")
    del xd


def test_linear_strided_and_batched():
    """x with a row stride wider than K and leading batch dimensions; y written into a wider output buffer."""
    M, N, K = 2 * 96, 256, 256
    x, w, b = wl.linear_host_inputs(M, N, K, seed=73)
    xw = torch.zeros((M, K + 64), dtype=torch.bfloat16)
    xw[:, :K] = x
    xd = xw.cuda()[:, :K]
    wq, sw = sattn.quantize_blocks(w.cuda())
    out = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    y = sattn.linear(xd, wq, sw, b.cuda(), mode=sattn.SATTN_LINEAR_W8A8, out=out[:, :N])
    ref = sattn.linear(x.cuda(), wq, sw, b.cuda(), mode=sattn.SATTN_LINEAR_W8A8)
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    assert torch.all(out[:, N:] == 7.0)  # columns past N untouched
    y3 = sattn.linear(x.cuda().view(2, 96, K), wq, sw, b.cuda(), mode=sattn.SATTN_LINEAR_W8A16)
    assert y3.shape == (2, 96, N)
    ref16 = sattn.linear(x.cuda(), wq, sw, b.cuda(), mode=sattn.SATTN_LINEAR_W8A16)
    assert torch.equal(y3.reshape(M, N).view(torch.int16), ref16.view(torch.int16))


@pytest.mark.parametrize("name", ["wan14b-720p-ffn-up", "wan14b-720p-ffn-down"])
def test_linear_full_size_sampled(name):
    """The Wan-14B 720p shapes through the same launches as the benchmark; the oracle checks three row tiles (first,
    middle, last and ragged) against three column tiles."""
    w = wl.LINEAR_WORKLOADS[name]
    dev = torch.device("cuda")
    x, wt, b = wl.linear_device_inputs(w, dev)
    wq, sw = sattn.quantize_blocks(wt)
    say(f"[linear full] {name}: M {w.M} N {w.N} K {w.K}")
    mt, nt = -(-w.M // BLK), -(-w.N // BLK)
    rows = np.concatenate([np.arange(t * BLK, min((t + 1) * BLK, w.M)) for t in (0, mt // 2, mt - 1)])
    cols = np.concatenate([np.arange(t * BLK, min((t + 1) * BLK, w.N)) for t in (0, nt // 2, nt - 1)])
    ri, ci = torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)
    xs, ws_, bs = bits(x[ri]), bits(wt[ci]), bits(b[ci])
    wq_s, sw_s = oracle.quant_blocks(ws_)
    assert np.array_equal(wq[ci].cpu().numpy(), wq_s)
    for mode, w8a8 in ((sattn.SATTN_LINEAR_W8A8, True), (sattn.SATTN_LINEAR_W8A16, False)):
        y = sattn.linear(x, wq, sw, b, mode=mode)
        torch.cuda.synchronize()
        got = bits(y[ri][:, ci])
        if w8a8:
            xq_s, sx_s = oracle.quant_blocks(xs)
            ref, mag = oracle.linear_w8a8(xq_s, sx_s, wq_s, sw_s, bs)
        else:
            ref, mag = oracle.linear_w8a16(xs, wq_s, sw_s, bs)
        check(got, ref, mag, w.K, w8a8, f"{name} {'W8A8' if w8a8 else 'W8A16'}")
        del y
