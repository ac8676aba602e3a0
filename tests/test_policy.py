"""Layer-selective quantization policy (TMAP I2V write-up, section "保持视频质量": layers whose attention error is
large over the denoising iterations keep full precision).  CPU pins of the host-side pieces: the error metrics
from probe sums, the oracle's probe sums, and the layer choice."""
import numpy as np
import pytest
import torch

from quantized_attention_05_amd import policy
from quantized_attention_05_amd import workloads as wl


def bf(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_metrics_closed_forms():
    r = np.array([1.0, -2.0, 0.5])
    s = lambda a: np.array([np.sum((a - r) ** 2), np.sum(r * r), np.sum(a * r), np.sum(a * a)])
    assert policy.rel_l2_and_cos(s(r)) == (0.0, 1.0)
    rel, cos = policy.rel_l2_and_cos(s(2 * r))
    assert rel == 1.0 and abs(cos - 1.0) < 1e-15
    rel, cos = policy.rel_l2_and_cos(s(-r))
    assert rel == 2.0 and abs(cos + 1.0) < 1e-15
    # sums over several heads are added before the ratios
    rel, _ = policy.rel_l2_and_cos(np.stack([s(r), s(2 * r)]))
    assert abs(rel - np.sqrt(np.sum(r * r) / (2 * np.sum(r * r)))) < 1e-15


def test_oracle_error_stats_closed_forms(orc):
    rng = np.random.default_rng(3)
    r = bf(rng.standard_normal((40, 64)))
    rv = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    st = orc.error_stats(r, r)
    assert st[0] == 0 and st[1] == st[2] == st[3] == np.sum(rv * rv)
    two = bf(2 * rv)  # doubling is exact in bf16
    st = orc.error_stats(two, r)
    assert st[0] == st[1] and st[2] == 2 * st[1] and st[3] == 4 * st[1]
    st = orc.error_stats(bf(-rv), r)
    assert st[0] == 4 * st[1] and st[2] == -st[1]
    # disjoint supports: orthogonal, so the error energy is the sum of both energies and the cosine is 0
    a = rv.copy()
    a[:, :32] = 0
    b = rv.copy()
    b[:, 32:] = 0
    st = orc.error_stats(bf(a), bf(b))
    assert st[2] == 0 and st[0] == st[1] + st[3] and policy.rel_l2_and_cos(st)[1] == 0.0


def test_select_bf16_layers():
    e = np.array([[0.01, 0.02], [0.30, 0.20], [0.05, 0.06], [0.30, 0.20], [0.10, 0.50]])
    # means: 0.015, 0.25, 0.055, 0.25, 0.30 -> layer 4 first, then the tie of layers 1 and 3 goes to layer 1
    assert policy.select_bf16_layers(e, 2) == [2, 0, 2, 2, 0]
    assert policy.select_bf16_layers(e, 3) == [2, 0, 2, 0, 0]
    assert policy.select_bf16_layers(e, 1, statistic="max") == [2, 2, 2, 2, 0]
    assert policy.select_bf16_layers(e, 1, statistic="min") == [2, 0, 2, 2, 2]  # min: 0.2 (layer 1, tie with 3)
    assert policy.select_bf16_layers(e, 0) == [2] * 5
    assert policy.select_bf16_layers(e, 5, quant_mode=1) == [0] * 5
    assert policy.select_bf16_layers(e[:, 0], 1) == [2, 0, 2, 2, 2]  # a single iteration as a 1-D table
    with pytest.raises(ValueError):
        policy.select_bf16_layers(e, 6)


def test_probe_layers_recipe():
    base = wl.scaled(wl.WORKLOADS["wan1.3b-480p"], H=2, Nq=256, Nkv=256)
    layers = wl.probe_layers(8, base)
    assert len({w.seed for w in layers}) == 8
    assert {w.outlier_scale for w in layers} <= {1.0, 3.0, 10.0, 30.0, 100.0}
    assert layers == wl.probe_layers(8, base)  # seeded
    q0, k0, _ = wl.head_inputs(layers[0], 0, 0)
    assert torch.equal(k0, wl.head_inputs(layers[0], 0, 0)[1])
