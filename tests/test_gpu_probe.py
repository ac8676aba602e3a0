"""GPU parity of the per-layer attention-error probe behind layer-selective quantization (TMAP I2V write-up, section
"保持视频质量"): sattn_error_stats against the oracle's sums by definition, and the probe's per-layer errors and
layer choice against the same quantities computed from the oracle's emulations of mode 2 and mode 0."""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_05_amd import policy
from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

from parity_helpers import device_inputs, head_bits, say, u16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,layout,n,batch", [(128, "bhnd", 300, 1), (64, "bhnd", 300, 1), (128, "bnhd", 300, 1),
                                              (128, "bhnd", 16500, 1), (64, "bnhd", 16500, 1), (128, "bhnd", 255, 1),
                                              (128, "bnhd", 700, 2)])
def test_error_stats_match_the_definition(d, layout, n, batch):
    """N = 300 sums each head in 2 row chunks, N = 16500 in 64 chunks of 258 rows with a ragged last one (246),
    N = 255 in a single chunk shorter than the workgroup's stride; B = 2 puts the (batch, head) pairs in the grid's
    second dimension."""
    w = wl.scaled(wl.WORKLOADS["wan14b-720p"], name="probe-stats", B=batch, H=3, Nq=n, Nkv=n, d=d, seed=61)
    q, k, v = device_inputs(w, layout=layout)
    stats = sattn.error_stats(q, k).cpu().numpy()  # any two bf16 tensors of one shape
    qh, kh = u16(q), u16(k)
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle.error_stats(qh[b, h], kh[b, h])
            assert np.allclose(stats[b, h], ref, rtol=1e-12, atol=0), (b, h, stats[b, h], ref)
    same = sattn.error_stats(q, q).cpu().numpy()
    assert np.all(same[..., 0] == 0) and np.all(same[..., 1] == same[..., 2]) and np.all(same[..., 2] == same[..., 3])
    # deterministic, and independent of what the workspace held before the call
    dirty = torch.full((sattn.sattn_error_stats_workspace_bytes(w.B, w.H, n) + 512,), 0x7F, dtype=torch.uint8,
                       device=q.device)
    again = sattn.error_stats(q, k, workspace=dirty).cpu().numpy()
    assert np.array_equal(again.view(np.uint64), stats.view(np.uint64))


def oracle_layer_error(w, iteration):
    """rel-L2 of the oracle's mode-2 emulation against its mode-0 emulation over all rows and heads of a layer."""
    tot = np.zeros(4)
    rows = np.arange(w.Nq, dtype=np.int32)
    for h in range(w.H):
        qb, kb, vb = head_bits(w, 0, h, seed=w.seed + iteration)
        qz = oracle.quantize_head(qb, kb, vb, w.blk_q, 64, 2)
        e2 = oracle.attn_emulate(2, rows, tile=64, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=64, nkv=w.Nkv,
                                 quant=qz, v_bf16=vb)
        e0 = oracle.attn_emulate(0, rows, tile=64, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=64, nkv=w.Nkv,
                                 q_bf16=qb, k_bf16=kb, v_bf16=vb)
        tot += oracle.error_stats(e2, e0)
    return policy.rel_l2_and_cos(tot)[0]


def test_probe_errors_and_layer_choice_match_the_oracle():
    base = wl.scaled(wl.WORKLOADS["wan1.3b-480p"], H=2, Nq=384, Nkv=384)
    layers = wl.probe_layers(6, base)
    gpu, orc = np.zeros((6, 2)), np.zeros((6, 2))
    for l, w in enumerate(layers):
        for t in range(2):
            q, k, v = device_inputs(w, seed=w.seed + t)
            gpu[l, t] = policy.probe_error(q, k, v, mode=2, sm_scale=w.sm_scale, blk_q=w.blk_q)[0]
            orc[l, t] = oracle_layer_error(w, t)
        say(f"  layer {l} (K outliers x{w.outlier_scale:g}): GPU rel-L2 {gpu[l]}, oracle {orc[l]}")
    # the GPU modes match the oracle to ~1e-4 of the output, far below the probe's errors (1e-2)
    assert np.all(np.abs(gpu - orc) <= 0.05 * orc + 2e-4), (gpu, orc)
    # the choice agrees wherever the oracle's ranking has a clear gap (>10 %) after the n-th layer
    score = np.sort(orc.mean(axis=1))[::-1]
    clear = [n for n in range(1, 6) if score[n - 1] > 1.1 * score[n]]
    assert clear, score
    for n in clear:
        assert policy.select_bf16_layers(gpu, n) == policy.select_bf16_layers(orc, n), n
