"""Layer-selective quantization: the per-layer attention-error probe and the choice of the layers that keep full
precision (TMAP I2V write-up, section "保持视频质量").  The page visualises each attention layer's error over all
denoising iterations, finds a few layers whose error is large in every iteration while most layers stay small, and
keeps those few layers at the original precision in every iteration.

The probe runs a layer's self-attention on the same inputs in the quantized mode and in mode 0 (bf16, the original
precision) through the C ABI, and reduces the two outputs with ``sattn_error_stats`` (fp64 sums per head, on the
GPU).  The policy is host arithmetic on the resulting small [layers, iterations] error table.
"""
from __future__ import annotations

import numpy as np

from . import sattn


def rel_l2_and_cos(stats) -> tuple[float, float]:
    """Relative L2 error sqrt(sum (a-r)^2 / sum r^2) and cosine sum a*r / sqrt(sum r^2 * sum a^2) from error-stat
    sums (any leading shape; the sums are added over it first)."""
    s = np.asarray(stats, dtype=np.float64).reshape(-1, 4).sum(axis=0)
    rel = float(np.sqrt(s[0] / s[1])) if s[1] > 0 else (0.0 if s[0] == 0 else float("inf"))
    den = np.sqrt(s[1] * s[3])
    cos = float(s[2] / den) if den > 0 else float(s[0] == 0)
    return rel, cos


def probe_error(q, k, v, mode: int = sattn.SATTN_MODE_I8_FP8, sm_scale=None, blk_q: int = 128, workspace=None,
                ref_mode: int = sattn.SATTN_MODE_BF16):
    """(rel-L2, cosine, per-head [B, H, 4] sums) of ``mode`` against ``ref_mode`` on one layer's q, k, v."""
    o = sattn.fwd(q, k, v, mode=mode, sm_scale=sm_scale, blk_q=blk_q, workspace=workspace)
    r = sattn.fwd(q, k, v, mode=ref_mode, sm_scale=sm_scale, blk_q=blk_q, workspace=workspace)
    stats = sattn.error_stats(o, r).cpu().numpy()
    rel, cos = rel_l2_and_cos(stats)
    return rel, cos, stats


def select_bf16_layers(errors, n_bf16: int, quant_mode: int = sattn.SATTN_MODE_I8_FP8, statistic: str = "mean"):
    """Per-layer modes from an error table ``errors`` [layers, iterations] (e.g. rel-L2 of the quantized mode): the
    ``n_bf16`` layers with the largest ``statistic`` of their error over the iterations ("mean", "max" or "min")
    keep mode 0, the others run ``quant_mode``.  Ties go to the lower layer index."""
    e = np.asarray(errors, dtype=np.float64)
    if e.ndim == 1:
        e = e[:, None]
    n_layers = e.shape[0]
    if not 0 <= n_bf16 <= n_layers:
        raise ValueError(f"n_bf16 = {n_bf16} outside [0, {n_layers}]")
    reduce = {"mean": np.mean, "max": np.max, "min": np.min}[statistic]
    score = reduce(e, axis=1)
    order = sorted(range(n_layers), key=lambda l: (-score[l], l))
    keep = set(order[:n_bf16])
    return [sattn.SATTN_MODE_BF16 if l in keep else quant_mode for l in range(n_layers)]
