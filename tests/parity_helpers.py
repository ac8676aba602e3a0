"""Shared helpers of the GPU parity tests: seeded inputs, runs through the C ABI, oracle references and the
comparison metrics.  The GPU side only ever receives the generated bf16 tensors; every expected value
comes from ``oracle``."""
from __future__ import annotations

import functools
import math
import sys

import numpy as np
import torch

import oracle
from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

REL_L2_GATE = 2e-3   # GPU output vs the oracle's step-by-step emulation, pooled over the compared rows
COS_GATE = 0.999     # GPU output vs fp64 exact attention, where the emulation itself reaches it
# Per query row (rel-L2 of that row vs the emulation), so that a wrong row cannot hide inside the pooled figure.  A
# row legitimately differs by bf16 rounding ties of its outputs (at most one ulp each, i.e. 2^-8 relative) and by the
# rare P roundings that the hardware exp2 and the MFMA summation order flip.  One E4M3 step of the weight w_j of key j
# is at most w_j / 8, and w_j <= 1/2 for every key whose P is rounded at all (the running max of its tile has P = 448
# exactly), so one flip moves a row by at most |v_j| / 16; with N_eff effective keys it moves it by about
# 1 / (8 sqrt(N_eff)) of its norm: 7e-4 at 75 600 keys, 7e-3 at 1 000.  Hence every row within ROW_GATE, and all but
# max(1, ROW_FRAC of the rows) within ROW_SOFT: a systematic fault (a lane, a tile, a block scale) moves many rows.
ROW_GATE = 2e-2
ROW_SOFT = 5e-3
ROW_FRAC = 0.01


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def host_inputs(w: wl.Workload, seed: int | None = None):
    return wl.full_inputs(w, seed)


def device_inputs(w: wl.Workload, seed: int | None = None, layout: str = "bhnd"):
    q, k, v = host_inputs(w, seed)
    if layout == "bhnd":
        return tuple(t.cuda() for t in (q, k, v))
    # [B, N, H, d] storage, viewed as [B, H, N, d]
    return tuple(t.transpose(1, 2).contiguous().cuda().transpose(1, 2) for t in (q, k, v))


def head_bits(w: wl.Workload, b: int, h: int, seed: int | None = None):
    q, k, v = host_inputs(w, seed)
    return wl.bits(q[b, h]), wl.bits(k[b, h]), wl.bits(v[b, h])


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def untile_v(tiled: np.ndarray) -> np.ndarray:
    """[nkb, d, 64] per-tile transposed layout -> [nkb*64, d] natural layout."""
    nkb, d, t = tiled.shape
    return tiled.transpose(0, 2, 1).reshape(nkb * t, d)


def sample_rows(nq: int, blk: int = 128) -> np.ndarray:
    """First, middle and last (ragged) query blocks."""
    nqb = -(-nq // blk)
    blocks = sorted({0, nqb // 2, nqb - 1})
    rows = np.concatenate([np.arange(b * blk, min((b + 1) * blk, nq)) for b in blocks])
    return rows.astype(np.int32)


def sample_heads(H: int):
    return sorted({0, H // 2, H - 1})


def oracle_quant(w: wl.Workload, b: int, h: int, mode: int, blk_q: int, seed=None):
    q, k, v = head_bits(w, b, h, seed)
    return oracle.quantize_head(q, k, v, blk_q, 64, mode)


def oracle_outputs(w: wl.Workload, b: int, h: int, mode: int, rows, blk_q: int, sm_scale: float, seed=None,
                   mask=None):
    """(E as fp32 values of its bf16 output, R in fp64) for the given rows of one head (with a block-sparse
    mask: the [query blocks, key blocks] mask of this head)."""
    q, k, v = head_bits(w, b, h, seed)
    mk = {} if mask is None else {"mask": mask, "mask_qblk": wl.MASK_QBLK}
    if mode == 0:
        E = oracle.attn_emulate(0, rows, tile=64, sm_scale=sm_scale, blk_q=blk_q, blk_k=64, nkv=w.Nkv,
                                q_bf16=q, k_bf16=k, v_bf16=v, **mk)
    else:
        qz = oracle.quantize_head(q, k, v, blk_q, 64, mode)
        E = oracle.attn_emulate(mode, rows, tile=64, sm_scale=sm_scale, blk_q=blk_q, blk_k=64, nkv=w.Nkv,
                                quant=qz, v_bf16=v, **mk)
    R = oracle.attn_ref_fp64(q, k, v, rows, sm_scale, **mk)
    return f32(E).astype(np.float64), R


def metrics(gpu: np.ndarray, E: np.ndarray, R: np.ndarray):
    gpu = gpu.astype(np.float64)
    rel = float(np.linalg.norm(gpu - E) / max(np.linalg.norm(E), 1e-300))
    cos = float(np.sum(gpu * R) / max(np.linalg.norm(gpu) * np.linalg.norm(R), 1e-300))
    cos_e = float(np.sum(E * R) / max(np.linalg.norm(E) * np.linalg.norm(R), 1e-300))
    return rel, cos, cos_e


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (the normal range; 2^-133 below it)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def row_metrics(gpu: np.ndarray, E: np.ndarray):
    """Per query row (last axis = channels): rel-L2 of the row vs the emulation (a row of zeros in E compares its
    absolute norm), and the largest element difference in bf16 ulps of the emulation's value."""
    gpu = gpu.astype(np.float64).reshape(-1, gpu.shape[-1])
    E = E.astype(np.float64).reshape(-1, E.shape[-1])
    num = np.linalg.norm(gpu - E, axis=1)
    den = np.linalg.norm(E, axis=1)
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    ulps = np.abs(gpu - E) / bf16_ulp(E)
    return rel, ulps


def check_output(gpu_rows: np.ndarray, E: np.ndarray, R: np.ndarray, label: str):
    assert np.all(np.isfinite(gpu_rows)), f"{label}: non-finite output"
    rel, cos, cos_e = metrics(gpu_rows, E, R)
    rrel, ulps = row_metrics(gpu_rows, E)
    worst = int(np.argmax(rrel))
    say(f"  {label}: rel-L2 vs emulation {rel:.3e}, cos vs fp64 {cos:.6f} (emulation {cos_e:.6f}); worst row "
        f"{worst} rel-L2 {rrel[worst]:.3e}, max |diff| {ulps.max():.0f} bf16 ulp, "
        f"{np.count_nonzero(ulps.max(axis=1) > 1)} of {rrel.size} rows beyond 1 ulp")
    assert rel <= REL_L2_GATE, f"{label}: rel-L2 {rel:.3e} > {REL_L2_GATE}"
    assert rrel[worst] <= ROW_GATE, f"{label}: row {worst} rel-L2 {rrel[worst]:.3e} > {ROW_GATE}"
    n_soft = int(np.count_nonzero(rrel > ROW_SOFT))
    allowed = max(1, int(ROW_FRAC * rrel.size))
    assert n_soft <= allowed, f"{label}: {n_soft} rows beyond rel-L2 {ROW_SOFT} (at most {allowed})"
    # the cosine gate applies where the method itself (the emulation) reaches it; elsewhere the GPU must be as close
    # to exact attention as the emulation is
    if cos_e >= COS_GATE:
        assert cos >= COS_GATE, f"{label}: cosine {cos:.6f} < {COS_GATE}"
    else:
        assert cos >= cos_e - 1e-4, f"{label}: cosine {cos:.6f} below the emulation's {cos_e:.6f}"
    return rel, cos
