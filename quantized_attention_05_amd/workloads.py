"""Seeded synthetic attention inputs shaped like the self- and cross-attention of Wan-style video DiTs.

This module draws random numbers and nothing else: it holds none of the attention or quantization
arithmetic.  Both the GPU path (tests, benchmark) and the CPU oracle are fed from it, so they see the
identical bf16 bit patterns.

Every (batch, head) slice is drawn from its own PCG64 stream seeded with ``SeedSequence([seed, b, h])``,
so a single head can be regenerated on its own (the oracle only ever needs a few heads of a large
workload).  Per slice, the draw order is: Q, K, V (``standard_normal`` float32, ``[N, d]``), then the
per-channel K offsets, then the outlier-channel picks, then the zero-block picks.  K is formed in fp32
(base + offset, outlier channels multiplied by 10), then every tensor is rounded to bf16 (round to
nearest even, via torch's CPU cast), then zeroed channels / blocks are set to exact zero.

Sequence lengths follow Wan's latent grids: 21 x 30 x 52 = 32 760 tokens (480p, 81 frames) and
21 x 45 x 80 = 75 600 tokens (720p); cross-attention keys are 512 text + 257 image tokens = 769.
"""
from __future__ import annotations

import dataclasses
from typing import Tuple

import numpy as np
import torch

# Distribution recipes (K offset per channel; extras):
#   "tiny"     : Q, V ~ N(0,1); K ~ N(0,1) + U(-4, 4) per channel; channel 0 of K is all zeros.
#   "outlier"  : Q, K, V ~ N(0,1); K + N(0, 3^2) per channel; 4 distinct channels of K scaled x10
#                (x outlier_scale).
#   "zeroblk"  : Q, K, V ~ N(0,1); K + N(0, 3^2) per channel; 1 % of the 64-token K blocks all zero.
#   "plain"    : Q, K, V ~ N(0,1).
DISTS = ("tiny", "outlier", "zeroblk", "plain")

MODE_NAMES = {0: "bf16", 1: "i8-qk+bf16-pv", 2: "i8-qk+fp8-pv"}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    d: int
    blk_q: int
    blk_k: int
    dist: str
    seed: int
    modes: Tuple[int, ...]
    outlier_scale: float = 10.0  # factor of the 4 outlier channels of K ("outlier" recipe)

    @property
    def ops(self) -> float:
        """Effective attention operations per call: 4 * Nq * Nkv * d * H * B (QK^T and PV, 2 ops/MAC)."""
        return 4.0 * self.Nq * self.Nkv * self.d * self.H * self.B

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 2, 256, 256, 64, 64, 64, "tiny", 0, (1,)),
        Workload("wan1.3b-480p", 1, 12, 32760, 32760, 128, 128, 64, "outlier", 1, (1,)),
        # Wan-14B 480p: "the same distributions as config 1" read with 1-based numbering, i.e. the tiny recipe
        # (U(-4, 4) channel offsets, K channel 0 zeroed) at the 14B shape ...
        Workload("wan14b-480p", 1, 40, 32760, 32760, 128, 128, 64, "tiny", 2, (0, 1, 2)),
        # ... and read with 0-based numbering, the Wan-1.3B recipe (N(0, 3^2) offsets, 4 outlier channels x10)
        Workload("wan14b-480p-outlier", 1, 40, 32760, 32760, 128, 128, 64, "outlier", 202, (0, 1, 2)),
        Workload("wan14b-720p", 1, 40, 75600, 75600, 128, 128, 64, "zeroblk", 3, (2,)),
        # one self-attention layer of the layer-selective pass (layer l uses seed 1000 + l) ...
        Workload("layersel-720p-self", 1, 40, 75600, 75600, 128, 128, 64, "plain", 1000, (0, 2)),
        # ... and its cross-attention call (layer l uses seed 2000 + l): 512 text + 257 image keys
        Workload("layersel-720p-cross", 1, 40, 75600, 769, 128, 128, 64, "plain", 2000, (0, 1, 2)),
    ]
}

LAYERSEL_LAYERS = 40
LAYERSEL_BF16_LAYERS = 8
LAYERSEL_MASK_SEED = 999


def layer_modes(n_layers: int = LAYERSEL_LAYERS, n_bf16: int = LAYERSEL_BF16_LAYERS,
                seed: int = LAYERSEL_MASK_SEED) -> list:
    """Fixed seeded per-layer mode mask: ``n_bf16`` layers stay in bf16 (mode 0), the rest INT8+FP8 (2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    keep = set(int(i) for i in rng.choice(n_layers, size=n_bf16, replace=False))
    return [0 if i in keep else 2 for i in range(n_layers)]


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x).to(torch.bfloat16)


def head_inputs(w: Workload, b: int, h: int, seed: int | None = None):
    """Q [Nq, d], K [Nkv, d], V [Nkv, d] as CPU bf16 tensors for one (batch, head) slice."""
    s = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([s, b, h])))
    d = w.d
    q = rng.standard_normal((w.Nq, d), dtype=np.float32)
    k = rng.standard_normal((w.Nkv, d), dtype=np.float32)
    v = rng.standard_normal((w.Nkv, d), dtype=np.float32)
    zero_channels = []
    zero_blocks = []
    if w.dist == "tiny":
        k += rng.uniform(-4.0, 4.0, size=(1, d)).astype(np.float32)
        zero_channels = [0]
    elif w.dist in ("outlier", "zeroblk"):
        k += (3.0 * rng.standard_normal((1, d))).astype(np.float32)
        if w.dist == "outlier":
            ch = rng.choice(d, size=4, replace=False)
            k[:, ch] *= np.float32(w.outlier_scale)
        else:
            nblk = (w.Nkv + 63) // 64
            nzero = int(round(0.01 * nblk))
            zero_blocks = [int(i) for i in rng.choice(nblk, size=nzero, replace=False)]
    elif w.dist != "plain":
        raise ValueError(f"unknown distribution {w.dist!r}")
    qt, kt, vt = _to_bf16(q), _to_bf16(k), _to_bf16(v)
    for c in zero_channels:
        kt[:, c] = 0
    for blk in zero_blocks:
        kt[blk * 64:(blk + 1) * 64, :] = 0
    return qt, kt, vt


def full_inputs(w: Workload, seed: int | None = None):
    """Q [B, H, Nq, d], K/V [B, H, Nkv, d] CPU bf16 tensors, head by head from ``head_inputs``."""
    q = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.bfloat16)
    k = torch.empty((w.B, w.H, w.Nkv, w.d), dtype=torch.bfloat16)
    v = torch.empty((w.B, w.H, w.Nkv, w.d), dtype=torch.bfloat16)
    for b in range(w.B):
        for h in range(w.H):
            q[b, h], k[b, h], v[b, h] = head_inputs(w, b, h, seed)
    return q, k, v


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a CPU bf16 tensor as a numpy uint16 array (no copy of the values' meaning)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def scaled(w: Workload, **changes) -> Workload:
    """The same recipe at other sizes (for tests that need a smaller instance of a workload)."""
    return dataclasses.replace(w, **changes)


# ---------------------------------------------------------------- block-sparse masks
# A block mask is [B, H, ceil(Nq / 128), ceil(Nkv / 64)] bytes: 1 = query block i attends to key block j.
MASK_QBLK = 128
MASK_KBLK = 64


def mask_dims(w: Workload) -> Tuple[int, int, int, int]:
    return (w.B, w.H, -(-w.Nq // MASK_QBLK), -(-w.Nkv // MASK_KBLK))


def random_block_mask(w: Workload, density: float, seed: int) -> np.ndarray:
    """Each block kept independently with probability ``density`` (PCG64 stream of ``seed``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.random(mask_dims(w)) < density).astype(np.uint8)


def band_block_mask(w: Workload, half_width: int, sink_blocks: int = 1) -> np.ndarray:
    """Local attention: query block i keeps key block j when their token centres lie within ``half_width`` tokens,
    plus the first ``sink_blocks`` key blocks; the same pattern for every (batch, head)."""
    B, H, nqm, nkm = mask_dims(w)
    qc = np.arange(nqm) * MASK_QBLK + MASK_QBLK // 2
    kc = np.arange(nkm) * MASK_KBLK + MASK_KBLK // 2
    keep = np.abs(qc[:, None] - kc[None, :]) <= half_width
    keep[:, :sink_blocks] = True
    return np.ascontiguousarray(np.broadcast_to(keep, (B, H, nqm, nkm)).astype(np.uint8))


def kept_pairs(w: Workload, mask: np.ndarray) -> int:
    """(query, key) pairs a block mask keeps, counting the ragged last blocks at their true sizes."""
    B, H, nqm, nkm = mask_dims(w)
    rq = np.minimum(MASK_QBLK, w.Nq - np.arange(nqm) * MASK_QBLK)
    rk = np.minimum(MASK_KBLK, w.Nkv - np.arange(nkm) * MASK_KBLK)
    return int(np.einsum("bhij,i,j->", (np.asarray(mask) != 0).astype(np.int64), rq, rk))


# ---------------------------------------------------------------- per-layer error probe
PROBE_SEED = 3000


def probe_layers(n_layers: int, base: Workload, seed: int = PROBE_SEED):
    """Synthetic layers of different quantization sensitivity for the per-layer error probe: every layer follows the
    "outlier" recipe of ``base``'s shape with its own K outlier factor, drawn from (1, 3, 10, 30, 100) by a seeded
    PCG64 stream; iteration t of layer l draws its tensors with seed ``seed + 100 * l + t``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    factors = rng.choice(np.array([1.0, 3.0, 10.0, 30.0, 100.0]), size=n_layers)
    return [dataclasses.replace(base, name=f"{base.name}-layer{l}", dist="outlier", outlier_scale=float(f),
                                seed=seed + 100 * l) for l, f in enumerate(factors)]


# ---------------------------------------------------------------- quantized linear layer
# Wan-14B linear shapes at the 720p sequence (75 600 tokens): hidden 5120, FFN 13 824.  Recipe (random numbers only):
# x ~ N(0, 1) with 8 seeded outlier input channels scaled x20 (the channel outliers of DiT activations that make
# per-block scales matter); W ~ N(0, 1/K); bias ~ N(0, 0.02^2).  Host draws use PCG64(seed) in the order x, outlier
# picks, W, bias; device draws (for the full-size shapes, where values do not change the timing or the sampled
# parity) use a torch generator seeded with the same seed.
@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    name: str
    M: int
    N: int
    K: int
    seed: int

    @property
    def ops(self) -> float:
        return 2.0 * self.M * self.N * self.K


LINEAR_WORKLOADS = {
    "wan14b-720p-ffn-up": LinearWorkload("wan14b-720p-ffn-up", 75600, 13824, 5120, 4000),
    "wan14b-720p-ffn-down": LinearWorkload("wan14b-720p-ffn-down", 75600, 5120, 13824, 4001),
    "wan14b-720p-proj": LinearWorkload("wan14b-720p-proj", 75600, 5120, 5120, 4002),
}
LINEAR_OUTLIERS = 8
LINEAR_OUTLIER_SCALE = 20.0


def linear_host_inputs(M: int, N: int, K: int, seed: int, with_bias: bool = True):
    """(x [M, K], W [N, K], bias [N] or None) as bf16 CPU tensors from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    ch = rng.choice(K, size=min(LINEAR_OUTLIERS, K), replace=False)
    x[:, ch] *= np.float32(LINEAR_OUTLIER_SCALE)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    b = rng.standard_normal(N, dtype=np.float32) * np.float32(0.02)
    return _to_bf16(x), _to_bf16(w), (_to_bf16(b) if with_bias else None)


def linear_device_inputs(w: LinearWorkload, device):
    """(x, W, bias) of a full-size linear workload drawn on the GPU (torch generator seeded with w.seed)."""
    gen = torch.Generator(device=device).manual_seed(w.seed)
    x = torch.randn((w.M, w.K), generator=gen, device=device)
    ch = torch.randperm(w.K, generator=gen, device=device)[:LINEAR_OUTLIERS]
    x[:, ch] *= LINEAR_OUTLIER_SCALE
    wt = torch.randn((w.N, w.K), generator=gen, device=device) * (1.0 / np.sqrt(w.K))
    b = torch.randn(w.N, generator=gen, device=device) * 0.02
    return x.to(torch.bfloat16), wt.to(torch.bfloat16), b.to(torch.bfloat16)
