"""Output parity of block-sparse attention (sattn_fwd_block_sparse, through the C ABI) with the CPU oracle's masked
emulation: the attention layer computes only the regions its sparse block mask selects (page
"视频生成模型的高效推理加速机制解析", section "核心组成与关键能力", item 3 "稀疏注意力").

Same gates as the dense tests (rel-L2 <= 2e-3 vs the emulation, cosine vs fp64 where the emulation reaches it),
plus: a mask that keeps everything reproduces the dense call bit for bit, and query blocks whose mask row keeps
nothing are exactly zero."""
import numpy as np
import pytest
import torch

from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

from parity_helpers import check_output, device_inputs, f32, oracle_outputs, sample_heads, sample_rows, say, u16

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS

SMALL = [
    ("sp-d128", dict(H=2, Nq=300, Nkv=333, d=128)),    # 6 key blocks (ragged), 3 query blocks (ragged)
    ("sp-d64", dict(H=2, Nq=260, Nkv=200, d=64)),
    ("sp-long", dict(H=1, Nq=256, Nkv=9601, d=128)),   # 151 key blocks: the tile list spans several chunks
]


def run_sparse(w, mode, mask: np.ndarray):
    q, k, v = device_inputs(w)
    o = sattn.fwd_block_sparse(q, k, v, torch.from_numpy(mask).cuda(), mode=mode, sm_scale=w.sm_scale,
                               blk_q=w.blk_q)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_sparse_small_all_rows(name, shape, mode):
    w = wl.scaled(W["wan14b-720p"], name=name, seed=51, **shape)
    mask = wl.random_block_mask(w, density=0.4, seed=52)
    mask[0, 0, 1] = 0          # head 0: query block 1 attends to nothing
    mask[0, -1, 0, -1] = 1     # last head: query block 0 keeps the ragged last key block
    say(f"[sparse small] {name} mode {mode} kept {mask.mean():.2f}")
    o = run_sparse(w, mode, mask)
    got = f32(u16(o)).astype(np.float64)
    assert not got[0, 0, 128:256].any(), "a query block with an empty mask row must be zero"
    rows = np.arange(w.Nq, dtype=np.int32)
    for h in range(w.H):
        E, R = oracle_outputs(w, 0, h, mode, rows, w.blk_q, w.sm_scale, mask=mask[0, h])
        check_output(got[0, h], E, R, f"{name} h{h} mode {mode}")


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_full_mask_is_the_dense_call(mode):
    w = wl.scaled(W["wan14b-720p"], name="sp-full", H=2, Nq=300, Nkv=333, seed=53)
    q, k, v = device_inputs(w)
    dense = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=w.blk_q)
    o = run_sparse(w, mode, np.ones(wl.mask_dims(w), np.uint8))
    assert torch.equal(o.view(torch.int16), dense.view(torch.int16))


def test_empty_mask_is_zero():
    w = wl.scaled(W["wan14b-720p"], name="sp-empty", H=2, Nq=300, Nkv=333, seed=54)
    o = run_sparse(w, 2, np.zeros(wl.mask_dims(w), np.uint8))
    assert not o.view(torch.int16).any()


def test_sparse_full_size_band_sampled():
    """The 720p shape with a local band mask (~24 % of the key blocks), sampled heads and query blocks."""
    w = W["wan14b-720p"]
    mask = wl.band_block_mask(w, half_width=9450)
    say(f"[sparse full] {w.name} band mask, kept {mask.mean():.3f}")
    o = run_sparse(w, 2, mask)
    rows = sample_rows(w.Nq, w.blk_q)
    for h in sample_heads(w.H):
        E, R = oracle_outputs(w, 0, h, 2, rows, w.blk_q, w.sm_scale, mask=mask[0, h])
        got = f32(u16(o[0, h][torch.from_numpy(rows).long().to(o.device)])).astype(np.float64)
        check_output(got, E, R, f"720p band h{h}")
