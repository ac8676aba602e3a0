"""Pins for the oracle's block-sparse attention: a [query blocks of 128 rows, key blocks of 64 keys] byte mask
selects the regions each query block attends to (page "视频生成模型的高效推理加速机制解析", section "核心组成与关键能力",
item 3 "稀疏注意力", and step 3 of "工作原理与执行流程": the attention layer computes only what its sparse mask
selects).

Pins, none of which retypes the masked loop:
* leaving key blocks out is the same computation as attending densely to the concatenation of the kept blocks
  (codes, scales and V gathered by block), bit for bit, for the emulation of all three modes and for R;
* a mask that keeps everything is the dense result, bit for bit;
* a query block whose mask keeps nothing gets exactly 0;
* keeping one block of identical keys gives uniform attention over that block: the plain mean of its V rows
  (mode 0, bf16 values exact), computed here with numpy;
* the mask is read per query block of mask_qblk rows (rows of one block share a mask row).
"""
import numpy as np
import pytest

from quantized_attention_05_amd import workloads as wl

KB = 64  # keys per mask block


def head(n, d, seed):
    w = wl.scaled(wl.WORKLOADS["tiny"], name="sparse", H=1, Nq=n, Nkv=n, d=d, seed=seed)
    q, k, v = wl.head_inputs(w, 0, 0)
    return w, wl.bits(q), wl.bits(k), wl.bits(v)


def gather_blocks(a, blocks, nkv):
    """Rows of the kept 64-key blocks of a per-key array (the last block may be ragged)."""
    idx = np.concatenate([np.arange(b * KB, min((b + 1) * KB, nkv)) for b in blocks])
    return a[idx]


def emulate(orc, mode, w, qb, kb, vb, rows, nkv, quant=None, **kw):
    if mode == 0:
        return orc.attn_emulate(0, rows, tile=64, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=64, nkv=nkv,
                                q_bf16=qb, k_bf16=kb, v_bf16=vb, **kw)
    return orc.attn_emulate(mode, rows, tile=64, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=64, nkv=nkv,
                            quant=quant, v_bf16=vb, **kw)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_masked_equals_dense_over_gathered_blocks(orc, mode):
    n, d = 300, 64  # 5 key blocks, the last one ragged (44 keys); 3 query blocks of 128 rows (the last ragged)
    w, qb, kb, vb = head(n, d, seed=31)
    qz = orc.quantize_head(qb, kb, vb, w.blk_q, 64, max(mode, 1)) if mode else None
    nkb = -(-n // KB)
    rng = np.random.default_rng(7)
    mask = (rng.random((3, nkb)) < 0.55).astype(np.uint8)
    mask[0, nkb - 1] = 1  # one query block keeps the ragged block, one drops it
    mask[1, nkb - 1] = 0
    mask[1, 0] = 1
    for qblk in range(3):
        rows = np.arange(qblk * 128, min((qblk + 1) * 128, n), dtype=np.int32)
        got = emulate(orc, mode, w, qb, kb, vb, rows, n, quant=qz, mask=mask, mask_qblk=128)
        kept = np.flatnonzero(mask[qblk])
        nk = sum(min((b + 1) * KB, n) - b * KB for b in kept)
        if mode == 0:
            ref = emulate(orc, 0, w, qb, gather_blocks(kb, kept, n), gather_blocks(vb, kept, n), rows, nk)
        else:
            gz = dict(qz)
            gz["k_codes"] = gather_blocks(qz["k_codes"], kept, n)
            gz["k_scales"] = qz["k_scales"][kept]
            if mode == 2:
                gz["v_codes"] = gather_blocks(qz["v_codes"], kept, n)
            ref = emulate(orc, mode, w, qb, None, gather_blocks(vb, kept, n), rows, nk, quant=gz)
        assert np.array_equal(got, ref), (mode, qblk)
        r_got = orc.attn_ref_fp64(qb, kb, vb, rows, w.sm_scale, mask=mask, mask_qblk=128)
        r_ref = orc.attn_ref_fp64(qb, gather_blocks(kb, kept, n), gather_blocks(vb, kept, n), rows, w.sm_scale)
        assert np.array_equal(r_got, r_ref)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_full_mask_is_dense_and_empty_row_is_zero(orc, mode):
    n, d = 200, 64
    w, qb, kb, vb = head(n, d, seed=32)
    qz = orc.quantize_head(qb, kb, vb, w.blk_q, 64, max(mode, 1)) if mode else None
    rows = np.arange(n, dtype=np.int32)
    nkb = -(-n // KB)
    full = np.ones((2, nkb), np.uint8)
    dense = emulate(orc, mode, w, qb, kb, vb, rows, n, quant=qz)
    assert np.array_equal(emulate(orc, mode, w, qb, kb, vb, rows, n, quant=qz, mask=full), dense)
    half = full.copy()
    half[1] = 0  # the second query block (rows 128..199) keeps nothing
    got = emulate(orc, mode, w, qb, kb, vb, rows, n, quant=qz, mask=half)
    assert np.array_equal(got[:128], dense[:128])
    assert not got[128:].any()
    r = orc.attn_ref_fp64(qb, kb, vb, rows, w.sm_scale, mask=half)
    assert not r[128:].any() and np.array_equal(r[:128], orc.attn_ref_fp64(qb, kb, vb, rows[:128], w.sm_scale))


def test_single_block_of_equal_keys_gives_its_mean(orc):
    n, d = 256, 64
    w, qb, kb, vb = head(n, d, seed=33)
    kb = kb.copy()
    kb[128:192] = kb[128]  # block 2: 64 identical keys
    mask = np.zeros((2, 4), np.uint8)
    mask[:, 2] = 1
    rows = np.arange(0, n, 5, dtype=np.int32)
    got = emulate(orc, 0, w, qb, kb, vb, rows, n, mask=mask)
    v2 = (vb[128:192].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mean = v2.mean(axis=0)  # every p = 1 exactly (x = m), P = 1 in bf16, so O = sum(v) / 64
    expect = ((mean.astype(np.float32).view(np.uint32) + 0x7FFF + ((mean.astype(np.float32).view(np.uint32) >> 16) & 1))
              >> 16).astype(np.uint16)
    assert np.array_equal(got, np.broadcast_to(expect, got.shape))
    r = orc.attn_ref_fp64(qb, kb, vb, rows, w.sm_scale, mask=mask)
    assert np.allclose(r, mean[None, :], rtol=0, atol=1e-12)


def test_mask_rows_follow_query_blocks(orc):
    """With mask_qblk = 64, rows 0..63 and 64..127 read different mask rows."""
    n, d = 192, 64
    w, qb, kb, vb = head(n, d, seed=34)
    mask = np.zeros((3, 3), np.uint8)
    mask[0, 0] = mask[1, 1] = mask[2, 2] = 1
    rows = np.arange(n, dtype=np.int32)
    got = emulate(orc, 0, w, qb, kb, vb, rows, n, mask=mask, mask_qblk=64)
    for blk in range(3):
        r = rows[blk * 64:(blk + 1) * 64]
        ref = emulate(orc, 0, w, qb, kb[blk * 64:(blk + 1) * 64], vb[blk * 64:(blk + 1) * 64], r, 64)
        assert np.array_equal(got[blk * 64:(blk + 1) * 64], ref)
