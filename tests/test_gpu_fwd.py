"""Output parity of the attention kernels (through the C ABI) with the CPU oracle.

Gate: relative L2 <= 2e-3 against the oracle's step-by-step emulation of the same quantized algorithm,
cosine >= 0.999 against exact fp64 attention wherever the emulation itself reaches 0.999, every output
finite.  Small cases compare every output; the Wan-sized workloads compare the first, middle and last
(ragged) query blocks of three heads, run in the same launch configuration as the benchmark."""
import numpy as np
import pytest
import torch

import oracle
from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

from parity_helpers import (check_output, device_inputs, f32, head_bits, oracle_outputs, sample_heads, sample_rows,
                            say, u16)

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


def run_fwd(w, mode, blk_q, layout="bhnd", cross=False):
    q, k, v = device_inputs(w, layout=layout)
    if cross:
        o = sattn.cross_fwd(q, k, v, mode=mode, sm_scale=w.sm_scale)
    else:
        o = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=blk_q)
    torch.cuda.synchronize()
    return o


def compare(w, mode, blk_q, o, heads=None, rows=None, label=""):
    heads = range(w.H) if heads is None else heads
    for b in range(w.B):
        for h in heads:
            rr = np.arange(w.Nq, dtype=np.int32) if rows is None else rows
            E, R = oracle_outputs(w, b, h, mode, rr, blk_q, w.sm_scale)
            got = f32(u16(o[b, h][torch.from_numpy(rr).long().to(o.device)])).astype(np.float64)
            check_output(got, E, R, f"{label} b{b} h{h} mode {mode}")


SMALL = [
    ("tiny", W["tiny"], 64),
    ("ragged-d128", wl.scaled(W["wan14b-720p"], name="ragged-d128", H=3, Nq=1000, Nkv=1000, seed=11), 128),
    ("ragged-d64", wl.scaled(W["tiny"], name="ragged-d64", H=2, Nq=333, Nkv=197, seed=12), 64),
    ("outlier-q64", wl.scaled(W["wan1.3b-480p"], name="outlier-q64", H=2, Nq=700, Nkv=650, seed=13), 64),
    ("plain-b2", wl.scaled(W["layersel-720p-self"], name="plain-b2", B=2, H=2, Nq=520, Nkv=300, seed=14), 128),
]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("name,w,blk_q", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small_all_rows(name, w, blk_q, mode):
    say(f"[fwd] {name} mode {mode}")
    o = run_fwd(w, mode, blk_q)
    compare(w, mode, blk_q, o, label=name)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 129, 769])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_fwd_sequence_tails(n, mode):
    w = wl.scaled(W["layersel-720p-self"], name=f"tail{n}", H=1, Nq=n, Nkv=n, seed=100 + n)
    say(f"[fwd tail] N={n} mode {mode}")
    o = run_fwd(w, mode, 128)
    compare(w, mode, 128, o, label=f"N{n}")


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_cross_attention_short_keys(mode):
    w = wl.scaled(W["layersel-720p-cross"], name="cross-small", H=2, Nq=700, seed=31)
    say(f"[cross] Nq {w.Nq} Nkv {w.Nkv} mode {mode}")
    o = run_fwd(w, mode, 128, cross=True)
    compare(w, mode, 128, o, label="cross")


# Wan-sized workloads: sampled heads x (first, middle, last) query blocks
LARGE = [
    ("wan1.3b-480p", W["wan1.3b-480p"], 1),
    ("wan14b-480p", W["wan14b-480p"], 0),
    ("wan14b-480p", W["wan14b-480p"], 1),
    ("wan14b-480p", W["wan14b-480p"], 2),
    ("wan14b-480p-outlier", W["wan14b-480p-outlier"], 0),
    ("wan14b-480p-outlier", W["wan14b-480p-outlier"], 1),
    ("wan14b-480p-outlier", W["wan14b-480p-outlier"], 2),
    ("wan14b-720p", W["wan14b-720p"], 2),
    ("wan14b-720p", W["wan14b-720p"], 1),
    ("wan14b-720p", W["wan14b-720p"], 0),
    ("layersel-720p-self", W["layersel-720p-self"], 2),
    ("layersel-720p-self", W["layersel-720p-self"], 0),
    ("layersel-720p-cross", W["layersel-720p-cross"], 0),
    ("layersel-720p-cross", W["layersel-720p-cross"], 1),
    ("layersel-720p-cross", W["layersel-720p-cross"], 2),
]


@pytest.mark.parametrize("name,w,mode", LARGE, ids=[f"{c[0]}-m{c[2]}" for c in LARGE])
def test_fwd_full_size_sampled(name, w, mode):
    say(f"[fwd full] {name} mode {mode} H{w.H} Nq{w.Nq} Nkv{w.Nkv}")
    o = run_fwd(w, mode, w.blk_q, cross=name.endswith("cross"))
    compare(w, mode, w.blk_q, o, heads=sample_heads(w.H), rows=sample_rows(w.Nq, w.blk_q), label=name)


# ------------------------------------------------------------------------------------- degenerate inputs
@pytest.mark.parametrize("mode", [1, 2])
def test_zero_blocks_and_channels(mode):
    """All-zero Q block, constant K (every K' block guarded), all-zero V channel: finite, matches oracle."""
    w = wl.scaled(W["wan14b-720p"], name="degenerate", H=2, Nq=300, Nkv=200, seed=41)
    q, k, v = (t.clone() for t in wl.full_inputs(w))
    q[0, 0, 128:256] = 0                       # a whole Q block of head 0
    k[0, 1] = k[0, 1, :1].expand_as(k[0, 1])   # head 1: K constant over tokens -> K' == 0
    v[0, :, :, 7] = 0                          # V channel 7 of both heads
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = sattn.fwd(qd, kd, vd, mode=mode, sm_scale=w.sm_scale, blk_q=128)
    torch.cuda.synchronize()
    for h in range(2):
        qb, kb, vb = wl.bits(q[0, h]), wl.bits(k[0, h]), wl.bits(v[0, h])
        rows = np.arange(w.Nq, dtype=np.int32)
        qz = oracle.quantize_head(qb, kb, vb, 128, 64, mode)
        E = f32(oracle.attn_emulate(mode, rows, tile=64, sm_scale=w.sm_scale, blk_q=128, blk_k=64, nkv=w.Nkv,
                                    quant=qz, v_bf16=vb)).astype(np.float64)
        R = oracle.attn_ref_fp64(qb, kb, vb, rows, w.sm_scale)
        got = f32(u16(o[0, h])).astype(np.float64)
        check_output(got, E, R, f"degenerate h{h}")
        assert np.all(got[:, 7] == 0.0)


def test_deterministic_and_no_out_of_bounds_writes():
    w = wl.scaled(W["wan14b-720p"], name="canary", H=3, Nq=333, Nkv=444, seed=51)
    q, k, v = device_inputs(w)
    for mode in (0, 1, 2):
        big = torch.full((w.B * w.H * w.Nq * w.d + 4096,), 0x7ABC, dtype=torch.int16, device="cuda")
        o1 = big[:w.B * w.H * w.Nq * w.d].view(torch.bfloat16).view(w.B, w.H, w.Nq, w.d)
        sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, out=o1)
        o2 = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"mode {mode} not deterministic"
        assert torch.all(big[w.B * w.H * w.Nq * w.d:] == 0x7ABC), f"mode {mode} wrote past O"


def test_calls_follow_the_current_stream():
    """The entry points enqueue on the caller's current stream: quantize + attention and the linear layer called under
    a side stream (default priority) give the same bits as on the default stream once that stream alone is waited for."""
    w = wl.scaled(W["wan14b-720p"], name="stream", H=2, Nq=300, Nkv=260, seed=41)
    q, k, v = device_inputs(w)
    x = torch.randn((300, 256), device="cuda").to(torch.bfloat16)
    wt = (torch.randn((136, 256), device="cuda") * 0.06).to(torch.bfloat16)
    ref_o = sattn.fwd(q, k, v, mode=2, sm_scale=w.sm_scale)
    wq, sw = sattn.quantize_blocks(wt)
    ref_y = sattn.linear(x, wq, sw, mode=sattn.SATTN_LINEAR_W8A8)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = sattn.fwd(q, k, v, mode=2, sm_scale=w.sm_scale)
        y = sattn.linear(x, wq, sw, mode=sattn.SATTN_LINEAR_W8A8)
    side.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16))


def test_strided_layout_matches_dense():
    w = wl.scaled(W["wan14b-720p"], name="nhd", H=4, Nq=300, Nkv=260, seed=21)
    for mode in (0, 1, 2):
        a = run_fwd(w, mode, 128, layout="bhnd")
        b = run_fwd(w, mode, 128, layout="bnhd")
        assert torch.equal(a.view(torch.int16), b.contiguous().view(torch.int16))


def test_layer_selective_sequence_has_no_state():
    """Calls in the per-layer mode pattern give exactly what each call gives alone."""
    modes = wl.layer_modes(10, 3, seed=5)
    ws = None
    outs = []
    base = wl.scaled(W["layersel-720p-self"], name="ls", H=2, Nq=256, Nkv=256)
    need = max(sattn.sattn_workspace_bytes(1, 2, 256, 256, 128, 128, 64, m) for m in range(3))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for i, m in enumerate(modes):
        w = wl.scaled(base, seed=1000 + i)
        q, k, v = device_inputs(w)
        outs.append((m, w, sattn.fwd(q, k, v, mode=m, sm_scale=w.sm_scale, workspace=ws)))
    torch.cuda.synchronize()
    for m, w, o in outs:
        q, k, v = device_inputs(w)
        alone = sattn.fwd(q, k, v, mode=m, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), alone.view(torch.int16))


# ------------------------------------------------------------------------------------- prepared operands
QUANTIZED = [
    ("tiny", W["tiny"], 64),
    ("ragged-d128", wl.scaled(W["wan14b-720p"], name="ragged-d128", H=3, Nq=1000, Nkv=1000, seed=11), 128),
    ("ragged-d64", wl.scaled(W["tiny"], name="ragged-d64", H=2, Nq=333, Nkv=197, seed=12), 64),
    ("ragged-q64-d128", wl.scaled(W["wan1.3b-480p"], name="ragged-q64-d128", H=2, Nq=700, Nkv=650, seed=13), 64),
]


def run_fwd_quantized(w, mode, blk_q, q, k, v):
    qz = sattn.quantize(q, k, v, mode=mode, blk_q=blk_q)
    o = sattn.fwd_quantized(qz, q if mode == 0 else None, k if mode == 0 else None, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("name,w,blk_q", QUANTIZED, ids=[c[0] for c in QUANTIZED])
def test_fwd_quantized_matches_fwd_and_oracle(name, w, blk_q, mode):
    """sattn_quantize + sattn_fwd_quantized (the attention kernel on prepared operands, as the benchmark times it)
    gives exactly the bits of the drop-in sattn_fwd, and every row passes the oracle's gate."""
    say(f"[fwd_quantized] {name} mode {mode}")
    q, k, v = device_inputs(w)
    o = run_fwd_quantized(w, mode, blk_q, q, k, v)
    ref = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=blk_q)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"{name} mode {mode}: differs from sattn_fwd"
    compare(w, mode, blk_q, o, label=f"{name} prepared")


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_fwd_quantized_full_size(mode):
    """The headline 720p shape through sattn_fwd_quantized: bit-identical to sattn_fwd on the whole output, and the
    sampled rows of three heads pass the oracle's gate."""
    w = W["wan14b-720p"]
    say(f"[fwd_quantized full] {w.name} mode {mode}")
    q, k, v = device_inputs(w)
    o = run_fwd_quantized(w, mode, w.blk_q, q, k, v)
    ref = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=w.blk_q)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"mode {mode}: differs from sattn_fwd"
    del ref
    compare(w, mode, w.blk_q, o, heads=sample_heads(w.H), rows=sample_rows(w.Nq, w.blk_q), label=f"{w.name} prepared")
