"""The drop-in calls under HIP graph capture.  The library enqueues kernels only (no memset, no copy, no allocation
inside sattn_fwd / sattn_fwd_noalloc / sattn_cross_fwd), so a captured call must replay to the bits of the eager
call.  Each graph is replayed several times, with other eager work of the process and synchronisations between the
replays, and every replay is checked against the eager result."""
import pytest
import torch

from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

from parity_helpers import device_inputs, say

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


def bits(t):
    return t.view(torch.int16)


def replay_and_check(g, out, ref, noise):
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        noise()  # other eager work of the process between replays
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_captured_fwd_replays_to_the_eager_bits(mode):
    w = wl.scaled(W["wan14b-720p"], name="graph", H=2, Nq=700, Nkv=650, seed=41)
    say(f"[graph] sattn_fwd mode {mode} H{w.H} Nq{w.Nq} Nkv{w.Nkv}")
    q, k, v = device_inputs(w)
    ws = torch.empty(sattn.sattn_workspace_bytes(w.B, w.H, w.Nq, w.Nkv, w.d, 128, 64, mode), dtype=torch.uint8,
                     device="cuda")
    ref = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, workspace=ws)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, out=out, workspace=ws)
    q2, k2, v2 = device_inputs(wl.scaled(w, seed=42))
    replay_and_check(g, out, ref, lambda: sattn.fwd(q2, k2, v2, mode=mode, sm_scale=w.sm_scale, workspace=ws))


@pytest.mark.parametrize("mode", [2, 0])
def test_captured_noalloc_and_cross_replay_to_the_eager_bits(mode):
    w = wl.scaled(W["wan14b-720p"], name="graph-na", H=2, Nq=520, Nkv=300, seed=43)
    wc = wl.scaled(W["layersel-720p-cross"], name="graph-x", H=2, Nq=520, seed=44)
    say(f"[graph] sattn_fwd_noalloc + sattn_cross_fwd mode {mode}")
    q, k, v = device_inputs(w)
    _, kc, vc = device_inputs(wc)
    wsx = torch.empty(sattn.sattn_workspace_bytes(wc.B, wc.H, wc.Nq, wc.Nkv, wc.d, 128, 64, mode), dtype=torch.uint8,
                      device="cuda")
    ref = sattn.fwd_noalloc(q, k, v, torch.empty_like(q), mode=mode, sm_scale=w.sm_scale)
    refx = sattn.cross_fwd(q, kc, vc, mode=mode, sm_scale=wc.sm_scale, workspace=wsx)
    out, outx = torch.empty_like(q), torch.empty_like(q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # a self-attention layer followed by its cross-attention, as in the pass
        sattn.fwd_noalloc(q, k, v, out, mode=mode, sm_scale=w.sm_scale)
        sattn.cross_fwd(q, kc, vc, mode=mode, sm_scale=wc.sm_scale, out=outx, workspace=wsx)
    qn, kn, vn = device_inputs(wl.scaled(w, seed=45))
    for rep in range(3):
        out.zero_()
        outx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), f"replay {rep}: self-attention differs"
        assert torch.equal(bits(outx), bits(refx)), f"replay {rep}: cross-attention differs"
        # eager work between replays, sharing the library's scratch array with the graph's call
        sattn.fwd_noalloc(qn, kn, vn, torch.empty_like(qn), mode=mode, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
