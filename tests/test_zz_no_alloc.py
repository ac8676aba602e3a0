"""sattn_fwd_noalloc (the drop-in self-attention with the library's own per-GPU scratch array as its workspace, for
callers that cannot allocate) against sattn_fwd on the same inputs, through the C ABI: two calls in a row, the
second on a smaller input, in every mode; the outputs must be bit-identical to sattn_fwd's (the same kernels on the
same inputs), which passes the oracle's gates in the other tests."""
import pytest
import torch

from quantized_attention_05_amd import sattn
from quantized_attention_05_amd import workloads as wl

from parity_helpers import device_inputs, say

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
BIG = wl.scaled(W["wan14b-720p"], name="noalloc-big", H=3, Nq=1000, Nkv=1000, seed=61)
SMALL = wl.scaled(W["tiny"], name="noalloc-small", H=2, Nq=333, Nkv=197, seed=62)


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_noalloc_matches_fwd_twice_then_smaller(mode):
    for w, blk_q in ((BIG, 128), (SMALL, 64)):
        say(f"[noalloc] {w.name} mode {mode} H{w.H} Nq{w.Nq} Nkv{w.Nkv} d{w.d}")
        q, k, v = device_inputs(w)
        need = sattn.sattn_workspace_bytes(w.B, w.H, w.Nq, w.Nkv, w.d, blk_q, 64, mode)
        assert 0 < need <= sattn.NOALLOC_SCRATCH_BYTES
        o = torch.full_like(q, 7.0)
        sattn.fwd_noalloc(q, k, v, o, mode=mode, sm_scale=w.sm_scale, blk_q=blk_q)
        ref = sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=blk_q)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"{w.name} mode {mode}"


def test_noalloc_full_headline_heads_fit_or_are_refused():
    """A call whose workspace exceeds the array is refused with SATTN_ERR_WORKSPACE and leaves the output untouched;
    the largest number of 720p heads that fits runs and matches sattn_fwd."""
    w = W["wan14b-720p"]
    per_head = sattn.sattn_workspace_bytes(1, 1, w.Nq, w.Nkv, w.d, 128, 64, 2)
    heads = sattn.NOALLOC_SCRATCH_BYTES // per_head
    assert heads >= 1
    while sattn.sattn_workspace_bytes(1, heads, w.Nq, w.Nkv, w.d, 128, 64, 2) > sattn.NOALLOC_SCRATCH_BYTES:
        heads -= 1
    fit = wl.scaled(w, name="noalloc-720p", H=heads)
    q, k, v = device_inputs(fit)
    o = torch.empty_like(q)
    sattn.fwd_noalloc(q, k, v, o, mode=2, sm_scale=fit.sm_scale)
    ref = sattn.fwd(q, k, v, mode=2, sm_scale=fit.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    say(f"[noalloc] {heads} heads of the 720p shape fit")
    # one head more does not fit: refused on the host (the descriptors reuse head 0 with zero head strides, so even a
    # launch would stay inside q and o)
    before = o.clone()
    qd = sattn.sattn_tensor(q.data_ptr(), 1, heads + 1, w.Nq, w.d, 0, 0, 128)
    od = sattn.sattn_tensor(o.data_ptr(), 1, heads + 1, w.Nq, w.d, 0, 0, 128)
    with pytest.raises(sattn.SattnError) as ei:
        sattn.sattn_fwd_noalloc(qd, qd, qd, od, 0.0, 2, 128, 64, sattn._stream())
    assert ei.value.status == sattn.SATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), before.view(torch.int16))
