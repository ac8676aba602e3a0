"""Benchmark of the quantized self-attention hot path on one MI355X.

One step = one ``sattn_fwd`` call (quantization of Q/K/V followed by the fused attention kernel) on the
Wan-14B 720p self-attention shape (B=1, H=40, N=75600 latent tokens, d=128), INT8 Q*K^T + FP8-E4M3 P*V,
inputs resident in HBM.  Prints one JSON line with the effective attention throughput
(4*Nq*Nkv*d*H ops per call), the roofline position of the attention kernel (timed alone with HIP events on
the stream it runs on) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TOPS + % INT8 MFMA peak, Wan-14B 720p self-attn"
PEAK_TOPS = {0: 2500.0, 1: 5000.0, 2: 5000.0}  # dense MFMA peak of the kernel's dominant op (bf16 / int8+fp8)
INT8_PEAK_TOPS = 5000.0
HBM_PEAK_GBPS = 8000.0
MODE_DTYPE = {0: "bf16", 1: "int8+bf16", 2: "int8+fp8e4m3"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_attention_05_amd", "csrc", f) for f in ("attn.hip", "sattn_internal.h", "quant_rules.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, mode: int, launches_ops: float):
    """HBM bytes per launch of the attention kernel from committed rocprofv3 counter runs, or None when the
    counters were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{workload}/mode{mode}")
    if not rec or rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
            "total_bytes": rec["fetch_bytes"] + rec["write_bytes"], "source": rec.get("source", TRAFFIC_FILE)}


def record_traffic(root: str, workload: str, mode: int):
    """Writes the measured HBM traffic of the timed attention kernel into the traffic table, from four rocprofv3 runs
    under root (csv output, file prefix "run"): pmc_FETCH_SIZE and pmc_WRITE_SIZE of this benchmark (--steps 1
    --warmup 0 --kernel-reps 1, so the timed instance runs as the kernel-alone reps) and copy_FETCH_SIZE and
    copy_WRITE_SIZE of --calibrate-copy.  A counter's values are summed per dispatch over its instances; the copy of
    a known byte count turns counter units into bytes.  Needs no GPU."""
    import csv

    from quantized_attention_05_amd import workloads as wl

    def per_dispatch(run: str, match: str):
        sums = {}
        with open(os.path.join(root, run, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if match in r["Kernel_Name"]:
                    k = int(r["Dispatch_Id"])
                    sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
        return [sums[k] for k in sorted(sums)]

    kernel = f"attn_pipe_kernel<{mode}, 128, 4, false, false>"
    copy_bytes = 1 << 28
    fetch, write = per_dispatch("pmc_FETCH_SIZE", kernel), per_dispatch("pmc_WRITE_SIZE", kernel)
    cf, cw = per_dispatch("copy_FETCH_SIZE", "copyBuffer"), per_dispatch("copy_WRITE_SIZE", "copyBuffer")
    if not (fetch and write and cf and cw):
        raise SystemExit(f"record-traffic: missing dispatches of {kernel} or of the copy under {root}")
    ff = copy_bytes / 1024 / (sum(cf) / len(cf))  # counter unit -> KiB of traffic
    fw = copy_bytes / 1024 / (sum(cw) / len(cw))
    w = wl.WORKLOADS[workload]
    nqb, nkb = -(-w.Nq // w.blk_q), -(-w.Nkv // 64)
    # codes read once (Q, K, V: one byte per element), O written once (bf16), and the scales
    algorithmic = w.B * w.H * (w.Nq * w.d + 2 * w.Nkv * w.d + 2 * w.Nq * w.d + 4 * (nqb + nkb + w.d))
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[f"{workload}/mode{mode}"] = {
        "kernel": kernel,
        "kernel_source_sha": kernel_source_hash(),
        "fetch_kib_per_dispatch": [round(x, 1) for x in fetch],
        "write_kib_per_dispatch": [round(x, 1) for x in write],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": round(sum(cf) / len(cf), 1),
                             "write_kib": round(sum(cw) / len(cw), 1), "fetch_factor": round(ff, 5),
                             "write_factor": round(fw, 5)},
        "fetch_bytes": round(sum(fetch) / len(fetch) * ff * 1024),
        "write_bytes": round(sum(write) / len(write) * fw * 1024),
        "algorithmic_bytes": algorithmic,
        "source": "profiles/attn_kernel_wan14b-720p_i8fp8_traffic.md",
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print(json.dumps(table[f"{workload}/mode{mode}"]))


def layer_selective(args):
    """The layer-selective pass: 40 self-attention calls on fresh tensors in a fixed seeded per-layer mode
    pattern (8 layers bf16, 32 layers INT8+FP8), each followed by a cross-attention call over 769 keys.
    Values do not change the timing, so the tensors are drawn on the GPU (torch generator seeded per layer)."""
    import torch

    from quantized_attention_05_amd import sattn
    from quantized_attention_05_amd import workloads as wl

    ws_ = wl.WORKLOADS["layersel-720p-self"]
    wc_ = wl.WORKLOADS["layersel-720p-cross"]
    modes = wl.layer_modes()
    dev = torch.device("cuda:0")
    shape_q = (ws_.B, ws_.H, ws_.Nq, ws_.d)
    shape_c = (wc_.B, wc_.H, wc_.Nkv, wc_.d)
    layers = []
    for i in range(wl.LAYERSEL_LAYERS):
        gen = torch.Generator(device=dev).manual_seed(ws_.seed + i)
        q, k, v = (torch.randn(shape_q, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
        genc = torch.Generator(device=dev).manual_seed(wc_.seed + i)
        kc, vc = (torch.randn(shape_c, generator=genc, device=dev).to(torch.bfloat16) for _ in range(2))
        layers.append((q, k, v, kc, vc))
    o = torch.empty(shape_q, dtype=torch.bfloat16, device=dev)
    ws_bytes = max(sattn.sattn_workspace_bytes(ws_.B, ws_.H, ws_.Nq, ws_.Nkv, ws_.d, 128, 64, m) for m in range(3))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def one_pass():
        for (q, k, v, kc, vc), m in zip(layers, modes):
            sattn.fwd(q, k, v, mode=m, sm_scale=ws_.sm_scale, out=o, workspace=ws)
            sattn.cross_fwd(q, kc, vc, mode=0, sm_scale=wc_.sm_scale, out=o, workspace=ws)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = GpuSampler(pci=gpu_pci_address()).start()
    e0.record(stream)
    for _ in range(args.steps):
        one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_state = sampler.stop()
    ms = e0.elapsed_time(e1) / args.steps
    ops = wl.LAYERSEL_LAYERS * (ws_.ops + wc_.ops)
    print(json.dumps({
        "metric": "effective attention TOPS, layer-selective Wan-14B 720p pass (40 self + 40 cross calls)",
        "value": round(ops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8+fp8e4m3 / bf16 per layer",
        "data": "synthetic: N(0,1) drawn on the GPU, torch generator seeded per layer",
        "config": {"workload": "layer-selective pass", "layers": wl.LAYERSEL_LAYERS,
                   "modes": "".join(str(m) for m in modes), "self": [ws_.H, ws_.Nq, ws_.d],
                   "cross_nkv": wc_.Nkv, "cross_mode": "bf16"},
        "pct_int8_mfma_peak": round(100.0 * ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
        "gpu_clock_power": gpu_state,
    }), flush=True)


def block_sparse(args):
    """Block-sparse self-attention at the Wan-14B 720p shape (INT8+FP8 unless --mode says otherwise) with a local
    band mask (query block i keeps the key blocks within 9450 tokens of it, plus the first block: ~24 % of the
    blocks).  Reports the TOPS of the work actually done (kept query-key pairs) and, for comparison, the dense call
    on the same inputs.  Inputs are drawn on the GPU (values do not change the timing)."""
    import torch

    from quantized_attention_05_amd import sattn
    from quantized_attention_05_amd import workloads as wl

    w = wl.WORKLOADS["wan14b-720p"]
    mode = args.mode
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    shape = (w.B, w.H, w.Nq, w.d)
    q, k, v = (torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    mask_np = wl.band_block_mask(w, half_width=9450)
    mask = torch.from_numpy(mask_np).to(dev)
    pairs = wl.kept_pairs(w, mask_np)
    ops_kept = 4.0 * pairs * w.d
    o = torch.empty_like(q)
    ws = torch.empty(sattn.sattn_workspace_bytes(w.B, w.H, w.Nq, w.Nkv, w.d, w.blk_q, 64, mode), dtype=torch.uint8,
                     device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = timed(lambda: sattn.fwd_block_sparse(q, k, v, mask, mode=mode, sm_scale=w.sm_scale, blk_q=w.blk_q, out=o,
                                              workspace=ws))
    ms_dense = timed(lambda: sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=w.blk_q, out=o, workspace=ws))
    print(json.dumps({
        "metric": "block-sparse attention TOPS on the kept blocks, Wan-14B 720p self-attn, local band mask",
        "value": round(ops_kept / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": MODE_DTYPE[mode],
        "data": ("synthetic: N(0,1) drawn on the GPU; band block mask "
                 "(recipe in quantized_attention_05_amd/workloads.py)"),
        "config": {"workload": "wan14b-720p block-sparse self-attention", "B": w.B, "H": w.H, "Nq": w.Nq,
                   "Nkv": w.Nkv, "d": w.d, "mode": wl.MODE_NAMES[mode], "mask": "band, half-width 9450 tokens, 1 sink",
                   "kept_block_fraction": round(float(mask_np.mean()), 4),
                   "kept_pair_fraction": round(pairs / (w.B * w.H * w.Nq * w.Nkv), 4)},
        "dense_ms_per_step": round(ms_dense, 3),
        "speedup_vs_dense": round(ms_dense / ms, 3),
        "dense_equivalent_tops": round(w.ops / (ms * 1e-3) / 1e12, 2),
    }), flush=True)


def layer_probe(args):
    """The per-layer attention-error probe of layer-selective quantization at the Wan-14B 720p layer shape: the
    layer's self-attention in mode 2 and in mode 0 on the same inputs, then the per-head error sums on the GPU.
    Reports the time of one layer's probe and, separately, of the error-sum kernel (which reads both outputs)."""
    import torch

    from quantized_attention_05_amd import policy
    from quantized_attention_05_amd import sattn
    from quantized_attention_05_amd import workloads as wl

    w = wl.WORKLOADS["wan14b-720p"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    shape = (w.B, w.H, w.Nq, w.d)
    q, k, v = (torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    ws = torch.empty(max(sattn.sattn_workspace_bytes(w.B, w.H, w.Nq, w.Nkv, w.d, w.blk_q, 64, m) for m in (0, 2)),
                     dtype=torch.uint8, device=dev)
    o2 = sattn.fwd(q, k, v, mode=2, sm_scale=w.sm_scale, workspace=ws)
    o0 = sattn.fwd(q, k, v, mode=0, sm_scale=w.sm_scale, workspace=ws)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        sattn.error_stats(o2, o0)
    e0.record(stream)
    for _ in range(args.steps):
        sattn.error_stats(o2, o0)
    e1.record(stream)
    torch.cuda.synchronize()
    stats_ms = e0.elapsed_time(e1) / args.steps
    for _ in range(args.warmup):
        policy.probe_error(q, k, v, mode=2, sm_scale=w.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rel, cos, _ = policy.probe_error(q, k, v, mode=2, sm_scale=w.sm_scale, workspace=ws)
    probe_ms = (time.perf_counter() - t0) * 1e3 / args.steps  # includes the host copy of the 40 x 4 sums
    out_bytes = 2 * w.B * w.H * w.Nq * w.d * 2
    print(json.dumps({
        "metric": "per-layer attention-error probe time (mode 2 vs bf16 + per-head error sums), Wan-14B 720p layer",
        "value": round(probe_ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(probe_ms, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+fp8e4m3 vs bf16; sums in f64", "data": "synthetic: N(0,1) drawn on the GPU",
        "config": {"workload": "wan14b-720p layer probe", "B": w.B, "H": w.H, "N": w.Nq, "d": w.d},
        "error_stats_ms": round(stats_ms, 4),
        "error_stats_gbps": round(out_bytes / (stats_ms * 1e-3) / 1e9, 1),
        "rel_l2_mode2_vs_bf16": rel, "cos_mode2_vs_bf16": cos,
    }), flush=True)


def linear_layers(args):
    """The quantized linear layer at the Wan-14B 720p shapes (75 600 tokens): one JSON line per shape with W8A8 (the
    headline: effective TOPS over 2 M N K), W8A16, the GEMM kernel alone on prepared codes, the activation
    quantization alone, and, as context, torch's bf16 linear and its plain INT8 matrix product (`torch._int_mm`:
    int32 out, no block scales, no bias; both hipBLASLt) on the same tensors and codes."""
    import torch

    from quantized_attention_05_amd import sattn
    from quantized_attention_05_amd import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(max(args.warmup, 1)):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for name in ("wan14b-720p-ffn-up", "wan14b-720p-ffn-down", "wan14b-720p-proj"):
        w = wl.LINEAR_WORKLOADS[name]
        x, wt, b = wl.linear_device_inputs(w, dev)
        wq, sw = sattn.quantize_blocks(wt)
        y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(sattn.sattn_linear_workspace_bytes(w.M, w.N, w.K, m) for m in (0, 1)), dtype=torch.uint8,
                         device=dev)
        xq, sx = sattn.quantize_blocks(x)
        ms8 = timed(lambda: sattn.linear(x, wq, sw, b, mode=sattn.SATTN_LINEAR_W8A8, out=y, workspace=ws), args.steps)
        ms16 = timed(lambda: sattn.linear(x, wq, sw, b, mode=sattn.SATTN_LINEAR_W8A16, out=y, workspace=ws),
                     args.steps)
        gemm8 = timed(lambda: sattn.linear_quantized(xq, sx, wq, sw, b, out=y), args.steps)
        quant = timed(lambda: sattn.quantize_blocks(x), args.steps)
        bf16 = timed(lambda: torch.nn.functional.linear(x, wt, b), args.steps)
        # the vendor library's plain INT8 GEMM on the same codes (int32 out, no block scales, no bias)
        int8mm = timed(lambda: torch._int_mm(xq, wq.t()), args.steps)
        tops = lambda ms: round(w.ops / (ms * 1e-3) / 1e12, 1)
        print(json.dumps({
            "metric": f"quantized linear layer TOPS (2 M N K), Wan-14B 720p {name.split('720p-')[1]}",
            "value": tops(ms8), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms8, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int8 (W8A8, 128x128 blocks)", "data": "synthetic: N(0,1) x with x20 outlier channels, "
            "N(0,1/K) weights, drawn on the GPU (recipe in quantized_attention_05_amd/workloads.py)",
            "config": {"workload": f"{name} linear", "M": w.M, "N": w.N, "K": w.K},
            "pct_int8_mfma_peak": round(100 * w.ops / (ms8 * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
            "w8a8_ms": round(ms8, 4), "w8a16_ms": round(ms16, 4), "w8a16_tops": tops(ms16),
            "gemm_w8a8_kernel_ms": round(gemm8, 4), "gemm_w8a8_kernel_tops": tops(gemm8),
            "quantize_x_ms": round(quant, 4),
            "quantize_x_gbps": round(w.M * w.K * 3 / (quant * 1e-3) / 1e9, 1),
            "torch_bf16_linear_ms": round(bf16, 4), "torch_bf16_linear_tops": tops(bf16),
            "torch_int8_mm_ms": round(int8mm, 4), "torch_int8_mm_tops": tops(int8mm),
        }), flush=True)
        del x, wt, b, wq, sw, y, ws, xq, sx
        torch.cuda.empty_cache()


def cpu_baseline(w, mode: int, budget_s: float):
    """The oracle, as it stands, on a bounded sample: heads {0, H/2, H-1} are quantized in full, then query blocks
    {first, middle, last} of each of them are emulated against all keys, followed by further blocks of the three
    heads in turn, until about `budget_s` seconds of CPU time are spent.  Extrapolated linearly to the whole call
    (H heads x all query rows) and reported as effective TOPS."""
    import numpy as np

    import oracle
    from quantized_attention_05_amd import workloads as wl

    heads = sorted({0, w.H // 2, w.H - 1})
    nqb = -(-w.Nq // w.blk_q)
    t_quant, data = 0.0, []
    for h in heads:
        q, k, v = (wl.bits(t) for t in wl.head_inputs(w, 0, h))
        t0 = time.perf_counter()
        quant = oracle.quantize_head(q, k, v, w.blk_q, w.blk_k, mode) if mode != 0 else None
        t_quant += time.perf_counter() - t0
        data.append((q, k, v, quant))
    # blocks {0, middle, last} of every sampled head first, then spread blocks of each head in turn
    extra = sorted({int(i) for i in np.linspace(1, nqb - 2, 64).astype(int)})
    order = [(hi, blk) for blk in (0, nqb // 2, nqb - 1) for hi in range(len(heads))]
    order += [(hi, blk) for blk in extra for hi in range(len(heads)) if blk not in (0, nqb // 2, nqb - 1)]
    rows_done, t_attn, done = 0, 0.0, []
    for hi, blk in order:
        q, k, v, quant = data[hi]
        rows = np.arange(blk * w.blk_q, min((blk + 1) * w.blk_q, w.Nq), dtype=np.int32)
        t0 = time.perf_counter()
        if mode == 0:
            oracle.attn_emulate(0, rows, tile=64, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=w.blk_k, nkv=w.Nkv,
                                q_bf16=q, k_bf16=k, v_bf16=v)
        else:
            oracle.attn_emulate(mode, rows, tile=64, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=w.blk_k, nkv=w.Nkv,
                                quant=quant, v_bf16=v)
        t_attn += time.perf_counter() - t0
        rows_done += rows.size
        done.append((heads[hi], blk))
        if t_quant + t_attn >= budget_s and len(done) >= 3 * len(heads):
            break
    # per head: its quantization plus all Nq rows at the measured rate
    t_call = w.H * w.B * (t_quant / len(heads) + t_attn * (w.Nq / rows_done))
    return {
        "value": w.ops / t_call / 1e12,
        "unit": "TOPS",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": (f"heads {heads} of {w.name}: full quantization ({t_quant:.2f} s) + step-by-step emulation of "
                   f"{rows_done} query rows in {len(done)} blocks (first/middle/last of each head, then spread) "
                   f"against all {w.Nkv} keys ({t_attn:.2f} s); extrapolated to {w.B * w.H} heads x {w.Nq} rows = "
                   f"{t_call:.1f} s per call"),
        "seconds_measured": round(t_quant + t_attn, 2),
    }


def gpu_pci_address(index: int = 0) -> str | None:
    """The PCI address of torch's GPU `index` as sysfs names it ("0000:75:00.0"), or None if torch does not say."""
    import torch

    p = torch.cuda.get_device_properties(index)
    try:
        return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    except AttributeError:
        return None


class GpuSampler:
    """Samples the GPU's power draw and its current core clock from sysfs (hwmon `power1_input`, `power1_cap`; the
    current level of `pp_dpm_sclk`) on a host thread while the timed steps run; reads files only, no GPU calls.
    Reports None where the files are missing (not an AMD GPU driver, or no permission)."""

    def __init__(self, period_s: float = 0.01, pci: str | None = None):
        """pci: the PCI address ("0000:75:00.0") of the GPU to read."""
        import glob
        import os
        import threading

        self.period_s, self.samples, self._stop = period_s, [], threading.Event()
        cards = []
        for d in sorted(glob.glob("/sys/class/drm/card*/device")):
            try:
                if open(f"{d}/vendor").read().strip() == "0x1002" and glob.glob(f"{d}/hwmon/hwmon*/power1_input"):
                    cards.append(d)
            except OSError:
                continue
        match = [d for d in cards if pci is not None and os.path.basename(os.path.realpath(d)).lower() == pci.lower()]
        # the card at that PCI address; else the only AMD card there is; else none (rather than another GPU's)
        self.dev = match[0] if match else (cards[0] if len(cards) == 1 else None)
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        import glob

        hw = glob.glob(f"{self.dev}/hwmon/hwmon*")[0]
        power = int(open(f"{hw}/power1_input").read()) / 1e6
        mhz = None
        for line in open(f"{self.dev}/pp_dpm_sclk"):
            if line.rstrip().endswith("*"):
                mhz = int(line.split(":")[1].strip().split("M")[0])
        return power, mhz

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except (OSError, ValueError, IndexError):
                return
            self._stop.wait(self.period_s)

    def start(self):
        if self.dev:
            self._thread.start()
        return self

    def stop(self):
        if not self.dev:
            return None
        self._stop.set()
        self._thread.join()
        try:
            hw = __import__("glob").glob(f"{self.dev}/hwmon/hwmon*")[0]
            cap = int(open(f"{hw}/power1_cap").read()) / 1e6
        except (OSError, ValueError, IndexError):
            cap = None
        pw = sorted(p for p, _ in self.samples)
        mhz = sorted(c for _, c in self.samples if c is not None)
        med = lambda xs: xs[len(xs) // 2] if xs else None
        return {"power_cap_w": cap, "power_w_median": med(pw), "power_w_max": pw[-1] if pw else None,
                "sclk_mhz_median": med(mhz), "sclk_mhz_min": mhz[0] if mhz else None,
                "sclk_mhz_max": mhz[-1] if mhz else None, "samples": len(self.samples),
                "source": f"{self.dev}: hwmon power1_input / power1_cap, current pp_dpm_sclk level, "
                          f"every {self.period_s * 1e3:.0f} ms during the timed steps"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b-720p",
                    help="a name from quantized_attention_05_amd.workloads.WORKLOADS, 'layersel', 'sparse', 'probe' or "
                         "'linear'")
    ap.add_argument("--mode", type=int, default=2, choices=[0, 1, 2])
    ap.add_argument("--nkv", type=int, default=None,
                    help="key sequence length instead of the workload's own (same recipe; e.g. a cross-attention sweep)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=None, help="attention-kernel-only timing reps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run one plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--record-traffic", metavar="DIR", default=None,
                    help="no GPU run: write the attention kernel's HBM traffic from the rocprofv3 counter runs under "
                         "DIR into profiles/traffic.json")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.record_traffic, args.workload, args.mode)
        return

    if args.calibrate_copy:
        import torch

        x = torch.full((1 << 28,), 1, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": x.numel()}))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the attention of one (batch, head) never "
                                   "leaves its GPU, and no multi-GPU path is built; run with --gpus 1"}))
        sys.exit(2)
    if args.workload == "layersel":
        layer_selective(args)
        return
    if args.workload == "sparse":
        block_sparse(args)
        return
    if args.workload == "probe":
        layer_probe(args)
        return
    if args.workload == "linear":
        linear_layers(args)
        return

    import torch

    from quantized_attention_05_amd import sattn
    from quantized_attention_05_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if args.nkv is not None and args.nkv != w.Nkv:
        w = wl.scaled(w, name=f"{w.name}-nkv{args.nkv}", Nkv=args.nkv)
    mode = args.mode
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    q, k, v = wl.full_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    gen_s = time.perf_counter() - t0
    o = torch.empty_like(q)
    ws_bytes = sattn.sattn_workspace_bytes(w.B, w.H, w.Nq, w.Nkv, w.d, w.blk_q, w.blk_k, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        sattn.fwd(q, k, v, mode=mode, sm_scale=w.sm_scale, blk_q=w.blk_q, blk_k=w.blk_k, out=o, workspace=ws)

    # warm-up: the W steps asked for and, unless W is 0, more until 0.1 s of them have run, so that a short call (a
    # cross-attention call takes about 1 ms) is timed at the clock the GPU settles to under load, not while it ramps up
    warm, w0 = 0, time.perf_counter()
    while warm < args.warmup or (args.warmup > 0 and time.perf_counter() - w0 < 0.1 and warm < 10000):
        step()
        torch.cuda.synchronize()
        warm += 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # one event between consecutive steps as well, for the per-step spread (median, min, max)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    sampler = GpuSampler(pci=gpu_pci_address()).start()
    wall0 = time.perf_counter()
    e0.record(stream)
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_state = sampler.stop()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = w.ops / (ms_per_step * 1e-3) / 1e12
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))

    # the dominant kernel alone: attention on prepared operands, HIP events on the same stream
    qz = sattn.Quantized(w.B, w.H, w.Nq, w.Nkv, w.d, w.blk_q, mode, dev)
    sattn.quantize(q, k, v, mode=mode, blk_q=w.blk_q, quant=qz)
    qarg = q if mode == 0 else None
    karg = k if mode == 0 else None
    reps = args.kernel_reps or max(5, args.steps)
    for _ in range(2):
        sattn.fwd_quantized(qz, qarg, karg, sm_scale=w.sm_scale, out=o)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        sattn.fwd_quantized(qz, qarg, karg, sm_scale=w.sm_scale, out=o)
    e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = e0.elapsed_time(e1) / reps
    # quantization alone (HBM-bound): algorithmic bytes = read Q, K, V (bf16) + write codes
    e0.record(stream)
    for _ in range(reps):
        sattn.quantize(q, k, v, mode=mode, blk_q=w.blk_q, quant=qz)
    e1.record(stream)
    torch.cuda.synchronize()
    quant_ms = e0.elapsed_time(e1) / reps
    elems_q, elems_kv = w.B * w.H * w.Nq * w.d, w.B * w.H * w.Nkv * w.d
    if mode == 0:
        quant_bytes = elems_kv * 2 * 2                       # V read + transposed V written
    elif mode == 1:
        quant_bytes = (elems_q + 2 * elems_kv) * 2 + elems_q + elems_kv + elems_kv * 2
    else:
        quant_bytes = (elems_q + 2 * elems_kv) * 2 + elems_q + 2 * elems_kv

    achieved = w.ops / (attn_ms * 1e-3) / 1e12
    traffic_detail = measured_traffic(w.name, mode, w.ops)
    line = {
        # the headline workload keeps the headline metric's name; the others name their own workload
        "metric": METRIC if w.name == "wan14b-720p" else f"effective attention TOPS + % INT8 MFMA peak, {w.name}",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median_min_max": [round(step_ms[len(step_ms) // 2], 4), round(step_ms[0], 4),
                                       round(step_ms[-1], 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": MODE_DTYPE[mode],
        "data": ("synthetic: seeded Wan-shaped N(0,1) Q/K/V, K per-channel offsets, zeroed K blocks "
                 "(recipe in quantized_attention_05_amd/workloads.py)"),
        "config": {"workload": f"{w.name} self-attention" if "cross" not in w.name else f"{w.name} attention",
                   "B": w.B, "H": w.H, "Nq": w.Nq, "Nkv": w.Nkv, "d": w.d, "mode": wl.MODE_NAMES[mode],
                   "blk_q": w.blk_q, "blk_k": w.blk_k, "parallelism": "single GPU"},
        "pct_int8_mfma_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "attn_kernel_ms": round(attn_ms, 4),
        "quantize_ms": round(quant_ms, 4),
        "quantize_gbps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_TOPS[mode],
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TOPS[mode], 4),
            "traffic": traffic_detail["total_bytes"] if traffic_detail else None,
            "traffic_detail": traffic_detail,
            "kernel": f"attn_pipe_kernel<{mode}, {w.d}, 4, false, false>",
            "ops_per_launch": w.ops,
        },
        "wall_s_timed_region": round(wall, 3),
        "gpu_clock_power": gpu_state,
        "input_generation_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, mode, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
