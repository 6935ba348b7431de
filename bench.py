"""Benchmark of the grouped NF4 MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload olmoe]
                    [--no-cpu-baseline] [--no-decode] [--no-backward]
                    [--no-control] [--no-mxfp4] [--copy-calibration]
    python bench.py --summarize-trace DIR
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR
    python bench.py --summarize-pmc DIR KERNEL_SUBSTR
    python bench.py --summarize-decode-fetch FETCH_DIR

A step is one full routed-expert layer forward (route + permute, gate_up with
SwiGLU, down, combine) over the whole batch, inputs resident in HBM.  The
headline workload is the OLMoE-1B-7B-shaped prefill layer (E=64, H=2048,
I=1024, top-8, T=4096 tokens); the value is its algorithmic TFLOP/s
(6*T*k*H*I per forward).  The same JSON line carries:

  roofline      the dominant kernel (the gate_up grouped GEMM) timed alone
                with HIP events on the stream it runs on, against the fp16
                dense MFMA peak;
  decode        the batch-1 decode layer (Qwen3-30B-A3B shape, 8 routed
                experts) as packed-weight GB/s over 48 distinct layer stacks
                replayed from a HIP graph;
  mxfp4         the same prefill layer on released-MXFP4-format stacks
                (e2m1 + e8m0 bytes multiplied in place);
  storage_modes the same layer with the stacks stored as fp4, int8, fp8 and
                as plain bf16 / fp16 weights (the passthrough modes);
  backward      the QLoRA training backward of a layer (olmoe without
                adapters, qlora with r=8 adapters): time per backward and
                its two dgrad kernels timed alone;
  cpu_baseline  the CPU oracle timed on this host on the same layer shape.

Prints exactly one JSON line.

--copy-calibration first copies a 512 MiB buffer three times (a plain copy
of known size: its FETCH_SIZE / WRITE_SIZE counters scale the GEMM's).  The
two --summarize modes turn rocprofv3 output (a --kernel-trace --stats run, or
a FETCH_SIZE and a WRITE_SIZE --pmc run of this script with
--copy-calibration) into the markdown summaries kept under profiles/; the
counter summary carries the HBM bytes per gate_up launch that the roofline
line reports as `traffic` while the GEMM source is unchanged.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped NF4 MoE layer TFLOP/s (prefill) + packed-weight GB/s (decode M=1)"
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
DECODE_LAYERS = 48
COPY_BYTES = 512 << 20
COUNTERS_MD = os.path.join(ROOT, "profiles", "gate_up_gemm_olmoe_counters.md")
GEMM_SRC = os.path.join(ROOT, "grouped_nf4_gemm_quantize_amd", "csrc", "gemm.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def gpu_stacks(cfg, dev, seed=0, group=16):
    """Quantise the layer's fp32 weights on the GPU, a few experts at a time."""
    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    out = {}
    for which, (n, kk) in (("gu", (2 * cfg.I, cfg.H)), ("dn", (cfg.H, cfg.I))):
        p = torch.empty((cfg.E, n, kk // 2), dtype=torch.uint8, device=dev)
        a = torch.empty((cfg.E, n, kk // 64), dtype=torch.float32, device=dev)
        for e0 in range(0, cfg.E, group):
            ex = range(e0, min(e0 + group, cfg.E))
            w = torch.from_numpy(synth.stack_weights(cfg, which, seed, ex)).to(dev)
            pp, aa = binding.quantize(w)
            p[e0:e0 + len(ex)] = pp
            a[e0:e0 + len(ex)] = aa
            del w
        out[which] = (p, a)
    return out


def time_events(fn, iters: int, stream) -> float:
    """Average milliseconds per call of fn(), HIP events on `stream`."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def traffic_from_profiles(kernel_src: str):
    """HBM bytes per launch of the gate_up GEMM from the committed counter
    summary (the JSON block of profiles/gate_up_gemm_olmoe_counters.md).

    Returns None when no counter summary exists or when the kernel source
    changed since the counters were taken.
    """
    if not os.path.exists(COUNTERS_MD):
        return None
    text = open(COUNTERS_MD).read()
    if "```json" not in text:
        return None
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _csv_rows(directory: str, suffix: str):
    paths = glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)
    if not paths:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def summarize_trace(directory: str) -> int:
    """Markdown table of a rocprofv3 --kernel-trace --stats run."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    print("| kernel | calls | avg us | min us | max us | total % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows[:16]:
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.2f} |")
    return 0


def _counter_means(directory: str, counter: str):
    """Mean counter value per dispatch for the gate_up GEMM and the copy."""
    gemm, copy = [], []
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if "grouped_gemm_kernel<true, 0, false, 2, 0, false>" in name:  # the NF4 gate_up
            gemm.append(v)
        elif "copyBuffer" in name:
            copy.append(v)
    if not gemm or not copy:
        raise SystemExit(f"{counter}: gate_up GEMM or copy dispatches missing in {directory}")
    # the calibration copies are the largest copy dispatches
    copy.sort()
    return sum(gemm) / len(gemm), copy[-1], len(gemm)


def summarize_counters(fetch_dir: str, write_dir: str) -> int:
    """Markdown + JSON summary of the FETCH_SIZE and WRITE_SIZE runs."""
    f_gemm, f_copy, n_f = _counter_means(fetch_dir, "FETCH_SIZE")
    w_gemm, w_copy, n_w = _counter_means(write_dir, "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    f_scale, w_scale = kib / f_copy, kib / w_copy
    fetch_b = f_gemm * f_scale * 1024.0
    write_b = w_gemm * w_scale * 1024.0
    rec = {
        "kernel": "grouped_gemm_kernel<true,0,false,2,0,false> (gate_up + SwiGLU, olmoe prefill)",
        "kernel_source_sha256": hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest(),
        "fetch_kib_per_launch_raw": round(f_gemm, 1),
        "write_kib_per_launch_raw": round(w_gemm, 1),
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib_raw": round(f_copy, 1),
        "copy_write_kib_raw": round(w_copy, 1),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "hbm_fetch_bytes_per_launch": round(fetch_b),
        "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "gemm_dispatches": [n_f, n_w],
    }
    print("| quantity | FETCH_SIZE | WRITE_SIZE |")
    print("|---|---:|---:|")
    print(f"| gate_up GEMM, KiB per launch (raw) | {f_gemm:.0f} | {w_gemm:.0f} |")
    print(f"| 512 MiB copy, KiB (raw) | {f_copy:.0f} | {w_copy:.0f} |")
    print(f"| scale = 524288 KiB / copy reading | {f_scale:.4f} | {w_scale:.4f} |")
    print(f"| gate_up GEMM, HBM MB per launch (scaled) | {fetch_b / 1e6:.1f} | {write_b / 1e6:.1f} |")
    print()
    print("```json")
    print(json.dumps(rec, indent=1))
    print("```")
    return 0


def copy_calibration(dev) -> None:
    """Three copies of a 512 MiB buffer: the plain copy of known size."""
    import torch

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def cpu_baseline(cfg, seconds_target: float = 10.0):
    """Time the CPU oracle on the layer shape (random NF4 stacks; values do
    not change its cost).  Runs whole forwards until about `seconds_target`."""
    import numpy as np

    import oracle
    from grouped_nf4_gemm_quantize_amd import synth

    rng = np.random.default_rng(1)
    E, H, I = cfg.E, cfg.H, cfg.I
    gp = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    ga = rng.uniform(0.01, 0.05, size=(E, 2 * I, H // 64)).astype(np.float32)
    dp = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    da = rng.uniform(0.01, 0.05, size=(E, H, I // 64)).astype(np.float32)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    from threadpoolctl import threadpool_info, threadpool_limits

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    runs, elapsed = 0, 0.0
    while elapsed < seconds_target and runs < 5:
        t0 = time.perf_counter()
        oracle.moe_forward(x, lg, cfg.k, gp, ga, dp, da)
        elapsed += time.perf_counter() - t0
        runs += 1
    per = elapsed / runs
    # the same forward once more on one thread (BLAS limited to 1)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.moe_forward(x, lg, cfg.k, gp, ga, dp, da)
        per1 = time.perf_counter() - t0
    return {
        "value": round(cfg.flops() / per / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{runs} full {cfg.name} layer forward(s) (T={cfg.T}, E={E}, H={H}, "
                   f"I={I}, top-{cfg.k}) of the NumPy fp64 oracle, random NF4 stacks, "
                   f"{per:.2f} s each; cores = the BLAS threads (NumPy's own loops, "
                   f"the dequantisation included, run on one)"),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "blas_threads": int(threads),
        "one_thread": {"value": round(cfg.flops() / per1 / 1e12, 6), "unit": "TFLOP/s",
                       "seconds_per_forward": round(per1, 3)},
    }


def bench_decode(dev, steps: int, mx: bool = False):
    """48 distinct decode layers (8 routed experts each) replayed from a graph
    (NF4 stacks, or released-format MXFP4 stacks with ``mx``)."""
    import numpy as np
    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    cfg = synth.config("decode")
    if mx:
        gp, ga = (torch.from_numpy(t).to(dev) for t in synth.mxfp4_stack(cfg, "gu"))
        dp, da = (torch.from_numpy(t).to(dev) for t in synth.mxfp4_stack(cfg, "dn"))
        st = None
    else:
        st = gpu_stacks(cfg, dev)
        gp, ga = st["gu"]
        dp, da = st["dn"]
    layers = []
    for l in range(DECODE_LAYERS):
        lg = np.random.default_rng(1000 + l).standard_normal((1, cfg.E), dtype=np.float32)
        layers.append(dict(
            gp=gp.clone(), ga=ga.clone(), dp=dp.clone(), da=da.clone(),
            lg=torch.from_numpy(lg).to(dev),
            y=torch.empty((1, cfg.H), dtype=torch.bfloat16, device=dev),
            ws=torch.empty(binding.forward_workspace_bytes(1, cfg.H, cfg.I, cfg.E, cfg.k),
                           dtype=torch.uint8, device=dev)))
    del gp, ga, dp, da, st
    x = torch.from_numpy(synth.activations(cfg)).to(dev).to(torch.bfloat16)

    def run_all():
        for L in layers:
            if mx:
                binding.moe_forward_mxfp4(x, L["lg"], cfg.k, L["gp"], L["ga"], L["dp"], L["da"],
                                          y=L["y"], workspace=L["ws"])
            else:
                binding.moe_forward(x, L["lg"], cfg.k, L["gp"], L["ga"], L["dp"], L["da"],
                                    y=L["y"], workspace=L["ws"])

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            run_all()
        eager_ms = time_events(run_all, max(steps, 3), stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run_all()
    with torch.cuda.stream(stream):
        for _ in range(3):
            g.replay()
        graph_ms = time_events(g.replay, max(steps, 10), stream)
    # packed bytes + scales of the k routed experts: 4 bits + 4 bytes per 64
    # (NF4), 4 bits + 1 byte per 32 (MXFP4)
    per_elem_16ths = 9 if not mx else 10
    per_layer_bytes = cfg.k * (2 * cfg.I * cfg.H + cfg.H * cfg.I) * per_elem_16ths // 16
    gbs = DECODE_LAYERS * per_layer_bytes / (graph_ms * 1e-3) / 1e9
    del g
    torch.cuda.empty_cache()
    # context: a plain one-shot read of the same byte count from HBM, 48
    # distinct buffers read back to back on one stream (torch's sum reduction
    # as the reader, launched eagerly: its launches queue ahead of the GPU as
    # the decode layers' do), the ceiling of a single dependent-free pass at
    # this size
    stream = None
    if not mx:
        cols = 1024
        rows = per_layer_bytes // 4 // cols
        bufs = [torch.ones((rows, cols), dtype=torch.float32, device=dev)
                for _ in range(DECODE_LAYERS)]
        outs = torch.empty((DECODE_LAYERS, rows), dtype=torch.float32, device=dev)
        s2 = torch.cuda.Stream(device=dev)

        def read_all():
            for i, b in enumerate(bufs):
                torch.sum(b, dim=1, out=outs[i])  # one pass: a sum per 4 KB row

        with torch.cuda.stream(s2):
            for _ in range(3):
                read_all()
            read_ms = time_events(read_all, max(steps, 10), s2)
        torch.cuda.synchronize()
        nbytes = rows * cols * 4
        stream = {"what": f"one-shot read of {nbytes} B from HBM (torch row sums over "
                          f"{DECODE_LAYERS} distinct buffers, back to back)",
                  "us_per_read": round(read_ms * 1e3 / DECODE_LAYERS, 3),
                  "gbs": round(DECODE_LAYERS * nbytes / (read_ms * 1e-3) / 1e9, 2)}
        del bufs, outs
    out = {
        "metric": "packed-weight GB/s (decode M=1)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "workload": (f"Qwen3-30B-A3B-shaped decode layer x{DECODE_LAYERS} distinct "
                     f"{'MXFP4' if mx else 'NF4'} stacks (E={cfg.E}, H={cfg.H}, I={cfg.I}, "
                     f"top-{cfg.k}, T=1), HIP graph replay"),
        "bytes_per_layer": per_layer_bytes,
        "us_per_layer": round(graph_ms * 1e3 / DECODE_LAYERS, 3),
        "us_per_layer_eager": round(eager_ms * 1e3 / DECODE_LAYERS, 3),
        "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
    }
    if stream is not None:
        out["stream_read_ceiling"] = stream
    del layers
    torch.cuda.empty_cache()
    return out


def bench_backward(name: str, dev, steps: int):
    """The QLoRA training backward of one layer (route, down dgrad, gate_up
    recomputed with the SwiGLU backward as its epilogue, gate_up dgrad,
    combine, adapter gradients) and its three grouped kernels timed alone on
    the same routing."""
    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    cfg = synth.config(name)
    st = gpu_stacks(cfg, dev)
    gp, ga = st["gu"]
    dp, da = st["dn"]
    x = torch.from_numpy(synth.activations(cfg)).to(dev).to(torch.bfloat16)
    lg = torch.from_numpy(synth.router_logits(cfg)).to(dev)
    dy = torch.from_numpy(synth.output_grad(cfg)).to(dev).to(torch.bfloat16)
    glo = dlo = None
    lw = synth.lora_weights(cfg)
    if lw is not None:
        t = {k_: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k_, v in lw.items()}
        glo = (t["a_gu"], t["b_gu"], cfg.lora_scale)
        dlo = (t["a_dn"], t["b_dn"], cfg.lora_scale)
    r = cfg.lora_r
    dx = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.backward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, r),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.moe_backward(x, lg, dy, cfg.k, gp, ga, dp, da, glo, dlo, cfg.renormalize,
                             dx=dx, workspace=ws)

    for _ in range(3):
        step()
    bwd_ms = time_events(step, max(steps, 5), stream)

    # the backward's three grouped kernels alone (without adapters), on this
    # layer's routing: the down dgrad (dh), the gate_up GEMM recomputed with
    # the SwiGLU backward as its epilogue (dG), the gate_up dgrad (dX)
    fws = torch.empty(binding.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, r),
                      dtype=torch.uint8, device=dev)
    binding.moe_forward(x, lg, cfg.k, gp, ga, dp, da, glo, dlo, cfg.renormalize,
                        workspace=fws)
    ptr = binding.forward_routing(fws, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    base = fws.data_ptr()
    P = cfg.P
    sp = fws[ptr["sorted_pair"] - base: ptr["sorted_pair"] - base + 4 * P].view(torch.int32)
    off = fws[ptr["offsets"] - base: ptr["offsets"] - base + 4 * (cfg.E + 1)].view(torch.int32)
    x16 = x.to(torch.float16)
    dH = torch.empty((P, cfg.I), dtype=torch.float16, device=dev)
    dG = torch.empty((P, 2 * cfg.I), dtype=torch.float16, device=dev)
    dXp = torch.empty((P, cfg.H), dtype=torch.float16, device=dev)

    dy16 = dy.to(torch.float16)  # the layer backward converts dy once, as here

    def down_dgrad():
        binding.grouped_dgrad(dy16, dp, da, off, P, gather=sp, gather_div=cfg.k, out=dH)

    def recompute():
        binding.grouped_gemm_swiglu_bwd(x16, gp, ga, off, P, dH, gather=sp, gather_div=cfg.k,
                                        out=dG)

    def gate_up_dgrad():
        binding.grouped_dgrad(dG, gp, ga, off, P, scatter=sp, out=dXp)

    for _ in range(2):
        down_dgrad()
        recompute()
        gate_up_dgrad()
    dn_ms = time_events(down_dgrad, max(steps, 10), stream)
    rc_ms = time_events(recompute, max(steps, 10), stream)
    gu_ms = time_events(gate_up_dgrad, max(steps, 10), stream)
    phi = float(P) * cfg.H * cfg.I
    grad_flops = 6.0 * phi           # the two dgrads
    exec_flops = 10.0 * phi          # + the recomputed gate_up forward
    if r:
        # adapter work: gate_up (in H, out 2I) recomputed u and delta, u again,
        # v, the input-gradient term, dA, dB: 4 rank-r products over H and 3
        # over 2I; down (in I, out H): u, v, the input-gradient term, dA, dB:
        # 3 over I and 2 over H
        exec_flops += 2.0 * P * r * (6 * cfg.H + 9 * cfg.I)
    out = {
        "workload": (f"{cfg.name} layer backward: E={cfg.E} H={cfg.H} I={cfg.I} top-{cfg.k} "
                     f"T={cfg.T}" + (f" LoRA r={r} on gate_up and down" if r else "")
                     + ", routing and gate_up recomputed"),
        "us_per_backward": round(bwd_ms * 1e3, 2),
        "tflops_gradient": round(grad_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "tflops_executed": round(exec_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "down_dgrad_us": round(dn_ms * 1e3, 2),
        "down_dgrad_tflops": round(2.0 * phi / (dn_ms * 1e-3) / 1e12, 2),
        "recompute_swiglu_bwd_us": round(rc_ms * 1e3, 2),
        "recompute_swiglu_bwd_tflops": round(4.0 * phi / (rc_ms * 1e-3) / 1e12, 2),
        "gate_up_dgrad_us": round(gu_ms * 1e3, 2),
        "gate_up_dgrad_tflops": round(4.0 * phi / (gu_ms * 1e-3) / 1e12, 2),
        "gate_up_dgrad_frac_peak": round(4.0 * phi / (gu_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
    }
    del st, gp, ga, dp, da, dH, dG, dXp, ws, fws
    torch.cuda.empty_cache()
    return out


def bench_mxfp4(dev, steps: int):
    """The olmoe-shaped prefill layer on synthetic released-MXFP4 stacks
    (e2m1 + e8m0 bytes multiplied in place) and its gate_up GEMM alone."""
    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    cfg = synth.config("olmoe")
    gb, gs = (torch.from_numpy(t).to(dev) for t in synth.mxfp4_stack(cfg, "gu"))
    db, ds = (torch.from_numpy(t).to(dev) for t in synth.mxfp4_stack(cfg, "dn"))
    x = torch.from_numpy(synth.activations(cfg)).to(dev).to(torch.bfloat16)
    lg = torch.from_numpy(synth.router_logits(cfg)).to(dev)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.moe_forward_mxfp4(x, lg, cfg.k, gb, gs, db, ds, y=y, workspace=ws)

    for _ in range(3):
        step()
    ms = time_events(step, max(steps, 5), stream)
    ptr = binding.forward_routing(ws, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    base = ws.data_ptr()
    P = cfg.P
    sp = ws[ptr["sorted_pair"] - base: ptr["sorted_pair"] - base + 4 * P].view(torch.int32)
    off = ws[ptr["offsets"] - base: ptr["offsets"] - base + 4 * (cfg.E + 1)].view(torch.int32)
    x16 = x.to(torch.float16)
    h = torch.empty((P, cfg.I), dtype=torch.float16, device=dev)

    def gate_up():
        binding.grouped_gemm_mxfp4(x16, gb, gs, off, P, gather=sp, gather_div=cfg.k,
                                   swiglu=True, out=h)

    for _ in range(2):
        gate_up()
    gu_ms = time_events(gate_up, max(steps, 10), stream)
    out = {
        "workload": (f"olmoe layer prefill on MXFP4 stacks (e2m1 + e8m0 per 32): E={cfg.E} "
                     f"H={cfg.H} I={cfg.I} top-{cfg.k} T={cfg.T}"),
        "us_per_forward": round(ms * 1e3, 2),
        "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
        "gate_up_us": round(gu_ms * 1e3, 2),
        "gate_up_tflops": round(4.0 * P * cfg.H * cfg.I / (gu_ms * 1e-3) / 1e12, 2),
    }
    del gb, gs, db, ds, ws, h
    torch.cuda.empty_cache()
    out["decode"] = bench_decode(dev, steps, mx=True)
    return out


def bench_storage_modes(dev, steps: int):
    """The olmoe-shaped prefill layer with its stacks stored in each of the
    other modes (quantised on the GPU from the same fp32 weights)."""
    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    cfg = synth.config("olmoe")
    x = torch.from_numpy(synth.activations(cfg)).to(dev).to(torch.bfloat16)
    lg = torch.from_numpy(synth.router_logits(cfg)).to(dev)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for qt in ("fp4", "int8", "fp8", "bf16", "fp16"):
        st = {}
        for which, (n, kk) in (("gu", (2 * cfg.I, cfg.H)), ("dn", (cfg.H, cfg.I))):
            if qt in binding.PASSTHROUGH:  # the weights themselves, no absmax
                p = torch.empty((cfg.E, n, kk), device=dev,
                                dtype=torch.bfloat16 if qt == "bf16" else torch.float16)
                a = None
            else:
                per = 1 if qt in binding.EIGHT_BIT else 2
                p = torch.empty((cfg.E, n, kk // per), dtype=torch.uint8, device=dev)
                a = torch.empty((cfg.E, n, kk // 64), dtype=torch.float32, device=dev)
            for e0 in range(0, cfg.E, 16):
                ex = range(e0, min(e0 + 16, cfg.E))
                w = torch.from_numpy(synth.stack_weights(cfg, which, 0, ex)).to(dev)
                pp, aa = binding.quantize(w, quant_type=qt)
                p[e0:e0 + len(ex)] = pp
                if a is not None:
                    a[e0:e0 + len(ex)] = aa
                del w
            st[which] = (p, a)
        gp, ga = st["gu"]
        dp, da = st["dn"]

        def step():
            binding.moe_forward(x, lg, cfg.k, gp, ga, dp, da, y=y, workspace=ws,
                                quant_type=qt)

        for _ in range(3):
            step()
        ms = time_events(step, max(steps, 5), stream)
        out[qt] = {"us_per_forward": round(ms * 1e3, 2),
                   "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
                   "stack_bytes": int(sum(t.numel() * t.element_size()
                                          for t in (gp, ga, dp, da) if t is not None))}
        del st, gp, ga, dp, da
        torch.cuda.empty_cache()
    return out


def control_lane(cfg, st, x16, off, sp, stream, iters: int):
    """Dequantise-then-GEMM control (a benchmark control, never a product
    path): the whole stack is dequantised to fp16 with plain torch ops, then
    the experts run as padded batched library GEMMs (hipBLASLt through
    torch.bmm) with torch SwiGLU between them.  It measures the round trip
    the in-register decode removes (grouped-nf4-gemm solutions entry "How do
    I run a grouped GEMM directly on NF4 packed MoE expert weights"; README
    "The package family").  The dequantisation is an upper bound (several
    generic kernels); the GEMM part alone is a lower bound for any
    dequantise-first path."""
    import torch

    from grouped_nf4_gemm_quantize_amd import binding

    dev = x16.device
    levels = torch.tensor(binding.codebook(), dtype=torch.float32, device=dev)
    E = cfg.E
    offs = off.cpu().tolist()
    counts = [offs[e + 1] - offs[e] for e in range(E)]
    mmax = max(max(counts), 1)

    def dequant_t(p, a):
        # [E, N, K/2] codes + [E, N, K/64] absmax -> W^T [E, K, N] fp16
        n = p.shape[1]
        kk = p.shape[2] * 2
        codes = torch.stack(((p >> 4), (p & 15)), dim=-1).reshape(E, n, kk).long()
        w = levels[codes] * a.repeat_interleave(64, dim=-1)
        return w.to(torch.float16).transpose(1, 2).contiguous()

    (gp, ga), (dp, da) = st["gu"], st["dn"]
    out = {}

    def deq():
        out["wgu"] = dequant_t(gp, ga)
        out["wdn"] = dequant_t(dp, da)

    deq()
    deq_ms = time_events(deq, 2, stream)
    # activations gathered per expert into a padded [E, mmax, H] block
    xp = torch.zeros((E, mmax, cfg.H), dtype=torch.float16, device=dev)
    rows = (sp // cfg.k).long()
    for e in range(E):
        if counts[e]:
            xp[e, :counts[e]] = x16[rows[offs[e]:offs[e + 1]]]
    I = cfg.I

    def gemms():
        g = torch.bmm(xp, out["wgu"])
        hh = torch.nn.functional.silu(g[..., :I]) * g[..., I:]
        out["o"] = torch.bmm(hh, out["wdn"])
        out["h"] = hh

    gemms()
    gemm_ms = time_events(gemms, iters, stream)
    # HBM floor of any dequantisation: read codes + absmax, write fp16 W^T
    deq_bytes = sum(t.numel() * t.element_size() for t in (gp, ga, dp, da)) + \
        2 * (out["wgu"].numel() + out["wdn"].numel())
    floor_us = deq_bytes / (PEAK_HBM_GBS * 1e9) * 1e6
    # one dense fp16 library GEMM with the gate_up projection's flops (the
    # routed rows times one expert's dequantised weights): what the matrix
    # cores reach on this machine for a plain GEMM with real operands
    xa = x16[rows]
    wd = out["wgu"][0]

    def dense():
        out["dense"] = torch.matmul(xa, wd)

    dense()
    dense_ms = time_events(dense, iters, stream)
    dense_flops = 2.0 * xa.shape[0] * xa.shape[1] * wd.shape[1]
    res = {"dequant_us": round(deq_ms * 1e3, 1), "dequant_hbm_floor_us": round(floor_us, 1),
           "dequant_bytes": deq_bytes, "gemm_swiglu_us": round(gemm_ms * 1e3, 1),
           "total_us": round((deq_ms + gemm_ms) * 1e3, 1),
           "total_at_dequant_floor_us": round(floor_us + gemm_ms * 1e3, 1),
           "padded_rows_per_expert": mmax,
           "dense_fp16_gemm_same_flops": {
               "shape": f"[{xa.shape[0]}x{xa.shape[1]}] x [{wd.shape[0]}x{wd.shape[1]}]",
               "us": round(dense_ms * 1e3, 1),
               "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1)}}
    del out["dense"], xa
    del out["wgu"], out["wdn"], xp
    return res, out


def measure_prefill(cfg, dev, steps: int, warmup: int, keep: bool = False):
    """One prefill workload: the whole layer forward timed over `steps`
    forwards after `warmup` untimed ones (HIP events on the current stream,
    device syncs around the timed region), then its gate_up and down grouped
    GEMMs timed alone on the same routing."""
    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    st = gpu_stacks(cfg, dev)
    gp, ga = st["gu"]
    dp, da = st["dn"]
    x = torch.from_numpy(synth.activations(cfg)).to(dev).to(torch.bfloat16)
    lg = torch.from_numpy(synth.router_logits(cfg)).to(dev)
    glo = dlo = None
    lw = synth.lora_weights(cfg)
    if lw is not None:
        t = {k_: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k_, v in lw.items()}
        glo = (t["a_gu"], t["b_gu"], cfg.lora_scale)
        dlo = (t["a_dn"], t["b_dn"], cfg.lora_scale)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k,
                                                     cfg.lora_r),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.moe_forward(x, lg, cfg.k, gp, ga, dp, da, glo, dlo, cfg.renormalize,
                            y=y, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` forwards, bracketed by device syncs
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    tflops = cfg.flops() / (ms * 1e-3) / 1e12
    log(f"[bench] {cfg.name} layer forward {ms * 1e3:.1f} us  {tflops:.1f} TFLOP/s")

    # the two grouped GEMMs alone, on this forward's routing
    ptr = binding.forward_routing(ws, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    base = ws.data_ptr()
    P = cfg.P
    sp = ws[ptr["sorted_pair"] - base: ptr["sorted_pair"] - base + 4 * P].view(torch.int32)
    off = ws[ptr["offsets"] - base: ptr["offsets"] - base + 4 * (cfg.E + 1)].view(torch.int32)
    x16 = x.to(torch.float16)
    h = torch.empty((P, cfg.I), dtype=torch.float16, device=dev)
    o = torch.empty((P, cfg.H), dtype=torch.float16, device=dev)

    def gate_up():
        binding.grouped_gemm(x16, gp, ga, off, P, gather=sp, gather_div=cfg.k, lora=glo,
                             swiglu=True, out=h)

    def down():
        binding.grouped_gemm(h, dp, da, off, P, lora=dlo, scatter=sp, out=o)

    for _ in range(2):
        gate_up()
        down()
    gu_ms = time_events(gate_up, max(steps, 10), stream)
    dn_ms = time_events(down, max(steps, 10), stream)
    gu_flops = 4.0 * P * cfg.H * cfg.I
    dn_flops = 2.0 * P * cfg.H * cfg.I
    if glo is not None:
        gu_flops += 2.0 * P * cfg.lora_r * (cfg.H + 2 * cfg.I)
        dn_flops += 2.0 * P * cfg.lora_r * (cfg.I + cfg.H)
    gu_tf = gu_flops / (gu_ms * 1e-3) / 1e12
    dn_tf = dn_flops / (dn_ms * 1e-3) / 1e12
    log(f"[bench] {cfg.name} gate_up GEMM {gu_ms * 1e3:.1f} us {gu_tf:.1f} TFLOP/s; "
        f"down GEMM {dn_ms * 1e3:.1f} us {dn_tf:.1f} TFLOP/s")
    out = {
        "workload": (f"{cfg.name} layer prefill: E={cfg.E} H={cfg.H} I={cfg.I} top-{cfg.k} "
                     f"T={cfg.T}" + (f" LoRA r={cfg.lora_r}" if cfg.lora_r else "")
                     + (" (Zipf routing)" if cfg.logits == "zipf" else "")),
        "us_per_forward": round(ms * 1e3, 3),
        "tflops": round(tflops, 3),
        "frac_peak": round(tflops / PEAK_F16_TFLOPS, 4),
        "flops_per_forward": cfg.flops(),
        "gate_up_us": round(gu_ms * 1e3, 3), "gate_up_tflops": round(gu_tf, 3),
        "gate_up_frac_peak": round(gu_tf / PEAK_F16_TFLOPS, 4),
        "down_us": round(dn_ms * 1e3, 3), "down_tflops": round(dn_tf, 3),
        "gate_up_flops": gu_flops,
    }
    del o, y, ws, gp, ga, dp, da
    if keep:
        out["_keep"] = (st, x16, off, sp, h)
    else:
        del st, x16, off, sp, h
    return out


def summarize_pmc(directory: str, kernel_substr: str) -> int:
    """Markdown table of a rocprofv3 --pmc run: the mean of every counter per
    dispatch of the kernels whose name contains `kernel_substr`."""
    per = {}
    names = set()
    for r in _csv_rows(directory, "counter_collection.csv"):
        if kernel_substr not in r["Kernel_Name"]:
            continue
        names.add(r["Kernel_Name"])
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel containing {kernel_substr!r} in {directory}")
    sums, counts = {}, {}
    for (_, c), v in per.items():
        sums[c] = sums.get(c, 0.0) + v
        counts[c] = counts.get(c, 0) + 1
    print(f"kernel(s): {', '.join(sorted('`' + n + '`' for n in names))}")
    print()
    print("| counter | dispatches | mean per dispatch |")
    print("|---|---:|---:|")
    for c in sorted(sums):
        print(f"| {c} | {counts[c]} | {sums[c] / counts[c]:.6g} |")
    return 0


def summarize_decode_fetch(fetch_dir: str) -> int:
    """HBM bytes read per decode-layer launch (FETCH_SIZE, scaled by what the
    counter reads for the 512 MiB calibration copy) against its algorithmic
    packed-weight bytes."""
    dec, copy = [], []
    for r in _csv_rows(fetch_dir, "counter_collection.csv"):
        if r["Counter_Name"] != "FETCH_SIZE":
            continue
        if "decode_layer_kernel" in r["Kernel_Name"]:
            dec.append(float(r["Counter_Value"]))
        elif "copyBuffer" in r["Kernel_Name"]:
            copy.append(float(r["Counter_Value"]))
    if not dec or not copy:
        raise SystemExit(f"decode or copy dispatches missing in {fetch_dir}")
    copy.sort()
    scale = COPY_BYTES / 1024.0 / copy[-1]
    mean = sum(dec) / len(dec)
    algo = 21233664
    fetch_b = mean * scale * 1024.0
    print("| quantity | value |")
    print("|---|---:|")
    print(f"| decode layer launches | {len(dec)} |")
    print(f"| FETCH_SIZE per launch, KiB (raw) | {mean:.0f} |")
    print(f"| 512 MiB copy, KiB (raw) | {copy[-1]:.0f} |")
    print(f"| scale = 524288 KiB / copy reading | {scale:.4f} |")
    print(f"| HBM bytes fetched per launch (scaled) | {fetch_b:.0f} |")
    print(f"| algorithmic packed bytes per layer | {algo} |")
    print(f"| fetched / algorithmic | {fetch_b / algo:.3f} |")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: about 30 ms of untimed warmup (the clock ramps up under load
    # over the first tens of milliseconds) and 55 ms of timed forwards
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="olmoe",
                    choices=["olmoe", "qwen3_zipf", "qlora"])
    ap.add_argument("--prefill-workloads", default="qwen3_zipf,qlora",
                    help="comma-separated further prefill workloads timed the same way")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-control", action="store_true",
                    help="skip the dequantise-then-GEMM control lane")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training-backward section")
    ap.add_argument("--backward-workloads", default="olmoe,qlora",
                    help="comma-separated workloads of the backward section")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the MXFP4 and storage-mode sections")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("DIR", "KERNEL_SUBSTR"))
    ap.add_argument("--summarize-decode-fetch", metavar="FETCH_DIR")
    args = ap.parse_args()
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc)
    if args.summarize_decode_fetch:
        return summarize_decode_fetch(args.summarize_decode_fetch)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the expert path here runs on a single GPU "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    from grouped_nf4_gemm_quantize_amd import binding, synth

    binding.load()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
    cfg = synth.config(args.workload)
    log(f"[bench] workload {cfg}")
    pf = measure_prefill(cfg, dev, args.steps, args.warmup, keep=True)
    ms, tflops = pf["us_per_forward"] / 1e3, pf["tflops"]
    gu_ms, dn_ms = pf["gate_up_us"] / 1e3, pf["down_us"] / 1e3
    gu_tf, dn_tf = pf["gate_up_tflops"], pf["down_tflops"]
    gu_flops = pf["gate_up_flops"]
    flops = cfg.flops()
    st, x16, off, sp, h = pf.pop("_keep")
    stream = torch.cuda.current_stream(dev)
    glo = None if not cfg.lora_r else True
    # the counter summary covers the olmoe gate_up kernel only
    traffic = traffic_from_profiles(GEMM_SRC) if cfg.name == "olmoe" else None
    control = None
    if glo is None and not args.no_control:
        control, cout = control_lane(cfg, st, x16, off, sp, stream, max(args.steps, 10))
        control["fused_gemms_us"] = round((gu_ms + dn_ms) * 1e3, 1)
        control["speedup_vs_control_total"] = round(control["total_us"] / control["fused_gemms_us"], 3)
        control["speedup_vs_control_gemm_only"] = round(control["gemm_swiglu_us"] / control["fused_gemms_us"], 3)
        control["speedup_vs_control_at_dequant_floor"] = round(
            control["total_at_dequant_floor_us"] / control["fused_gemms_us"], 3)
        # the control computes the same thing: expert 0's h rows against ours
        offs0 = off[:2].cpu().tolist()
        n0 = offs0[1] - offs0[0]
        if n0:
            ref = cout["h"][0, :n0].float()
            got = h[offs0[0]:offs0[1]].float()
            control["h_rel_fro_vs_fused"] = float(((got - ref).norm() / ref.norm()).item())
        del cout
        log(f"[bench] dequantise-then-GEMM control {control}")
    del h, x16

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name} layer prefill: E={cfg.E} H={cfg.H} I={cfg.I} "
                         f"top-{cfg.k} T={cfg.T}" + (f" LoRA r={cfg.lora_r}" if cfg.lora_r else "")),
            "E": cfg.E, "H": cfg.H, "I": cfg.I, "k": cfg.k, "T": cfg.T,
            "routing": cfg.logits, "lora_r": cfg.lora_r,
            "flops_per_step": flops,
        },
        "roofline": {
            "kernel": "grouped_gemm_kernel (gate_up + SwiGLU)",
            "bound": "mfma",
            "achieved": round(gu_tf, 3),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gu_tf / PEAK_F16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "flops_per_launch": gu_flops,
        },
        "kernels": {
            "gate_up_us": round(gu_ms * 1e3, 3), "gate_up_tflops": round(gu_tf, 3),
            "down_us": round(dn_ms * 1e3, 3), "down_tflops": round(dn_tf, 3),
        },
    }
    if control is not None:
        result["control_dequant_then_gemm"] = control
    del st, off, sp
    torch.cuda.empty_cache()
    others = [n_ for n_ in args.prefill_workloads.split(",") if n_ and n_ != cfg.name]
    if others:
        result["prefill_workloads"] = {}
        for n_ in others:
            r_ = measure_prefill(synth.config(n_), dev, args.steps, args.warmup)
            r_.pop("gate_up_flops")
            result["prefill_workloads"][n_] = r_
            log(f"[bench] prefill {n_} {r_}")
            torch.cuda.empty_cache()
    if not args.no_decode:
        result["decode"] = bench_decode(dev, args.steps)
        log(f"[bench] decode {result['decode']}")
    if not args.no_mxfp4:
        result["mxfp4"] = bench_mxfp4(dev, args.steps)
        log(f"[bench] mxfp4 {result['mxfp4']}")
        result["storage_modes"] = bench_storage_modes(dev, args.steps)
        log(f"[bench] storage modes {result['storage_modes']}")
    bwd_names = [n_ for n_ in args.backward_workloads.split(",") if n_]
    if not args.no_backward and bwd_names:
        result["backward"] = {n_: bench_backward(n_, dev, args.steps) for n_ in bwd_names}
        log(f"[bench] backward {result['backward']}")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg)
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
