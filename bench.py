#!/usr/bin/env python3
"""Benchmark of the bidirectional Mamba-2 SSD mixer on one MI355X.

A step is one bidirectional bimamba_ssd_fwd call (every kernel of the scan:
segment states, state passing, outputs) over one batch of synthetic input
already resident in HBM. The headline workload is the long-sequence prefill
at 131 072 tokens (batch 1, 64 heads x headdim 64 = d_inner 4096 of a
1.3B-shaped model, d_state 128, chunk 256, bf16 inputs, fp32 accumulation and
output), the largest single-GPU configuration and the one the >= 60 % HBM
roofline target is set on.

Prints ONE JSON line. Besides the contract fields it carries:
  settle        the untimed fixed-duration phase that brings the clocks to
                their steady state before the warm-up and the timed steps
  roofline      HBM roofline of the dominant kernel (algorithmic bytes per
                launch / its average HIP-event duration over the timed steps);
                `traffic` is the measured HBM bytes per launch from the
                committed counter summary of that kernel and workload when it
                was taken on the kernel source as it stands, else null
  mfma          the same launches against the dense fp16/bf16 matrix-core
                peak, counting the algorithmic flops of the chunked form
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded
                sample of the same inputs (a subset of the heads, every
                token), with its parity against the GPU
  extra         the training-length layer, the 32k prefill, the latency fit
                time(L) = a + bL + cL^2, slowly decaying heads, the packed
                batch, the cached block step and the follow-on kernels
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3   # dense fp32 matrix (and vector) peak
METRIC = "BiMamba-2 SSD tokens/s + % HBM/MFMA roofline; block-cached step ms"
KERNEL_SOURCE = os.path.join(ROOT, "bidirectional_mamba_ssm_amd", "csrc", "ssd_chunked.hip")
TILE = 64   # block length of the matrix-core kernel's decomposition (every chunk size)


def summary_path(kernel, workload, kind):
    """Committed rocprofv3 summary of one kernel on one workload."""
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_{kind}.md")


def bytes_per_token(H, P, N, G, elem):
    """Algorithmic bytes per token: every input of both directions read once
    (x, dt, B, C), y (fp32) written once."""
    per_dir = H * P * elem + H * elem + 2 * G * N * elem
    return 2 * per_dir + H * P * 4


def flops_per_token(H, P, N, G, Q):
    """Algorithmic flops per token of the chunked SSD form, both directions:
    per chunk of Q tokens the Gram matrix C B^T over its causal half (once per
    group), the masked product with x, the chunk's state contribution and the
    carried-state output (per head)."""
    per_dir = G * (Q + 1) * N + H * ((Q + 1) * P + 4 * N * P)
    return 2 * per_dir


def summary_field(path, key):
    """An integer field of a committed counter summary, if the summary was
    taken on the kernel source as it stands (else None)."""
    import hashlib
    try:
        text = open(path).read()
        src_hash = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return int(fields[key])
    except (KeyError, ValueError):
        return None


def measured_traffic(kernel, workload):
    """HBM bytes per launch of a kernel (FETCH_SIZE + WRITE_SIZE), from its
    committed counter summary, or None."""
    return summary_field(summary_path(kernel, workload, "hbm_traffic"), "traffic_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU takes some tens of milliseconds of work to reach its steady
    # clock; the default warm-up covers that
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed seconds of steps before the warm-up (steady clocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--prefix", type=int, default=262144,
                    help="prefix length of the block-step state")
    ap.add_argument("--block-step-only", action="store_true",
                    help="only the block-decode step lines (one JSON object)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="only the training-backward line (one JSON object)")
    ap.add_argument("--epilogue-only", action="store_true",
                    help="only the gated-norm epilogue line (one JSON object)")
    ap.add_argument("--merge-only", action="store_true",
                    help="only the concatenating-merge lines (one JSON object)")
    ap.add_argument("--conv-only", action="store_true",
                    help="only the short-convolution line (one JSON object)")
    ap.add_argument("--workload", default="long_128k",
                    help="workload of the main line (a name in synth.WORKLOADS)")
    ap.add_argument("--chunk", type=int, default=None, help="chunk of the main line (default: the workload's)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    return ap.parse_args()


def settle(fn, seconds, torch):
    """Runs fn untimed for at least `seconds` (the GPU reaches its steady
    clock after some tens of milliseconds of work). Returns the calls made."""
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_steps(bm, fn, steps, warmup, torch, live=True):
    """Times `steps` calls after `warmup`. With `live`, the library's
    per-launch HIP events (recorded on the stream each kernel is launched on)
    run over the same timed steps; otherwise (workloads of a few
    microseconds, where recording events per launch would add host time to
    the step) the steps are timed bare and the per-launch events are taken
    over a second, identical set of steps. Returns ms per step, wall seconds,
    per-kernel (launches, total ms) and the dominant kernel."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    if live:
        with bm.profile() as prof:
            e0.record(s)
            for _ in range(steps):
                fn()
            e1.record(s)
            torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        e0.record(s)
        for _ in range(steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        with bm.profile() as prof:
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
    ker = {k: (c, t) for k, (c, t) in prof.kernels.items()}
    dom = max(ker, key=lambda k: ker[k][1])
    return e0.elapsed_time(e1) / steps, wall, ker, dom


def graph_step_ms(fn, torch, per_graph=20, replays=50):
    """GPU time per call with the host out of the way: `per_graph` calls
    captured once into a HIP graph (the calls launch kernels only: no
    allocation, no memset, no synchronization) and the graph replayed
    `replays` times between two events. Returns ms per call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * per_graph)
    del g
    return ms


def step_stats(fn, steps, torch, flush=None):
    """Per-step times (ms) from a pair of events around each step: median,
    p10, p90. With `flush`, a 512 MiB write evicts the L2s and the 256 MB
    MALL before each step (outside the events): the cold-cache time."""
    s = torch.cuda.current_stream()
    times = []
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    q = lambda f: times[min(len(times) - 1, int(f * len(times)))]  # noqa: E731
    return {"median_ms": round(q(0.5), 4), "p10_ms": round(q(0.1), 4), "p90_ms": round(q(0.9), 4)}


def roofline_for(ker, dom, bytes_per_launch, traffic=None):
    launches, total_ms = ker[dom]
    avg_s = total_ms / launches / 1e3
    achieved = bytes_per_launch / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "kernel": dom, "avg_us": round(avg_s * 1e6, 2)}


def mfma_for(ker, dom, flops_per_launch, executed=None):
    """Algorithmic flops per launch over the kernel's time against the dense
    bf16 peak; with `executed` (matrix-core flops per launch counted by
    rocprofv3, SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 x 2) also the executed
    rate."""
    launches, total_ms = ker[dom]
    sec = total_ms / launches / 1e3
    tflops = flops_per_launch / sec / 1e12
    out = {"achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "kernel": dom,
           "flops_per_launch": flops_per_launch}
    if executed:
        ex = executed / sec / 1e12
        out.update({"executed_flops_per_launch": executed, "executed_achieved": round(ex, 1),
                    "executed_frac": round(ex / MFMA_BF16_PEAK_TFLOPS, 4)})
    return out


def calibrate_copy(torch, dev):
    """A plain copy of known size (256 MiB read, 256 MiB written), so that a
    counter run can scale its byte counters."""
    src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bidirectional_mamba_ssm_amd as bm
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.epilogue_only:
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        print(json.dumps({"gated_norm_layer_1p3b_train": epilogue_bench(args, bm, synth, torch, dev, args.steps)}),
              flush=True)
        return
    if args.merge_only:
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        print(json.dumps({"merge_layer_1p3b_train": merge_bench(args, bm, synth, torch, dev, args.steps)}),
              flush=True)
        return
    if args.bwd_only:
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        print(json.dumps({"bwd_layer_1p3b_train": bwd_bench(args, bm, synth, torch, dev, args.steps)}),
              flush=True)
        return
    if args.conv_only:
        if args.calibrate_copy:
            calibrate_copy(torch, dev)
        print(json.dumps({"conv1d_layer_1p3b_train": conv_bench(args, bm, synth, torch, dev, args.steps)}),
              flush=True)
        return
    if args.block_step_only:
        print(json.dumps({"block_step": block_step_bench(args, bm, synth, torch, dev, args.steps)}),
              flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if args.chunk:
        import dataclasses
        w = dataclasses.replace(w, chunk=args.chunk)
    f, b = synth.make_workload(w, device=dev)
    torch.cuda.synchronize()
    y = torch.empty(w.batch, w.seqlen, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    shape = bm.make_shape(f["x"], f["B"], w.chunk)
    ws_bytes = bm.workspace_size(shape, 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def step():
        bm.ssd_fwd(f, b, chunk=w.chunk, y=y, workspace=ws)

    if args.calibrate_copy:
        calibrate_copy(torch, dev)

    t0 = time.perf_counter()
    n_settle = settle(step, args.settle_s, torch)
    settle_s = time.perf_counter() - t0
    ms, wall, ker, dom = time_steps(bm, step, args.steps, args.warmup, torch)
    tokens = w.batch * w.seqlen
    bpt = bytes_per_token(w.nheads, w.headdim, w.d_state, w.ngroups, 2)
    fpt = flops_per_token(w.nheads, w.headdim, w.d_state, w.ngroups, TILE)
    # the dominant kernel reads every input of the step once and writes y
    roof = roofline_for(ker, dom, bpt * tokens, measured_traffic(dom, w.name))

    out = {
        "metric": METRIC,
        "value": round(tokens / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": w.batch, "seq_len": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "d_state": w.d_state,
                   "ngroups": w.ngroups, "chunk": w.chunk, "bidirectional": True,
                   "parallelism": "none (1 GPU)"},
        "settle": {"seconds": round(settle_s, 3), "steps": n_settle},
        "roofline": roof,
        # (the token-sequential kernels use no matrix cores)
        "mfma": None if dom.startswith("seq_") else
        mfma_for(ker, dom, fpt * tokens,
                 summary_field(summary_path(dom, w.name, "instruction_mix"),
                               "executed_mfma_flops_per_launch")),
        "algorithmic_bytes_per_token": bpt,
        "algorithmic_flops_per_token": fpt,
        "hbm_roofline_frac_step": round(bpt * tokens / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_ms_per_step": {k: round(t / args.steps, 4) for k, (c, t) in ker.items()},
        "wall_s_timed": round(wall, 3),
    }

    if not args.no_extra:
        # per-step distribution, warm and with the caches flushed before each
        # step (after the timed loop, so a profile of --no-extra sees only it)
        flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        out["step_ms_warm"] = step_stats(step, 30, torch)
        out["step_ms_cold_cache"] = step_stats(step, 30, torch, flush=flush)
        del flush
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(f, b, y, w, torch, np)
    del f, b, y, ws
    torch.cuda.empty_cache()
    if not args.no_extra:
        out["extra"] = extras(args, bm, synth, torch, dev)
    print(json.dumps(out), flush=True)


def scan_line(bm, torch, f, b, w, chunk, steps, warmup, cu=None, traffic=True):
    """Times one bidirectional scan workload; its own roofline line."""
    y = torch.empty(w.batch, w.seqlen, w.nheads, w.headdim, dtype=torch.float32, device=f["x"].device)
    shape = bm.make_shape(f["x"], f["B"], chunk)
    nseq = len(cu) - 1 if cu is not None else 0
    ws = torch.empty(max(bm.workspace_size(shape, nseq), 256), dtype=torch.uint8, device=f["x"].device)
    fn = lambda: bm.ssd_fwd(f, b, chunk=chunk, cu_seqlens=cu, y=y, workspace=ws)  # noqa: E731
    settle(fn, 0.2, torch)
    ms, _, ker, dom = time_steps(bm, fn, steps, warmup, torch)
    tok = w.batch * w.seqlen
    bpt = bytes_per_token(w.nheads, w.headdim, w.d_state, w.ngroups, 2)
    fpt = flops_per_token(w.nheads, w.headdim, w.d_state, w.ngroups, TILE)
    res = {"tokens_per_s": round(tok / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
           "hbm_roofline_frac_step": round(bpt * tok / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "kernels_ms_per_step": {k: round(t / steps, 4) for k, (c, t) in ker.items()},
           "roofline": roofline_for(ker, dom, bpt * tok, measured_traffic(dom, w.name) if traffic else None),
           "mfma": mfma_for(ker, dom, fpt * tok)}
    del y, ws
    return res


def ceilings(torch, dev):
    """Practical ceilings on this machine, next to the vendor peaks (context for
    the roofline fractions; library kernels, not this path): a plain device
    copy of 1 GiB (bytes read + written per second) and a dense bf16 matrix
    product of 8192 x 8192 x 8192 (torch.mm on contiguous operands)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    src = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 20 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    g = torch.Generator(device=dev).manual_seed(7)
    n = 8192
    a = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16).contiguous()
    for _ in range(3):
        c = torch.mm(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    mm_tflops = 2 * n ** 3 * 10 / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_1gib": {"achieved": round(copy_gbs, 1), "unit": "GB/s",
                          "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4)},
            "bf16_mm_8192": {"achieved": round(mm_tflops, 1), "unit": "TFLOP/s",
                             "frac_of_peak": round(mm_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}


def extras(args, bm, synth, torch, dev):
    import numpy as np
    res = {}
    steps = max(3, args.steps // 2)
    res["ceilings"] = ceilings(torch, dev)
    # one mixer layer at the training length (8 x 1024 tokens), and the 32k prefill
    for name in ("layer_1p3b_train", "long_32k"):
        w = synth.WORKLOADS[name]
        f, b = synth.make_workload(w, device=dev)
        res[name] = scan_line(bm, torch, f, b, w, w.chunk, max(steps, 50), 10)
        del f, b
        torch.cuda.empty_cache()

    # latency against length at batch 1 (the long-prefill shape): the fit
    # time(L) = a + b L + c L^2 splits it into a constant, a linear and a
    # quadratic part; a scan's quadratic part should be ~0
    base = synth.WORKLOADS["long_128k"]
    lens = [1024, 4096, 16384, 32768, 65536, 131072]
    times = []
    import dataclasses
    for L in lens:
        w = dataclasses.replace(base, seqlen=L)
        f, b = synth.make_workload(w, device=dev)
        r = scan_line(bm, torch, f, b, w, w.chunk, max(10, min(200, 4 * 131072 // L)), 5, traffic=False)
        times.append(r["ms_per_step"])
        del f, b
        torch.cuda.empty_cache()
    Lv = np.array(lens, dtype=np.float64)
    coef, *_ = np.linalg.lstsq(np.stack([np.ones_like(Lv), Lv, Lv ** 2], 1), np.array(times), rcond=None)
    a, bl, c = (float(v) for v in coef)
    res["latency_fit"] = {"lengths": lens, "ms_per_step": times,
                          "fit_ms": {"a": round(a, 5), "b_per_token": bl, "c_per_token2": c},
                          "quadratic_share_at_131072": round(c * 131072 ** 2 / times[-1], 5),
                          "linear_share_at_131072": round(bl * 131072 / times[-1], 5)}

    # slowly decaying heads (A scaled by 1e-2): the carried state reaches far,
    # so no exact-zero decay lets any work be skipped
    w = base
    f, b = synth.make_workload(w, device=dev)
    f = dict(f, A=(f["A"] * 1e-2).contiguous())
    b = dict(b, A=(b["A"] * 1e-2).contiguous())
    res["long_128k_slow_decay"] = dict(scan_line(bm, torch, f, b, w, w.chunk, steps, 5, traffic=False),
                                       A_scale=1e-2)
    del f, b
    torch.cuda.empty_cache()

    # the secondary reading of the long-prefill shape: the tiny head shape
    # (4 heads x headdim 16, d_state 16) at 131 072 tokens, chunk 256, bf16
    # (served by the token-sequential kernel in segments: the matrix-core
    # path is built for headdim 64 / d_state 128)
    f, b = synth.make_workload(synth.WORKLOADS["long_128k_small_heads"], device=dev)
    y = torch.empty(1, 131072, 4, 16, dtype=torch.float32, device=dev)
    shape = bm.make_shape(f["x"], f["B"], 256)
    ws = torch.empty(max(bm.workspace_size(shape, 0), 256), dtype=torch.uint8, device=dev)
    fn = lambda: bm.ssd_fwd(f, b, chunk=256, y=y, workspace=ws)  # noqa: E731
    ms, _, ker, dom = time_steps(bm, fn, 20, 5, torch)
    bpt = bytes_per_token(4, 16, 16, 1, 2)
    res["long_128k_small_heads"] = {"tokens_per_s": round(131072 / (ms / 1e3), 1),
                                    "ms_per_step": round(ms, 4), "bytes_per_token": bpt,
                                    "hbm_roofline_frac_step": round(bpt * 131072 / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                    "kernels_ms_per_step": {k: round(t / 20, 4) for k, (c, t) in ker.items()}}
    del f, b, y, ws
    torch.cuda.empty_cache()

    # packed variable-length batch with per-sequence resets
    w = synth.packed_workload()
    f, b = synth.make_inputs(1, w.seqlen, w.nheads, w.headdim, w.d_state, w.ngroups,
                             w.dtype, w.seed, device=dev)
    cu = synth.cu_seqlens_of(w.seqlens)
    res["packed_varlen"] = dict(scan_line(bm, torch, f, b, w, w.chunk, steps, 5, cu=cu),
                                tokens=w.seqlen, nseq=len(cu) - 1)
    del f, b
    torch.cuda.empty_cache()

    res["block_step"] = block_step_bench(args, bm, synth, torch, dev, max(steps, 100))
    res["conv1d_layer_1p3b_train"] = conv_bench(args, bm, synth, torch, dev, max(steps, 20))
    res["bwd_layer_1p3b_train"] = bwd_bench(args, bm, synth, torch, dev, max(3, steps // 4))
    res["gated_norm_layer_1p3b_train"] = epilogue_bench(args, bm, synth, torch, dev, max(steps, 20))
    res["merge_layer_1p3b_train"] = merge_bench(args, bm, synth, torch, dev, max(steps, 20))
    return res


def block_step_bench(args, bm, synth, torch, dev, steps):
    c = synth.BLOCK_STEP
    H, P, N, G, Lb = c["nheads"], c["headdim"], c["d_state"], c["ngroups"], c["block"]
    out = {}
    seg = 8192
    for nseq, prefix in ((1, args.prefix), (16, args.prefix), (1, 4096)):
        st = bm.State(nseq, H, P, N)
        done, s = 0, 0
        # the forward state after the prefix, built in segments chained through the cache
        while done < prefix:
            n = min(seg, prefix - done)
            pf, _ = synth.make_inputs(nseq, n, H, P, N, G, "bf16", c["seed"] * 1000 + s,
                                      device=dev, bidirectional=False)
            bm.ssd_fwd(pf, None, chunk=256, init_state=st.tensor(), final_state=st.tensor())
            done += n
            s += 1
            del pf
        torch.cuda.synchronize()
        f, b = synth.make_inputs(nseq, Lb, H, P, N, G, "bf16", c["seed"], device=dev)
        y = torch.empty(nseq, Lb, H, P, dtype=torch.float32, device=dev)
        fn = lambda: bm.block_step(st, f, b, commit=False, chunk=64, y=y)  # noqa: E731
        ms, _, ker, dom = time_steps(bm, fn, max(steps, 10), max(3, args.warmup), torch,
                                     live=False)
        per_seq = H * P * N * 4 + bytes_per_token(H, P, N, G, 2) * Lb
        key = f"b{nseq}_prefix{prefix}"
        out[key] = {"ms_per_step": round(ms, 5), "bytes_per_step": per_seq * nseq,
                    "hbm_roofline_frac_step": round(per_seq * nseq / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                    "roofline": roofline_for(ker, dom, per_seq * nseq)}
        # the same step with the host out of the way (graph replay): the
        # launch-bound batch-1 step is mostly host time when called one by one
        msg = graph_step_ms(fn, torch)
        out[key]["ms_per_step_graph"] = round(msg, 5)
        out[key]["hbm_roofline_frac_graph"] = round(per_seq * nseq / (msg / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
        # the same step through a plan bound once (no per-call argument checks)
        plan = bm.BlockStepPlan(st, f, b, commit=False, chunk=64, y=y)
        msp, _, _, _ = time_steps(bm, plan.run, max(steps, 10), max(3, args.warmup), torch, live=False)
        out[key]["ms_per_step_plan"] = round(msp, 5)
        fc = lambda: bm.block_step(st, f, b, commit=True, chunk=64, y=y)  # noqa: E731
        msc, _, _, _ = time_steps(bm, fc, 20, 5, torch, live=False)
        out[key]["ms_per_commit_step"] = round(msc, 5)
        out[key]["ms_per_commit_step_graph"] = round(graph_step_ms(fc, torch), 5)
        st.free()
        del f, b, y
        torch.cuda.empty_cache()
    return out


def bwd_bytes_per_token(H, P, N, G, e):
    """Algorithmic bytes of the training backward per token, both streams:
    read x, dt, B, C of each stream and dy once; write dx, ddt, dB, dC of
    each stream once (fp32)."""
    return 2 * (H * P * e + H * e + 2 * G * N * e) + H * P * 4 + 2 * (H * P + H + 2 * G * N) * 4


def bwd_flops_per_token(H, P, N, G, Q=64):
    """Algorithmic flops of the training backward per token, both streams,
    counting the block products on the parts they use (triangles for the
    within-block ones): per block of Q positions and head, C.B^T and dy.x^T
    and the within-block dxd, dC, dB over the lower triangle, the four
    entering/leaving-state products and the block state and gradient feed
    over the full block."""
    tri = Q * (Q + 1) // 2
    mac = tri * N + tri * P + tri * P + 2 * tri * N + 6 * Q * N * P
    return 2 * 2 * H * mac // Q


def bwd_bench(args, bm, synth, torch, dev, steps):
    """The training backward at the training layer's shape (8 x 1024 tokens,
    64 heads x 64, d_state 128, bf16, both streams)."""
    w = synth.WORKLOADS["layer_1p3b_train"]
    f, b = synth.make_workload(w, device=dev)
    g = torch.Generator(device=dev).manual_seed(82)
    dy = torch.randn(w.batch, w.seqlen, w.nheads, w.headdim, generator=g, device=dev)
    shape = bm.make_shape(f["x"], f["B"], 64)
    ws = torch.empty(bm.bwd_workspace_size(shape, True), dtype=torch.uint8, device=dev)
    grads = bm.ssd_bwd(f, b, dy, workspace=ws)
    fn = lambda: bm.ssd_bwd(f, b, dy, grads=grads, workspace=ws)  # noqa: E731
    ms, _, ker, dom = time_steps(bm, fn, steps, max(3, args.warmup // 10), torch)
    tok = w.batch * w.seqlen
    bpt = bwd_bytes_per_token(w.nheads, w.headdim, w.d_state, w.ngroups, 2)
    fpt = bwd_flops_per_token(w.nheads, w.headdim, w.d_state, w.ngroups)
    tfl = fpt * tok / (ms / 1e3) / 1e12
    res = {"workload": f"training backward, {w.name} (8 x 1024 tokens, 64 x 64 heads, d_state 128, bf16 in, fp32 gradients, both streams)",
           "tokens_per_s": round(tok / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
           "algorithmic_bytes_per_token": bpt,
           "hbm_roofline_frac_step": round(bpt * tok / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "algorithmic_flops_per_token": fpt,
           "mfma_fp32": {"achieved": round(tfl, 1), "peak": MFMA_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tfl / MFMA_FP32_PEAK_TFLOPS, 4)},
           "kernels_ms_per_step": {k: round(t / steps, 4) for k, (c, t) in ker.items()},
           "dominant_kernel": dom}
    if not args.no_cpu_baseline:
        # the oracle's adjoint (C, fp64) on one row of the same inputs; its
        # work is spread over rows, so one row runs on one core
        import oracle
        fr = {k: (v[:1] if v.dim() > 1 else v) for k, v in f.items()}
        br = {k: (v[:1] if v.dim() > 1 else v) for k, v in b.items()}
        t0 = time.perf_counter()
        oracle.bissd_bwd(fr, br, dy[:1])
        sec = time.perf_counter() - t0
        res["cpu_oracle"] = {"tokens_per_s": round(w.seqlen / sec, 1), "kind": "oracle", "cores": 1,
                             "sample": f"1 of {w.batch} rows ({w.seqlen} tokens), both streams, fp64 adjoint, {sec:.1f} s"}
    del f, b, dy, ws, grads
    torch.cuda.empty_cache()
    return res


def epilogue_bench(args, bm, synth, torch, dev, steps):
    """The gated-norm epilogue at the layer's shape: 8 x 1024 tokens, 4096
    channels, one group, fp32 y, bf16 gate and output. Algorithmic bytes:
    y, z read once, the output written once, plus the weight."""
    rows, C = 8 * 1024, 4096
    y, z, w = synth.make_epilogue_inputs(rows, C, "bf16", 108, device=dev)
    out = torch.empty(rows, C, dtype=torch.bfloat16, device=dev)
    fn = lambda: bm.gated_norm(y, z, w, out=out)  # noqa: E731
    ms, _, ker, dom = time_steps(bm, fn, steps, max(3, args.warmup // 10), torch)
    nbytes = rows * C * (4 + 2 + 2) + C * 4
    res = {"workload": f"gated RMS norm, {rows} tokens x {C} channels, one group, bf16 gate and output",
           "tokens_per_s": round(rows / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
           "bytes_per_launch": nbytes, "roofline": roofline_for(ker, dom, nbytes),
           "ms_per_step_graph": round(graph_step_ms(fn, torch), 5)}
    if not args.no_cpu_baseline:
        from oracle import epilogue as oepi
        n = 1024
        t0 = time.perf_counter()
        oepi.gated_rmsnorm(y[:n], z[:n], w, C)
        sec = time.perf_counter() - t0
        res["cpu_oracle"] = {"tokens_per_s": round(n / sec, 1), "kind": "oracle",
                             "sample": f"{n} of {rows} tokens, numpy fp64, {sec:.2f} s"}
    del y, z, w, out
    torch.cuda.empty_cache()
    return res


def merge_bench(args, bm, synth, torch, dev, steps):
    """The concatenating merge at the layer's shape. (1) The scan with the
    two streams written apart (8 x 1024 tokens, 64 heads x 64, d_state 128,
    bf16), against the summing scan. (2) The Linear merge over the block
    outputs: 8 x 1024 tokens, 2 x 2048 channels in, 2048 out (d_model 2048),
    bf16 weight, fp32 streams and output; bound by the matrix cores
    (2 x 4096 x 2048 flops per token)."""
    w = synth.WORKLOADS["layer_1p3b_train"]
    f, b = synth.make_workload(w, device=dev)
    tok = w.batch * w.seqlen
    yf = torch.empty(w.batch, w.seqlen, w.nheads, w.headdim, dtype=torch.float32, device=dev)
    yb = torch.empty_like(yf)
    shape = bm.make_shape(f["x"], f["B"], w.chunk)
    ws = torch.empty(max(bm.workspace_size(shape, 0), 256), dtype=torch.uint8, device=dev)
    fn = lambda: bm.ssd_fwd_streams(f, b, chunk=w.chunk, y_fwd=yf, y_bwd=yb, workspace=ws)  # noqa: E731
    ms_s, _, ker_s, dom_s = time_steps(bm, fn, steps, max(3, args.warmup // 10), torch)
    fn = lambda: bm.ssd_fwd(f, b, chunk=w.chunk, y=yf, workspace=ws)  # noqa: E731
    ms_f, _, _, _ = time_steps(bm, fn, steps, max(3, args.warmup // 10), torch)
    # one more fp32 output of y: the streams written apart
    bpt = bytes_per_token(w.nheads, w.headdim, w.d_state, w.ngroups, 2) + w.nheads * w.headdim * 4
    res = {"streams": {"workload": "scan with the streams kept apart, 8 x 1024 tokens, 64 heads x 64, "
                                   "d_state 128, bf16",
                       "tokens_per_s": round(tok / (ms_s / 1e3), 1), "ms_per_step": round(ms_s, 4),
                       "ms_per_step_summed_scan": round(ms_f, 4),
                       "roofline": roofline_for(ker_s, dom_s, bpt * tok)}}
    del f, b, yf, yb, ws
    torch.cuda.empty_cache()

    rows, cin, cout = tok, 2048, 2048
    g = torch.Generator(device=dev).manual_seed(109)
    yf = torch.randn(rows, cin, generator=g, device=dev)
    yb = torch.randn(rows, cin, generator=g, device=dev)
    wt = (torch.randn(cout, 2 * cin, generator=g, device=dev) / (2 * cin) ** 0.5).to(torch.bfloat16)
    bias = torch.randn(cout, generator=g, device=dev)
    out = torch.empty(rows, cout, dtype=torch.float32, device=dev)
    fn = lambda: bm.merge_linear(yf, yb, wt, bias, out=out)  # noqa: E731
    ms, _, ker, dom = time_steps(bm, fn, steps, max(3, args.warmup // 10), torch)
    flops = 2 * rows * 2 * cin * cout
    nbytes = rows * (2 * cin + cout) * 4 + cout * 2 * cin * 2 + cout * 4
    m = mfma_for(ker, dom, flops)
    m["bound"] = "mfma"
    res["linear"] = {"workload": f"Linear merge, {rows} tokens, 2 x {cin} -> {cout}, bf16 weight, "
                                "fp32 streams and output",
                     "tokens_per_s": round(rows / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
                     "roofline": m, "hbm": roofline_for(ker, dom, nbytes)}
    if not args.no_cpu_baseline:
        from oracle import merge as omerge
        n = 512
        a, c, wc, bc = yf[:n].cpu(), yb[:n].cpu(), wt.float().cpu(), bias.cpu()
        t0 = time.perf_counter()
        omerge.merge_linear(a, c, wc, bc)
        sec = time.perf_counter() - t0
        res["linear"]["cpu_oracle"] = {"tokens_per_s": round(n / sec, 1), "kind": "oracle",
                                       "sample": f"{n} of {rows} tokens, numpy fp64, {sec:.2f} s"}
    del yf, yb, wt, bias, out
    torch.cuda.empty_cache()
    return res


def conv_bench(args, bm, synth, torch, dev, steps):
    """The short convolution in front of the scan at the layer's shape (8 x
    1024 tokens, 64 x 64 + 2 x 128 = 4352 channels, width 4, bf16, SiLU, both
    directions in one launch). Algorithmic bytes: every input element read
    once, every output element written once, plus the taps and biases."""
    c = synth.CONV_LAYER
    H, P, G, N, W = c["nheads"], c["headdim"], c["ngroups"], c["d_state"], c["width"]
    ch = bm.conv_channels(H, P, G, N)
    batch, L = c["batch"], c["seqlen"]
    f, b = synth.make_conv_inputs(batch, L, ch, W, c["dtype"], c["seed"], device=dev)

    def outs():
        return dict(x=torch.empty(batch, L, H, P, dtype=torch.bfloat16, device=dev),
                    B=torch.empty(batch, L, G, N, dtype=torch.bfloat16, device=dev),
                    C=torch.empty(batch, L, G, N, dtype=torch.bfloat16, device=dev))
    out = (outs(), outs())
    fn = lambda: bm.conv1d(f, b, H, P, G, N, out=out)  # noqa: E731
    ms, _, ker, dom = time_steps(bm, fn, steps, max(3, args.warmup // 10), torch)
    nbytes = 2 * (2 * batch * L * ch * 2 + ch * (W + 1) * 4)
    tok = batch * L
    res = {"workload": f"conv1d {batch}x{L} tokens, {ch} channels, width {W}, bf16, SiLU, both directions",
           "tokens_per_s": round(tok / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
           "bytes_per_launch": nbytes,
           "roofline": roofline_for(ker, dom, nbytes)}
    res["ms_per_step_graph"] = round(graph_step_ms(fn, torch), 5)
    if not args.no_cpu_baseline:
        # the oracle (numpy, fp64) on one row of the same inputs, both directions
        from oracle import conv as oconv
        fr = {k: (v[:1] if k == "xbc" else v) for k, v in f.items()}
        br = {k: (v[:1] if k == "xbc" else v) for k, v in b.items()}
        t0 = time.perf_counter()
        oconv.conv1d(fr["xbc"], fr["weight"], fr["bias"])
        oconv.conv1d(br["xbc"], br["weight"], br["bias"], reverse=True)
        sec = time.perf_counter() - t0
        res["cpu_oracle"] = {"tokens_per_s": round(L / sec, 1), "kind": "oracle",
                             "sample": f"1 of {batch} rows ({L} tokens), both directions, numpy fp64, {sec:.2f} s"}
    del f, b, out
    torch.cuda.empty_cache()
    return res


def cpu_baseline(f, b, y, w, torch, np):
    """The fp64 oracle on this host's cores on a bounded sample of the same
    inputs, about 10-20 s of CPU work: whole rows where the batch has several,
    else a subset of the heads over every token of the row (heads are
    independent units of the oracle's work, each a full pass over the
    sequence in both directions). The rate is scaled to tokens/s of the whole
    workload (all heads), with the parity of the sample against the GPU."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    oracle.set_num_threads(cores)

    def sample(lo, hi, heads):
        def cut(d):
            out = {}
            for k, v in d.items():
                if k in ("x", "dt"):
                    out[k] = v[lo:hi][:, :, heads].contiguous().cpu()
                elif k in ("B", "C"):
                    out[k] = v[lo:hi].contiguous().cpu()
                else:
                    out[k] = v[heads].contiguous().cpu()
            return out
        return cut(f), cut(b)

    H = w.nheads
    if w.batch > 1:
        rows, heads = (0, 1), list(range(H))
    else:
        rows, heads = (0, 1), list(range(0, H, max(1, H // cores)))[:cores]
    fr, br = sample(rows[0], rows[1], heads)
    t0 = time.perf_counter()
    ref = oracle.bissd(fr, br)
    t1 = time.perf_counter() - t0
    # grow the sample to about 10 s of CPU time
    if w.batch > 1:
        n_rows = int(min(w.batch, max(1, math.ceil(10.0 / max(t1, 1e-3)))))
        rows = (0, n_rows)
    else:
        n_heads = int(min(H, max(len(heads), math.ceil(len(heads) * 10.0 / max(t1, 1e-3)))))
        heads = list(range(0, H, max(1, H // n_heads)))[:n_heads]
    fr, br = sample(rows[0], rows[1], heads)
    t0 = time.perf_counter()
    ref = oracle.bissd(fr, br)
    sec = time.perf_counter() - t0
    got = y[rows[0]:rows[1]][:, :, heads].double().cpu().numpy()
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)) / rms)
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    nrow = rows[1] - rows[0]
    # tokens/s of the whole workload: sample work / whole work = rows * heads / (batch * H)
    value = nrow * w.seqlen * (len(heads) / H) / sec
    return {"value": round(value, 2), "unit": "tokens/s",
            "cores": int(oracle.num_threads()), "kind": "oracle",
            "sample": f"{nrow} of {w.batch} rows x {w.seqlen} tokens, {len(heads)} of {H} heads, "
                      f"both directions, of the same inputs; fp64 sequential recurrence, {sec:.1f} s; "
                      f"rate scaled to all {H} heads",
            "cpu_model": cpu_model,
            "parity_max_abs_err_over_rms": err, "parity_ok": err <= 1e-2}


if __name__ == "__main__":
    main()
