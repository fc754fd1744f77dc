"""Benchmark of the W4A8 hot path on one MI355X.

Default workload: the 70B-like FFN-down layer at M = 2048 (K = 28672,
N = 8192), the largest configuration, MFMA-bound.  A bf16 [2048, 28672] unit
Student t(3); W bf16 [8192, 28672] ~ N(0, 0.02^2) packed once to two-level
int4 (group 64).  One step = w4a8_gemm_bf16act: per-token int8 quantization of
A plus the W4A8 GEMM with bf16 output (for m <= 16 one kernel does both).
Weight packing is offline (once per weight) and not part of a step.  The steps
are captured into a HIP graph and the timed region replays it, so host-side
launch cost does not stand in for device time.  Exactly --warmup untimed steps
run first (one eager step loads the kernels, the rest replay graphs), then
exactly --steps timed steps.

Inputs are resident in HBM before timing.  To keep the 256 MB MALL and the L2s
from serving the weights, each step uses the next of R distinct copies of the
packed weights and activations (R copies total > 512 MB).

Printed: one JSON line with the step throughput (TOPS = 2*M*N*K / step time),
the dominant kernel's roofline (algorithmic ops or bytes per launch / average
launch time from HIP events on the launch stream, against the vendor peak and
against references measured in the same run: a device copy and an MFMA-only
loop with its shader clock), the other workloads (decode, prefill, FFN-down
M = 1 and 64) as sub-objects with their own rooflines, the standalone
quantizer (64M bf16 elements, block 32 and 128: GB/s, dequantization round
trip and its MSE), the extension paths (LQQ weights, W8A8 against W4A8 on
memory-bound and compute-bound shapes, per-block activation scales in the
GEMM, the EQuARX dequantize-add-requantize step), and the CPU oracle timed on
the host cores on a bounded sample (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
INT8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA, vendor figure
METRIC = "W4A8 GEMM TOPS + quantizer GB/s; % of int8-MFMA / HBM roofline, 1 MI355X"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="ffn_down_m2048",
                   choices=["decode", "prefill", "ffn_down_m1", "ffn_down_m64", "ffn_down_m2048",
                            "tiny"])
    p.add_argument("--sub-steps", type=int, default=50,
                   help="timed steps of each other workload (sub-objects of the line)")
    p.add_argument("--sub-warmup", type=int, default=50)
    p.add_argument("--no-subworkloads", action="store_true")
    p.add_argument("--no-probes", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-quantizer", action="store_true")
    p.add_argument("--no-extensions", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (reference for the "
                        "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def gemm_algorithmic_bytes(m, n, k, out_bytes, fused):
    """Bytes the W4A8 GEMM must move: int4 weights, uint8 group scales, fp32 channel
    scales and the output, each once; plus the activations once: bf16 when
    quantization is fused into the kernel (the int8 codes it also leaves in the
    workspace are not counted), else the int8 codes + fp32 row scales."""
    act = 2 * m * k if fused else (m * k + 4 * m)
    return n * k // 2 + n * (k // 64) + 4 * n + act + m * n * out_bytes


def quantizer_algorithmic_bytes(elems, block):
    """bf16 in (2 B), int8 out (1 B), one fp32 scale per block."""
    return elems * 3 + 4 * (elems // block)


def copy_probe_gbps(torch, dev, reps=10):
    """Measured HBM reference: a 256 MiB device-to-device copy (bytes read +
    bytes written per second), timed with HIP events after a warmup."""
    x = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * 4 * x.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    return gbps


def time_graph(torch, fn, copies, reps, min_calls=20):
    """Capture fn(r % copies, stream) for r in range(calls) into one HIP graph,
    with calls the smallest multiple of `copies` that is at least min_calls
    (so the gap between graph launches is spread over many kernels), replay it
    once untimed, then `reps` times between HIP events on the capture stream.
    Returns the average milliseconds per fn call."""
    calls = copies * max(1, -(-min_calls // copies))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in range(copies):
            fn(r, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        for r in range(calls):
            fn(r % copies, s)
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * calls)


def n_copies(per_copy_bytes):
    """Distinct buffer sets needed for > 512 MB in rotation (cold MALL and L2)."""
    return max(2, min(64, (512 << 20) // max(per_copy_bytes, 1) + 1))


def profile_traffic(kernel_key: str, workload: str):
    """HBM traffic per launch measured by rocprofv3 counters, if a committed profile
    for this kernel and workload exists and the GEMM sources are unchanged since."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    msha = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    mbytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (msha and mbytes) or msha.group(1) != sources_sha256():
        return None
    return float(mbytes.group(1))


def sources_sha256() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a8_quantized_gemm_quantize_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def cpu_baseline(a_bits, w_bits, spec, seconds):
    """The CPU oracle (plain C, OpenMP over output rows), timed on the host cores:
    per-token quantization + GEMM on the same workload, repeated for ~`seconds`;
    then each stage on its own (weight packing once, activation quantization and
    the int8 GEMM for about a second each)."""
    import oracle
    m, n, k = spec["m"], spec["n"], spec["k"]
    t_pack = time.perf_counter()
    q, sg, sch = oracle.quantize_w4_grouped(w_bits, 64)          # offline step, timed once
    t_pack = time.perf_counter() - t_pack
    rows = m
    if m > 64:                                                     # bound the sample
        rows = 64
    a = np.ascontiguousarray(a_bits[:rows])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.w4a8_gemm_bf16act(a, q, sg, sch, 64, want_y=True)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    ops = 2.0 * rows * n * k * reps

    def repeat(fn, budget=1.0):
        count, t1 = 0, time.perf_counter()
        while True:
            out = fn()
            count += 1
            dt = time.perf_counter() - t1
            if dt >= budget:
                return out, dt / count

    (a_q, a_s), t_quant = repeat(lambda: oracle.quantize_act_blockwise(a, k))
    _, t_gemm = repeat(lambda: oracle.w4a8_gemm(a_q, a_s, q, sg, sch, 64, want_y=True))
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} runs of per-token quantize + GEMM on rows [0,{rows}) of the "
                      f"{m}x{n}x{k} workload ({el:.1f} s wall)",
            "stages": {
                "pack_weights_gbps": 2.0 * n * k / t_pack / 1e9,          # bf16 weights in
                "quantize_gbps": (3.0 * rows * k + 4.0 * rows) / t_quant / 1e9,
                "gemm_tops": 2.0 * rows * n * k / t_gemm / 1e12,
            }}


def mfma_probe_leg(torch, w4a8, dev, stream, reps=40):
    """The int8 matrix-core reference (MFMA-only loop built with the library): one
    workgroup of 8 wavefronts per compute unit, timed with HIP events on the
    launch stream; the shader clock is read inside the kernel.  About 40 ms of
    launches: a GPU coming out of idle takes some 30 ms of sustained load to
    reach its steady clock, and this leg runs right before the headline's
    warmup steps."""
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4096
    for _ in range(3):
        w4a8.probe_mfma_i8(ncu, iters, device=dev, stream=stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ops, _, clocks = w4a8.probe_mfma_i8(ncu, iters, device=dev, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ticks, rt = [int(v) for v in clocks.cpu().tolist()]
    clock_ghz = ticks / rt * 0.1 if rt > 0 else None
    tops = ops / (ms * 1e-3) / 1e12
    res = {"kind": "int8 MFMA-only loop (w4a8_probe_mfma_i8), 8 wavefronts per CU",
           "compute_units": ncu, "kernel_ms": ms, "achieved": tops, "unit": "TFLOP/s",
           "frac_of_spec": tops / INT8_PEAK_TOPS, "clock_ghz": clock_ghz}
    if clock_ghz:
        res["peak_at_clock"] = ncu * 8192 * clock_ghz * 1e9 / 1e12
    return res


def measure_workload(torch, w4a8, dev, name, a_bits, w_bits, spec, steps, warmup,
                     packed=None, probes=None, prime=None):
    """One workload: `warmup` untimed steps, then exactly `steps` timed steps, each
    step = w4a8_gemm_bf16act (per-token quantization of A + the W4A8 GEMM) over
    the next of R rotating weight/activation copies (> 512 MB in rotation).
    Returns the step time, the step throughput and the dominant kernel's roofline.
    `prime` (optional) runs after set-up and graph capture, right before the
    warmup steps."""
    m, n, k = spec["m"], spec["n"], spec["k"]
    out_dtype = torch.bfloat16 if spec["out"] == "bf16" else torch.float32
    out_bytes = 2 if spec["out"] == "bf16" else 4

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    a0 = to_dev(a_bits)
    wp0, gs0, cs0 = packed if packed is not None else w4a8.pack_w4_grouped(to_dev(w_bits))
    per_copy = wp0.numel() + gs0.numel() + 4 * cs0.numel() + 2 * m * k
    copies = n_copies(per_copy)
    wps = [wp0] + [wp0.clone() for _ in range(copies - 1)]
    gss = [gs0] + [gs0.clone() for _ in range(copies - 1)]
    css = [cs0] + [cs0.clone() for _ in range(copies - 1)]
    acts = [a0] + [a0.clone() for _ in range(copies - 1)]
    # codes and scales of the quantized activations, then (decode batches at
    # large K) the int32 partial sums of the split-K GEMM
    ws_base = w4a8.workspace_bytes(m, k)
    split = w4a8.gemm_workspace_bytes(m, n, k) > 0
    wss = [torch.empty(w4a8.workspace_bytes(m, k, n), dtype=torch.uint8, device=dev)
           for _ in range(copies)]
    out = torch.empty((m, n), dtype=out_dtype, device=dev)
    stream = torch.cuda.current_stream()

    def step(r, st):
        # one pass of the path: per-token quantization of A + W4A8 GEMM
        w4a8.w4a8_gemm_bf16act(acts[r], wps[r], gss[r], css[r], n, out=out, workspace=wss[r],
                               stream=st)

    def gemm_only(r, st):
        a_q, a_s = w4a8.workspace_views(wss[r], m, k)
        if split:
            w4a8.w4a8_gemm_ws(a_q, a_s, wps[r], gss[r], css[r], n, out=out,
                              workspace=wss[r][ws_base:], stream=st)
        else:
            w4a8.w4a8_gemm(a_q, a_s, wps[r], gss[r], css[r], n, out=out, stream=st)

    # One graph holds `per_graph` steps (a multiple of the copy count, at least
    # 20), cycling through the copies, so the gap between graph launches is
    # spread over many steps.
    per_graph = copies * max(1, -(-20 // copies))

    def capture(fn, count=per_graph):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream()
            for r in range(count):
                fn(r % copies, s)
        return g

    # Warmup: exactly `warmup` untimed steps.  The first is an eager step on
    # copy 0 (it loads the kernels before graph capture); the others replay
    # graphs: whole graphs of `per_graph` steps, then a graph of the first
    # (count mod per_graph) steps, captured beforehand.  The timed region
    # replays exactly `steps` steps the same way.
    eager = 1 if warmup >= 1 else 0
    if eager:
        step(0, stream)
        torch.cuda.synchronize()
    g_step = capture(step)
    warm_graph = warmup - eager
    partial = {r: capture(step, r) for r in {steps % per_graph, warm_graph % per_graph} if r}

    def run_steps(count):
        for _ in range(count // per_graph):
            g_step.replay()
        if count % per_graph:
            partial[count % per_graph].replay()

    if prime is not None:
        prime()
    run_steps(warm_graph)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    run_steps(steps)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps

    # Dominant kernel: with m <= 16 the step is one fused kernel (quantization in
    # the GEMM's prologue), so its average duration is the step time; otherwise
    # the GEMM launches alone are replayed from their own graph (after one
    # untimed replay) and timed with HIP events on the same stream (with split
    # K: the K-sliced GEMM and the pass that sums its partials, together).
    fused = m <= 16
    if fused:
        gemm_ms = ms_per_step
        gemm_launches = steps
    else:
        g_gemm = capture(gemm_only)
        g_gemm.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // per_graph)
        e0.record(stream)
        for _ in range(reps):
            g_gemm.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        gemm_ms = e0.elapsed_time(e1) / (reps * per_graph)
        gemm_launches = reps * per_graph

    ops = 2.0 * m * n * k
    tops = ops / (ms_per_step * 1e-3) / 1e12
    gemm_bytes = gemm_algorithmic_bytes(m, n, k, out_bytes, fused)
    hbm_bound = m <= 64
    if hbm_bound:
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS}
        if probes and probes.get("copy_gbps"):
            roof["probe"] = {"kind": "256 MiB device copy, read + written",
                             "achieved": probes["copy_gbps"], "unit": "GB/s",
                             "frac_of_probe": achieved / probes["copy_gbps"]}
    else:
        achieved = ops / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": achieved / INT8_PEAK_TOPS}
        mp = (probes or {}).get("mfma")
        if mp:
            roof["probe"] = {"kind": mp["kind"], "achieved": mp["achieved"], "unit": "TFLOP/s",
                             "frac_of_probe": achieved / mp["achieved"],
                             "clock_ghz": mp["clock_ghz"]}
    if split:
        kernel_key = "gemm_splitk"
    elif hbm_bound:
        kernel_key = "gemm_skinny_fused" if fused else "gemm_skinny"
    else:
        kernel_key = "gemm_tiled"
    roof["kernel"] = kernel_key
    if split:
        roof["kernel_launches"] = ["gemm_tiled_kernel over K slices", "splitk_finalize_kernel"]
        roof["splitk_partial_bytes"] = w4a8.gemm_workspace_bytes(m, n, k)
    roof["kernel_ms"] = gemm_ms
    roof["kernel_launches_timed"] = gemm_launches
    roof["algorithmic_bytes_per_launch"] = gemm_bytes
    roof["algorithmic_ops_per_launch"] = ops
    roof["traffic"] = profile_traffic(kernel_key, name)
    res = {"workload": f"{name} W4A8 GEMM M={m} K={k} N={n}, per-token int8 activations "
                       f"(quantized in the call), int4 weights group 64, {spec['out']} out",
           "m": m, "n": n, "k": k, "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
           "value": tops, "unit": "TOPS", "weight_copies_rotated": copies,
           "steps_per_graph": per_graph, "roofline": roof}
    del wps, gss, css, acts, wss, out, g_step, partial
    return res


SUB_WORKLOADS = ["ffn_down_m1", "ffn_down_m64", "decode", "prefill"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build "
              "runs the hot path on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    from w4a8_quantized_gemm_quantize_amd import binding as w4a8
    from w4a8_quantized_gemm_quantize_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        x = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": 4 * x.numel(),
                          "bytes_written_per_launch": 4 * x.numel(), "launches": 5}))
        return
    stream = torch.cuda.current_stream()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # Measured references on this GPU: a device copy (HBM) and the MFMA-only loop.
    # They run inside the headline measurement, after its set-up and graph
    # capture and right before its warmup steps, so the timed steps start on a
    # GPU that has just been under load (clocks as in steady use), not on one
    # that sat idle while the host captured the graphs.
    probes = {}

    def run_probes():
        probes["copy_gbps"] = copy_probe_gbps(torch, dev)
        probes["mfma"] = mfma_probe_leg(torch, w4a8, dev, stream)
        log("probes done")

    a_bits, w_bits, spec = inputs.workload_inputs(args.workload, seed=0)
    head = measure_workload(torch, w4a8, dev, args.workload, a_bits, w_bits, spec,
                            max(1, args.steps), max(0, args.warmup), probes=probes,
                            prime=None if args.no_probes else run_probes)
    log(f"{args.workload}: {head['ms_per_step'] * 1e3:.1f} us/step")
    m, n, k = spec["m"], spec["n"], spec["k"]
    line = {
        "metric": METRIC, "value": head["value"], "unit": "TOPS", "n_gpus": 1,
        "steps": head["steps"], "warmup": head["warmup"], "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": head["workload"], "m": m, "n": n, "k": k, "group": 64,
                   "weight_copies_rotated": head["weight_copies_rotated"],
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
    }
    if probes:
        line["probes"] = {"hbm_copy_gbps": probes["copy_gbps"], "mfma": probes["mfma"]}

    if not args.no_subworkloads:
        # The other workloads of the path, each with its own roofline.  The FFN
        # shapes share the head workload's weights when it is an FFN shape.
        subs = {}
        ffn_packed = None
        head_ffn = args.workload.startswith("ffn_down")
        for name in SUB_WORKLOADS:
            if name == args.workload:
                continue
            packed = None
            if name.startswith("ffn_down") and head_ffn:
                # same weights (seed 0, 8192 x 28672): packed once, shared
                sspec = inputs.WORKLOADS[name]
                sa = inputs.activations(sspec["m"], sspec["k"], 0, sspec["dist"],
                                        sspec["outlier_frac"])
                sw = w_bits
                if ffn_packed is None:
                    wdev = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
                    ffn_packed = w4a8.pack_w4_grouped(wdev)
                    del wdev
                packed = ffn_packed
            else:
                sa, sw, sspec = inputs.workload_inputs(name, seed=0)
            subs[name] = measure_workload(torch, w4a8, dev, name, sa, sw, sspec,
                                          args.sub_steps, args.sub_warmup, packed=packed,
                                          probes=probes)
            log(f"{name}: {subs[name]['ms_per_step'] * 1e3:.2f} us/step")
        del ffn_packed
        torch.cuda.empty_cache()
        line["workloads"] = subs

    if not args.no_quantizer:
        line["quantizer"] = quantizer_leg(torch, w4a8, inputs, dev, stream)
        log("quantizer done")
    if not args.no_extensions:
        line["extensions"] = extensions_leg(
            torch, w4a8, inputs, dev,
            ffn_w_bits=w_bits if args.workload.startswith("ffn_down") else None)
        log("extensions done")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a_bits, w_bits, spec, args.cpu_seconds)
        line["cpu_baseline"]["gpu_over_cpu"] = head["value"] / line["cpu_baseline"]["value"]
    print(json.dumps(line), flush=True)


def quantizer_leg(torch, w4a8, inputs, dev, stream, reps=20):
    """Standalone quantizer workload: 64M bf16 ~ N(0,1) as [65536, 1024], blocks 32
    and 128.  Input/output sets of ~200 MB rotate, more than 512 MB in all, so
    reads come from HBM (not the 256 MB last-level cache)."""
    spec = inputs.QUANTIZER
    rows, cols = spec["rows"], spec["cols"]
    x0 = torch.from_numpy(inputs.activations(rows, cols, seed=0).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    ncp = n_copies(rows * cols * 3 + 4 * (rows * cols // 32))
    xs = [x0] + [x0.clone() for _ in range(ncp - 1)]
    res = {"workload": f"{rows}x{cols} bf16 ~ N(0,1) (64M elements, seed 0), "
                       f"{ncp} buffer sets rotated"}
    for block in spec["blocks"]:
        qs = [torch.empty((rows, cols), dtype=torch.int8, device=dev) for _ in range(ncp)]
        ss = [torch.empty((rows, cols // block), dtype=torch.float32, device=dev)
              for _ in range(ncp)]
        def quant(r, st, block=block, qs=qs, ss=ss):
            w4a8.quantize_act_blockwise(xs[r], block, q=qs[r], scales=ss[r], stream=st)
        # graph replays of the input/output sets in turn, as for the GEMMs
        # (per-call events would add the launch gaps to a 35-40 us kernel)
        ms = time_graph(torch, quant, ncp, reps)
        gbps = quantizer_algorithmic_bytes(rows * cols, block) / (ms * 1e-3) / 1e9
        entry = {"kernel_ms": ms, "achieved": gbps, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS}
        # dequantization round trip: q, scales -> fp32 and bf16; MSE against x
        elems = rows * cols
        for name, dt, ob in (("dequant_f32", torch.float32, 4), ("dequant_bf16", torch.bfloat16, 2)):
            outs = [torch.empty((rows, cols), dtype=dt, device=dev) for _ in range(ncp)]

            def deq(r, st, outs=outs, dt=dt):
                w4a8.dequantize_act_blockwise(qs[r], ss[r], block, dt, out=outs[r], stream=st)
            dms = time_graph(torch, deq, ncp, 10)
            dbytes = elems * (1 + ob) + 4 * (elems // block)
            x64 = xs[0].double()
            mse = float(((outs[0].double() - x64) ** 2).mean())
            entry[name] = {"kernel_ms": dms, "achieved": dbytes / (dms * 1e-3) / 1e9,
                           "unit": "GB/s", "mse": mse}
        res[f"block{block}"] = entry
    return res


def extensions_leg(torch, w4a8, inputs, dev, ffn_w_bits=None):
    """The extension paths, each timed from a HIP graph over rotating buffer sets:
    LQQ weights (decode shape, fused step), W8A8 against W4A8 (decode: memory-bound;
    prefill: compute-bound, int8 activations), the GEMM with per-block activation
    scales (decode shape, blocks 32 and 128; prefill shape, block 128) and the
    EQuARX receive step (64M elements, bf16 partial sums, blocks 32 and 128)."""
    res = {}

    def bf16_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- decode shape: LQQ, W8A8 and per-block scales
    a_bits, w_bits, spec = inputs.workload_inputs("decode", seed=0)
    m, n, k = spec["m"], spec["n"], spec["k"]
    a = bf16_dev(a_bits)
    w = bf16_dev(w_bits)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(w4a8.workspace_bytes(m, k), dtype=torch.uint8, device=dev)
    act_bytes = 2 * m * k + m * n * 2 + 4 * n

    wp, gp, cs = w4a8.pack_w4_lqq(w)
    c = n_copies(wp.numel() + 2 * gp.numel())
    sets = [(wp, gp, cs)] + [(wp.clone(), gp.clone(), cs.clone()) for _ in range(c - 1)]
    ms = time_graph(torch, lambda r, st: w4a8.w4a8_gemm_lqq_bf16act(
        a, *sets[r], n, out=out, workspace=ws, stream=st), c, 4)
    byt = n * k // 2 + 2 * n * (k // 64) + act_bytes
    res["lqq_decode"] = {"shape": [m, n, k], "kernel_ms": ms, "achieved": byt / (ms * 1e-3) / 1e9,
                         "unit": "GB/s", "frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del sets

    w4p, g4, c4 = w4a8.pack_w4_grouped(w)
    c = n_copies(w4p.numel() + g4.numel())
    sets4 = [(w4p, g4, c4)] + [(w4p.clone(), g4.clone(), c4.clone()) for _ in range(c - 1)]
    ms4 = time_graph(torch, lambda r, st: w4a8.w4a8_gemm_bf16act(
        a, *sets4[r], n, out=out, workspace=ws, stream=st), c, 4)
    w8p, c8 = w4a8.pack_w8_channel(w)
    c = n_copies(w8p.numel())
    sets8 = [(w8p, c8)] + [(w8p.clone(), c8.clone()) for _ in range(c - 1)]
    ms8 = time_graph(torch, lambda r, st: w4a8.w8a8_gemm_bf16act(
        a, *sets8[r], n, out=out, workspace=ws, stream=st), c, 4)
    res["w8a8_vs_w4a8_decode"] = {
        "shape": [m, n, k], "w4a8_ms": ms4, "w8a8_ms": ms8, "w4a8_speedup": ms8 / ms4,
        "w8a8_achieved": (n * k + act_bytes) / (ms8 * 1e-3) / 1e9, "unit": "GB/s"}
    del sets8

    for block in (32, 128):
        a_q, a_s = w4a8.quantize_act_blockwise(a, block)
        ms = time_graph(torch, lambda r, st: w4a8.w4a8_gemm_blockact(
            a_q, a_s, *sets4[r], n, block, out=out, stream=st), len(sets4), 4)
        byt = n * k // 2 + n * (k // 64) + 4 * n + m * k + 4 * m * (k // block) + m * n * 2
        res[f"blockact{block}_decode"] = {"shape": [m, n, k], "kernel_ms": ms,
                                          "achieved": byt / (ms * 1e-3) / 1e9, "unit": "GB/s",
                                          "frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                          "per_token_ms": ms4}
    del sets4

    # ---- prefill shape: W8A8 vs W4A8 (compute-bound) and per-block scales
    a_bits, w_bits, spec = inputs.workload_inputs("prefill", seed=0)
    m, n, k = spec["m"], spec["n"], spec["k"]
    a = bf16_dev(a_bits)
    w = bf16_dev(w_bits)
    a_q, a_s = w4a8.quantize_act_blockwise(a, k)
    a_s = a_s.reshape(-1)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ops = 2.0 * m * n * k
    w4p, g4, c4 = w4a8.pack_w4_grouped(w)
    c = n_copies(w4p.numel() + m * k)
    sets4 = [(w4p, g4, c4)] + [(w4p.clone(), g4.clone(), c4.clone()) for _ in range(c - 1)]
    ms4 = time_graph(torch, lambda r, st: w4a8.w4a8_gemm(
        a_q, a_s, *sets4[r], n, out=out, stream=st), c, 2)
    w8p, c8 = w4a8.pack_w8_channel(w)
    c8n = n_copies(w8p.numel() + m * k)
    sets8 = [(w8p, c8)] + [(w8p.clone(), c8.clone()) for _ in range(c8n - 1)]
    ms8 = time_graph(torch, lambda r, st: w4a8.w8a8_gemm(
        a_q, a_s, *sets8[r], n, out=out, stream=st), c8n, 2)
    del sets8
    res["w8a8_vs_w4a8_prefill"] = {
        "shape": [m, n, k], "w4a8_ms": ms4, "w8a8_ms": ms8, "w4a8_speedup": ms8 / ms4,
        "w4a8_achieved": ops / (ms4 * 1e-3) / 1e12, "w8a8_achieved": ops / (ms8 * 1e-3) / 1e12,
        "unit": "TFLOP/s", "peak": INT8_PEAK_TOPS}
    a_qb, a_sb = w4a8.quantize_act_blockwise(a, 128)
    ms = time_graph(torch, lambda r, st: w4a8.w4a8_gemm_blockact(
        a_qb, a_sb, *sets4[r], n, 128, out=out, stream=st), c, 2)
    res["blockact128_prefill"] = {"shape": [m, n, k], "kernel_ms": ms,
                                  "achieved": ops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                                  "frac": ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                                  "per_token_ms": ms4}
    del sets4, a, w

    # ---- the regime claim where the weights dominate: 70B FFN-down weights
    # (8192 x 28672), fused per-token activations, M = 1 and M = 16
    n, k = 8192, 28672
    wf = ffn_w_bits if ffn_w_bits is not None else inputs.weights(n, k, 0)
    w = bf16_dev(wf)
    w4p, g4, c4 = w4a8.pack_w4_grouped(w)
    c4n = n_copies(w4p.numel() + g4.numel())
    sets4 = [(w4p, g4, c4)] + [(w4p.clone(), g4.clone(), c4.clone()) for _ in range(c4n - 1)]
    w8p, c8 = w4a8.pack_w8_channel(w)
    del w
    c8n = n_copies(w8p.numel())
    sets8 = [(w8p, c8)] + [(w8p.clone(), c8.clone()) for _ in range(c8n - 1)]
    for m in (1, 16):
        a = bf16_dev(inputs.activations(m, k, 0, "student_t"))
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(w4a8.workspace_bytes(m, k, n), dtype=torch.uint8, device=dev)
        ms4 = time_graph(torch, lambda r, st: w4a8.w4a8_gemm_bf16act(
            a, *sets4[r], n, out=out, workspace=ws, stream=st), c4n, 10)
        ms8 = time_graph(torch, lambda r, st: w4a8.w8a8_gemm_bf16act(
            a, *sets8[r], n, out=out, workspace=ws, stream=st), c8n, 10)
        act_bytes = 2 * m * k + m * n * 2 + 4 * n
        b4 = n * k // 2 + n * (k // 64) + act_bytes
        b8 = n * k + act_bytes
        res[f"w8a8_vs_w4a8_ffn_down_m{m}"] = {
            "shape": [m, n, k], "w4a8_ms": ms4, "w8a8_ms": ms8, "w4a8_speedup": ms8 / ms4,
            "w4a8_achieved": b4 / (ms4 * 1e-3) / 1e9, "w8a8_achieved": b8 / (ms8 * 1e-3) / 1e9,
            "unit": "GB/s", "peak": HBM_PEAK_GBPS}
        del a, out, ws
    del sets4, sets8, w4p, g4, c4, w8p, c8
    torch.cuda.empty_cache()

    # ---- EQuARX receive step on the quantizer's 64M elements
    qspec = inputs.QUANTIZER
    rows, cols = qspec["rows"], qspec["cols"]
    xs = [bf16_dev(inputs.activations(rows, cols, seed=s)) for s in (1, 2)]
    for block in (32, 128):
        qi, si = w4a8.quantize_act_blockwise(bf16_dev(inputs.activations(rows, cols, seed=3)),
                                             block)
        qo = [torch.empty_like(qi) for _ in range(2)]
        so = [torch.empty_like(si) for _ in range(2)]
        qis = [qi, qi.clone()]
        sis = [si, si.clone()]
        ms = time_graph(torch, lambda r, st: w4a8.dequant_add_requant(
            qis[r], sis[r], xs[r], block, q_out=qo[r], s_out=so[r], stream=st), 2, 10)
        elems = rows * cols
        byt = elems * (1 + 2 + 1) + 2 * 4 * (elems // block)
        res[f"equarx_step_block{block}"] = {
            "elements": elems, "kernel_ms": ms, "achieved": byt / (ms * 1e-3) / 1e9,
            "unit": "GB/s", "frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    return res


if __name__ == "__main__":
    main()
