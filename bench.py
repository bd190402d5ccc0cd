#!/usr/bin/env python3
"""Benchmark of the block-scaled cast hot path on one MI355X.

Default workload: the MXFP8 cast of a 16384 x 16384 bf16 tensor (log-uniform
row magnitudes), row-wise (dim0) and column-wise (dim1, transposed output) in
one pass, block size 32 -- one step is one mx_quantize call over the whole
tensor, inputs resident in HBM.  The metric follows the torchao "Multiply
with inverse scale" page ("Performance" section): GB/s = algorithmic bytes
read + written / kernel time, where the bytes are 2 per input element plus,
per direction, 1 per E4M3 element and 1 per 32-element E8M0 scale.

Prints ONE JSON line.  `--config` times one of the other workloads instead;
`--copy` runs the plain device copy used to calibrate the HBM byte counters.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s

# What the metric kernel is built from: its translation unit, the headers it
# includes, and the host code that picks its launch shape.  The stored HBM
# traffic is valid only while their hash matches the one it was taken with.
KERNEL_SOURCES = ["block_scaled_precision_bf16_amd/csrc/mx_cast_fmt_e4m3.hip",
                  "block_scaled_precision_bf16_amd/csrc/mx_cast.h",
                  "block_scaled_precision_bf16_amd/csrc/stage_flush.h",
                  "block_scaled_precision_bf16_amd/csrc/rag_flush.h",
                  "block_scaled_precision_bf16_amd/csrc/device_math.h",
                  "block_scaled_precision_bf16_amd/csrc/launch.h",
                  "block_scaled_precision_bf16_amd/csrc/bufio.h",
                  "block_scaled_precision_bf16_amd/csrc/api.cpp"]
TRAFFIC_FILE = os.path.join(HERE, "profiles", "counters_mxfp8_dim0_dim1_16384.md")


def mx_bytes(M, K, directions, extra_inputs=0):
    """Algorithmic bytes of an MXFP8 cast: 2 B per bf16 input element (per
    input tensor), 1 B per E4M3 element and 1 B per E8M0 scale (one per block
    of up to 32 elements of a line) for each output direction (directions 2:
    row-wise and transposed, 1: transposed only)."""
    n = M * K
    row, col = n + M * -(-K // 32), n + K * -(-M // 32)
    return 2 * n * (1 + extra_inputs) + (row + col if directions == 2 else col)


def nvfp4_bytes(M, K, directions):
    """2 B per bf16 input, 1/2 B per E2M1 element (a line of n codes in
    ceil(n/2) bytes) and 1 B per E4M3 scale (one per block of up to 16
    elements of a line) for each direction (directions 2: row-wise and
    transposed, 1: transposed only; the absmax pre-pass is timed
    separately)."""
    row = M * (-(-K // 2) + -(-K // 16))
    col = K * (-(-M // 2) + -(-M // 16))
    return 2 * M * K + (row + col if directions == 2 else col)


CONFIGS = {
    # name: (workload generator key, shape, kind, bytes)
    "mxfp8_dim0_dim1_16384": ("c2_dim1_16384", (16384, 16384), "mx", 3),
    "mxfp8_dim1_16384": ("c2_dim1_16384", (16384, 16384), "mx", 2),
    "mxfp8_gelu_dbias_8192": ("c3_gelu_dbias_8192", (8192, 8192), "mx_gelu", 3),
    "mxfp8_dgelu_dbias_8192": ("c3_gelu_dbias_8192", (8192, 8192), "mx_dgelu", 3),
    "mxfp8_swiglu_8192": ("c4_gated_8192", (8192, 8192), "gated_swiglu", 3),
    "mxfp8_geglu_8192": ("c4_gated_8192", (8192, 8192), "gated_geglu", 3),
    "nvfp4_16384": ("c5_nvfp4_16384", (16384, 16384), "nvfp4", 3),
    "nvfp4_2d_16384": ("c5_nvfp4_16384", (16384, 16384), "nvfp4_2d", 3),
    "mxfp8_dsilu_dbias_8192": ("f1_dsilu_dbias_8192", (8192, 8192), "mx_dsilu", 3),
    "mxfp8_dswiglu_8192": ("f1_dgated_8192", (8192, 4096), "dgated_swiglu", 3),
    "mxfp8_dgeglu_8192": ("f1_dgated_8192", (8192, 4096), "dgated_geglu", 3),
    "mxfp8_e5m2_dim0_dim1_16384": ("c2_dim1_16384", (16384, 16384), "mx", 3),
    "mxfp8_e4m3_roundup_dim0_dim1_16384": ("c2_dim1_16384", (16384, 16384), "mx", 3),
    "mxfp8_e5m2_roundup_dim0_dim1_16384": ("c2_dim1_16384", (16384, 16384), "mx", 3),
    "mxfp8_tiled_dim0_dim1_16384": ("c2_dim1_16384", (16384, 16384), "mx", 3),
    "mxfp8_grouped_8x_16384x7168": ("f4_grouped_moe", (16384, 7168), "mx_grouped", 3),
    "nvfp4_grouped_8x_16384x7168": ("f4_grouped_moe", (16384, 7168), "nvfp4_grouped", 3),
    "mxfp8_grouped_swiglu_8x_16384x4096": ("f4_grouped_moe", (16384, 4096), "mx_grouped_swiglu", 3),
    # the any-shape kernels: rows and row lengths that are not multiples of 16 and 8
    "mxfp8_dim0_dim1_16383": ("c2_dim1_16384", (16383, 16383), "mx", 3),
    "nvfp4_16383": ("c5_nvfp4_16384", (16383, 16383), "nvfp4", 3),
    # rows that are not multiples of 16, row lengths that are multiples of 8
    # (MXFP8) or 16 (NVFP4): the tiled kernels, transposed rows at any byte
    "mxfp8_dim0_dim1_16383x16384": ("c2_dim1_16384", (16383, 16384), "mx", 3),
    "mxfp8_grouped_ragged_8x_16384x7168": ("f4_grouped_moe", (16384, 7168), "mx_grouped", 3),
    "nvfp4_grouped_ragged_8x_16384x7168": ("f4_grouped_moe", (16384, 7168), "nvfp4_grouped", 3),
    "nvfp4_16383x16384": ("c5_nvfp4_16384", (16383, 16384), "nvfp4", 3),
}

# Row counts of the 8 experts in the grouped workloads: shares of a seeded
# Dirichlet draw, rounded down to multiples of 16 -- or, for the ragged
# workloads, not rounded (the token counts of a real MoE layer).
MOE_GROUPS = dict(groups=8, seed=8)
MOE_RAGGED = ("mxfp8_grouped_ragged_8x_16384x7168", "nvfp4_grouped_ragged_8x_16384x7168")


def group_rows(config, M):
    import workloads as W
    return W.moe_group_rows(M, **MOE_GROUPS, step=1 if config in MOE_RAGGED else 16)

# MXFP8 flags OR-ed into the axis mask (E5M2 elements = 4, round-up E8M0
# rule = 8, GEMM-ready tiled scales = 16), and the format each plain MXFP8
# workload names.
FORMAT_FLAGS = {"mxfp8_e5m2_dim0_dim1_16384": 4, "mxfp8_e4m3_roundup_dim0_dim1_16384": 8,
                "mxfp8_e5m2_roundup_dim0_dim1_16384": 12, "mxfp8_tiled_dim0_dim1_16384": 16}
FORMAT_NAMES = {0: "mxfp8 e4m3 + e8m0", 4: "mxfp8 e5m2 + e8m0",
                8: "mxfp8 e4m3 + e8m0 (round-up rule)", 12: "mxfp8 e5m2 + e8m0 (round-up rule)",
                16: "mxfp8 e4m3 + e8m0 in MFMA scale tiles"}


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(HERE, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != kernel_source_hash():
        return None
    return int(m.group(1))


def gpu_us_per_call(fn, stream, calls=4):
    """Mean GPU time of `calls` back-to-back calls of fn (microseconds)."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(calls):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    return max(s.elapsed_time(e) * 1e3 / calls, 1.0)


def lead_calls(us_per_call, timed, at_least):
    """Untimed calls to queue right before `timed` timed calls: at least
    50 ms of GPU work (host stalls of about 33 ms have been seen while the
    timed calls were being queued), and 100 us per timed call (more than the
    host needs to queue one), so the host stays ahead of the GPU throughout."""
    return max(at_least, int(max(50000.0, 100.0 * timed) / us_per_call) + 1)


def run_environment(dev):
    """What the numbers were measured on: host, GPU, ROCm / HIP version, and
    the md5 of the loaded libmxcast.so."""
    import socket
    import torch
    import block_scaled_precision_bf16_amd as mx
    with open(mx.LIB_PATH, "rb") as f:
        lib_md5 = hashlib.md5(f.read()).hexdigest()
    props = torch.cuda.get_device_properties(dev)
    return {"host": socket.gethostname(), "gpu": torch.cuda.get_device_name(dev),
            "arch": getattr(props, "gcnArchName", None), "hip": torch.version.hip,
            "torch": torch.__version__, "libmxcast_md5": lib_md5}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="mxfp8_dim0_dim1_16384", choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy", action="store_true", help="run the byte-counter calibration copy")
    ap.add_argument("--prewarm-ms", type=float, default=100.0,
                    help="untimed steps for at least this much GPU time before the warm-up "
                         "steps (the GPU leaves its idle clocks over ~10 ms of work)")
    ap.add_argument("--cold", type=int, default=20, help="cold-cache samples (0: none)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the cast shards by rows with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_precision_bf16_amd as mx
    import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy:
        n = 512 * 1024 * 1024
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    key, (M, K), kind, dirs = CONFIGS[args.config]
    pre_pass = None   # NVFP4: the tensor absmax pass, timed on its own
    print(f"[bench] generating {args.config} inputs {M}x{K}", file=sys.stderr, flush=True)
    inputs = W.make(key, M, K)
    if kind in ("mx_gelu", "mx_dgelu", "mx_dsilu"):
        x_h, g_h = inputs
    elif kind.startswith("dgated"):
        g_h, x_h = inputs
    else:
        x_h, g_h = inputs, None
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    x = to_dev(x_h)
    grad = to_dev(g_h) if g_h is not None else None

    # outputs and workspace allocated once, outside the timed region
    if kind == "mx_grouped":
        grp_rows = group_rows(args.config, M)
        out = mx.mx_quantize_grouped(x, grp_rows)
        step = lambda: mx.mx_quantize_grouped(x, grp_rows, out=out)
        nbk = -(-K // 32)
        alg_bytes = 2 * M * K + (M * K + M * nbk) + (M * K + sum(K * -(-m // 32) for m in grp_rows))
        desc = dict(workload=args.config, M=M, K=K, groups=grp_rows, block=32,
                    directions="row+col per group", format="mxfp8 e4m3 + e8m0")
    elif kind == "mx_grouped_swiglu":
        # an MoE layer's expert FFN input [gate | linear] (N = K / 2 per half)
        grp_rows = group_rows(args.config, M)
        out = mx.mx_quantize_gated_grouped(x, grp_rows, mx.GATED_SWIGLU)
        step = lambda: mx.mx_quantize_gated_grouped(x, grp_rows, mx.GATED_SWIGLU, out=out)
        N = K // 2
        nbn = -(-N // 32)
        alg_bytes = 2 * M * K + (M * N + M * nbn) + (M * N + sum(N * -(-m // 32) for m in grp_rows))
        desc = dict(workload=args.config, M=M, K=K, N=N, groups=grp_rows, block=32,
                    directions="row+col per group", format="mxfp8 e4m3 + e8m0",
                    activation="swiglu")
    elif kind == "nvfp4_grouped":
        grp_rows = group_rows(args.config, M)
        amax = mx.mx_absmax_bf16_grouped(x, grp_rows)
        pre_pass = ("absmax (per group)", lambda: mx.mx_absmax_bf16_grouped(x, grp_rows, out=amax),
                    2 * M * K)
        out = mx.nvfp4_quantize_transpose_grouped(x, grp_rows, amax)
        step = lambda: mx.nvfp4_quantize_transpose_grouped(x, grp_rows, amax, out=out)
        # each group's transpose: [K][ceil(m/2)] codes, [K][ceil(m/16)] scales
        alg_bytes = nvfp4_bytes(M, K, 2) - K * (-(-M // 2) + -(-M // 16)) + \
            K * sum(-(-m // 2) + -(-m // 16) for m in grp_rows)
        desc = dict(workload=args.config, M=M, K=K, groups=grp_rows, block=16,
                    directions="row+transpose per group",
                    format="nvfp4 (e2m1 + e4m3 scales + fp32 scale per group)")
    elif kind.startswith("nvfp4"):
        two_d = kind == "nvfp4_2d"
        amax = mx.mx_absmax_bf16(x)
        pre_pass = ("absmax", lambda: mx.mx_absmax_bf16(x, out=amax), 2 * M * K)
        out = mx.nvfp4_quantize_transpose(x, amax, two_d=two_d)
        step = lambda: mx.nvfp4_quantize_transpose(x, amax, out=out, two_d=two_d)
        alg_bytes = nvfp4_bytes(M, K, 2)
        desc = dict(workload=args.config, M=M, K=K, block="16x16" if two_d else 16,
                    directions="row+transpose",
                    format="nvfp4 (e2m1 + e4m3 scales + fp32 tensor scale)")
    elif kind.startswith("dgated"):
        act = mx.GATED_SWIGLU if kind.endswith("swiglu") else mx.GATED_GEGLU
        out = mx.mx_quantize_dgated(grad, x, act)
        step = lambda: mx.mx_quantize_dgated(grad, x, act, out=out)
        N = K
        alg_bytes = 2 * M * N + 4 * M * N + 2 * (2 * M * N + 2 * M * N // 32)
        desc = dict(workload=args.config, M=M, N=N, block=32, directions="row+col",
                    format="mxfp8 e4m3 + e8m0", activation="d" + kind.split("_")[1],
                    output="[d_gate | d_linear] M x 2N")
    elif kind.startswith("gated"):
        act = mx.GATED_SWIGLU if kind.endswith("swiglu") else mx.GATED_GEGLU
        out = mx.mx_quantize_gated(x, act)
        step = lambda: mx.mx_quantize_gated(x, act, out=out)
        N = K // 2
        alg_bytes = 2 * M * K + 2 * (M * N + M * N // 32)
        desc = dict(workload=args.config, M=M, K=K, N=N, block=32, directions="row+col",
                    format="mxfp8 e4m3 + e8m0", activation=kind.split("_")[1])
    else:
        axis = (mx.COLWISE if dirs == 2 else mx.ROWWISE | mx.COLWISE) | FORMAT_FLAGS.get(args.config, 0)
        fusion = {"mx": mx.FUSE_NONE, "mx_gelu": mx.FUSE_GELU | mx.FUSE_DBIAS,
                  "mx_dgelu": mx.FUSE_DGELU | mx.FUSE_DBIAS,
                  "mx_dsilu": mx.FUSE_DSILU | mx.FUSE_DBIAS}[kind]
        ws = torch.empty(max(16, mx.mx_quantize_workspace_size(M, K, axis, fusion)),
                         dtype=torch.uint8, device=dev)
        out = mx.mx_quantize(x, grad, axis=axis, fusion=fusion, workspace=ws)
        step = lambda: mx.mx_quantize(x, grad, axis=axis, fusion=fusion, out=out, workspace=ws)
        ndir = 1 if dirs == 2 else 2
        alg_bytes = mx_bytes(M, K, ndir, extra_inputs=1 if kind in ("mx_dgelu", "mx_dsilu") else 0)
        if fusion & mx.FUSE_DBIAS:
            alg_bytes += 4 * K
        desc = dict(workload=args.config, M=M, K=K, block=32,
                    directions="col" if ndir == 1 else "row+col",
                    format=FORMAT_NAMES[FORMAT_FLAGS.get(args.config, 0)],
                    fusion={"mx": "none", "mx_gelu": "gelu+dbias", "mx_dgelu": "dgelu+dbias",
                            "mx_dsilu": "dsilu+dbias"}[kind])

    stream = torch.cuda.current_stream(dev)
    # Bring the GPU to its working clocks first: from idle, the first ~50
    # launches of the 16384^2 cast run ~5% slower while the clocks ramp (a
    # per-launch trace shows 200 us on average for launches 1-50, 188 us from
    # launch 50 on), which is power management, not the kernel.  Untimed.
    prewarm = 0
    if args.prewarm_ms > 0:
        t_end = time.perf_counter() + args.prewarm_ms / 1e3
        while time.perf_counter() < t_end or prewarm < 8:
            for _ in range(8):
                step()
            prewarm += 8
            torch.cuda.synchronize()
    step_us = gpu_us_per_call(step, stream)

    # The timed launches follow, with no pause, a run of untimed launches of
    # the same step (the warm-up) long enough for the host to queue all of
    # them first: the GPU stays busy at its working clocks and no host-side
    # pause (the binding's argument checks, the interpreter) lands between a
    # launch's two events.
    lead = lead_calls(step_us, args.steps, args.warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for _ in range(lead):
        step()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    # the K steps on the GPU's clock: first launch's start to last launch's end
    span_ms = starts[0].elapsed_time(ends[-1])
    per = sorted(s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends))   # us per launch
    mean_us = sum(per) / len(per)
    median_us = per[len(per) // 2]
    gbs = alg_bytes / (mean_us * 1e3)

    # Cold caches: before each sample, 1 GiB is written (every line the
    # previous call left in L2 or the 256 MB MALL is evicted) and then a second
    # 1 GiB buffer is read, so that the fill's own dirty lines are written back
    # before the timed call rather than inside it.  Both outside the events.
    cold = []
    if args.cold > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        sweep = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        for _ in range(args.cold):
            flush.fill_(0)
            _ = torch.amax(sweep)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            step()
            e.record(stream)
            torch.cuda.synchronize()
            cold.append(s.elapsed_time(e) * 1e3)
        del flush, sweep
    cold.sort()

    def pct(v, q):
        return round(v[min(len(v) - 1, int(q * len(v)))], 2) if v else None

    pre_stats = None
    if pre_pass is not None:
        # the absmax pre-pass of the NVFP4 casts: a pure read of the input,
        # timed like the cast (back to back, events per launch)
        name, fn, nbytes = pre_pass
        n_pre = max(20, args.steps)
        pre_lead = lead_calls(gpu_us_per_call(fn, stream, 8), n_pre, 5)
        ps = [torch.cuda.Event(enable_timing=True) for _ in range(n_pre)]
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(n_pre)]
        torch.cuda.synchronize()
        for _ in range(pre_lead):
            fn()
        for i in range(n_pre):
            ps[i].record(stream)
            fn()
            pe[i].record(stream)
        torch.cuda.synchronize()
        pt = sorted(a.elapsed_time(b) * 1e3 for a, b in zip(ps, pe))
        pm = sum(pt) / len(pt)
        pre_stats = {"pass": name, "launches": n_pre, "us_mean": round(pm, 2),
                     "us_median": round(pt[len(pt) // 2], 2), "bytes": nbytes,
                     "GB/s": round(nbytes / (pm * 1e3), 1),
                     "frac": round(nbytes / (pm * 1e3) / HBM_PEAK_GBS, 4)}

    traffic = measured_traffic() if args.config == "mxfp8_dim0_dim1_16384" else None
    result = {
        "metric": "MXFP8 cast GB/s (bytes rd+wr / kernel \u00b5s) and % HBM peak at 16384\u00b2 bf16",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(span_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": desc,
        "us_per_launch": {"mean": round(mean_us, 2), "median": round(median_us, 2),
                          "p10": pct(per, 0.1), "p90": pct(per, 0.9),
                          "cold_mean": round(sum(cold) / len(cold), 2) if cold else None,
                          "cold_median": pct(cold, 0.5), "cold_p10": pct(cold, 0.1),
                          "cold_p90": pct(cold, 0.9), "cold_samples": len(cold)},
        "timing": {"warm": "back-to-back launches right after untimed launches of the same step that keep the GPU busy while the host queues them, HIP events per launch on the cast's stream",
                   "cold": "1 GiB write then 1 GiB read of other buffers before each sample",
                   "prewarm_launches": prewarm, "lead_launches": lead},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "algorithmic_bytes": alg_bytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernel_source_sha256": kernel_source_hash(),
        "env": run_environment(dev),
    }

    if pre_stats is not None:
        result["pre_pass"] = pre_stats
    if not args.no_cpu:
        import oracle as O
        cores = min(16, len(os.sched_getaffinity(0)))
        O.set_threads(cores)
        # the whole workload: about 1 s on 16 host threads for the 16384^2 cast
        rows = M
        xs = np.ascontiguousarray(x_h[:rows])
        print(f"[bench] oracle CPU baseline on {rows}x{K}, {cores} threads",
              file=sys.stderr, flush=True)
        c0 = time.process_time()
        t0 = time.perf_counter()
        if kind == "mx_grouped":
            O.mx_quantize_grouped(xs, group_rows(args.config, M))
            sb = alg_bytes
        elif kind == "nvfp4_grouped":
            O.nvfp4_quantize_transpose_grouped(xs, group_rows(args.config, M))
            sb = alg_bytes
        elif kind == "mx_grouped_swiglu":
            O.mx_quantize_gated_grouped(xs, group_rows(args.config, M), mx.GATED_SWIGLU)
            sb = alg_bytes
        elif kind.startswith("nvfp4"):
            O.nvfp4_quantize_transpose(xs, tensor_amax=O.absmax(x_h), two_d=kind == "nvfp4_2d")
            sb = nvfp4_bytes(rows, K, 2)
        elif kind.startswith("dgated"):
            O.mx_quantize_dgated(np.ascontiguousarray(g_h[:rows]), xs,
                                 mx.GATED_SWIGLU if kind.endswith("swiglu") else mx.GATED_GEGLU)
            sb = 6 * rows * K + 2 * (2 * rows * K + 2 * rows * K // 32)
        elif kind.startswith("gated"):
            O.mx_quantize_gated(xs, mx.GATED_SWIGLU if kind.endswith("swiglu") else mx.GATED_GEGLU)
            sb = 2 * rows * K + 2 * (rows * (K // 2) + rows * (K // 2) // 32)
        else:
            gs = np.ascontiguousarray(g_h[:rows]) if g_h is not None else None
            O.mx_quantize(xs, grad=gs, axis=axis, fusion=fusion)
            sb = mx_bytes(rows, K, ndir, extra_inputs=1 if kind in ("mx_dgelu", "mx_dsilu") else 0)
        dt = time.perf_counter() - t0
        cpu_s = time.process_time() - c0
        result["cpu_baseline"] = {"value": round(sb / (dt * 1e9), 3), "unit": "GB/s",
                                  "cores": cores, "kind": "oracle",
                                  "sample": f"the whole {M}x{K} workload, same recipe and seed",
                                  "seconds": round(dt, 3), "cpu_seconds": round(cpu_s, 1),
                                  "cpu": cpu_model()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
