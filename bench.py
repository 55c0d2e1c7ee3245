"""Throughput of the fused fp16 GEMM + epilogue on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload x_acc_8192]
                    [--no-cpu-baseline] [--no-configs] [--all] [--compare-unfused]

A step is one call of the fused kernel (one gemm_epi_run_ext) on the workload,
with every input already resident in HBM.  The timed region is K steps on one
stream, bracketed by torch.cuda.synchronize(); HIP events recorded on that
same stream give the average launch duration that the roofline uses.
Prints ONE JSON line (the headline workload).  Unless --no-configs (or
--workload) is given, the line's "configs" entry also reports the other four
configurations (128^3, 1024^3, 2400 x 3232 x 4096, the 16-batch case), each
timed the same way just before the headline: kernel us, TFLOP/s, roofline
and the epilogue's HBM GB/s.  --all also reports every other workload, one
JSON line each on stderr.

The CPU baseline is the oracle as it stands (plain fp64 triple loop),
timed on a bounded slice of the same workload on this host's cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6  # MI355X dense fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# workloads that --all also times with fp32 and bfloat16 epilogue tensors
EPI_TYPE_WORKLOADS = ("x_acc_8192", "relu_square_16x2048x2048x1024")
KERNEL_SOURCES = ("dense_gemm_elementwise_amd/csrc/gemm_epi_kernels.hpp", "dense_gemm_elementwise_amd/csrc/gemm_epi.hip",
                  "dense_gemm_elementwise_amd/csrc/gemm_epi_launch.hpp", "dense_gemm_elementwise_amd/csrc/gemm_epi_bf16.hip")


def kernel_source_hash():
    """sha256 of the kernel sources with comments and blank lines removed, so
    that a change of wording does not invalidate counters taken on the same
    code."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes")


def _device_args(w, t, D, Aux, Acc, stream, ge):
    """Arguments of gemm_epi_run_ext for workload w on device tensors t."""
    def ptr(x):
        return x.data_ptr() if x is not None else None
    return (w.L, w.M, w.N, w.K, ptr(t["A"]), ptr(t["B"]), ptr(t["C"]), ptr(t["X"]), ptr(t["row_bias"]),
            ptr(t["col_bias"]), (w.alpha, w.beta, w.s3), ge.KINDS[w.kind], ptr(D), ptr(Aux), ptr(Acc),
            stream.cuda_stream)


def _upload(p, w, dev):
    """Host inputs of workload w as device tensors (bfloat16 workloads hold
    uint16 bit patterns on the host)."""
    import torch

    def one(v):
        if v is None:
            return None
        if w.dtype == "bf16":
            return torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(v).to(dev)
    return {k: one(v) for k, v in p.items()}


def _launcher(w, ge, args):
    """The call of workload w with arguments `args` (those of gemm_epi_run_ext),
    converted to ctypes once: gemm_epi_run_ext, or gemm_epi_run_typed with
    the workload's element type.  Host cost per call on MI355X: about 3.8 us
    against 4.4 us converting the arguments on every call, and 3.4 us for any
    HIP launch API from C++; it bounds the launch rate of the smallest
    workloads."""
    if w.dtype == "f16":
        return ge.prepared("gemm_epi_run_ext", *args)
    return ge.prepared("gemm_epi_run_typed", *args[:-1], ge.DTYPES[w.dtype], args[-1])


def _outputs(w, ge, dev):
    import torch
    D = torch.empty((w.L, w.M, w.N), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float16, device=dev)
    Aux = torch.empty_like(D) if w.kind in ge.HAS_AUX else None
    Acc = torch.empty((w.L, w.M, w.N), dtype=torch.float32, device=dev) if w.kind in ge.HAS_ACC else None
    return D, Aux, Acc


def _plan(args, ge):
    return ge.gemm_epi_plan_ext(*args[:10], args[11], args[12], args[13], args[14])


def _timed_launches(launch, steps, stream):
    """Times `steps` launches between two synchronisations: one HIP event on
    the launch stream before the first launch and one after the last give
    the average launch duration (what the roofline uses), and the wall clock
    covers the whole timed region.  The median and minimum of single
    launches come from a second pass of `steps` launches with an event
    before each, after the timed region, so that those events (a few us per
    launch on short kernels) stay out of it.  launch(i) is called with
    i = 0 .. 2*steps - 1 across the two passes."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = e0.elapsed_time(e1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(stream)
        launch(steps + i)
    ev[steps].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return wall * 1e3 / steps, total / steps, {"median": per[steps // 2], "min": per[0], "mean": total / steps}


def bench_gpu(w, steps, warmup):
    import torch
    import dense_gemm_elementwise_amd as ge
    from dense_gemm_elementwise_amd import workloads

    dev = torch.device("cuda:0")
    p = workloads.make_inputs(w)
    t = _upload(p, w, dev)
    D, Aux, Acc = _outputs(w, ge, dev)
    stream = torch.cuda.current_stream(dev)
    args = _device_args(w, t, D, Aux, Acc, stream, ge)
    run = _launcher(w, ge, args)
    for _ in range(warmup):
        rc = run()
        if rc:
            raise RuntimeError(ge.gemm_epi_status_string(rc))
    wall_ms, ev_ms, stats = _timed_launches(lambda i: run(), steps, stream)
    rc, plan = _plan(args, ge)
    return {"ms_per_step": wall_ms, "kernel_ms": ev_ms, "launch_ms": stats, "plan": plan}


def bench_gpu_stream_k(w, steps, warmup):
    """The same workload through gemm_epi_run_ws_typed, which splits K across
    workgroups (stream-K) when the problem has too few tiles; None when no
    split is planned for it."""
    import torch
    import dense_gemm_elementwise_amd as ge
    from dense_gemm_elementwise_amd import workloads

    dev = torch.device("cuda:0")
    p = workloads.make_inputs(w)
    t = _upload(p, w, dev)
    dt = ge.DTYPES[w.dtype]
    D, Aux, Acc = _outputs(w, ge, dev)
    stream = torch.cuda.current_stream(dev)
    args = _device_args(w, t, D, Aux, Acc, stream, ge)
    rc, plan = ge.gemm_epi_plan_ws(*args[:10], args[11], args[12], args[13], args[14])
    if rc or plan["workspace_bytes"] == 0:
        return None
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    wargs = args[:15] + (ws.data_ptr(), plan["workspace_bytes"], dt, args[15])
    for _ in range(warmup):
        rc = ge.gemm_epi_run_ws_typed(*wargs)
        if rc:
            raise RuntimeError(ge.gemm_epi_status_string(rc))
    _, ev_ms, stats = _timed_launches(lambda i: ge.gemm_epi_run_ws_typed(*wargs), steps, stream)
    return {"tile": [plan["bm"], plan["bn"], plan["bk"]], "workgroups": plan["workgroups"],
            "workspace_bytes": plan["workspace_bytes"], "kernel_ms": round(ev_ms, 5),
            "launch_ms": {k: round(v, 5) for k, v in stats.items()},
            "tflops": round(w.flops / (ev_ms * 1e-3) / 1e12, 2), "roofline": roofline(w, ev_ms)}


def bench_gpu_epi_types(w, steps, warmup):
    """Context: the same fp16 workload with its epilogue tensors (C, X, the
    biases, D, Aux) in fp32 and in bfloat16 instead (gemm_epi_run_mixed): the
    workload's C and X converted on the device (exactly to fp32, rounded to
    bfloat16).  Launch times and TFLOP/s per epilogue type."""
    import torch
    import dense_gemm_elementwise_amd as ge
    from dense_gemm_elementwise_amd import workloads

    if w.dtype != "f16":
        return None
    dev = torch.device("cuda:0")
    t16 = _upload(workloads.make_inputs(w), w, dev)
    out = {}
    for name, tt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        t = {k: (v.to(tt) if (v is not None and k not in ("A", "B")) else v) for k, v in t16.items()}
        D = torch.empty((w.L, w.M, w.N), dtype=tt, device=dev)
        Aux = torch.empty_like(D) if w.kind in ge.HAS_AUX else None
        Acc = torch.empty((w.L, w.M, w.N), dtype=torch.float32, device=dev) if w.kind in ge.HAS_ACC else None
        stream = torch.cuda.current_stream(dev)
        args = _device_args(w, t, D, Aux, Acc, stream, ge)
        margs = args[:15] + (ge.DTYPES["f16"], ge.DTYPES[name], args[15])
        for _ in range(warmup):
            rc = ge.gemm_epi_run_mixed(*margs)
            if rc:
                raise RuntimeError(ge.gemm_epi_status_string(rc))
        _, ev_ms, stats = _timed_launches(lambda i: ge.gemm_epi_run_mixed(*margs), steps, stream)
        out[name] = {"kernel_ms": round(ev_ms, 5), "tflops": round(w.flops / (ev_ms * 1e-3) / 1e12, 2)}
    return out


MALL_BYTES = 256 << 20  # MI355X Infinity Cache


def bench_gpu_cold(w, steps, warmup):
    """The same launches with every step on its own copy of the inputs and
    outputs, rotating through enough copies (more than twice the 256 MB
    MALL) that no step finds its operands in a cache."""
    import torch
    import dense_gemm_elementwise_amd as ge
    from dense_gemm_elementwise_amd import workloads

    dev = torch.device("cuda:0")
    p = workloads.make_inputs(w)
    base = _upload(p, w, dev)
    sets = min(4096, -(-2 * MALL_BYTES // w.hbm_bytes) + 1)
    copies = []
    for _ in range(sets):
        t = {k: (v.clone() if v is not None else None) for k, v in base.items()}
        copies.append((t,) + _outputs(w, ge, dev))
    stream = torch.cuda.current_stream(dev)
    calls = [_launcher(w, ge, _device_args(w, t, D, Aux, Acc, stream, ge)) for (t, D, Aux, Acc) in copies]
    for i in range(warmup):
        calls[i % sets]()
    _, ev_ms, stats = _timed_launches(lambda i: calls[(i + warmup) % sets](), steps, stream)
    del copies
    return {"copies": sets, "kernel_ms": round(ev_ms, 5), "launch_ms": {k: round(v, 5) for k, v in stats.items()},
            "tflops": round(w.flops / (ev_ms * 1e-3) / 1e12, 2),
            "epilogue_hbm_gbs": round(w.epilogue_bytes / (ev_ms * 1e-3) / 1e9, 1)}


def bench_unfused_own(w, steps, warmup):
    """Context, not the metric: the same workload through this library's own
    unfused composition (gemm_epi_run_unfused_typed: the GEMM writes the fp32
    accumulator to HBM, a second launch applies the epilogue).  Same
    results as the fused kernel; the difference is the fusion's saving."""
    import torch
    import dense_gemm_elementwise_amd as ge
    from dense_gemm_elementwise_amd import workloads

    dev = torch.device("cuda:0")
    p = workloads.make_inputs(w)
    t = _upload(p, w, dev)
    dt = ge.DTYPES[w.dtype]
    D, Aux, Acc = _outputs(w, ge, dev)
    ws = torch.empty(w.L * w.M * w.N, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    args = _device_args(w, t, D, Aux, Acc, stream, ge)
    uargs = args[:15] + (ws.data_ptr(), ws.numel() * 4, dt, args[15])
    for _ in range(warmup):
        rc = ge.gemm_epi_run_unfused_typed(*uargs)
        if rc:
            raise RuntimeError(ge.gemm_epi_status_string(rc))
    _, ev_ms, stats = _timed_launches(lambda i: ge.gemm_epi_run_unfused_typed(*uargs), steps, stream)
    return {"what": "own GEMM kernel writing the fp32 accumulator + own elementwise epilogue kernel",
            "ms_per_step": round(ev_ms, 5), "tflops": round(w.flops / (ev_ms * 1e-3) / 1e12, 2)}


def bench_unfused_library(w, steps, warmup):
    """Context, not the metric: the same workload run unfused through the
    vendor library -- torch.matmul (hipBLASLt, fp16 output) followed by the
    epilogue as separate torch elementwise kernels -- on the same inputs.
    This is the three-kernel composition the fusion replaces; its
    intermediate Y = A @ B is rounded to the 16-bit element type before the
    epilogue."""
    import torch
    from dense_gemm_elementwise_amd import workloads

    dev = torch.device("cuda:0")
    p = workloads.make_inputs(w)
    t = _upload(p, w, dev)
    A, B, C, X = t["A"], t["B"], t["C"], t["X"]
    rb, cb = t["row_bias"], t["col_bias"]
    a, b, s3 = w.alpha, w.beta, w.s3

    def step():
        Y = torch.matmul(A, B)
        if w.kind == "BIAS_ROW_COL":
            return (a * Y + rb[None, None, :] + cb[None, :, None],)
        if w.kind == "RELU_AUX_STORE":
            f = a * Y + b * C
            return (torch.relu(f), f)
        if w.kind == "RELU_SCALE_ACC":
            f = torch.relu(a * Y + b * C)
            return (s3 * f, f, Y.float())
        if w.kind == "LINCOMB":
            return (a * Y + b * C,)
        if w.kind == "AUX_SCALE":
            aux = a * Y + b * C
            return (s3 * aux, aux)
        if w.kind == "LINCOMB_X_ACC":
            return (a * Y + b * C + s3 * X, Y)
        if w.kind == "RELU":
            return (torch.relu(a * Y + b * C),)
        d = a * Y + b * C
        if w.kind == "RELU_SQUARE":
            d = torch.relu(d)
        return (d, d * d)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the GEMM alone, for reference
    for _ in range(warmup):
        torch.matmul(A, B)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        torch.matmul(A, B)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_gemm = e0.elapsed_time(e1) / steps
    return {"what": "torch.matmul (hipBLASLt) + torch elementwise epilogue, unfused",
            "ms_per_step": round(ms, 5), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2),
            "gemm_only_ms": round(ms_gemm, 5), "gemm_only_tflops": round(w.flops / (ms_gemm * 1e-3) / 1e12, 2)}


def bench_cpu_oracle(w, rows):
    """The oracle on the first `rows` output rows of batch entry 0 (all N
    columns, full K): a bounded slice of the same workload."""
    import numpy as np
    import oracle
    from dense_gemm_elementwise_amd import workloads

    p = workloads.make_inputs(w)
    rows = min(rows, w.M)
    sl = {k: (np.ascontiguousarray(v[:1, :rows]) if (v is not None and k != "B") else v) for k, v in p.items()}
    sl["B"] = np.ascontiguousarray(p["B"][:1])
    t0 = time.perf_counter()
    oracle.gemm_epi(sl["A"], sl["B"], sl["C"], sl["X"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return flops / dt / 1e12, dt, rows


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def config_summary(w, steps, warmup):
    """One of the other report configurations, timed like the headline:
    mean launch, TFLOP/s, its roofline and the epilogue's HBM bytes per
    second (warm: the inputs were just used)."""
    g = bench_gpu(w, steps, warmup)
    ms = g["kernel_ms"]
    return {"kernel_us": round(ms * 1e3, 2), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2),
            "roofline": roofline(w, ms), "epilogue_gbs_warm": round(w.epilogue_bytes / (ms * 1e-3) / 1e9, 1),
            "tile": [g["plan"]["bm"], g["plan"]["bn"], g["plan"]["bk"]], "workgroups": g["plan"]["workgroups"],
            "shape": [w.L, w.M, w.N, w.K], "epilogue": w.kind}


def omp_threads():
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


def measured_mfma_busy(workload_name):
    """The share of SIMD cycles with the MFMA unit busy (rocprofv3's MfmaUtil)
    from the committed profile summary, if it was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha256") != kernel_source_hash() or "mfma_util_pct" not in rec:
        return None
    return round(rec["mfma_util_pct"] / 100.0, 4)


def roofline(w, kernel_ms):
    """The bound of this workload's kernel (the larger of its MFMA time and
    its algorithmic-bytes time at peak) and what the measured launch
    reaches against it."""
    t_mfma = w.flops / (PEAK_FP16_TFLOPS * 1e12)
    t_hbm = w.hbm_bytes / (PEAK_HBM_GBS * 1e9)
    t = kernel_ms * 1e-3
    if t_mfma >= t_hbm:
        achieved, peak, unit, bound = w.flops / t / 1e12, PEAK_FP16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = w.hbm_bytes / t / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name),
            "attainable_frac": round(max(t_mfma, t_hbm) / t, 4), "mfma_busy": measured_mfma_busy(w.name)}


def result_line(w, g, steps, warmup, cpu):
    tflops = w.flops / (g["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": "fused GEMM+epilogue TFLOP/s at 8192^3 fp16; % of fp16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "L": w.L, "M": w.M, "N": w.N, "K": w.K, "epilogue": w.kind,
            "alpha": w.alpha, "beta": w.beta, "s3": w.s3, "init": f"{w.init} seed {w.seed}",
            "accumulate": "f32", "tile": [g["plan"]["bm"], g["plan"]["bn"], g["plan"]["bk"]],
            "workgroups": g["plan"]["workgroups"], "parallelism": "single GPU",
        },
        "roofline": roofline(w, g["kernel_ms"]),
        "launch_ms": {k: round(v, 5) for k, v in g["launch_ms"].items()},
        "epilogue_hbm_gbs": round(w.epilogue_bytes / (g["kernel_ms"] * 1e-3) / 1e9, 1),
        "cpu_baseline": cpu,
    }
    return line


def copy_calibration(mib, steps):
    """A plain copy of known size: reading and writing mib MiB per launch.
    Profiling it gives the scale of the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda:0").to(torch.float16)
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        torch.neg(src, out=dst)  # one elementwise kernel: reads n halves, writes n halves
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "bytes_read": n * 2, "bytes_written": n * 2, "launches": steps}))


# Shapes off the fast path's 16-byte rule (LINCOMB, fp16, Gaussian inputs):
# (M, N, K, element offset of every tensor from a 256-byte boundary)
RAGGED_SHAPES = [(4096, 4096, 4095, 0), (4096, 4095, 4096, 0), (4096, 4100, 4096, 0), (4096, 4096, 4096, 1),
                 (1001, 1001, 1001, 0), (256, 256, 65535, 0)]


def bench_ragged(steps, warmup):
    """One JSON line per shape: the general kernel (gemm_epi_run_ext), the
    same call with its operands staged through a workspace so that the fast
    kernel runs (gemm_epi_run_ws_typed, the workspace gemm_epi_plan_ws
    reports), and torch.matmul (hipBLASLt) followed by torch.add; mean launch
    times from HIP events over `steps` calls after `warmup`."""
    import torch
    import dense_gemm_elementwise_amd as ge

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator().manual_seed(2025)

    def tensor(shape, off):
        n = 1
        for x in shape:
            n *= x
        return torch.randn(n + off, generator=g).half().to(dev)[off:].view(shape)

    for (M, N, K, off) in RAGGED_SHAPES:
        A, B, C, D = tensor((1, M, K), off), tensor((1, K, N), off), tensor((1, M, N), off), tensor((1, M, N), off)
        P = [t.data_ptr() for t in (A, B, C)]
        rc, plan = ge.gemm_epi_plan_ws(1, M, N, K, P[0], P[1], P[2], None, None, None, "LINCOMB", D.data_ptr(), None,
                                       None)
        if rc:
            raise RuntimeError(ge.gemm_epi_status_string(rc))
        ws = torch.zeros(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device=dev)
        args = (1, M, N, K, P[0], P[1], P[2], None, None, None, (1.0, 1.0, 0.0), "LINCOMB", D.data_ptr(), None, None)
        general = ge.prepared("gemm_epi_run_ext", *args, stream.cuda_stream)
        staged = ge.prepared("gemm_epi_run_ws_typed", *args, ws.data_ptr(), ws.numel(), "f16", stream.cuda_stream)
        line = {"shape": [1, M, N, K], "offset_elems": off, "plan_ws": plan}
        for name, fn in (("general", general), ("staged", staged), ("torch", lambda: torch.add(torch.matmul(A, B), C))):
            for _ in range(warmup):
                fn()
            _, ev_ms, stats = _timed_launches(lambda i: fn(), steps, stream)
            line[name + "_us"] = round(ev_ms * 1e3, 1)
        line["flops"] = 2 * M * N * K
        print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 50 launches pass before the clock and the caches settle on a fresh process
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other four report configurations (timed before the headline by default)")
    ap.add_argument("--cpu-rows", type=int, default=6144)
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--compare-unfused", action="store_true",
                    help="also time the unfused compositions, this library's own and the vendor library's "
                         "(context, not the metric)")
    ap.add_argument("--copy-kernel", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--ragged", action="store_true",
                    help="only time shapes off the fast path's 16-byte rule: general kernel, staged operands, "
                         "library (one JSON line each)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    if a.copy_kernel:
        copy_calibration(a.copy_kernel, a.steps)
        return
    if a.ragged:
        bench_ragged(a.steps, a.warmup)
        return

    from dense_gemm_elementwise_amd import workloads
    name = a.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]

    if a.all:
        for other in workloads.WORKLOADS.values():
            if other.name == name:
                continue
            g = bench_gpu(other, a.steps, a.warmup)
            line = result_line(other, g, a.steps, a.warmup, None)
            line["cold"] = bench_gpu_cold(other, a.steps, a.warmup)
            sk = bench_gpu_stream_k(other, a.steps, a.warmup)
            if sk is not None:
                line["stream_k"] = sk
            if other.name in EPI_TYPE_WORKLOADS:
                line["epi_types"] = bench_gpu_epi_types(other, a.steps, a.warmup)
            if a.compare_unfused:
                line["unfused_own"] = bench_unfused_own(other, a.steps, a.warmup)
                line["unfused_library"] = bench_unfused_library(other, a.steps, a.warmup)
            print(json.dumps(line), file=sys.stderr, flush=True)

    # The other report configurations first (their launches also bring the
    # GPU to its working clock before the headline is timed).
    configs = None
    if not a.no_configs and a.workload is None:
        configs = {c: config_summary(workloads.WORKLOADS[c], max(a.steps, 20), max(a.warmup, 20))
                   for c in workloads.CONFIGS if c != name}

    g = bench_gpu(w, a.steps, a.warmup)
    cpu = None
    if not a.no_cpu_baseline:
        threads = omp_threads()
        os.environ["OMP_NUM_THREADS"] = str(threads)
        v, dt, rows = bench_cpu_oracle(w, a.cpu_rows)
        cpu = {"value": round(v, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"first {rows} of {w.M} output rows of {w.name} (all {w.N} columns, K={w.K}), "
                         f"fp64 i-k-j triple loop + epilogue, {dt:.1f} s"}
    line = result_line(w, g, a.steps, a.warmup, cpu)
    if configs is not None:
        line["configs"] = configs
    if a.all and w.name in EPI_TYPE_WORKLOADS:
        line["epi_types"] = bench_gpu_epi_types(w, a.steps, a.warmup)
    if a.compare_unfused:
        line["unfused_own"] = bench_unfused_own(w, a.steps, a.warmup)
        line["unfused_library"] = bench_unfused_library(w, a.steps, a.warmup)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
