"""Benchmark of the fused GEMM + bias + GELU on one MI355X.

    python bench.py [--steps 50] [--warmup 300] [--workload c3_gelu] [--unfused]
                    [--transpose-b] [--transpose-a]

One step is one gemm_bias_act call over the whole workload (schedule choice,
global->LDS loads, MFMA main loop, fused epilogue, store), with inputs already
resident in HBM. W untimed steps, then K timed steps between two device
synchronisations. Two HIP events on the launch stream bracket the K timed
launches and give the kernel's average launch duration (the roofline's
"achieved"); a separate pass with an event per launch gives the median latency,
as the pages' bench helper reports it.

The default W is 300, not the pages' 10: an MI355X coming out of idle raises
its clocks over the first ~300 launches of this kernel (~40 ms). Measured per
100-launch window from cold at 4096^3: 0.149, 0.125, 0.122, then 0.120 ms
flat through 1500 launches. With 10 warmups the timed steps sit in the ramp.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = {"f16": 2516.6, "bf16": 2516.6,    # dense, 256 CU x 2.4 GHz x 4096 flop/clk
                    "e4m3": 5033.2, "e5m2": 5033.2}    # dense fp8: twice the 16-bit rate
PEAK_HBM_GBS = 8000.0
METRIC = "TFLOP/s fused fp16 GEMM+bias+GELU at 4096³; % of MI355X fp16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu() -> dict:
    """Model name and usable core count of the host this process runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"model": model, "cores": cores, "nproc": os.cpu_count()}


def _smi_handle(dev_index: int):
    """amdsmi handle of torch device dev_index (matched by PCI bus), or None."""
    import amdsmi
    import torch
    amdsmi.amdsmi_init()
    handles = amdsmi.amdsmi_get_processor_handles()
    props = torch.cuda.get_device_properties(dev_index)
    bus = getattr(props, "pci_bus_id", None)
    for h in handles:
        bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)   # "dddd:bb:dd.f"
        if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
            return h
    return handles[0] if len(handles) == 1 else None


def gpu_stack(dev_index: int) -> dict:
    """Software stack and device identity, best effort (a field that cannot be
    read is None, with the reason under "errors")."""
    import torch
    out = {"torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None),
           "rocm": None, "driver": None, "gpu": None, "cus": None, "arch": None,
           "max_sclk_mhz": None, "errors": {}}
    try:
        props = torch.cuda.get_device_properties(dev_index)
        out["gpu"] = props.name
        out["cus"] = props.multi_processor_count
        out["arch"] = getattr(props, "gcnArchName", None)
    except Exception as e:   # noqa: BLE001 - report, do not fail the bench
        out["errors"]["device"] = repr(e)
    try:
        with open("/opt/rocm/.info/version") as f:
            out["rocm"] = f.read().strip()
    except OSError as e:
        out["errors"]["rocm"] = repr(e)
    try:
        import amdsmi
        h = _smi_handle(dev_index)
        if h is not None:
            d = amdsmi.amdsmi_get_gpu_driver_info(h)
            out["driver"] = "%s %s" % (d.get("driver_name"), d.get("driver_version"))
            c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            out["max_sclk_mhz"] = c.get("max_clk")
    except Exception as e:   # noqa: BLE001
        out["errors"]["amdsmi"] = repr(e)
    if not out["errors"]:
        del out["errors"]
    return out


class ClockProbe:
    """The core clock the power manager has set at a point of the stream, read
    on the device by the library's clock probe (one wave per workgroup, 4
    workgroups per CU, each dividing elapsed s_memtime core cycles by elapsed
    constant-rate wall-clock ticks over spin_us), enqueued on the launch stream
    right behind the launches it describes. The probe itself is a light load:
    under the GEMM's full matrix-core load the chip's current limiting runs the
    clock lower than the set point this reads."""

    def __init__(self, dev, n_wg=1024, spin_us=10):
        import torch
        self.n_wg, self.spin_us = n_wg, spin_us
        self.buf = [torch.zeros(2 * n_wg, dtype=torch.int64, device=dev) for _ in range(2)]
        self.khz = None

    def enqueue(self, slot: int):
        import tiled_dense_gemm_bias_amd as gba
        self.khz = gba.clock_probe(self.buf[slot], self.n_wg, self.spin_us)

    def read(self, slot: int) -> dict:
        """Per-workgroup MHz after the stream has finished: median, min, max."""
        v = self.buf[slot].cpu().numpy().reshape(-1, 2).astype(np.float64)
        ok = v[:, 1] > 0
        if not ok.any() or not self.khz:
            return {"median": None}
        mhz = v[ok, 0] / v[ok, 1] * self.khz / 1000.0
        return {"median": round(float(np.median(mhz)), 1), "min": round(float(mhz.min()), 1),
                "max": round(float(mhz.max()), 1)}


# Sources each kernel family is compiled from (the schedule table and host code
# are left out: they do not change what a launch of the kernel does).
KERNEL_HEADERS = {0: ["gba_kernels.hpp"],
                  3: ["gba_kernels.hpp", "gba_dma.hpp", "gemm_v3.hpp"],
                  4: ["gba_kernels.hpp", "gba_dma.hpp", "gemm_v3.hpp", "gemm_v5.hpp"],
                  "f8": ["gba_kernels.hpp", "gba_dma.hpp", "gemm_v3.hpp", "gemm_v5.hpp",
                         "gemm_f8.hpp"]}


def instance_file(s: dict) -> str:
    """The csrc file that instantiates schedule s."""
    if s["kernel"] == "f8":
        return "f8_256x256x128_w2x2_persistent_%s.hip" % s["fmt"]
    if s["kernel"] == 4:
        return "v5_%dx%dx%d_w%dx%d_persistent.hip" % (s["bm"], s["bn"], s["bk"], s["wm"], s["wn"])
    if s["kernel"] == 3:
        return "v3_%dx%dx%d_w%dx%d_s%d_l%d_p%d_m16.hip" % (
            s["bm"], s["bn"], s["bk"], s["wm"], s["wn"], s["stages"], s["loaders"], s["spread"])
    return "inst_%dx%dx%d_w%dx%d.hip" % (s["bm"], s["bn"], s["bk"], s["wm"], s["wn"])


def kernel_source_hash(sched: dict) -> str:
    """sha256 over the sources of the kernel that schedule `sched` launches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_bias_amd", "csrc")
    for fn in KERNEL_HEADERS[sched["kernel"]] + [instance_file(sched)]:
        h.update(fn.encode())
        h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sched: dict):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current sources of the kernel `sched` launches; else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(workload)
    if not rec or rec.get("kernel_hash") != kernel_source_hash(sched):
        return None
    return rec.get("bytes_per_launch")


def time_launches(fn, steps, warmup, stream, clock=None):
    """W untimed calls, then K timed ones between two device synchronisations.

    Returns (wall_ms, avg_ms, per):
      wall_ms  host clock over the K timed calls (sync before and after);
      avg_ms   average launch duration: two HIP events on the launch stream
               bracket the K launches, divided by K (each launch's kernel plus
               the dispatch gap before the next);
      per      per-launch durations from a second, separate pass of K calls
               with an event before each (for the median). An event record
               between launches costs ~3 us on this device, so those intervals
               run a little longer; they are not part of the timed region.
    clock, a ClockProbe, if given, is enqueued right behind the warmup calls
    (slot 0: the clock the timed region starts at) and right behind the second
    pass (slot 1: the clock at its end); neither probe is inside a timed interval.
    """
    import torch
    for _ in range(warmup):
        fn()
    if clock is not None:
        clock.enqueue(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3
    avg_ms = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(stream)
        fn()
    ev[steps].record(stream)
    if clock is not None:
        clock.enqueue(1)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return wall_ms, avg_ms, per


def cpu_baseline(w, A, B, bias, got_bits, target_s=12.0, transpose_b=False, scale=None,
                 transpose_a=False):
    """The fp64 oracle on a bounded sample of rows, timed on the host cores
    (8-bit inputs when scale is given)."""
    import oracle
    from oracle import compare
    import synth

    def run(rows, with_abs=False):
        if scale is not None:
            return oracle.gemm_bias_act_fp8(A, B, bias, scale, w.act, w.fmt, w.dtype, rows=rows,
                                            nthreads=cores, with_abs=with_abs)
        return oracle.gemm_bias_act(A, B, bias, w.act, w.dtype, rows=rows, nthreads=cores,
                                    with_abs=with_abs, transpose_b=transpose_b,
                                    transpose_a=transpose_a)

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    rows = synth.sample_rows(w.M, 16, seed=w.seed)
    t0 = time.perf_counter()
    run(rows)
    t_probe = time.perf_counter() - t0
    n = int(min(w.M, max(16, 16 * target_s / max(t_probe, 1e-3))))
    n = max(16, (n // cores) * cores if n > cores else n)
    rows = synth.sample_rows(w.M, n, seed=w.seed)
    t0 = time.perf_counter()
    R, S = run(rows, with_abs=True)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * w.N * w.K
    rep = compare.check(oracle.decode(got_bits[rows], w.dtype), R, K=w.K, dtype=w.dtype,
                        act=oracle.ACTS[w.act], S=S,
                        sum_rel=None if scale is None else compare.fp8_sum_rel(w.K))
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d output rows of %dx%dx%d %s %s (fp64 triple loop, %.1f s)"
                      % (len(rows), w.M, w.M, w.N, w.K,
                         w.dtype if scale is None else w.fmt + "->" + w.dtype, w.act, dt)}
    parity = {k: rep[k] for k in ("ok", "strict_ok", "rel_frobenius", "max_abs", "max_ulp")}
    parity["rows"] = len(rows)
    return base, parity


def cpu_single_thread() -> dict:
    """The oracle on one host thread over the two small workloads, whole (256^3
    with and without bias+GELU, 1024^3 plain): median of 5 runs at 256^3, one
    run at 1024^3."""
    import oracle
    import synth
    res = {}
    for name, reps in (("c1_plain", 5), ("c1_gelu", 5), ("c2_plain", 1)):
        w = synth.WORKLOADS[name]
        A, B, bias = synth.make_inputs(w)
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.gemm_bias_act(A, B, bias, w.act, w.dtype, nthreads=1)
            ts.append(time.perf_counter() - t0)
        t = statistics.median(ts)
        res[name] = {"seconds": round(t, 4), "GFLOP/s": round(w.flops / t / 1e9, 3),
                     "runs": reps, "threads": 1}
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="c3_gelu")
    ap.add_argument("--unfused", action="store_true", help="also time gemm + bias_act")
    ap.add_argument("--workspace", action="store_true",
                    help="pass a split-K workspace (gemm_bias_act_ex): shapes with fewer tiles "
                         "than CUs split K")
    ap.add_argument("--transpose-b", action="store_true",
                    help="B stored [N,K] (transpose_B): time gemm_bias_act_nt on the same numbers")
    ap.add_argument("--transpose-a", action="store_true",
                    help="A stored [K,M] (transpose_A): time gemm_bias_act_ex with GBA_TRANSPOSE_A "
                         "on the same numbers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--act", default=None,
                    help="replace the workload's activation (none, relu, sigmoid, gelu, softplus, gelu_tanh)")
    ap.add_argument("--tune", action="store_true", help="autotune before timing")
    ap.add_argument("--schedule", default=None, help="force bm,bn,bk,wm,wn,stages,kernel,loaders,spread[,raster,group_m]")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain device copy of the workload's C size (counter scaling)")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print("bench.py measures one GPU: this build runs the fused GEMM on a single MI355X "
              "(no multi-GPU path); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import synth
    import tiled_dense_gemm_bias_amd as gba

    if not os.path.exists(gba.LIB_PATH):
        from tiled_dense_gemm_bias_amd import build as gba_build
        gba_build.build()

    fp8 = a.workload in synth.FP8_WORKLOADS
    w = synth.FP8_WORKLOADS[a.workload] if fp8 else synth.WORKLOADS[a.workload]
    if a.act:
        w = dataclasses.replace(w, act=a.act)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] generating %s inputs %dx%dx%d %s" % (w.name, w.M, w.N, w.K, w.dtype))
    scale = None
    if fp8:
        A, B, bias, scale = synth.make_inputs_fp8(w)   # B is W [N,K]
    else:
        A, B, bias = synth.make_inputs(w)
    tb = a.transpose_b and not fp8
    ta = a.transpose_a and not fp8
    if tb:
        B = np.ascontiguousarray(B.T)   # the same operand, stored as the [N,K] weight W
    if ta:
        A = np.ascontiguousarray(A.T)   # the same operand, stored as At [K,M]
    wl_key = (w.name + ("_t" + ("t" if tb else "n") if ta else ("_nt" if tb else ""))
              + ("_" + a.act if a.act else ""))
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16

    def dev_t(bits):
        return None if bits is None else torch.from_numpy(bits.view(np.int16)).view(tdt).to(dev)

    if fp8:
        a_t, b_t = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        bias_t = dev_t(bias)
    else:
        a_t, b_t, bias_t = dev_t(A), dev_t(B), dev_t(bias)
    c_t = torch.empty((w.M, w.N), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)

    if a.copy_calibration:
        src = torch.empty((w.M, w.N), dtype=tdt, device=dev).fill_(1.0)
        for _ in range(a.warmup + a.steps):
            c_t.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: %d copies of %d bytes" % (a.warmup + a.steps,
                                                                   c_t.numel() * 2))
        return 0

    if a.schedule and not fp8:
        f = [int(x) for x in a.schedule.split(",")]
        keys = ["bm", "bn", "bk", "wm", "wn", "stages", "kernel", "loaders", "spread", "raster",
                "group_m"]
        sched = dict(zip(keys, f))
        sched.setdefault("raster", 1)
        sched.setdefault("group_m", 4)
        gba.set_schedule(sched)
    elif a.tune and not fp8:
        best, ms = gba.autotune(a_t, b_t, bias_t, c_t, w.act, all_groups=True, transpose_b=tb,
                                transpose_a=ta)
        log("[bench] autotune best %s %.4f ms" % (best, ms))
    if fp8:
        sched = {"kernel": "f8", "fmt": w.fmt, "bm": 256, "bn": 256, "bk": 128, "wm": 2, "wn": 2,
                 "stages": 2, "raster": 1, "group_m": 4}
        ws_t = None
        if a.workspace:
            nb = gba.workspace_size(w.M, w.N, w.K, w.act, w.dtype, fp8=True)
            ws_t = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
            sched = dict(sched, splits_workspace_bytes=nb)
        step = gba.bind_gemm_bias_act_fp8(a_t, b_t, bias_t, c_t, scale, w.act, w.fmt,
                                          workspace=ws_t)
    else:
        sched = gba.get_schedule(w.M, w.N, w.K, w.act, w.dtype, transpose_b=tb, transpose_a=ta)
        ws_t = None
        if a.workspace:
            nb = gba.workspace_size(w.M, w.N, w.K, w.act, w.dtype, transpose_b=tb,
                                    transpose_a=ta)
            ws_t = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
            plan, splits = gba.split_plan(w.M, w.N, w.K, w.act, w.dtype, transpose_b=tb,
                                          transpose_a=ta)
            sched = dict(plan, splits=splits, splits_workspace_bytes=nb)
        step = gba.bind_gemm_bias_act(a_t, b_t, bias_t, c_t, w.act, transpose_b=tb, workspace=ws_t,
                                      transpose_a=ta)
    log("[bench] schedule %s%s%s" % (sched, " (A stored [K,M])" if ta else "",
                                     " (B stored [N,K])" if tb else ""))
    clock = ClockProbe(dev)
    wall_ms, kern_avg, per = time_launches(step, a.steps, a.warmup, stream, clock)
    sclk = {"at_start": clock.read(0), "at_end": clock.read(1),
            "source": "device clock probe (s_memtime / s_memrealtime per workgroup, %d "
                      "workgroups over %d us) enqueued behind the warmups and behind the "
                      "per-launch-event pass" % (clock.n_wg, clock.spin_us),
            "meaning": "the clock the power manager has set at those two moments, read under "
                       "the probe's light load; under the GEMM's full matrix-core load the "
                       "chip runs below it (GRBM_GUI_ACTIVE cycles per dispatch in the "
                       "committed counter profile)"}
    ms_per_step = wall_ms / a.steps
    kern_med = statistics.median(per)
    flops = float(w.flops)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg * 1e-3) / 1e12
    tflops_med = flops / (kern_med * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[w.fmt if fp8 else w.dtype]
    in_bytes = 1 if fp8 else 2
    alg_bytes = (w.M * w.K + w.K * w.N) * in_bytes + (w.M * w.N + (w.N if w.bias else 0)) * 2
    log("[bench] %d steps after %d warmups: wall %.4f ms/step -> %.1f TFLOP/s (value); "
        "event-bracketed kernel avg %.4f ms -> %.1f TFLOP/s (%.1f%% of peak, roofline); "
        "per-launch-event median %.4f ms -> %.1f TFLOP/s; sclk %s"
        % (a.steps, a.warmup, ms_per_step, value, kern_avg, achieved, 100 * achieved / peak,
           kern_med, tflops_med, sclk["at_end"]["median"]))
    got_bits = c_t.view(torch.int16).cpu().numpy().view(np.uint16)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8_" + w.fmt + "->" + w.dtype) if fp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": ("%s: C = %s(scale * A.W^T + bias), W stored [N,K], M=%d N=%d K=%d, "
                                "%s in, %s out, fp32 accumulate"
                                % (wl_key, w.act, w.M, w.N, w.K, w.fmt, w.dtype)) if fp8 else
                               ("%s: C = %s(%s.%s + bias), M=%d N=%d K=%d, %s in/out, fp32 accumulate"
                                % (wl_key, w.act, "At^T, At stored [K,M]" if ta else "A",
                                   "W^T, W stored [N,K]" if tb else "B", w.M, w.N, w.K, w.dtype)),
                   "M": w.M, "N": w.N, "K": w.K, "act": w.act, "bias": w.bias,
                   "a_layout": "KM (transpose_A)" if ta else "MK",
                   "b_layout": "NK (transpose_B)" if (tb or fp8) else "KN",
                   "schedule": sched, "flop_model": "2*M*N*K (epilogue not counted)"},
        "median_ms": round(kern_med, 5),
        "pct_of_peak": round(100 * achieved / peak, 2),
        "timing": {
            "value": "2*M*N*K / (host wall clock over the K timed steps / K); ms_per_step",
            "kernel_avg_ms": round(kern_avg, 5),
            "kernel_avg": "two HIP events on the launch stream bracket the K timed launches, "
                          "divided by K; gives roofline.achieved and pct_of_peak",
            "tflops_kernel_avg": round(achieved, 2),
            "median_ms": round(kern_med, 5),
            "median": "separate untimed pass of K launches with one HIP event before each; "
                      "every interval includes one event record (~3 us at this size)",
            "tflops_median": round(tflops_med, 2),
        },
        "sclk_mhz": sclk,
        "spec_sclk_mhz": 2400,
        "stack": gpu_stack(dev.index),
        "host": host_cpu(),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(wl_key, sched),
                     "algorithmic_bytes": alg_bytes, "kernel_avg_ms": round(kern_avg, 5)},
    }

    if a.unfused and not fp8:
        t_t = torch.empty_like(c_t)
        y_t = torch.empty_like(c_t)
        _, g_ms, _ = time_launches(lambda: gba.gemm(a_t, b_t, t_t, transpose_b=tb, transpose_a=ta),
                                   a.steps,
                                   a.warmup, stream)
        _, b_ms, _ = time_launches(lambda: gba.bias_act(t_t, bias_t, y_t, w.act), a.steps,
                                   a.warmup, stream)
        ba_bytes = 2 * w.M * w.N * 2 + (w.N * 2 if w.bias else 0)
        out["unfused"] = {
            "gemm_ms": round(g_ms, 5), "bias_act_ms": round(b_ms, 5),
            "total_ms": round(g_ms + b_ms, 5), "fused_ms": round(kern_avg, 5),
            "speedup_fused": round((g_ms + b_ms) / kern_avg, 3),
            "bias_act_GBps": round(ba_bytes / (b_ms * 1e-3) / 1e9, 1),
            "bias_act_frac_hbm_peak": round(ba_bytes / (b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "hbm_bytes_saved": 2 * w.M * w.N * 2,
        }
        log("[bench] unfused: gemm %.4f ms + bias_act %.4f ms (%.0f GB/s) vs fused %.4f ms"
            % (g_ms, b_ms, out["unfused"]["bias_act_GBps"], kern_avg))

    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a row sample")
        base, parity = cpu_baseline(w, A, B, bias, got_bits, transpose_b=tb, scale=scale,
                                    transpose_a=ta)
        out["cpu_baseline"] = base
        out["parity_sampled"] = parity
        if not fp8:
            out["cpu_baseline"]["single_thread"] = cpu_single_thread()
        log("[bench] cpu baseline %.4f TFLOP/s on %d threads; parity %s"
            % (base["value"], base["cores"], parity))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
