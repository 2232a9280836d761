"""Benchmark of the persistent tile-scheduled GEMM on one MI355X.

One step = one tsgemm_run over the 8192^3 bf16 workload (A, B i.i.d.
normal(0,1)/sqrt(K), tiles 256x256x64, group_size 8, 3 stages requested, one
persistent workgroup per CU).  Inputs are resident in HBM before timing starts.
Before the W warm-up steps the step runs back to back for --prewarm-ms (150 ms;
reported as "prewarm"): the GPU raises its clocks over the first tens of ms
under load, and the timed steps should see the steady state.
Prints one JSON line:
  value      whole-job TFLOP/s = 2*M*N*K*steps / wall time of the timed steps
  roofline   the GEMM kernel against the dense bf16 MFMA peak: achieved =
             2*M*N*K per launch / mean launch time from HIP events recorded on
             the launch stream around every timed launch
  context    torch's own A @ B (hipBLASLt) on the same device inputs, for
             reference only
  cpu_baseline  the CPU oracle (fp64 triple loop) timed on this host on a
             bounded sample of the same product (its first R rows of C)
--workload picks another of the six shapes, or the block-scaled FP8 shape
mx_8192_mxfp8 (E4M3 elements with E8M0 scales per 32 along K, bf16 output;
one step = tsgemm_mx_pack_scales of SFA and of SFB from their row-major layout
plus tsgemm_run_mx_packed, or with --mx-scales rowmajor tsgemm_run_mx alone;
roofline: the GEMM kernel against the dense fp8 MFMA peak; cpu_baseline the MX
oracle; context torch's per-tensor-scaled fp8 product when available).  --cold
rewrites a 512 MiB buffer before every timed launch so the small shapes are not
served from the Infinity Cache.  --power S (4 s by default, 0 = off; after the
timed steps, so the timed region is the same) runs the step back to back for S
seconds while `amd-smi metric` samples the board's socket power and graphics
clocks, and does the same for torch's A @ B; it reports watts, clocks and
joules per step ("power").
"""

from __future__ import annotations

import argparse
import json
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "mxfp8": 5000.0}   # MI355X dense MFMA, published
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "cfg3_8192_bf16"
_CSRC = "persistent_tile_scheduled_amd/csrc/"
KERNEL_SOURCES = {
    "gemm": tuple(_CSRC + f for f in ("tsgemm_kernel.h", "tsgemm_device.h", "tile_scheduler.h", "tsgemm_gemm_tu.hip")),
    "mx": tuple(_CSRC + f for f in ("tsgemm_mx_kernel.h", "tsgemm_device.h", "tile_scheduler.h", "tsgemm_mx_tu.hip")),
}
PROFILE_FOR = {"cfg3_8192_bf16": "profiles/gemm_8192_bf16.md", "mx_8192_mxfp8": "profiles/gemm_8192_mxfp8.md"}


def recorded_traffic(workload: str, kind: str = "gemm"):
    """HBM bytes per launch measured with rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    calibrated on a plain copy) as recorded in profiles/, or None when there is
    no record or the kernel sources changed since it was taken."""
    import hashlib
    path = PROFILE_FOR.get(workload)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    fields = {}
    for line in open(os.path.join(ROOT, path)):
        if ":" in line and line.strip().split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            k, v = line.strip().split(":", 1)
            fields[k] = v.strip()
    if fields.get("kernel_source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def _rows_for(run, M: int, target_s: float):
    """Rows of C whose oracle product takes about target_s seconds, and the time
    per row.  Calibrated twice: on 64 rows, whose time is dominated by starting
    the oracle's threads, then on enough rows for ~2 s."""
    rows = min(M, 64)  # enough rows to keep every oracle thread busy
    t0 = time.perf_counter()
    run(rows)
    dt = max(time.perf_counter() - t0, 1e-4)
    r2 = int(min(M, rows * 2.0 / dt))
    if r2 > rows:
        t0 = time.perf_counter()
        run(r2)
        rows, dt = r2, max(time.perf_counter() - t0, 1e-4)
    return int(max(8, min(M, rows * target_s / dt))), dt / rows


def cpu_baseline(w, A, B, target_s: float = 15.0):
    """Time the oracle on the first R rows of C, R sized for ~target_s seconds;
    a whole product smaller than that is repeated to fill the window."""
    import numpy as np
    import oracle
    B64 = B.double().numpy()
    rows, per_row = _rows_for(lambda r: oracle.gemm_f64(A[:r].double().numpy(), B64), w.M, target_s)
    # a product too small to fill the window is repeated whole (the small shapes)
    reps = 1
    if rows == w.M:
        reps = int(max(1, min(1000, target_s / max(per_row * w.M, 1e-4))))
    A64 = A[:rows].double().numpy()
    t0 = time.perf_counter()
    for _ in range(reps):
        c = oracle.gemm_f64(A64, B64)
    dt = time.perf_counter() - t0
    assert np.isfinite(c).all()
    flops = 2.0 * rows * w.N * w.K * reps
    what = f"first {rows} of {w.M} rows of C" if reps == 1 else f"the whole product {reps} times"
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{what} ({flops / 1e9:.1f} GFLOP, fp64 triple loop, {dt:.1f} s)",
    }


def cpu_baseline_mx(w, A, SFA, B, SFB, target_s: float = 15.0):
    """Time the MX oracle on the first R rows of C, R sized for ~target_s seconds."""
    import numpy as np
    import oracle
    rows, _ = _rows_for(lambda r: oracle.mx_gemm_f64(A[:r], SFA[:r], B, SFB), w.M, target_s)
    t0 = time.perf_counter()
    c = oracle.mx_gemm_f64(A[:rows], SFA[:rows], B, SFB)
    dt = time.perf_counter() - t0
    assert np.isfinite(c).all()
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"first {rows} of {w.M} rows of C ({flops / 1e9:.1f} GFLOP, MX decode + fp64 sum, {dt:.1f} s)",
    }


def torch_context_fp8(torch, Ad, Bd, w, stream, warmup, steps):
    """torch._scaled_mm on the same E4M3 codes with one fp32 scale per tensor
    (hipBLASLt fp8; not the block-scaled product), as context only."""
    try:
        a = Ad.view(torch.float8_e4m3fn)
        b = Bd.view(torch.float8_e4m3fn).t()
        one = torch.ones((), dtype=torch.float32, device=Ad.device)

        def f():
            return torch._scaled_mm(a, b, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        for _ in range(min(warmup, 10)):
            f()
        torch.cuda.synchronize()
        n = max(5, min(steps, 20))
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(n):
            f()
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / n
        return {"torch_scaled_mm_fp8_per_tensor_ms": round(ms, 4),
                "torch_scaled_mm_fp8_per_tensor_tflops": round(w.flops / (ms * 1e-3) / 1e12, 2)}
    except Exception as exc:  # context only: an unsupported op is reported, not fatal
        return {"torch_scaled_mm_fp8_per_tensor": f"unavailable: {type(exc).__name__}: {str(exc)[:120]}"}


def torch_context(torch, Ad, Bd, w, stream, warmup, steps):
    """torch's own A @ B (hipBLASLt) on the same device inputs, as context only."""
    for _ in range(min(warmup, 10)):
        torch.matmul(Ad, Bd)
    torch.cuda.synchronize()
    n = max(5, min(steps, 20))
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(n):
        torch.matmul(Ad, Bd)
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / n
    return {"torch_matmul_ms": round(ms, 4), "torch_matmul_tflops": round(w.flops / (ms * 1e-3) / 1e12, 2)}


def parse_smi(text: str):
    """(socket watts, [GFX clock MHz per XCD]) from the text of `amd-smi metric -p -c`, or None
    when it holds no socket-power reading."""
    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    clks = [float(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    return (float(m.group(1)), clks) if m else None


def _smi_sample():
    """One `amd-smi metric -p -c` reading (see parse_smi), or None."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=15)
    except (OSError, subprocess.SubprocessError):
        return None
    return parse_smi(r.stdout)


def measure_power(torch, enqueue, seconds: float, settle: float = 1.5):
    """Run `enqueue` (which queues a few launches) back to back for `seconds`
    and sample board power from a side thread once the load has run `settle`
    seconds.  Returns watts, clocks, launches and the mean time per launch."""
    stop = threading.Event()
    samples = []

    def sampler():
        if stop.wait(settle):
            return
        while not stop.is_set():
            s = _smi_sample()
            if s is None:
                return
            samples.append(s)
            stop.wait(0.25)

    th = threading.Thread(target=sampler, daemon=True)
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        n += enqueue()
        torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stop.set()
    th.join()
    if not samples:
        return {"error": "amd-smi gave no socket-power reading"}
    watts = sum(s[0] for s in samples) / len(samples)
    clks = [c for s in samples for c in s[1]]
    ms = dt / n * 1e3
    return {"samples": len(samples), "socket_w": round(watts, 1),
            "gfx_mhz_mean": round(sum(clks) / len(clks)) if clks else None,
            "gfx_mhz_range": [round(min(clks)), round(max(clks))] if clks else None,
            "launches": n, "ms_per_launch": round(ms, 4), "joules_per_launch": round(watts * ms * 1e-3, 4)}


def copy_mode(args, torch):
    """Plain device-to-device copy of a known size: reads and writes
    copy-mib MiB per launch.  Its FETCH_SIZE / WRITE_SIZE counter readings give
    the factor that turns those counters into bytes."""
    dev = torch.device("cuda:0")
    n = args.copy_mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "ms_per_launch": round(ms, 4), "GB/s (read+write)": round(2 * n / ms / 1e6, 1)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads for the CPU-oracle baseline (0 = all the host offers)")
    ap.add_argument("--mode", choices=["gemm", "copy"], default="gemm",
                    help="copy: time a plain device copy of --copy-mib MiB (calibrates HBM byte counters)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--cold", action="store_true",
                    help="rewrite a 512 MiB scratch buffer before every timed launch (caches cold); "
                         "the per-launch events still bracket only the GEMM")
    ap.add_argument("--no-torch-context", action="store_true")
    ap.add_argument("--epilogue", type=int, choices=[0, 64], default=0,
                    help="fp16/bf16 epilogue: 0 = direct stores, 64 = C staged through LDS in 64-column chunks")
    ap.add_argument("--prewarm-ms", type=float, default=150.0,
                    help="before the --warmup steps, run the step back to back for this long: the GPU raises its "
                         "clocks over the first tens of ms under load (0: none)")
    ap.add_argument("--series", action="store_true",
                    help="also print every timed launch's kernel time, in launch order, to stderr")
    ap.add_argument("--mx-scales", choices=["packed", "rowmajor"], default="packed",
                    help="MX workload: pack the scales on the device each step (default) or feed them row-major")
    ap.add_argument("--no-l2-prefetch", action="store_true",
                    help="workers without a tile leave at once instead of warming their XCD's L2")
    ap.add_argument("--power", type=float, default=4.0, metavar="SECONDS",
                    help="after the timed steps, run the step (and torch's A @ B) back to back this long while "
                         "amd-smi samples socket power and clocks (0: off)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.mode == "copy":
        copy_mode(args, torch)
        return
    import persistent_tile_scheduled_amd as tsg
    from workloads import MX_WORKLOADS, WORKLOADS, mx_workload_inputs, workload_inputs

    mx = args.workload in MX_WORKLOADS
    if not mx and args.workload not in WORKLOADS:
        sys.exit(f"unknown workload {args.workload!r}; have {sorted(WORKLOADS) + sorted(MX_WORKLOADS)}")
    dev = torch.device("cuda:0")
    if mx:
        w = MX_WORKLOADS[args.workload]
        A, SFA, B, SFB = mx_workload_inputs(w)
        operands = [torch.from_numpy(x).to(dev) for x in (A, SFA, B, SFB)]
        Ad, Bd = operands[0], operands[2]
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    else:
        w = WORKLOADS[args.workload]
        A, B = workload_inputs(w)
        Ad, Bd = A.to(dev), B.to(dev)
        C = torch.empty((w.M, w.N), dtype=w.torch_dtype, device=dev)
    plan = tsg.Plan(w.M, w.N, w.K, w.dtype, w.block_M, w.block_N, w.block_K, w.group_size,
                    w.num_stages, num_workgroups=w.num_workgroups, store_block_N=0 if mx else args.epilogue,
                    l2_prefetch=False if args.no_l2_prefetch else None)
    info = plan.info()
    P = plan.num_workgroups
    stream = torch.cuda.current_stream(dev)

    packed = mx and args.mx_scales == "packed"
    if packed:
        sfp = [torch.empty((plan.mx_packed_scale_bytes(op),), dtype=torch.uint8, device=dev) for op in (0, 1)]

    def launch(gemm_start=None, gemm_end=None):
        # the events bracket the GEMM kernel alone (the roofline's kernel time)
        if packed:
            plan.mx_pack_scales(operands[1], sfp[0], 0, stream)
            plan.mx_pack_scales(operands[3], sfp[1], 1, stream)
        if gemm_start is not None:
            gemm_start.record(stream)
        if packed:
            plan.run_mx_packed(operands[0], sfp[0], operands[2], sfp[1], C, stream)
        elif mx:
            plan.run_mx(*operands, C, stream)
        else:
            plan.run(Ad, Bd, C, stream)
        if gemm_end is not None:
            gemm_end.record(stream)

    # Device pre-warm (untimed, reported): under a fresh load the kernel time
    # falls for the first ~40 launches of this workload (0.94 -> 0.72 ms at
    # 8192^3) while the chip raises its clocks; the W warm-up steps follow.
    prewarm_launches = 0
    t_end = time.perf_counter() + args.prewarm_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(4):
            launch()
        prewarm_launches += 4
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        launch(starts[i], ends[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    series = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if args.series:
        print("kernel_ms in launch order: " + " ".join(f"{x:.4f}" for x in series), file=sys.stderr, flush=True)
    launch_ms = sorted(series)
    mean_ms = sum(launch_ms) / len(launch_ms)
    if scratch is not None:
        # wall time includes the cache flushes: report the GEMM launches only
        # (and, for packed MX scales, not the packing either)
        wall = sum(launch_ms) * 1e-3

    flops = float(w.flops)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (mean_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    out = {
        "metric": ("MXFP8 block-scaled GEMM TFLOP/s and % of dense fp8 MFMA peak, 1xMI355X" if mx
                   else "GEMM TFLOP/s and % of dense fp16/bf16 MFMA peak, 1xMI355X"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "prewarm": {"ms": args.prewarm_ms, "launches": prewarm_launches},
        "config": {
            "workload": w.name, "M": w.M, "N": w.N, "K": w.K,
            "tile": [w.block_M, w.block_N, w.block_K], "group_size": w.group_size,
            "num_stages": w.num_stages, "lds_slots": info["lds_slots"], "num_workgroups": P,
            "store_block_N": info["store_block_N"], "l2_prefetch": info["l2_prefetch"],
            "inputs": (f"normal(0,1) MX-encoded (E4M3 + E8M0 per 32 along K), seed {w.seed}" if mx
                       else f"{w.dist}, seed {w.seed}"),
            **({"scales": ("row-major, packed on the device inside every step" if packed else "row-major")}
               if mx else {}),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(w.name, "mx" if mx else "gemm"),
            "kernel_ms": {"mean": round(mean_ms, 4), "min": round(launch_ms[0], 4),
                          "median": round(launch_ms[len(launch_ms) // 2], 4),
                          "p90": round(launch_ms[min(len(launch_ms) - 1, (9 * len(launch_ms)) // 10)], 4)},
            "hbm_gbs_algorithmic": round(w.algorithmic_bytes / (mean_ms * 1e-3) / 1e9, 1),
            "caches": "cold (512 MiB rewritten before each launch)" if args.cold else "warm",
        },
        "context": None,
        "cpu_baseline": None,
    }
    if not args.no_torch_context:
        out["context"] = (torch_context_fp8 if mx else torch_context)(torch, Ad, Bd, w, stream,
                                                                      args.warmup, args.steps)
    if args.power > 0:
        def ours():
            for _ in range(8):
                launch()
            return 8
        pw = {"kernel": measure_power(torch, ours, args.power)}
        if not mx and not args.no_torch_context:
            def lib():
                for _ in range(8):
                    torch.matmul(Ad, Bd)
                return 8
            pw["torch_matmul"] = measure_power(torch, lib, args.power)
        for v in pw.values():
            if "joules_per_launch" in v:
                v["tflops_per_w"] = round(w.flops / v["joules_per_launch"] / 1e12, 3)
        out["power"] = pw
    if not args.no_cpu_baseline:
        if args.cpu_threads > 0:
            import oracle
            oracle.set_num_threads(args.cpu_threads)
        out["cpu_baseline"] = cpu_baseline_mx(w, A, SFA, B, SFB) if mx else cpu_baseline(w, A, B)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
