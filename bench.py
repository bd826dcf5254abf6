"""Throughput of libgemm on one MI355X.

One step is one pass of the whole hot path over synthetic, seeded inputs
already resident in HBM:

  * bf16-operand / fp32-accumulate GEMM, M = N = K = 8192 (alpha 1, beta 0,
    N(0,1) rounded to bf16, seed 4)                                   -- tiled MFMA path
  * fp32 GEMM, M = N = K = 4096 (alpha 1, beta 0, N(0,1), seed 2)  -- tiled MFMA path
  * fp32 GEMM, M = 16, N = K = 8192 (alpha 1, beta 0, U[-1,1], seed 3) -- skinny streaming path

``value`` is the step's total arithmetic (2*M*N*K summed over the three
calls) divided by the wall time of the timed steps, in GFLOP/s.  Each launch
is also bracketed by HIP events on the stream it runs on, giving every
kernel's average duration; ``roofline`` reports the kernel with the largest
share of the step against its own roof (fp32 or bf16 matrix peak, or HBM
bandwidth for the skinny path) and ``parts`` reports all three.

The skinny call cycles through three copies of B (3 x 268 MB) so every call
streams B from HBM rather than from the 256 MB last-level cache, and passes a
preallocated workspace so the library takes its split-K path (partial sums,
then a reduce kernel; the event pair brackets both).

``cold`` times each workload again, call by call, after reading a 1 GiB
buffer that evicts L2 and the last-level cache, and reports the median and
the minimum (``--cold-calls``; it does not enter ``value``).

``cpu_baseline`` times the CPU oracle (fp64, OpenMP) on a bounded sample of
the same step: all 4096 rows of the fp32 problem, the first 4096 rows of the
bf16 problem and the whole skinny problem.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GFLOP/s (2MNK/t) fp32 4096^3 + bf16 8192^3, % of MI355X MFMA peak"
PEAK_TFLOPS = {"f32": 157.3, "bf16f32": 2500.0, "fp8f32": 5000.0}
PEAK_HBM_GBS = 8000.0
# The skinny call runs after the fp32 GEMM (64 MB of C written) rather than
# right after the bf16 GEMM, whose 256 MB of freshly written C would still be
# draining from the last-level cache to HBM while the skinny kernel streams B.
STEP = ["bf16f32_8192", "f32_4096", "f32_16x8192x8192"]
# Timed on their own with --only (not part of the step): other operand types,
# layouts and shapes.
EXTRA = ["fp8f32_8192_nt", "bf16f32_8192_nt", "bf16f32_8192_tn", "bf16f32_16x8192x8192", "bf16f32_16x8192x8192_nt",
         "f32_16x8192x8192_nt", "fp8f32_16x8192x8192_nt", "f32_4096_nt", "f32_4096_tn",
         "fp8f32_8192_nn", "fp8f32_8192_tn", "bf16f32_2048x4096x4096", "bf16f32_2048x4096x4096_nt",
         "f32_2048x4096x4096"]
# The other configurations of the workload set, timed call by call after the
# step (they do not enter ``value``): (workload, whether a workspace is passed).
# The M = 16 shape is timed here through the plain call as well, which has no
# workspace and so no K split.
CONFIGS = [("f32_256", True), ("f32_4092_beta", True), ("f32_1000x3000x777", True),
           ("f32_16x8192x8192", False)]
CONFIG_NAMES = [n for n, _ in CONFIGS if n not in STEP]
SKINNY_COPIES = 3
CPU_SAMPLE_ROWS = {"f32_4096": 4096, "bf16f32_8192": 4096, "f32_16x8192x8192": 16}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=STEP + EXTRA + CONFIG_NAMES, default=None,
                    help="time a single workload (of the step, an extra one, or one of the other configurations)")
    ap.add_argument("--no-workspace", action="store_true",
                    help="with --only: call without a workspace (the plain call; no K split)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--observe-clocks", type=float, default=6.0,
                    help="after the timed steps, keep running the step this many seconds while amd-smi samples "
                         "the GFX clocks and socket power (0: off)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="after the timed steps, time this many calls of each workload one at a time, each "
                         "after reading a 1 GiB buffer that evicts L2 and the last-level cache (0: skip)")
    ap.add_argument("--config-calls", type=int, default=50,
                    help="after the timed steps, time this many back-to-back calls of each of the other "
                         "configurations (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (a plain kernel of known traffic) so hardware "
                         "byte counters can be scaled against it")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"f32_mfma32": "gemm_f32_tiled.hip", "bf16_mfma32": "gemm_bf16_tiled.hip",
                  "bf16_mfma32_256x256x64_w2x2_a8b8_lines": "gemm_bf16_lines.hip",
                  "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines": "gemm_bf16_lines.hip",
                  "bf16_mfma32_256x256x32_w2x2_a8b8_tn_lines": "gemm_bf16_lines.hip",
                  "bf16_mfma32_128x128x64_w2x2_a8b8_lines": "gemm_bf16_lines.hip",
                  "bf16_mfma32_128x128x64_w2x2_a8b8_nt_lines": "gemm_bf16_lines.hip",
                  "bf16_mfma32_128x128x32_w2x2_a8b8_tn_lines": "gemm_bf16_lines.hip",
                  "fp8_mfma32_256x256x128_w2x2_nt_lines": "gemm_fp8_lines.hip",
                  "fp8_mfma32_128x128x128_w2x2_nt_lines": "gemm_fp8_lines.hip",
                  "f32_skinny": "gemm_f32_skinny.hip", "fp8_mfma32": "gemm_fp8_tiled.hip",
                  "bf16_skinny": "gemm_bf16_skinny.hip", "f32_skinny_nt": "gemm_skinny_nt.hip",
                  "bf16_skinny_nt": "gemm_skinny_nt.hip", "fp8_skinny_nt": "gemm_skinny_nt.hip",
                  "fp8_skinny_kn": "gemm_fp8_skinny.hip"}


# Headers that only some kernel sources include (the whole-line epilogue).
OWN_HEADERS = ["gemm_lines.hpp"]
# Headers every kernel source includes: a change there changes the kernels too.
KERNEL_HEADERS = [os.path.join("tiled_gemm_f32_amd", "csrc", "gemm_device.hpp"),
                  os.path.join("tiled_gemm_f32_amd", "csrc", "gemm_kernels.hpp"),
                  os.path.join("include", "gemm.h")]


def kernel_source_sha(kernel_name: str):
    """sha256 over the source file a kernel is built from, the shared headers
    every source includes and the headers of its own that the source
    includes (to spot stale counter data)."""
    import hashlib
    # The longest matching prefix names the source.
    for prefix, src in sorted(KERNEL_SOURCES.items(), key=lambda kv: -len(kv[0])):
        if kernel_name.startswith(prefix):
            src_path = os.path.join("tiled_gemm_f32_amd", "csrc", src)
            with open(os.path.join(ROOT, src_path), "rb") as f:
                text = f.read()
            own = [os.path.join("tiled_gemm_f32_amd", "csrc", hdr) for hdr in OWN_HEADERS
                   if b'#include "' + hdr.encode() + b'"' in text]
            h = hashlib.sha256()
            for path in [src_path] + KERNEL_HEADERS + own:
                with open(os.path.join(ROOT, path), "rb") as f:
                    h.update(f.read())
            return h.hexdigest()
    return None


def measured_traffic(kernel_name: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's source changed after the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get("kernels", {}).get(kernel_name)
    if not rec or rec.get("source_sha256") != kernel_source_sha(kernel_name):
        return None
    return rec.get("bytes_per_launch")


def _amd_smi_sample(exe):
    """(socket power W, [GFX clock MHz per XCD]) from one amd-smi metric call, or None."""
    import re
    import subprocess
    try:
        out = subprocess.run([exe, "metric", "-g", "0", "--clock", "--power"], capture_output=True, text=True,
                             timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    power = re.search(r"SOCKET_POWER:\s*(\d+(?:\.\d+)?)\s*W", out)
    clocks, in_gfx = [], False
    for line in out.splitlines():
        if re.match(r"^\s*GFX_\d+:\s*$", line):
            in_gfx = True
            continue
        m = re.match(r"^\s*CLK:\s*(\d+)\s*MHz", line)
        if m and in_gfx:
            clocks.append(int(m.group(1)))
        in_gfx = False if m else in_gfx
    if power is None or not clocks:
        return None
    return float(power.group(1)), clocks


def observe_clocks(run_step, seconds):
    """Run the step for `seconds` while a thread samples amd-smi; median GFX
    clock (mean over XCDs) and socket power, or None when unavailable."""
    import shutil
    import statistics
    import threading
    exe = shutil.which("amd-smi")
    if exe is None or seconds <= 0:
        return None
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        stop.wait(0.5)                   # let the clocks settle on the load first
        while not stop.is_set():
            s = _amd_smi_sample(exe)
            if s is not None:
                samples.append(s)
            stop.wait(0.25)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            run_step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    mean_clk = [sum(c) / len(c) for _, c in samples]
    return {"gfx_mhz_median": round(statistics.median(mean_clk)), "gfx_mhz_min": min(min(c) for _, c in samples),
            "gfx_mhz_max": max(max(c) for _, c in samples),
            "socket_power_w_median": round(statistics.median(p for p, _ in samples)), "samples": len(samples),
            "seconds": seconds, "tool": "amd-smi metric --clock --power"}


def _to_device(t, dev):
    """Host tensor to the device; fp8 moves as bytes (no fp8 kernel involved)."""
    import torch
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).to(dev).view(torch.float8_e4m3fn)
    return t.to(dev)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library is single-GPU (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_gemm_f32_amd as tg
    from tiled_gemm_f32_amd import _lib
    from tiled_gemm_f32_amd.workloads import WORKLOADS, make_inputs

    if not os.path.exists(_lib.LIB_PATH):
        from tiled_gemm_f32_amd import build as hip_build
        hip_build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = [args.only] if args.only else STEP

    DTYPES = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32, "fp8f32": tg.GEMM_DTYPE_FP8F32}
    # Inputs resident in HBM before timing.
    def make_call(name, with_ws=None):
        w = WORKLOADS[name]
        A, B, C0 = make_inputs(w)
        Ad, C = _to_device(A, dev), C0.to(dev)
        copies = SKINNY_COPIES if w.M <= 16 else 1
        Bs = [_to_device(B, dev) for _ in range(copies)]
        ws = None
        if with_ws is None:
            with_ws = w.dtype == "f32" or w.M <= 16
        if with_ws:
            ws = tg.workspace(w.M, w.N, w.K, device=dev, dtype=DTYPES[w.dtype])
        return {"w": w, "A": Ad, "B": Bs, "C": C, "ws": ws, "i": 0, "durs": []}

    calls = [make_call(name, False if args.no_workspace else None) for name in names]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def ldb_of(w):
        return w.K if w.op_b == "T" else w.N

    def lda_of(w):
        return w.M if w.op_a == "T" else w.K

    def ops_of(w):
        return (tg.GEMM_OP_T if w.op_a == "T" else tg.GEMM_OP_N, tg.GEMM_OP_T if w.op_b == "T" else tg.GEMM_OP_N)

    def launch(c, record):
        w = c["w"]
        B = c["B"][c["i"] % len(c["B"])]
        c["i"] += 1
        fn = tg.gemm_f32 if w.dtype == "f32" else tg.gemm_bf16f32
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        if w.dtype == "fp8f32" or w.op_b == "T" or w.op_a == "T":
            st = tg.gemm_general(DTYPES[w.dtype], *ops_of(w), w.M, w.N, w.K, w.alpha, c["A"].data_ptr(), lda_of(w),
                                 B.data_ptr(), ldb_of(w), w.beta, c["C"].data_ptr(), w.N, 0, None,
                                 c["ws"].data_ptr() if c["ws"] is not None else 0,
                                 c["ws"].numel() if c["ws"] is not None else 0, sh)
        elif c["ws"] is not None:
            fws = tg.gemm_f32_ws if w.dtype == "f32" else tg.gemm_bf16f32_ws
            st = fws(w.M, w.N, w.K, w.alpha, c["A"].data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                     c["C"].data_ptr(), w.N, c["ws"].data_ptr(), c["ws"].numel(), sh)
        else:
            st = fn(w.M, w.N, w.K, w.alpha, c["A"].data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                    c["C"].data_ptr(), w.N, sh)
        if st != tg.GEMM_OK:
            raise tg.GemmError(st, w.name)
        if record:
            e1.record(stream)
            c["durs"].append((e0, e1))

    def plan_of(c):
        w = c["w"]
        return tg.gemm_plan_query_general(DTYPES[w.dtype], *ops_of(w), w.M, w.N, w.K, w.alpha,
                                          c["A"].data_ptr(), lda_of(w), c["B"][0].data_ptr(), ldb_of(w), w.beta,
                                          c["C"].data_ptr(), w.N, 0,
                                          c["ws"].numel() if c["ws"] is not None else 0)[1]

    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for c in calls:
            launch(c, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for c in calls:
            launch(c, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    flops_step = sum(c["w"].flops for c in calls)
    value = flops_step * args.steps / elapsed / 1e9
    parts = {}
    for c in calls:
        w = c["w"]
        ms = sum(e0.elapsed_time(e1) for e0, e1 in c["durs"]) / len(c["durs"])
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9
        kname = tg.gemm_kernel_query(plan_of(c)["kernel_id"])["name"]
        bound = "hbm" if w.M <= 16 else "mfma"
        parts[w.name] = {
            "kernel": kname, "ms": round(ms, 5), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
            "bound": bound,
            "frac": round(gbs / PEAK_HBM_GBS if bound == "hbm" else tflops / PEAK_TFLOPS[w.dtype], 4),
            "flops": w.flops, "algorithmic_bytes": w.algorithmic_bytes,
        }

    def roofline_of(name):
        p = parts[name]
        w = WORKLOADS[name]
        if p["bound"] == "hbm":
            achieved, peak, unit = p["gbs"], PEAK_HBM_GBS, "GB/s"
        else:
            achieved, peak, unit = p["tflops"], PEAK_TFLOPS[w.dtype], "TFLOP/s"
        return {"kernel": p["kernel"], "workload": name, "bound": p["bound"], "achieved": achieved, "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4), "traffic": measured_traffic(p["kernel"]),
                "algorithmic_bytes": w.algorithmic_bytes}

    cold = cold_timings(calls, launch, args.cold_calls, dev) if args.cold_calls > 0 else None
    configs = None
    if args.config_calls > 0 and not args.only:
        configs = config_timings(make_call, launch, plan_of, args.config_calls)

    dominant = max(parts, key=lambda n: parts[n]["ms"])
    roof = roofline_of(dominant)

    def one_step():
        for c in calls:
            launch(c, False)

    observed = observe_clocks(one_step, args.observe_clocks)

    cpu = None
    if not args.no_cpu_baseline and not args.only:
        cpu = cpu_baseline(calls)

    dtypes = "+".join(d for d in ("f32", "bf16f32", "fp8f32") if any(c["w"].dtype == d for c in calls))
    single = args.only is not None and (args.only not in STEP or args.no_workspace)
    metric = METRIC if not single else f"GFLOP/s (2MNK/t) {args.only}" + (" (no workspace)" if args.no_workspace else "")
    line = {
        "metric": metric, "value": round(value, 1), "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtypes, "data": "synthetic",
        "config": {"workload": " + ".join(names), "parallelism": "single-gpu",
                   "shapes": {n: [WORKLOADS[n].M, WORKLOADS[n].N, WORKLOADS[n].K] for n in names}},
        "roofline": roof,
        "rooflines": [roofline_of(n) for n in parts],
        "parts": parts,
        "cold": cold,
        "configs": configs,
        "observed_clocks": observed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cold_timings(calls, launch, n, dev):
    """Each workload's calls timed one by one from cold caches: before every
    call a 1 GiB buffer is read (a sum), which evicts the XCDs' L2 and the
    256 MB last-level cache with clean lines, so no write-back lands in the
    timed call.  Median and minimum of the HIP-event times on the launch
    stream, after 5 untimed calls."""
    import statistics
    import torch
    scrub = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    out = {}
    for c in calls:
        w = c["w"]
        for _ in range(5):
            launch(c, False)
        saved, c["durs"] = c["durs"], []
        for _ in range(n):
            scrub.sum()
            launch(c, True)
        torch.cuda.synchronize()
        ts = [e0.elapsed_time(e1) for e0, e1 in c["durs"]]
        c["durs"] = saved
        med, lo = statistics.median(ts), min(ts)
        if w.M <= 16:
            rate, unit, peak = w.algorithmic_bytes / (med * 1e-3) / 1e9, "GB/s", PEAK_HBM_GBS
        else:
            rate, unit, peak = w.flops / (med * 1e-3) / 1e12, "TFLOP/s", PEAK_TFLOPS[w.dtype]
        out[w.name] = {"calls": n, "median_ms": round(med, 5), "min_ms": round(lo, 5), "rate_at_median": round(rate, 2),
                       "unit": unit, "frac_at_median": round(rate / peak, 4)}
    del scrub
    return out


def config_timings(make_call, launch, plan_of, n):
    """The other configurations, each timed over n back-to-back calls (HIP
    events per call on the launch stream, after 5 untimed calls): mean time,
    rate against the call's own roof, and the launch the library chose (tile,
    K split, workgroups and how many waves of the 256 compute units they
    make)."""
    import torch
    out = {}
    for name, with_ws in CONFIGS:
        c = make_call(name, with_ws)
        w = c["w"]
        for _ in range(5):
            launch(c, False)
        for _ in range(n):
            launch(c, True)
        torch.cuda.synchronize()
        ms = sum(e0.elapsed_time(e1) for e0, e1 in c["durs"]) / len(c["durs"])
        pl = plan_of(c)
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9
        bound = "hbm" if w.M <= 16 else "mfma"
        key = name if with_ws or w.M > 16 else name + "_no_workspace"
        out[key] = {
            "kernel": tg_kernel_name(pl["kernel_id"]), "workspace": with_ws, "calls": n, "ms": round(ms, 5),
            "tflops": round(tflops, 2), "gbs": round(gbs, 1), "bound": bound,
            "frac": round(gbs / PEAK_HBM_GBS if bound == "hbm" else tflops / PEAK_TFLOPS[w.dtype], 4),
            "tile": [pl["tile_m"], pl["tile_n"]], "k_splits": pl["splits"], "workgroups": pl["grid"],
            "waves_of_256": round(pl["grid"] / 256, 3), "flops": w.flops, "algorithmic_bytes": w.algorithmic_bytes,
        }
        del c
    return out


def tg_kernel_name(kernel_id):
    import tiled_gemm_f32_amd as tg
    return tg.gemm_kernel_query(kernel_id)["name"]


def cpu_baseline(calls):
    """The oracle on a bounded sample of the step, timed on the host cores."""
    import numpy as np
    import oracle
    from tiled_gemm_f32_amd.workloads import bf16_bits, make_inputs

    flops, secs, sample = 0, 0.0, []
    for c in calls:
        w = c["w"]
        rows = min(CPU_SAMPLE_ROWS.get(w.name, w.M), w.M)
        A, B, C0 = make_inputs(w)
        a = bf16_bits(A) if w.dtype == "bf16f32" else A.numpy()
        b = bf16_bits(B) if w.dtype == "bf16f32" else B.numpy()
        a = np.ascontiguousarray(a[:rows])
        c0 = np.ascontiguousarray(C0.numpy()[:rows])
        t0 = time.perf_counter()
        oracle.gemm_ref(a, b, w.alpha, w.beta, c0)
        secs += time.perf_counter() - t0
        flops += 2 * rows * w.N * w.K
        sample.append(f"{w.name}: rows 0..{rows - 1} of {w.M}")
    return {"value": round(flops / secs / 1e9, 2), "unit": "GFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(secs, 2), "sample": "; ".join(sample)}


if __name__ == "__main__":
    main()
