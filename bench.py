"""Benchmark of the multi-precision square GEMM on one MI355X.

One step is one pass of the precision sweep: C = A*B at N = 512, 1024, 2048,
4096 and 8192 (square) for FP16 (fp32 accumulate), INT8 and packed INT4
(int32 accumulate), 15 GEMMs on seeded synthetic inputs that are resident in
HBM before the timed region starts.  Two JSON lines go to stdout, the
headline last:

headline line
  value         whole-step throughput in TOPS (2*M*N*K per GEMM, summed over
                the sweep, divided by the wall time of a step)
  per_gemm      per (precision, N): mean kernel time from HIP events on the
                launch stream around every GEMM of K steps run right after the
                timed ones (the timed steps carry events around the dominant
                GEMM only), TOPS and fraction of peak; the same GEMM back to
                back (R launches captured in one HIP graph, median of 3
                replays, so that host launch cost is not timed); for N <= 2048
                also cold (each launch after a 512 MiB fill that evicts L2 and
                MALL, median of 10); and its sampled parity flag
  c3            (outside the step) the FP16 8192^3 GEMM on N(0,1)/sqrt(K)
                operands, timed between the sweep's other GEMMs and back to back
  roofline      the GEMM that takes the largest share of a step, timed by its
                HIP events inside the timed steps, against the MFMA peak of its
                own precision
  cpu_baseline  the CPU oracle (plain triple loop) timed on a row sample of
                every GEMM of the sweep and scaled to whole GEMMs, with the
                host CPU model

detail line ("kind": "bench_detail"; also written to --detail PATH)
  per_gemm      medians and minima of the in-step times, HBM rates, the
                pages' L4 figures as context
  dequant       (outside the step) the INT8 / INT4 GEMMs at N = 8192 with the
                dequantizing epilogue, ((float)S * scale_a[i]) * scale_b[j]
                rounded to binary16, timed back to back alternately with the
                plain GEMM (medians of 3), with a bit-exact sampled parity check
  layout        (outside the step) the N = 8192 GEMMs with B row-major (the
                paper's "transposed B", read with transposing LDS loads), timed
                back to back alternately with the column-major B kernel (medians
                of 3), checked bit-equal to it and against the oracle
  telemetry     (outside the step) socket power, graphics clock (mean over
                the XCDs) and hotspot temperature from amdsmi while the sweep
                runs back to back for 3 s, with the board's power limit
  shapes        (outside the step) non-square inference shapes M x 8192 x 8192,
                M in {16, 64, 256, 1024}: the first M rows of the sweep's
                N = 8192 operands, timed back to back and placed on their own
                roofline (HBM-bound below about M = 315 for f16 and i8, 157 for
                i4), with a sampled parity check; also timed with the
                dequantizing epilogue (i8, i4), with B row-major, and (i4)
                with B converted once into its FP6 image (gemm_i4_packed_b,
                checked bit-equal to the plain call)

Usage: python bench.py [--steps K] [--warmup W] [--case f16:8192] [--calib-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TOPS at N=512–8192 per precision (FP16/INT8/INT4) + % of MFMA peak"
SIZES = (512, 1024, 2048, 4096, 8192)
PRECS = ("f16", "i8", "i4")
# MI355X published dense MFMA peaks (TFLOP/s or TOPS).  gfx950 has no 4-bit
# integer MFMA; INT4 runs on the INT8 MFMA, so its peak is the INT8 one.
PEAK = {"f16": 2500.0, "i8": 5000.0, "i4": 5000.0}
HBM_PEAK_GBS = 8000.0
IN_BYTES = {"f16": 2.0, "i8": 1.0, "i4": 0.5}
SWEEP_CFG_ID = 4  # seeds of the sweep workload: (cfg_id << 32) ^ (N << 8) ^ operand
C3_CFG_ID, C3_N = 3, 8192   # FP16 8192^3 on N(0,1)/sqrt(K) operands, seeded as workload 3
# the pages' own durations for these GEMMs on an NVIDIA L4 (ms; best kernel per
# precision and size, Table I-c), reported as context only
L4_MS = {
    "f16": {512: 0.184, 1024: 1.430, 2048: 11.850, 4096: 102.350, 8192: 16500.0},
    "i8": {512: 0.109, 1024: 0.726, 2048: 5.410, 4096: 42.000, 8192: 480.060},
    "i4": {512: 0.056, 1024: 0.382, 2048: 2.810, 4096: 21.520, 8192: 167.100},
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--case", action="append", default=[],
                    help="time only prec:N (repeatable), e.g. f16:8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the power / clock sampling under sustained sweep load")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing of the N <= 2048 GEMMs")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-dequant", action="store_true",
                    help="skip the dequantizing-epilogue measurement")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the non-square (small M) measurement")
    ap.add_argument("--no-layout", action="store_true",
                    help="skip the row-major-B measurement")
    ap.add_argument("--cfg", type=int, default=None,
                    help="run every GEMM on this INT8-MFMA-path tile configuration (INT4 without the "
                         "FP6 path), e.g. 8 for the 4-wave form of the 256 x 256 tile (for profiling)")
    ap.add_argument("--no-c3", action="store_true",
                    help="skip the FP16 8192^3 N(0,1)/sqrt(K) workload")
    ap.add_argument("--detail", metavar="PATH",
                    help="also write the bench_detail JSON line to PATH")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of C per GEMM for the CPU baseline (default 192)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy, the reference for HBM counter scaling")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time every non-split tile configuration on 23 shapes x 3 precisions "
                         "(back to back, alternated) and report the picker's loss, then exit")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarise a rocprofv3 kernel_trace.csv (or counter_collection.csv) "
                         "per kernel and grid size, then exit (no GPU needed)")
    return ap.parse_args()


TILE_SWEEP_SHAPES = [(n, n, n) for n in (1024, 1536, 2048, 2560, 3072, 3584, 4096, 5120, 6144, 7168, 8192)] + [
    (8192, 6144, 8192), (4096, 8192, 4096), (12288, 4096, 4096), (2048, 8192, 8192), (1024, 8192, 8192),
    (6144, 4096, 8192), (3072, 8192, 4096), (8192, 3072, 8192), (1536, 4096, 8192), (5120, 3072, 4096),
    (10240, 2048, 4096), (2560, 6144, 4096), (256, 8192, 8192), (384, 8192, 8192), (512, 8192, 8192)]


def tile_sweep():
    """Every tile configuration without K split (and the picker's choice) on
    the shapes the picker's time model was fitted to: back-to-back time of a
    HIP graph of 10-200 launches (about 3e13 flops, at least 10), medians of
    three alternated rounds.  Prints one line per shape and the picker's mean and worst loss."""
    import torch
    import precision_dense_gemm_amd as pd
    dev = torch.device("cuda:0")
    cfgs = [0, 4, 1, 5, 2, 7, 8, 9, 10]
    compare_only = (8, 10)   # never picked: the 4-wave form of 0, and 0 on 32 x 32 MFMAs for FP16

    def graph_time(make, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            go = make()   # binds the capture stream
            for _ in range(reps):
                go()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    losses = []
    for prec in ("f16", "i8", "i4"):
        for (M, N, K) in TILE_SWEEP_SHAPES:
            if prec == "f16":
                A = (torch.rand((M, K), device=dev) * 2 - 1).half()
                B = (torch.rand((N, K), device=dev) * 2 - 1).half()
                C = torch.empty((M, N), dtype=torch.float32, device=dev)
            elif prec == "i8":
                A = torch.randint(-128, 128, (M, K), dtype=torch.int8, device=dev)
                B = torch.randint(-128, 128, (N, K), dtype=torch.int8, device=dev)
                C = torch.empty((M, N), dtype=torch.int32, device=dev)
            else:
                A = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev)
                B = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev)
                C = torch.empty((M, N), dtype=torch.int32, device=dev)
            reps = max(10, min(200, int(3e13 / (2.0 * M * N * K))))
            ts = {c: [] for c in cfgs}
            for _ in range(3):
                for c in cfgs:
                    ts[c].append(graph_time(lambda c=c: pd.prepare(prec, A, B, C, K=K, cfg=c), reps))
            med = {c: sorted(v)[1] for c, v in ts.items()}
            pick = pd.pick_config({"f16": 0, "i8": 1, "i4": 2}[prec], M, N, K)
            best = min((c for c in cfgs if c not in compare_only), key=med.get)
            loss = med[pick] / med[best] - 1
            losses.append(loss)
            print(f"{prec} {M}x{N}x{K} pick={pick} best={best} loss={100 * loss:.1f}% | "
                  + " ".join(f"{c}:{med[c]:.2f}" for c in cfgs), flush=True)
            del A, B, C
    print(f"picker loss over {len(losses)} shapes: mean {100 * sum(losses) / len(losses):.2f}%, "
          f"worst {100 * max(losses):.1f}%", flush=True)


def trace_summary(path):
    """Per (kernel, grid) dispatch statistics from rocprofv3 CSV output: durations
    from a kernel trace, and the mean of every counter from a counter collection."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(path)))
    if not rows:
        print("no rows")
        return
    keys = rows[0].keys()
    grid = [k for k in ("Grid_Size", "Grid_Size_X") if k in keys]
    wg = [k for k in ("Workgroup_Size", "Workgroup_Size_X") if k in keys]

    def short(name):
        return name.replace("(anonymous namespace)::", "").split("(")[0][:110]

    if "Start_Timestamp" in keys and "Counter_Name" not in keys:
        groups = defaultdict(list)
        for r in rows:
            g = (short(r["Kernel_Name"]), r[grid[0]] if grid else "?", r[wg[0]] if wg else "?")
            groups[g].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"{'calls':>6} {'mean_us':>10} {'min_us':>10} {'max_us':>10} {'grid':>10} {'wg':>5}  kernel")
        for (name, g, w), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            print(f"{len(d):6d} {np.mean(d):10.2f} {np.min(d):10.2f} {np.max(d):10.2f} {g:>10} {w:>5}  {name}")
    else:
        groups = defaultdict(lambda: defaultdict(list))
        for r in rows:
            g = (short(r["Kernel_Name"]), r[grid[0]] if grid else "?")
            groups[g][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for (name, g), ctrs in groups.items():
            print(f"grid {g:>10}  {name}")
            for c, v in sorted(ctrs.items()):
                print(f"    {c:28s} dispatches {len(v):5d}  mean {np.mean(v):18.1f}")


def sample_power(step, ms_per_step):
    """Run `step` back to back for about TELEMETRY_S seconds while a thread
    samples amdsmi's GPU metrics; return socket power, graphics clock and
    hotspot temperature during the load (medians / max), or None when amdsmi
    is not available."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                samples.append((time.time(), m.get("current_socket_power"), m.get("current_gfxclks"),
                                m.get("temperature_hotspot")))
            except Exception:
                pass
            stop.wait(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    steps = max(1, int(TELEMETRY_S * 1e3 / max(ms_per_step, 1e-3)))
    torch.cuda.synchronize()
    t0 = time.time()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.time()
    stop.set()
    th.join()
    try:
        limit_uw = amdsmi.amdsmi_get_power_info(handle).get("power_limit")
        amdsmi.amdsmi_shut_down()
    except Exception:
        limit_uw = None
    inside = [s for s in samples if t0 + 0.5 < s[0] < t1 - 0.1]
    power = [s[1] for s in inside if isinstance(s[1], (int, float))]
    clocks = [float(np.mean(s[2])) for s in inside if isinstance(s[2], (list, tuple)) and s[2]
              and all(isinstance(c, (int, float)) for c in s[2])]
    temps = [s[3] for s in inside if isinstance(s[3], (int, float))]
    return {
        "load_s": round(t1 - t0, 2),
        "samples": len(inside),
        "socket_power_w_median": float(np.median(power)) if power else None,
        "socket_power_w_max": float(max(power)) if power else None,
        "power_limit_w": round(limit_uw / 1e6, 1) if isinstance(limit_uw, (int, float)) else None,
        "gfxclk_mhz_median": round(float(np.median(clocks)), 1) if clocks else None,
        "temp_hotspot_c_max": float(max(temps)) if temps else None,
        "note": "amdsmi metrics refresh about once a second; samples from inside the load only",
    }


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gemm_ops(n):
    return 2.0 * n * n * n


SHAPE_MS = (16, 64, 256, 1024)   # rows of A for the non-square shapes M x 8192 x 8192
COLD_MAX_N, COLD_REPS = 2048, 10   # cold-cache timing: sweep sizes up to this N, launches each
TELEMETRY_S = 3.0                  # seconds of sustained sweep load sampled for power and clock


def kernel_name(pd, prec, n, i4_path=None):
    """The GEMM kernel the library runs for an n^3 GEMM of `prec` with column-major B."""
    if prec == "i4" and i4_path == "fp6":
        return "gemm_f6_kernel"
    cfg = pd.pick_config({"f16": pd.PREC_F16, "i8": pd.PREC_I8, "i4": pd.PREC_I4}[prec], n, n, n)
    # FP16 and INT8 run the 16 x 16 MFMA kernel on the 256 x 256, 256 x 128 and 128 x 128 tiles
    return "gemm_mf16_kernel" if prec in ("f16", "i8") and cfg in (0, 1, 4, 7) else "gemm_kernel"


def shape_roofline(prec, M, N, K, ms):
    """Achieved rate of one M x N x K GEMM against the roof that bounds it: HBM for
    algorithmic bytes / peak bandwidth above flops / peak MFMA, else MFMA."""
    flops = 2.0 * M * N * K
    nbytes = M * K * IN_BYTES[prec] + K * N * IN_BYTES[prec] + 4.0 * M * N
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (PEAK[prec] * 1e12)
    tops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    if t_hbm >= t_mfma:
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "tops": round(tops, 2)}
    return {"bound": "mfma", "achieved": round(tops, 2), "peak": PEAK[prec],
            "unit": "TFLOP/s" if prec == "f16" else "TOPS", "frac": round(tops / PEAK[prec], 4),
            "gbs": round(gbs, 1)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_n4096_n8192_hbm_counters.txt")
KERNEL_SOURCE = os.path.join(ROOT, "precision_dense_gemm_amd", "csrc", "pdgemm.hip")


def code_text(text):
    """C++ text without its // comments, indentation and blank lines (the kernel source
    holds no // inside string literals), so that a comment edit keeps the hash."""
    out = []
    for line in text.split("\n"):
        code = line.split("//", 1)[0].strip()
        if code:
            out.append(" ".join(code.split()))
    return "\n".join(out)


def kernel_source_sha(source=KERNEL_SOURCE):
    """sha256 of what decides the code a launch runs: the code (comments aside) of the
    device part of the kernel source (everything before its host-side section) and of the
    host's tile table, instantiation and tile choice (from the Config struct to the
    argument checks)."""
    import hashlib
    text = open(source, encoding="utf-8").read()
    device = text[:text.index("// host side")]
    tiles = text[text.index("struct Config {"):text.index("int validate(")]
    return hashlib.sha256(code_text(device + "\n" + tiles).encode()).hexdigest()


def measured_traffic(path=TRAFFIC_FILE, source=KERNEL_SOURCE):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    keyed "prec:N"; empty when the summary is missing or was taken on other kernels
    (its recorded kernel_source_sha differs from the current one)."""
    import re
    try:
        text = open(path).read()
        sha = kernel_source_sha(source)
    except (OSError, ValueError):
        return {}
    m = re.search(r"^source_sha256 = ([0-9a-f]{64})$", text, flags=re.M)
    if not m or m.group(1) != sha:
        return {}
    return {k: int(v) for k, v in re.findall(r"^traffic_bytes\[(\w+:\d+)\] = (\d+)$", text, flags=re.M)}


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.tile_sweep:
        tile_sweep()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(across GPUs the GEMM would shard by output panels, with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import precision_dense_gemm_amd as pd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cases = [(p, n) for n in SIZES for p in PRECS]
    if args.case:
        cases = [(c.split(":")[0], int(c.split(":")[1])) for c in args.case]

    # ---- inputs, resident in HBM before timing ----
    work = []
    host = {}
    for prec, n in cases:
        t0 = time.time()
        sa = synth.config_seed(SWEEP_CFG_ID, n, synth.OPERAND_A)
        sb = synth.config_seed(SWEEP_CFG_ID, n, synth.OPERAND_B)
        A, Bt = synth.operands(prec, n, n, n, sa, sb)
        Ad = torch.from_numpy(A).to(dev)
        Bd = torch.from_numpy(Bt).to(dev)
        C = torch.empty((n, n), dtype=torch.float32 if prec == "f16" else torch.int32, device=dev)
        host[(prec, n)] = (A, Bt)
        work.append((prec, n, Ad, Bd, C))
        log(f"[bench] inputs {prec} N={n} ready in {time.time() - t0:.1f}s")

    # config c3: the FP16 8192^3 GEMM on N(0,1)/sqrt(K) operands (its own
    # seeds), timed beside the sweep's uniform FP16 8192 entry (outside the step)
    c3 = None
    if not args.case and not args.no_c3:
        t0 = time.time()
        n3 = C3_N
        sa = synth.config_seed(C3_CFG_ID, n3, synth.OPERAND_A)
        sb = synth.config_seed(C3_CFG_ID, n3, synth.OPERAND_B)
        A3, B3 = synth.operands("f16", n3, n3, n3, sa, sb, dist="normal")
        c3 = (torch.from_numpy(A3).to(dev), torch.from_numpy(B3).to(dev),
              torch.empty((n3, n3), dtype=torch.float32, device=dev), A3, B3)
        log(f"[bench] inputs c3 f16 N={n3} N(0,1)/sqrt(K) ready in {time.time() - t0:.1f}s")

    # one prepared launcher per GEMM: arguments are checked and marshalled
    # once, so host time per launch stays far below the smallest kernel
    # INT4 runs through the workspace entry point: on the FP6 cores where the
    # library picks that path (large products), else on the INT8 MFMA; the
    # workspace is allocated here, once, outside any timed region
    workspaces = {} if args.cfg is not None else {
        (prec, n): pd.i4_workspace(n, n, n, dev) for prec, n, *_ in work if prec == "i4"}
    i4_path = {n: ("fp6" if (args.cfg is None and pd.i4_f6_pick(n, n, n) >= 0) else "i8-mfma")
               for p_, n, *_ in work if p_ == "i4"}

    def ws_of(prec, n):
        return workspaces.get((prec, n))

    launchers = {(prec, n): pd.prepare(prec, Ad, Bd, C, K=n, workspace=ws_of(prec, n), cfg=args.cfg)
                 for prec, n, Ad, Bd, C in work}
    torch.cuda.synchronize()

    def launch(prec, n, Ad, Bd, C):
        launchers[(prec, n)]()

    # ---- one parity check per GEMM (sampled entries against the oracle) ----
    parity = {}
    if not args.no_parity:
        import oracle
        for prec, n, Ad, Bd, C in work:
            launch(prec, n, Ad, Bd, C)
            torch.cuda.synchronize()
            A, Bt = host[(prec, n)]
            rng = np.random.default_rng(n)
            rows = rng.integers(0, n, 256)
            cols = rng.integers(0, n, 256)
            got = C.cpu().numpy()[rows, cols]
            if prec == "f16":
                R, S = oracle.entries_f16(A, Bt, rows, cols)
                ok = bool(np.all(np.abs(got.astype(np.float64) - R) <= 1e-3 * S))
            elif prec == "i8":
                ok = bool(np.array_equal(got.astype(np.int64), oracle.entries_i8(A, Bt, rows, cols)))
            else:
                ok = bool(np.array_equal(got.astype(np.int64), oracle.entries_i4(A, Bt, rows, cols)))
            parity[f"{prec}:{n}"] = ok
            log(f"[bench] parity {prec} N={n}: {'ok' if ok else 'FAIL'}")

    # ---- warmup, then exactly K timed steps ----
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for w in work:
            launch(*w)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    def instrumented_steps(count, only=None):
        """Run `count` steps with a HIP event pair on the launch stream around
        every GEMM (or only around `only`); return the event pairs per GEMM."""
        out = {(p, n): [] for p, n, *_ in work}
        pairs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  if only is None or (w[0], w[1]) == only else None for w in work] for _ in range(count)]
        for step in range(count):
            for w, se in zip(work, pairs[step]):
                if se is None:
                    launch(*w)
                    continue
                se[0].record(stream)
                launch(*w)
                se[1].record(stream)
                out[(w[0], w[1])].append(se)
        return out

    # The dominant GEMM (the largest share of a step) gets an event pair in
    # the timed steps, for the roofline; an event pair around every GEMM would
    # add its own cost to the step, so the per-GEMM in-step times come from
    # instrumented steps after the timed ones.
    probe = instrumented_steps(1)
    torch.cuda.synchronize()
    dom_key = max(probe, key=lambda k: probe[k][0][0].elapsed_time(probe[k][0][1]))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed = instrumented_steps(args.steps, only=dom_key)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    dom_ms = [s.elapsed_time(e) for s, e in timed[dom_key]]

    ev = instrumented_steps(args.steps)
    torch.cuda.synchronize()
    log(f"[bench] {args.steps} instrumented steps for the per-GEMM times")

    step_ops = sum(gemm_ops(n) for _, n, *_ in work)
    value = step_ops / (ms_per_step * 1e-3) / 1e12

    # Back-to-back timing of one GEMM on its own (after the timed steps): R
    # launches captured in one HIP graph and replayed, so that neither host
    # launch cost nor per-launch events enter the few-microsecond kernels;
    # inputs stay warm in L2/MALL.  make_go prepares the launch on the stream
    # current at its call (the capture stream); prepare() enqueues the first of
    # the R launches itself.  Median of `replays` replays, per launch.
    def time_b2b(make_go, est_ms, replays=3):
        reps = int(min(200, max(5, 2.0 / max(est_ms, 1e-3))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            go = make_go()
            for _ in range(reps - 1):
                go()
        g.replay()
        times = []
        for _ in range(replays):
            s0 = torch.cuda.Event(enable_timing=True)
            e0 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            g.replay()
            e0.record(stream)
            e0.synchronize()
            times.append(s0.elapsed_time(e0) / reps)
        del g, go
        return float(np.median(times))

    def plain(prec, n, Ad, Bd, C):
        return lambda: pd.prepare(prec, Ad, Bd, C, K=n, workspace=ws_of(prec, n), cfg=args.cfg)

    # Cold-cache timing of the small GEMMs (outside the step): before each
    # launch a 512 MiB fill evicts the L2s and the 256 MB MALL, so the operands
    # come from HBM; events bracket the launch alone.  Median of COLD_REPS.
    cold = {}
    if not args.no_cold:
        scrub = torch.empty(1 << 27, dtype=torch.float32, device=dev)   # 512 MiB
        for w in work:
            prec, n = w[0], w[1]
            if n > COLD_MAX_N:
                continue
            times = []
            for r in range(COLD_REPS):
                scrub.fill_(float(r))
                s0 = torch.cuda.Event(enable_timing=True)
                e0 = torch.cuda.Event(enable_timing=True)
                s0.record(stream)
                launch(*w)
                e0.record(stream)
                e0.synchronize()
                times.append(s0.elapsed_time(e0))
            cold[(prec, n)] = float(np.median(times))
        del scrub

    # config c3 (outside the step): events around each of `steps` launches
    # separated by the sweep's other GEMMs (as inside a step), and back to back
    c3_entry = None
    if c3 is not None:
        A3d, B3d, C3d, A3, B3 = c3
        go3 = pd.prepare("f16", A3d, B3d, C3d, K=C3_N)
        torch.cuda.synchronize()
        if not args.no_parity:
            import oracle
            rng = np.random.default_rng(C3_N + 3)
            rows, cols = rng.integers(0, C3_N, 256), rng.integers(0, C3_N, 256)
            R, S = oracle.entries_f16(A3, B3, rows, cols)
            got = C3d.cpu().numpy()[rows, cols]
            parity["c3"] = bool(np.all(np.abs(got.astype(np.float64) - R) <= 1e-3 * S))
            log(f"[bench] parity c3: {'ok' if parity['c3'] else 'FAIL'}")
        times = []
        for _ in range(args.steps):
            for w in work:
                if (w[0], w[1]) != ("f16", 8192):
                    launch(*w)
            s0 = torch.cuda.Event(enable_timing=True)
            e0 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            go3()
            e0.record(stream)
            times.append((s0, e0))
        torch.cuda.synchronize()
        ms3 = float(np.mean([a.elapsed_time(b) for a, b in times]))
        ms3_b = time_b2b(lambda: pd.prepare("f16", A3d, B3d, C3d, K=C3_N), ms3)
        tops3 = gemm_ops(C3_N) / (ms3 * 1e-3) / 1e12
        tops3_b = gemm_ops(C3_N) / (ms3_b * 1e-3) / 1e12
        c3_entry = {"workload": f"f16 {C3_N}^3, N(0,1)/sqrt(K)", "ms": round(ms3, 5), "tops": round(tops3, 1),
                    "frac": round(tops3 / PEAK["f16"], 4), "ms_b2b": round(ms3_b, 5),
                    "tops_b2b": round(tops3_b, 1), "frac_b2b": round(tops3_b / PEAK["f16"], 4)}
        if "c3" in parity:
            c3_entry["parity"] = parity["c3"]
        log(f"[bench] c3: {ms3:.4f} ms in sweep order, {ms3_b:.4f} ms back to back")
        del times

    b2b = {}
    for w in work:
        prec, n = w[0], w[1]
        est = float(np.mean([s.elapsed_time(e) for s, e in ev[(prec, n)]])) if ev[(prec, n)] else 1.0
        b2b[(prec, n)] = time_b2b(plain(*w), est)

    # ---- power and clock under sustained load (outside the timed steps) ----
    # amdsmi's metrics table refreshes about once a second, far slower than a
    # step, so the sweep runs for TELEMETRY_S while a thread samples it; only
    # samples taken well inside the load are kept.
    telemetry = None
    if not args.no_telemetry:
        telemetry = sample_power(lambda: [launch(*w) for w in work], ms_per_step)

    # ---- the dequantizing epilogue at N = 8192 (not part of the step) ----
    dequant = {}
    if not args.no_dequant:
        for prec, n, Ad, Bd, C in work:
            if prec == "f16" or n != 8192:
                continue
            sa_h = synth.f32_scales(n, synth.config_seed(SWEEP_CFG_ID, n, synth.OPERAND_A) + 2)
            sb_h = synth.f32_scales(n, synth.config_seed(SWEEP_CFG_ID, n, synth.OPERAND_B) + 3)
            sad, sbd = torch.from_numpy(sa_h).to(dev), torch.from_numpy(sb_h).to(dev)
            Ch = torch.empty((n, n), dtype=torch.float16, device=dev)
            def dequant_go():
                return pd.prepare(prec, Ad, Bd, Ch, K=n, scales=(sad, sbd), workspace=ws_of(prec, n))
            dequant_go()
            torch.cuda.synchronize()
            entry = {"out": "f16"}
            if not args.no_parity:
                import oracle
                A, Bt = host[(prec, n)]
                rng = np.random.default_rng(n + 1)
                rows, cols = rng.integers(0, n, 256), rng.integers(0, n, 256)
                S = (oracle.entries_i8 if prec == "i8" else oracle.entries_i4)(A, Bt, rows, cols)
                want = oracle.dequant_entries(S, sa_h[rows], sb_h[cols], half_out=True)
                got = Ch.cpu().numpy()[rows, cols]
                ok = bool(np.array_equal(got.view(np.uint16), want.view(np.uint16)))
                entry["parity"] = ok
                parity[f"{prec}:{n}:dequant"] = ok
                log(f"[bench] parity {prec} N={n} dequant->f16: {'ok' if ok else 'FAIL'}")
            # alternate the two so that clock and power drift hit both alike
            ds, rs = [], []
            for _ in range(3):
                ds.append(time_b2b(dequant_go, b2b[(prec, n)]))
                rs.append(time_b2b(plain(prec, n, Ad, Bd, C), b2b[(prec, n)]))
            ms_d, ms_r = float(np.median(ds)), float(np.median(rs))
            entry.update({
                "ms_back_to_back": round(ms_d, 5),
                "tops_back_to_back": round(gemm_ops(n) / (ms_d * 1e-3) / 1e12, 2),
                "frac_of_peak": round(gemm_ops(n) / (ms_d * 1e-3) / 1e12 / PEAK[prec], 4),
                "plain_ms_back_to_back": round(ms_r, 5),
                "time_vs_plain": round(ms_d / ms_r, 4),
            })
            dequant[f"{prec}:{n}"] = entry
            log(f"[bench] dequant {prec} N={n}: {ms_d:.4f} ms (plain {ms_r:.4f} ms)")
            del Ch, sad, sbd

    # ---- B row-major at N = 8192 (not part of the step) ----
    layout = {}
    brow_dev = {}   # the row-major B of each precision, reused by the shape section
    if not args.no_layout:
        for prec, n, Ad, Bd, C in work:
            if n != 8192:
                continue
            A, Bt = host[(prec, n)]
            if prec == "i4":
                Brow = synth.pack_int4(np.ascontiguousarray(synth.unpack_int4(Bt).T))
            else:
                Brow = np.ascontiguousarray(Bt.T)
            Brd = torch.from_numpy(Brow).to(dev)
            Cr = torch.empty_like(C)
            def rowb_go():
                return pd.prepare(prec, Ad, Brd, Cr, K=n, rowb=True, workspace=ws_of(prec, n))
            rowb_go()
            launchers[(prec, n)]()
            torch.cuda.synchronize()
            entry = {"same_as_column_major": bool(torch.equal(Cr.view(torch.int32), C.view(torch.int32)))}
            if not args.no_parity:
                import oracle
                rng = np.random.default_rng(n + 2)
                rows, cols = rng.integers(0, n, 256), rng.integers(0, n, 256)
                got = Cr.cpu().numpy()[rows, cols]
                if prec == "f16":
                    R, S = oracle.entries_f16_rowb(A, Brow, rows, cols)
                    ok = bool(np.all(np.abs(got.astype(np.float64) - R) <= 1e-3 * S))
                else:
                    ref = (oracle.entries_i8_rowb if prec == "i8" else oracle.entries_i4_rowb)(
                        A, Brow, rows, cols)
                    ok = bool(np.array_equal(got.astype(np.int64), ref))
                entry["parity"] = ok and entry["same_as_column_major"]
                parity[f"{prec}:{n}:rowb"] = entry["parity"]
            rs, cs = [], []
            for _ in range(3):
                rs.append(time_b2b(rowb_go, b2b[(prec, n)]))
                cs.append(time_b2b(plain(prec, n, Ad, Bd, C), b2b[(prec, n)]))
            ms_r, ms_c = float(np.median(rs)), float(np.median(cs))
            entry.update({
                "ms_back_to_back": round(ms_r, 5),
                "tops_back_to_back": round(gemm_ops(n) / (ms_r * 1e-3) / 1e12, 2),
                "frac_of_peak": round(gemm_ops(n) / (ms_r * 1e-3) / 1e12 / PEAK[prec], 4),
                "column_major_ms_back_to_back": round(ms_c, 5),
                "time_vs_column_major": round(ms_r / ms_c, 4),
            })
            layout[f"{prec}:{n}"] = entry
            log(f"[bench] row-major B {prec} N={n}: {ms_r:.4f} ms (column-major {ms_c:.4f} ms)")
            brow_dev[prec] = Brd
            del Cr

    # ---- non-square inference shapes (not part of the step) ----
    shapes = {}
    if not args.no_shapes:
        for prec, n, Ad, Bd, C in work:
            if n != 8192:
                continue
            # INT4 with B converted once into its FP6 image (weights packed ahead
            # of the calls); each call converts only A
            img_b = pd.i4_f6_pack(Bd, n) if prec == "i4" else None
            for M in SHAPE_MS:
                Cm = torch.empty((M, n), dtype=C.dtype, device=dev)
                def shape_go():
                    return pd.prepare(prec, Ad[:M], Bd, Cm, K=n)
                shape_go()
                torch.cuda.synchronize()
                entry = {"M": M, "N": n, "K": n,
                         "cfg": pd.pick_config({"f16": 0, "i8": 1, "i4": 2}[prec], M, n, n)}
                if not args.no_parity:
                    import oracle
                    A, Bt = host[(prec, n)]
                    rng = np.random.default_rng(M)
                    rows, cols = rng.integers(0, M, 256), rng.integers(0, n, 256)
                    got = Cm.cpu().numpy()[rows, cols]
                    if prec == "f16":
                        R, S = oracle.entries_f16(A, Bt, rows, cols)
                        ok = bool(np.all(np.abs(got.astype(np.float64) - R) <= 1e-3 * S))
                    else:
                        ref = (oracle.entries_i8 if prec == "i8" else oracle.entries_i4)(A, Bt, rows, cols)
                        ok = bool(np.array_equal(got.astype(np.int64), ref))
                    entry["parity"] = ok
                    parity[f"{prec}:{M}x{n}x{n}"] = ok
                ms = time_b2b(shape_go, 0.05)
                entry["ms_back_to_back"] = round(ms, 5)
                entry["roofline"] = shape_roofline(prec, M, n, n, ms)
                if prec != "f16":
                    # the same product with the dequantizing epilogue to binary16 (the
                    # scales of the dequant section, first M rows)
                    sah = synth.f32_scales(n, synth.config_seed(SWEEP_CFG_ID, n, synth.OPERAND_A) + 2)[:M]
                    sbh = synth.f32_scales(n, synth.config_seed(SWEEP_CFG_ID, n, synth.OPERAND_B) + 3)
                    Ch = torch.empty((M, n), dtype=torch.float16, device=dev)
                    scl = (torch.from_numpy(sah).to(dev), torch.from_numpy(sbh).to(dev))
                    entry["dequant_f16_ms_back_to_back"] = round(time_b2b(
                        lambda: pd.prepare(prec, Ad[:M], Bd, Ch, K=n, scales=scl), 0.05), 5)
                    del Ch, scl
                if img_b is not None:
                    Cp = torch.empty((M, n), dtype=torch.int32, device=dev)
                    wsp = torch.empty(max(pd.i4_f6_image_bytes(M, n), 16), dtype=torch.uint8, device=dev)
                    def packed_go():
                        go = lambda: pd.gemm_i4_packed_b(Ad[:M], img_b, n, n, out=Cp, workspace=wsp)
                        go()
                        return go
                    packed_go()
                    torch.cuda.synchronize()
                    entry["packed_b_same_bits"] = bool(torch.equal(Cp, Cm))
                    entry["packed_b_ms_back_to_back"] = round(time_b2b(packed_go, 0.05), 5)
                    del Cp, wsp
                if prec in brow_dev:
                    # the same product with B row-major (integers: K split across
                    # workgroups where pick_splits asks), checked on the same entries
                    entry["rowb_splits"] = list(pd.pick_splits({"f16": 0, "i8": 1, "i4": 2}[prec], M, n, n,
                                                               rowb=True))
                    rowb_go = pd.prepare(prec, Ad[:M], brow_dev[prec], Cm, K=n, rowb=True)
                    rowb_go()
                    torch.cuda.synchronize()
                    if not args.no_parity:
                        got = Cm.cpu().numpy()[rows, cols]
                        if prec == "f16":
                            ok = bool(np.all(np.abs(got.astype(np.float64) - R) <= 1e-3 * S))
                        else:
                            ok = bool(np.array_equal(got.astype(np.int64), ref))
                        entry["rowb_parity"] = ok
                        parity[f"{prec}:{M}x{n}x{n}:rowb"] = ok
                    entry["rowb_ms_back_to_back"] = round(time_b2b(
                        lambda: pd.prepare(prec, Ad[:M], brow_dev[prec], Cm, K=n, rowb=True), 0.05), 5)
                shapes[f"{prec}:{M}x{n}x{n}"] = entry
                log(f"[bench] shape {prec} {M}x{n}x{n}: {ms * 1e3:.1f} us "
                    f"({entry['roofline']['bound']} {entry['roofline']['frac']:.3f})")
                del Cm

    per = {}      # full per-GEMM detail (printed on the detail line)
    for (prec, n), pairs in ev.items():
        times = [s.elapsed_time(e) for s, e in pairs]
        ms = float(np.mean(times)) if times else float("nan")
        tops = gemm_ops(n) / (ms * 1e-3) / 1e12
        hbm_bytes = n * n * (2 * IN_BYTES[prec] + 4)
        ms_b = b2b[(prec, n)]
        per[f"{prec}:{n}"] = {
            "ms": round(ms, 5),
            "ms_median": round(float(np.median(times)), 5) if times else None,
            "ms_min": round(float(np.min(times)), 5) if times else None,
            "tops": round(tops, 2),
            "frac_of_peak": round(tops / PEAK[prec], 4),
            "ms_back_to_back": round(ms_b, 5),
            "tops_back_to_back": round(gemm_ops(n) / (ms_b * 1e-3) / 1e12, 2),
            "min_hbm_gbs": round(hbm_bytes / (ms * 1e-3) / 1e9, 1),
            **({"ms_cold": round(cold[(prec, n)], 5),
                "cold_min_hbm_gbs": round(hbm_bytes / (cold[(prec, n)] * 1e-3) / 1e9, 1)}
               if (prec, n) in cold else {}),
            "l4_tops_context": round(gemm_ops(n) / (L4_MS[prec][n] * 1e-3) / 1e12, 3),
        }
        if f"{prec}:{n}" in parity:
            per[f"{prec}:{n}"]["parity"] = parity[f"{prec}:{n}"]

    traffic = measured_traffic()
    for key, nbytes in traffic.items():
        if key in per:
            per[key]["hbm_bytes_profiled"] = nbytes

    # dominant kernel: the largest share of a step, timed by its own event
    # pairs inside the timed steps
    dprec, dn = dom_key
    dom = f"{dprec}:{dn}"
    dom_tops = gemm_ops(dn) / (float(np.mean(dom_ms)) * 1e-3) / 1e12
    per[dom]["ms_timed_steps"] = round(float(np.mean(dom_ms)), 5)
    roofline = {
        "bound": "mfma",
        "kernel": f"{kernel_name(pd, dprec, dn, i4_path.get(dn))} {dprec} N={dn}",
        "achieved": round(dom_tops, 2),
        "peak": PEAK[dprec],
        "unit": "TFLOP/s" if dprec == "f16" else "TOPS",
        "frac": round(dom_tops / PEAK[dprec], 4),
        # HBM bytes per launch, rocprofv3 counters scaled by a 1 GiB copy
        "traffic": traffic.get(dom),
    }

    # ---- CPU baseline: the oracle on a row sample of every GEMM ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        rows = args.cpu_rows or 192
        total_s = 0.0
        sampled_ops = 0.0
        for prec, n, *_ in work:
            A, Bt = host[(prec, n)]
            r = min(rows, n)
            t0 = time.perf_counter()
            if prec == "f16":
                oracle.gemm_f16(A[:r], Bt, threads=threads)
            elif prec == "i8":
                oracle.gemm_i8(A[:r], Bt, threads=threads)
            else:
                oracle.gemm_i4(A[:r], Bt, threads=threads)
            dt = time.perf_counter() - t0
            sampled_ops += 2.0 * r * n * n
            total_s += dt * (n / r)   # every row of C costs the same
            log(f"[bench] cpu oracle {prec} N={n}: {r} rows in {dt:.2f}s")
        cpu = {
            "value": round(step_ops / total_s / 1e12, 6),
            "unit": "TOPS",
            "cores": threads,
            "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"first {rows} rows of C for each of the {len(work)} GEMMs "
                      f"({sampled_ops / 1e9:.1f} GOP), time scaled by N/{rows} per GEMM",
        }

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 1 GiB device-to-device")

    # the headline line carries the metric for every GEMM of the sweep in a
    # compact form: in-step ms, TOPS and fraction of peak, back-to-back ms and
    # fraction of peak (cold times and the rest are on the detail line)
    compact = {}
    for key, e in per.items():
        c = {"ms": e["ms"], "tops": round(e["tops"], 1), "frac": e["frac_of_peak"],
             "ms_b2b": e["ms_back_to_back"],
             "frac_b2b": round(e["tops_back_to_back"] / PEAK[key.split(":")[0]], 4)}
        if key.startswith("i4:"):
            c["path"] = i4_path[int(key.split(":")[1])]
        compact[key] = c

    detail = {
        "kind": "bench_detail",
        "per_gemm": per,
        "dequant": dequant or None,
        "layout": layout or None,
        "shapes": shapes or None,
        "telemetry": telemetry,
    }
    detail_text = json.dumps(detail)
    if args.detail:
        with open(args.detail, "w") as f:
            f.write(detail_text + "\n")
    print(detail_text, flush=True)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16,i8,i4",
        "data": "synthetic (SplitMix64-seeded; f16 U[-1,1], i8 U[-128,127], i4 U[-8,7])",
        "config": {
            "workload": "square GEMM sweep N in {512,1024,2048,4096,8192} x {f16->f32, i8->i32, i4->i32}"
                        if not args.case else "square GEMM " + ", ".join(args.case),
            "gemms_per_step": len(work),
            "layout": "A row-major, B column-major, C row-major",
        },
        "per_gemm": compact,
        # every timed GEMM's sampled-entry check against the oracle (per GEMM on the detail line)
        "parity": (all(parity.values()) if parity else None),
        "c3": c3_entry,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out, separators=(",", ":")), flush=True)
    if parity and not all(parity.values()):
        sys.exit(1)


if __name__ == "__main__":
    main()
