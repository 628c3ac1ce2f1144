"""Benchmark of the BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
    python bench.py --counters            (run under rocprofv3 --pmc, see below)
    python bench.py --counter-summary FETCH_CSV WRITE_CSV

Headline workload: decode GEMV at batch 1 on the 2B-class shapes, K=2560 ->
N=6912 and K=6912 -> N=2560, bf16 activations with 1% x20 outliers.  One step
is the whole inference hot path for one token through both BitLinears:
per-token int8 quantization then the ternary product with fused dequant
(weights are packed once, before timing).  Inputs are resident in HBM; the
packed weights rotate over enough distinct copies (> 2x the 256 MB Infinity
Cache) that every step streams them from HBM.  The K timed steps are one HIP
graph replay (no host launch overhead inside the timed region).

value = packed weight bytes of the step x K / elapsed time, in GB/s.

Also printed on the same JSON line:
  roofline      the decode kernel: algorithmic bytes per launch / its average
                launch duration (HIP events on the launch stream around a
                graph of back-to-back launches), against the 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle (plain C, OpenMP over outputs) running the same
                step on the host cores, on a bounded number of repetitions, and
                on one thread (value_1thread);
  roofline.traffic  measured HBM bytes per launch of the same kernel, from two
                rocprofv3 --pmc runs of `bench.py --counters` (FETCH_SIZE, then
                WRITE_SIZE, KiB per dispatch), each scaled by the factor that
                makes the same counter read the known size of a 64 MiB device
                copy in the same run; `--counter-summary` turns the two CSV
                files into profiles/traffic_gemv_fused_decode_2b_m1.txt, which
                records a hash of the kernel sources; the field is null when
                the sources have changed since;
  also          the other workloads: one decode step over the 30-layer 2B-class
                stack (210 BitLinears + glue, batch 1 and 8) in tokens/s,
                checked bit for bit against the oracle's chain; 100B-class
                decode (M = 1, 8, 32) in GB/s; binary-weight (b1) and base-3
                (b3) decode on the 2B and 100B shapes (M = 1, 8); prefill GEMMs (2B M=2048,
                100B M=512), ternary and binary, in int8 TOPS; the training
                products (straight-through forward, input and weight
                gradients, 2B shapes, 2048 tokens) in bf16 TFLOP/s;
  clocks        the shader and memory clock levels the driver reported while
                the timed graphs ran (min / median / max of 1 ms samples).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

import bitlinear_matmul_02_amd as bl
import workloads

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_fused_decode_2b_m1.txt")
KERNEL_SOURCES = ("bitlinear_matmul_02_amd/csrc/gemv.hip", "bitlinear_matmul_02_amd/csrc/bl_internal.h")
CAL_BYTES = 64 << 20  # calibration copy
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA, MI355X
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--counters", action="store_true",
                    help="launch the headline kernels and a calibration copy for rocprofv3 --pmc, then exit")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 --pmc CSV files, then exit")
    ap.add_argument("--extras", default=None,
                    help="comma-separated secondary workloads to run beside the headline (default: all; "
                         "names as in the 'also' object)")
    ap.add_argument("--trace-summary", nargs="+", metavar=("DB", "REGEX"),
                    help="per-kernel table of a rocprofv3 --kernel-trace database (kernels whose name matches "
                         "REGEX), then exit")
    ap.add_argument("--pmc-table", nargs="+", metavar=("CSV", "REGEX"),
                    help="per-kernel means of the counters in a rocprofv3 --pmc CSV file (kernels whose name "
                         "matches REGEX), then exit")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
class Linear:
    """Device buffers of one BitLinear used in a timed step.

    mode "fused": one launch (bitlinear_forward_decode);
    mode "gemv" / "gemm": bitlinear_quant_act then the product call."""

    def __init__(self, M, K, N, packed_copies, beta, x, y_dtype=torch.float32, mode=None):
        dev = x.device
        self.M, self.K, self.N = M, K, N
        self.packed = packed_copies
        self.beta = beta
        self.x = x
        if mode is None:
            # the fused decode kernel wins while the quantization it repeats per
            # workgroup is small (measured: M <= 4); the GEMV otherwise
            mode = "fused" if (M <= 4 and bl.decode_fits(M, K)) else ("gemv" if M <= bl.GEMV_MAX_M else "gemm")
        self.mode = mode
        self.x_q = torch.empty((M, bl.act_stride(K)), dtype=torch.int8, device=dev)
        self.x_ds = torch.empty((M,), dtype=torch.float32, device=dev)
        self.y = torch.empty((M, N), dtype=y_dtype, device=dev)
        if mode == "gemm":
            nbytes, self.product = bl.gemm_workspace_bytes(M, N, K), bl.bitlinear_gemm
        else:
            nbytes, self.product = bl.gemv_workspace_bytes(M, N, K), bl.bitlinear_gemv
        self.ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev) if nbytes > 0 else None

    def weight_bytes(self):
        return self.N * self.K // 4

    def traffic_bytes(self):
        """Algorithmic HBM bytes of the timed kernel: packed weights once, its
        activation input once (bf16 x when fused, int8 rows otherwise), y once."""
        act = self.M * self.K * self.x.element_size() if self.mode == "fused" else self.M * bl.act_stride(self.K)
        return self.weight_bytes() + act + self.M * self.N * self.y.element_size()

    def quant(self):
        if self.mode != "fused":
            bl.bitlinear_quant_act(self.x, self.x_q, self.x_ds)

    def run_product(self, r):
        packed = self.packed[r % len(self.packed)]
        if self.mode == "fused":
            bl.bitlinear_forward_decode(self.x, packed, self.beta, self.N, self.y)
        else:
            self.product(self.x_q, self.x_ds, self.K, packed, self.beta, self.N, self.y, self.ws)

    def step(self, r):
        self.quant()
        self.run_product(r)


def rotation(per_step_bytes):
    return int(max(1, min(256, -(-2 * MALL_BYTES // max(per_step_bytes, 1)) + 1)))


def pack_from_host(w_np, dev):
    return bl.pack_weights(torch.from_numpy(w_np).to(dev))


def copies_of(packed, n):
    return [packed] + [packed.clone() for _ in range(n - 1)]


def capture(fn, nsteps):
    """One HIP graph holding fn(0) ... fn(nsteps - 1)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # one eager call first (loads code objects)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(nsteps):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def capture_steps(linears, nsteps):
    def one(i):
        for lin in linears:
            lin.step(i)
    return capture(one, nsteps)


class ClockSampler:
    """The GPU's current shader (sclk) and memory (mclk) clock levels, read
    from the driver's pp_dpm_* files by a background thread every `period`
    seconds, kept only while a timed graph replay is in flight."""

    def __init__(self, period=0.001):
        import glob
        import threading
        self.files = {}
        for key in ("sclk", "mclk"):
            found = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_" + key))
            if found:
                self.files[key] = found[0]
        self.samples = {k: [] for k in self.files}
        self.busy = False
        self.period = period
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if self.files else None
        if self._thread:
            self._thread.start()

    @staticmethod
    def _current(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().split("Mhz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.wait(self.period):
            if not self.busy:
                continue
            for k, path in self.files.items():
                v = self._current(path)
                if v is not None and self.busy:
                    self.samples[k].append(v)

    def summary(self):
        self._stop.set()
        out = {}
        for k, v in self.samples.items():
            if v:
                out[k + "_mhz"] = {"min": min(v), "median": float(np.median(v)), "max": max(v), "samples": len(v)}
        if not out:
            return None
        out["source"] = "current pp_dpm_sclk / pp_dpm_mclk level, polled every 1 ms during the timed graph replays"
        return out


CLOCKS = None


def time_graph(g, reps=1):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if CLOCKS:
        CLOCKS.busy = True
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    if CLOCKS:
        CLOCKS.busy = False
    return a.elapsed_time(b) / 1e3, time.perf_counter() - t0


def kernel_duration(lin, launches=200):
    """Average duration of the product kernel: HIP events on the launch stream
    around a graph of `launches` back-to-back launches (weight copies rotate)."""
    lin.quant()
    g = capture(lambda i: lin.run_product(i), launches)
    time_graph(g)
    el, _ = time_graph(g)
    return el / launches


# --------------------------------------------------------------- headline
def headline(args, dev):
    wl = workloads.DECODE_2B
    host = []
    for i, lin in enumerate(wl.linears):
        w = workloads.gen_weights(lin.N, lin.K, seed=2 * i)
        xb = workloads.gen_acts_bf16(lin.M, lin.K, seed=2 * i + 1, outliers=lin.outliers)
        host.append((w, xb))
    per_step = sum(l.N * l.K // 4 for l in wl.linears)
    R = rotation(per_step)
    linears = []
    for (w, xb), lin in zip(host, wl.linears):
        packed, beta = pack_from_host(w, dev)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        linears.append(Linear(lin.M, lin.K, lin.N, copies_of(packed, R), beta, x))

    # sanity: the timed path reproduces the oracle on this input
    import oracle
    for (w, xb), L in zip(host, linears):
        L.quant()
        L.run_product(0)
        torch.cuda.synchronize()
        ref = oracle.bitlinear_forward(xb, w, threads=8)
        if not np.array_equal(L.y.cpu().numpy(), ref["y"]):
            raise SystemExit("bench: GPU output differs from the oracle on the headline workload")

    g_warm = capture_steps(linears, max(args.warmup, 1))
    g_main = capture_steps(linears, args.steps)
    time_graph(g_warm)
    elapsed, wall = time_graph(g_main)
    value = per_step * args.steps / elapsed / 1e9

    durs = [kernel_duration(L) for L in linears]
    bytes_per = [L.traffic_bytes() for L in linears]
    # the same step with the standalone quantizer (two launches per BitLinear)
    split = [Linear(L.M, L.K, L.N, L.packed, L.beta, L.x, mode="gemv") for L in linears]
    g_split = capture_steps(split, args.steps)
    time_graph(g_split)
    el_split, _ = time_graph(g_split)
    achieved = sum(bytes_per) / sum(durs) / 1e9
    out = {
        "value": value, "ms_per_step": elapsed / args.steps * 1e3, "wall_s": wall,
        "rotation_copies": R,
        "unfused_us_per_step": round(el_split / args.steps * 1e6, 2),
        "kernel_us": {"%dx%d->%d" % (L.M, L.K, L.N): round(d * 1e6, 3) for L, d in zip(linears, durs)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "gemv_t2_kernel (fused quantization)", "bytes_per_launch": bytes_per},
    }
    return out, host, wl


# ------------------------------------------------------- HBM traffic counters
def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def headline_linears(dev, R):
    wl = workloads.DECODE_2B
    out = []
    for i, lin in enumerate(wl.linears):
        w = workloads.gen_weights(lin.N, lin.K, seed=2 * i)
        xb = workloads.gen_acts_bf16(lin.M, lin.K, seed=2 * i + 1, outliers=lin.outliers)
        packed, beta = pack_from_host(w, dev)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        out.append(Linear(lin.M, lin.K, lin.N, copies_of(packed, R), beta, x))
    return out


def counters_run(dev):
    """Dispatches for counter collection: a 64 MiB device copy (calibration),
    then each headline kernel COUNTER_LAUNCHES times over rotating weight copies."""
    launches = COUNTER_LAUNCHES
    src = torch.ones(CAL_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    linears = headline_linears(dev, rotation(sum(l.N * l.K // 4 for l in workloads.DECODE_2B.linears)))
    for L in linears:
        for i in range(launches):
            L.run_product(i)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": [L.traffic_bytes() for L in linears]}), flush=True)


def _counter_rows(path, counter):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return sorted(rows)


def _short_kernel(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("bl::", "")
    depth = 0
    for i, ch in enumerate(name):  # cut the argument list after the template arguments
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return name[:i]
    return name


def trace_summary(db, regex=None):
    """Markdown table of per-kernel dispatch durations from a rocprofv3 kernel trace."""
    import re
    import sqlite3
    pat = re.compile(regex) if regex else None
    con = sqlite3.connect(db)
    groups = {}
    for name, gx, wx, dur, lds, vgpr in con.execute(
            "select name, grid_x, workgroup_x, duration, lds_size, vgpr_count from kernels"):
        if pat and not pat.search(name):
            continue
        key = (_short_kernel(name), gx // max(wx, 1), wx, lds, vgpr)
        groups.setdefault(key, []).append(dur)
    print("| kernel | workgroups x threads | LDS B | VGPRs | dispatches | mean us | median us | min us |")
    print("|---|---|---|---|---|---|---|---|")
    for key, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        print("| `%s` | %d x %d | %d | %d | %d | %.2f | %.2f | %.2f |"
              % (key[0][:70], key[1], key[2], key[3], key[4], len(v), sum(v) / len(v) / 1e3, v[len(v) // 2] / 1e3,
                 v[0] / 1e3))


def pmc_table(path, regex=None):
    """Markdown table of per-kernel counter means (one row per kernel and grid)."""
    import re
    pat = re.compile(regex) if regex else None
    csv.field_size_limit(1 << 30)
    groups, counters = {}, []
    with open(path) as f:
        for r in csv.DictReader(f):
            if pat and not pat.search(r["Kernel_Name"]):
                continue
            key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1))
            c = r["Counter_Name"]
            if c not in counters:
                counters.append(c)
            groups.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    print("| kernel | workgroups | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for key, d in groups.items():
        vals = ["%.4g" % (sum(d[c]) / len(d[c])) if c in d else "" for c in counters]
        print("| `%s` | %d | %s |" % (key[0][:70], key[1], " | ".join(vals)))


COUNTER_LAUNCHES = 16  # dispatches per headline shape in counters_run, in workload order


def counter_summary(fetch_csv, write_csv):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the calibration copy
    and write the per-launch HBM traffic of the headline kernels."""
    lins = workloads.DECODE_2B.linears
    labels = ["%dx%d->%d" % (l.M, l.K, l.N) for l in lins]
    algo = [l.N * l.K // 4 + l.M * l.K * 2 + l.M * l.N * 4 for l in lins]  # packed + bf16 x + fp32 y
    factors, med, names = {}, {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        cal = [v for _, name, _, v in rows if "copyBuffer" in name and v * 1024 > CAL_BYTES / 4]
        if not cal:
            raise SystemExit("no calibration copy dispatch in %s" % path)
        factors[counter] = CAL_BYTES / (float(np.median(cal)) * 1024)
        gemv = [(name, grid, v) for _, name, grid, v in rows if "gemv_t2_kernel" in name]
        if len(gemv) != COUNTER_LAUNCHES * len(lins):
            raise SystemExit("expected %d kernel dispatches in %s, found %d" % (COUNTER_LAUNCHES * len(lins), path, len(gemv)))
        for i in range(len(lins)):
            part = gemv[i * COUNTER_LAUNCHES:(i + 1) * COUNTER_LAUNCHES]
            med[(counter, i)] = float(np.median([v for _, _, v in part]))
            names[i] = (part[0][0].split("(GemvArgs")[0].replace("void ", "").replace("(anonymous namespace)::", ""),
                        part[0][1])
    lines, traffic = [], []
    for i, lab in enumerate(labels):
        rd = med[("FETCH_SIZE", i)] * 1024 * factors["FETCH_SIZE"]
        wr = med[("WRITE_SIZE", i)] * 1024 * factors["WRITE_SIZE"]
        traffic.append(rd + wr)
        lines.append("%-14s %s grid=%d threads: FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB (median of %d dispatches)"
                     % (lab, names[i][0], names[i][1], med[("FETCH_SIZE", i)], med[("WRITE_SIZE", i)], COUNTER_LAUNCHES))
        lines.append("%-14s -> read %.0f B + write %.0f B = %.0f B per launch; algorithmic %d B; ratio %.3f"
                     % ("", rd, wr, rd + wr, algo[i], (rd + wr) / algo[i]))
    mean = sum(traffic) / len(traffic)
    text = [
        "HBM traffic of the fused decode kernel (gemv_t2_kernel, fused quantization), 2B-class shapes, batch 1",
        "",
        "commands (run from the repository root on one MI355X):",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- python bench.py --counters",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- python bench.py --counters",
        "  python bench.py --counter-summary gpurun_out/pmc_fetch/run_counter_collection.csv "
        "gpurun_out/pmc_write/run_counter_collection.csv",
        "",
        "calibration: a 64 MiB device copy (__amd_rocclr_copyBuffer) in the same run;",
        "  FETCH_SIZE factor %.5f (the counter reads %.0f KiB for 65536 KiB moved)" % (factors["FETCH_SIZE"], 65536 / factors["FETCH_SIZE"]),
        "  WRITE_SIZE factor %.5f" % factors["WRITE_SIZE"],
        "",
    ] + lines + [
        "",
        "traffic_bytes_per_launch_mean = %.0f" % mean,
        "kernel_source_hash = %s" % kernel_source_hash(),
    ]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def measured_traffic():
    """Mean measured HBM bytes per launch of the headline kernel, or None when
    the summary is missing or older than the kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(" = ", 1) for l in f.read().splitlines() if " = " in l)
    except OSError:
        return None
    if kv.get("kernel_source_hash", "").strip() != kernel_source_hash():
        return None
    return round(float(kv["traffic_bytes_per_launch_mean"]))


def cpu_baseline(host, wl, budget_s=10.0):
    import oracle
    threads = min(16, os.cpu_count() or 1)
    prepared = []
    for (w, xb), lin in zip(host, wl.linears):
        beta = oracle.absmean(w)
        prepared.append((oracle.ternarize(w, beta), beta, xb))
    per_step = sum(l.N * l.K // 4 for l in wl.linears)

    def run(nthreads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            for t, beta, xb in prepared:
                q, ds, _ = oracle.quant_act(xb, bf16_bits=True)
                acc = oracle.matmul_i32(q, t, threads=nthreads)
                oracle.dequant(acc, ds, beta)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    reps, el = run(threads, budget_s)
    reps1, el1 = run(1, budget_s / 3)
    return {"value": round(per_step * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d decode steps (quantize + int32 product + dequant, both 2B shapes, M=1) in %.1f s"
                      % (reps, el),
            "value_1thread": round(per_step * reps1 / el1 / 1e9, 3),
            "sample_1thread": "%d steps on one thread in %.1f s" % (reps1, el1)}


# ------------------------------------------------------------------- extras
def gpu_weights(N, K, seed, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * workloads.W_STD
    packed, beta = bl.pack_weights(w)
    del w
    return packed, beta


def gpu_acts(M, K, seed, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    return torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)


def decode_extra(shapes, Ms, dev, steps=100):
    res = {}
    packs = [gpu_weights(N, K, 100 + i, dev) for i, (K, N) in enumerate(shapes)]
    per_step = sum(N * K // 4 for K, N in shapes)
    R = rotation(per_step)
    copies = [copies_of(p, R) for p, _ in packs]
    for M in Ms:
        lins = [Linear(M, K, N, copies[i], packs[i][1], gpu_acts(M, K, 200 + i, dev))
                for i, (K, N) in enumerate(shapes)]
        g = capture_steps(lins, steps)
        time_graph(g)
        el, _ = time_graph(g)
        durs = [kernel_duration(L, 100) for L in lins]
        res["M%d" % M] = {"mode": lins[0].mode, "GB_s": round(per_step * steps / el / 1e9, 1),
                          "gemv_GB_s": round(sum(L.traffic_bytes() for L in lins) / sum(durs) / 1e9, 1),
                          "us_per_step": round(el / steps * 1e6, 2),
                          "frac_hbm": round(sum(L.traffic_bytes() for L in lins) / sum(durs) / 1e9 / HBM_PEAK_GBS, 4)}
        del lins, g
    del copies, packs
    torch.cuda.empty_cache()
    return res


def decode_step(Ms, dev, steps=50, n_layers=workloads.N_LAYERS):
    """One decode step over all BitLinears of the 30-layer stack, for each batch in Ms.

    Latent weights are drawn on the device (torch generator, one seed per
    matrix), packed, and copied to the host where the oracle advances its own
    chain layer by layer from the same bf16 input tokens; after one eager step
    the GPU's residual stream must equal the oracle's bit for bit.  A timed
    step restarts from the input tokens (a 10 KB device copy) and runs the
    210 BitLinears with their glue; `steps` of them form one HIP graph."""
    import oracle
    from bitlinear_matmul_02_amd.decoder import DecoderStack, PackedLinear
    threads = min(16, os.cpu_count() or 1)
    x0 = {M: workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, workloads.D_MODEL, workloads.DECODER_X0_SEED))
          for M in Ms}
    xr = dict(x0)
    layers, wbytes = [], 0
    for l in range(n_layers):
        L, lat = {}, {}
        for j, (name, K, N) in enumerate(workloads.LAYER_SHAPES):
            g = torch.Generator(device=dev).manual_seed(workloads.decoder_weight_seed(l, j))
            w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * workloads.W_STD
            packed, beta = bl.pack_weights(w)
            L[name] = PackedLinear(packed, beta, N, K)
            lat[name] = w.cpu().numpy()
            wbytes += packed.numel()
            del w
        tern = {}
        for name, w in lat.items():
            b = oracle.absmean(w)
            tern[name] = (b, oracle.ternarize(w, b))
        del lat

        def lin(inp, name):
            b, t = tern[name]
            q, ds, _ = oracle.quant_act(inp)
            return oracle.dequant(oracle.matmul_i32(q, t, threads=threads), ds, b)
        for M in Ms:
            x = xr[M]
            q = lin(oracle.rmsnorm(x), "q")  # k and v do not feed the residual stream
            x = oracle.add_f32(x, lin(q, "o"))
            xn = oracle.rmsnorm(x)
            x = oracle.add_f32(x, lin(oracle.relu2_mul(lin(xn, "gate"), lin(xn, "up")), "down"))
            xr[M] = x
        layers.append(L)
        del tern
    res = {"layers": n_layers, "bitlinears": 7 * n_layers, "weight_bytes": wbytes}
    for M in Ms:
        stack = DecoderStack(layers, M, dev)
        src = torch.from_numpy(x0[M]).to(dev)
        x = src.clone()
        stack.step(x)
        torch.cuda.synchronize()
        got = x.cpu().numpy()
        exact = bool(np.array_equal(got, xr[M]))
        rel = float(np.max(np.abs(got.astype(np.float64) - xr[M]) / np.maximum(np.abs(xr[M]), 1e-30)))
        if not np.all(np.isfinite(xr[M])) or not (exact or rel <= 1e-3):
            raise RuntimeError("decode step M=%d differs from the oracle (max rel %.3g)" % (M, rel))

        def one(i):
            x.copy_(src)
            stack.step(x)
        g = capture(one, steps)
        time_graph(g)
        el, _ = time_graph(g)
        t = el / steps
        res["M%d" % M] = {"tok_s": round(M / t, 1), "us_per_step": round(t * 1e6, 1),
                          "weight_GB_s": round(wbytes / t / 1e9, 1),
                          "frac_hbm": round(wbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                          "path": "fused" if stack.fused else "quant_act + gemv",
                          "oracle_match": "bit-exact" if exact else "rel %.2g" % rel}
        del g, stack, x, src
    del layers
    torch.cuda.empty_cache()
    return res


def decode_fmt_extra(fmt, shapes, Ms, dev, steps=100):
    """Other weight formats at decode: "b1" binary weights (BitNet b1, 1 bit
    per weight, bitlinear_gemv_b1) or "b3" ternary weights five to a byte
    (1.6 bits, bitlinear_gemv_b3); per BitLinear the standalone quantizer
    then the product.  GB/s counts the packed bytes; weights_per_s is the same
    stream in weights per second, comparable across formats."""
    pack_fn = bl.pack_weights_b1 if fmt == "b1" else bl.pack_weights_b3
    gemv_fn = bl.bitlinear_gemv_b1 if fmt == "b1" else bl.bitlinear_gemv_b3
    res = {}
    packs = []
    for i, (K, N) in enumerate(shapes):
        g = torch.Generator(device=dev).manual_seed(500 + i)
        w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * workloads.W_STD
        packs.append(pack_fn(w))
        del w
    per_step = sum(p.numel() for p, _ in packs)
    weights = sum(N * K for K, N in shapes)
    R = rotation(per_step)
    copies = [copies_of(p, R) for p, _ in packs]
    for M in Ms:
        bufs = []
        for i, (K, N) in enumerate(shapes):
            x = gpu_acts(M, K, 600 + i, dev)
            bufs.append((x, torch.empty((M, bl.act_stride(K)), dtype=torch.int8, device=dev),
                         torch.empty((M,), dtype=torch.float32, device=dev),
                         torch.empty((M,), dtype=torch.int32, device=dev),
                         torch.empty((M, N), dtype=torch.float32, device=dev)))

        def step(r, quant=True):
            for (K, N), (x, xq, xds, rs, y), c, (_, beta) in zip(shapes, bufs, copies, packs):
                if quant:
                    bl.bitlinear_quant_act(x, xq, xds, rs)
                gemv_fn(xq, xds, rs, K, c[r % R], beta, N, y)
        g = capture(step, steps)
        time_graph(g)
        el, _ = time_graph(g)
        step(0)
        gk = capture(lambda r: step(r, quant=False), steps)
        time_graph(gk)
        elk, _ = time_graph(gk)
        res["M%d" % M] = {"GB_s": round(per_step * steps / el / 1e9, 1),
                          "gemv_GB_s": round(per_step * steps / elk / 1e9, 1),
                          "us_per_step": round(el / steps * 1e6, 2),
                          "weights_per_s_T": round(weights * steps / el / 1e12, 3),
                          "frac_hbm_gemv": round(per_step * steps / elk / 1e9 / HBM_PEAK_GBS, 4)}
        del g, gk, bufs
    del copies, packs
    torch.cuda.empty_cache()
    return res


def train_extra(M, shapes, dev, reps=10):
    """Training step of one BitLinear with straight-through gradients, per
    shape: forward y = beta x t^T, input gradient dx = beta dy t, weight
    gradient dw = dy^T x (bf16 in, fp32 out, bf16 matrix cores); TFLOP/s on
    2 M N K per product against the dense bf16 peak."""
    res = {}
    for i, (K, N) in enumerate(shapes):
        packed, beta = gpu_weights(N, K, 900 + i, dev)
        x = gpu_acts(M, K, 910 + i, dev)
        dy = gpu_acts(M, N, 920 + i, dev)
        y = torch.empty((M, N), device=dev)
        dx = torch.empty((M, K), device=dev)
        dw = torch.empty((N, K), device=dev)
        ops = {"forward": lambda r: bl.bitlinear_train_forward(x, packed, beta, N, y),
               "backward_input": lambda r: bl.bitlinear_train_backward_input(dy, packed, beta, K, dx),
               "backward_weight": lambda r: bl.bitlinear_train_backward_weight(dy, x, dw)}
        flop = 2.0 * M * N * K
        row = {}
        for name, fn in ops.items():
            g = capture(fn, reps)
            time_graph(g)
            el, _ = time_graph(g)
            d = el / reps
            row[name] = {"us": round(d * 1e6, 1), "TFLOPS": round(flop / d / 1e12, 1),
                         "frac_mfma_bf16": round(flop / d / 1e12 / BF16_PEAK_TFLOPS, 4)}
            del g
        res["%dx%d->%d" % (M, K, N)] = row
        del packed, x, dy, y, dx, dw
        torch.cuda.empty_cache()
    return res


def prefill_b1_extra(M, shapes, dev, reps=20):
    """Binary-weight prefill GEMM (bitlinear_gemm_b1) TOPS on the same shapes."""
    res = {}
    for i, (K, N) in enumerate(shapes):
        g = torch.Generator(device=dev).manual_seed(700 + i)
        w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * workloads.W_STD
        packed, beta = bl.pack_weights_b1(w)
        del w
        x_q, x_ds, rs = bl.quant_act(gpu_acts(M, K, 800 + i, dev), with_rowsum=True)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        g2 = capture(lambda r: bl.bitlinear_gemm_b1(x_q, x_ds, rs, K, packed, beta, N, y), reps)
        time_graph(g2)
        el, _ = time_graph(g2)
        d = el / reps
        tops = 2.0 * M * N * K / d / 1e12
        res["%dx%d->%d" % (M, K, N)] = {"gemm_us": round(d * 1e6, 1), "TOPS": round(tops, 1),
                                        "frac_mfma": round(tops / INT8_PEAK_TOPS, 4)}
        del packed, x_q, y, g2
        torch.cuda.empty_cache()
    return res


def prefill_extra(M, shapes, dev, reps=20):
    res = {}
    for i, (K, N) in enumerate(shapes):
        packed, beta = gpu_weights(N, K, 300 + i, dev)
        L = Linear(M, K, N, [packed], beta, gpu_acts(M, K, 400 + i, dev))
        L.quant()
        L.run_product(0)
        torch.cuda.synchronize()
        d = kernel_duration(L, reps)
        # the quantizer alone, as a graph of back-to-back launches (no host
        # launch cost inside the timing)
        nq = 100
        gq = capture(lambda i: L.quant(), nq)
        time_graph(gq)
        elq, _ = time_graph(gq)
        tops = 2.0 * M * N * K / d / 1e12
        res["%dx%d->%d" % (M, K, N)] = {"gemm_us": round(d * 1e6, 1), "TOPS": round(tops, 1),
                                        "frac_mfma": round(tops / INT8_PEAK_TOPS, 4),
                                        "quant_us": round(elq / nq * 1e6, 2)}
        del gq
        del L, packed
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.counter_summary:
        counter_summary(*args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary[:2])
        return
    if args.pmc_table:
        pmc_table(*args.pmc_table[:2])
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the path has no sharding or collectives); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bl.lib()
    if args.counters:
        counters_run(dev)
        return

    global CLOCKS
    CLOCKS = ClockSampler()
    head, host, wl = headline(args, dev)
    result = {
        "metric": "ternary GEMV HBM GB/s + decode tok/s; prefill int8 TOPS; % of roofline",
        "value": round(head["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "shapes": ["1x2560->6912", "1x6912->2560"],
                   "step": "per BitLinear: absmax int8 quantization + ternary product + dequant (fp32 out), "
                           "one fused launch",
                   "rotation_copies": head["rotation_copies"], "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "kernel_us": head["kernel_us"],
        "unfused_us_per_step": head["unfused_us_per_step"],
    }
    shapes_2b = [(l.K, l.N) for l in workloads.DECODE_2B.linears]
    extras = {
        "decode_step_2b_30l": lambda: decode_step(workloads.DECODE_STEP_BATCHES, dev),
        "decode_100b": lambda: decode_extra(workloads.SHAPES_100B, (1, 8, 32), dev),
        "decode_b1_2b": lambda: decode_fmt_extra("b1", shapes_2b, (1, 8), dev),
        "decode_b1_100b": lambda: decode_fmt_extra("b1", workloads.SHAPES_100B, (1, 8), dev),
        "decode_b3_2b": lambda: decode_fmt_extra("b3", shapes_2b, (1, 8), dev),
        "decode_b3_100b": lambda: decode_fmt_extra("b3", workloads.SHAPES_100B, (1, 8), dev),
        "prefill_2b_m2048": lambda: prefill_extra(2048, ((2560, 6912), (6912, 2560)), dev),
        "prefill_100b_m512": lambda: prefill_extra(512, workloads.SHAPES_100B, dev),
        "prefill_b1_2b_m2048": lambda: prefill_b1_extra(2048, ((2560, 6912), (6912, 2560)), dev),
        "prefill_b1_100b_m512": lambda: prefill_b1_extra(512, workloads.SHAPES_100B, dev),
        "train_2b_m2048": lambda: train_extra(2048, ((2560, 6912), (6912, 2560)), dev),
    }
    if args.extras is not None:
        chosen = [e for e in args.extras.split(",") if e]
        unknown = [e for e in chosen if e not in extras]
        if unknown:
            print("bench.py: unknown --extras %s (known: %s)" % (",".join(unknown), ",".join(extras)), file=sys.stderr)
            sys.exit(2)
    else:
        chosen = [] if args.quick else list(extras)
    if chosen:
        result["also"] = {name: extras[name]() for name in chosen}
    result["clocks"] = CLOCKS.summary()
    # The oracle runs last: its host threads can keep the cores busy for a
    # while after it returns, which would delay the graph launches between
    # the timing events of the GPU measurements.
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(host, wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
