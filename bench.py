"""Benchmark of the BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
    python bench.py --counters            (run under rocprofv3 --pmc, see below)
    python bench.py --counter-summary FETCH_CSV WRITE_CSV

Headline workload: decode GEMV at batch 1 on the 100B-class shapes, the
largest configuration that fits one GPU: K=8192 -> N=28672 and K=28672 ->
N=8192, bf16 activations N(0, 1).  One step is the whole inference hot path
for one token through both BitLinears: per-token absmax int8 quantization,
the ternary product and the dequantization (fp32 out), one fused launch per
BitLinear (weights packed once, before timing).  Inputs are resident in HBM.
Every BitLinear cycles through its own R distinct copies of its packed
weights, R * (its bytes) >= 2x the 256 MB Infinity Cache, and its copy
counter runs on across every graph (warm-up, timed), so a copy is read again
only after at least twice the cache's capacity of its other copies: every
step streams its weights from HBM.  The W warm-up steps and the K timed steps
are two HIP graphs, each replayed once (no host launch cost inside).

value = packed weight bytes of the step x K / elapsed time, in GB/s.

Also printed on the same JSON line:
  roofline      the decode kernel, against the 8 TB/s HBM peak: achieved =
                the algorithmic bytes of the step's launches (packed weights,
                bf16 x, fp32 y of both BitLinears) / the timed step (HIP events
                on the launch stream around the timed graph, whose steps hold
                only these launches);
  roofline.traffic  measured HBM bytes per launch of the same kernel, from two
                rocprofv3 --pmc runs of `bench.py --counters` (FETCH_SIZE, then
                WRITE_SIZE, KiB per dispatch), each scaled by the factor that
                makes the same counter read the known size of a 64 MiB device
                copy in the same run; `--counter-summary` turns the two CSV
                files into profiles/traffic_gemv_decode_100b_m1.txt, which
                records a hash of the kernel sources; the field is null when
                the sources have changed since;
  cpu_baseline  the CPU oracle (plain C, OpenMP over outputs) on the host cores,
                on bounded samples: the headline step on all cores and on one
                thread, and every other configuration (see cpu_baseline());
  also          the other workloads: the 2B-class decode GEMV at batch 1; one
                decode step over the 30-layer 2B-class stack (210 BitLinears +
                glue, batch 1 and 8) in tokens/s, checked bit for bit against
                the oracle's chain; 100B-class decode (M = 1, 8, 32) in GB/s;
                binary-weight (b1) and base-3 (b3) decode on the 2B and 100B
                shapes (M = 1, 8); prefill GEMMs (2B M=2048, 100B M=512),
                ternary and binary, in int8 TOPS; the training products
                (straight-through forward, input and weight gradients, 2B
                shapes, 2048 tokens) in bf16 TFLOP/s;
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
HEADLINE = workloads.DECODE_100B
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_decode_100b_m1.txt")
KERNEL_SOURCES = ("bitlinear_matmul_02_amd/csrc/gemv.hip", "bitlinear_matmul_02_amd/csrc/bl_internal.h")
CAL_BYTES = 64 << 20  # calibration copy
CAL_COPIES = 3  # calibration copies, the first copy dispatches of a counter run
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA, MI355X
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
MALL_BYTES = 256 << 20
THREADS = max(1, min(16, os.cpu_count() or 1))  # host threads of the oracle


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
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
def rotation(weight_bytes):
    """Distinct copies of one matrix such that R copies span at least twice
    the Infinity Cache: a copy is read again only after >= 2x its capacity of
    other copies of the same matrix."""
    return int(max(2, min(512, -(-2 * MALL_BYTES // max(weight_bytes, 1)) + 1)))


class Linear:
    """Device buffers of one BitLinear used in a timed step.

    mode "fused": one launch (bitlinear_forward_decode);
    mode "gemv" / "gemm": bitlinear_quant_act then the product call.
    Each product call uses the next of the R weight copies (a counter that
    runs on across graphs)."""

    def __init__(self, M, K, N, packed_copies, beta, x, y_dtype=torch.float32, mode=None):
        dev = x.device
        self.M, self.K, self.N = M, K, N
        self.packed = packed_copies
        self.beta = beta
        self.x = x
        self.r = 0
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
        return algorithmic_bytes(self.M, self.K, self.N, self.mode, self.x.element_size(), self.y.element_size())

    def quant(self):
        if self.mode != "fused":
            bl.bitlinear_quant_act(self.x, self.x_q, self.x_ds)

    def run_product(self):
        packed = self.packed[self.r % len(self.packed)]
        self.r += 1
        if self.mode == "fused":
            bl.bitlinear_forward_decode(self.x, packed, self.beta, self.N, self.y)
        else:
            self.product(self.x_q, self.x_ds, self.K, packed, self.beta, self.N, self.y, self.ws)

    def step(self):
        self.quant()
        self.run_product()


def algorithmic_bytes(M, K, N, mode, x_bytes=2, y_bytes=4):
    act = M * K * x_bytes if mode == "fused" else M * bl.act_stride(K)
    return N * K // 4 + act + M * N * y_bytes


def pack_from_host(w_np, dev):
    return bl.pack_weights(torch.from_numpy(w_np).to(dev))


def copies_of(packed, n):
    return [packed] + [packed.clone() for _ in range(n - 1)]


def capture(fn, nsteps):
    """One HIP graph holding nsteps calls of fn."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # one eager call first (loads code objects)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(nsteps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


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


def time_graph(g):
    """Replay g once; HIP events on the current stream around it."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if CLOCKS:
        CLOCKS.busy = True
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    if CLOCKS:
        CLOCKS.busy = False
    return a.elapsed_time(b) / 1e3, time.perf_counter() - t0


def timed(fn, nsteps, warm):
    """Seconds for nsteps calls of fn: a graph of `warm` calls, then a graph of
    nsteps calls, each replayed once, in the order captured (so that weight
    copy counters run on without repeats); returns (elapsed, wall)."""
    g_warm = capture(fn, max(warm, 1))
    g_main = capture(fn, nsteps)
    time_graph(g_warm)
    out = time_graph(g_main)
    del g_warm, g_main
    return out


def kernel_duration(lin, launches=200):
    """Average duration of the product kernel alone: HIP events on the launch
    stream around a graph of `launches` back-to-back launches (its weight
    copies rotate)."""
    lin.quant()
    el, _ = timed(lin.run_product, launches, launches // 4)
    return el / launches


# --------------------------------------------------------------- headline
def build_linears(wl, dev, host=None):
    """Device buffers of the workload's BitLinears from host-drawn inputs
    (tensor i: weights seed 2i, activations seed 2i + 1); returns (linears, host)."""
    if host is None:
        host = []
        for i, lin in enumerate(wl.linears):
            w = workloads.gen_weights(lin.N, lin.K, seed=2 * i)
            xb = workloads.gen_acts_bf16(lin.M, lin.K, seed=2 * i + 1, outliers=lin.outliers)
            host.append((w, xb))
    linears = []
    for (w, xb), lin in zip(host, wl.linears):
        packed, beta = pack_from_host(w, dev)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        linears.append(Linear(lin.M, lin.K, lin.N, copies_of(packed, rotation(lin.N * lin.K // 4)), beta, x))
    return linears, host


def decode_workload(wl, args, dev, roofline=True):
    """Time a decode workload (one step = each BitLinear once) and check the
    timed path against the oracle on the whole output first."""
    import oracle
    linears, host = build_linears(wl, dev)
    prepared = []
    for (w, xb), L in zip(host, linears):
        L.quant()
        L.run_product()
        torch.cuda.synchronize()
        beta = oracle.absmean(w)
        t = oracle.ternarize(w, beta)
        q, ds, _ = oracle.quant_act(xb, bf16_bits=True)
        if not np.array_equal(L.y.cpu().numpy(), oracle.dequant(oracle.matmul_i32(q, t, threads=THREADS), ds, beta)):
            raise SystemExit("bench: GPU output differs from the oracle on %s" % wl.name)
        prepared.append((t, beta, xb))
    del host

    def step():
        for L in linears:
            L.step()
    elapsed, wall = timed(step, args.steps, args.warmup)
    per_w = sum(L.weight_bytes() for L in linears)
    per_alg = sum(L.traffic_bytes() for L in linears)
    durs = [kernel_duration(L) for L in linears]
    # one BitLinear call as the host sees it: enqueue, then wait for it
    # (eager, median of 50, each call on the next weight copy)
    single = []
    for L in linears:
        ts = []
        for _ in range(50):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            L.step()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        single.append(float(np.median(ts)))
    # the same step with the standalone quantizer (two launches per BitLinear)
    split = [Linear(L.M, L.K, L.N, L.packed, L.beta, L.x, mode="gemv") for L in linears]
    el_split, _ = timed(lambda: [L.step() for L in split], args.steps, args.warmup)
    achieved = per_alg * args.steps / elapsed / 1e9
    out = {
        "value": per_w * args.steps / elapsed / 1e9, "ms_per_step": elapsed / args.steps * 1e3, "wall_s": wall,
        "rotation_copies": [len(L.packed) for L in linears],
        "rotation_bytes_per_shape": [len(L.packed) * L.weight_bytes() for L in linears],
        "unfused_us_per_step": round(el_split / args.steps * 1e6, 2),
        "kernel_us": {"%dx%d->%d" % (L.M, L.K, L.N): round(d * 1e6, 3) for L, d in zip(linears, durs)},
        "single_call_us": {"%dx%d->%d" % (L.M, L.K, L.N): round(t * 1e6, 2) for L, t in zip(linears, single)},
        "mode": linears[0].mode,
    }
    if roofline:
        out["roofline"] = {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "kernel": "gemv_t2_kernel (%s)" % ("fused quantization" if linears[0].mode == "fused" else linears[0].mode),
            "bytes_per_launch": [L.traffic_bytes() for L in linears],
            "duration_us_per_launch": round(elapsed / args.steps / len(linears) * 1e6, 3),
            "timing": "HIP events on the launch stream around the timed graph; its steps hold only these launches",
        }
    else:
        out["frac_hbm"] = round(achieved / HBM_PEAK_GBS, 4)
    del linears, split
    torch.cuda.empty_cache()
    return out, prepared


# ------------------------------------------------------- HBM traffic counters
def kernel_source_hash():
    """Hash of the decode kernel's sources with comments and whitespace
    removed: an edit of a comment does not make the measured traffic stale."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def counters_run(dev):
    """Dispatches for counter collection: a 64 MiB device copy (calibration),
    then each headline kernel COUNTER_LAUNCHES times over its rotating weight copies."""
    launches = COUNTER_LAUNCHES
    # three copies of 64 MiB, each from a source no cache holds: a 1 GiB fill
    # (4x the Infinity Cache) runs before each, so the copy's reads all leave L2
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    for _ in range(CAL_COPIES):
        src = torch.ones(CAL_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        flush.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del flush
    linears, _ = build_linears(HEADLINE, dev)
    for L in linears:
        L.quant()
        for _ in range(launches):
            L.run_product()
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
    lins = HEADLINE.linears
    labels = ["%dx%d->%d" % (l.M, l.K, l.N) for l in lins]
    modes = ["fused" if (l.M <= 4 and bl.decode_fits(l.M, l.K)) else "gemv" for l in lins]
    algo = [algorithmic_bytes(l.M, l.K, l.N, m) for l, m in zip(lins, modes)]  # packed + x + fp32 y
    factors, med, names, cal_kib = {}, {}, {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        # the calibration copies are the first CAL_COPIES copy dispatches; the
        # weight rotation copies made later are copies too, of another size
        cal = [v for _, name, _, v in rows if "copyBuffer" in name][:CAL_COPIES]
        if len(cal) != CAL_COPIES:
            raise SystemExit("expected %d calibration copies in %s, found %d" % (CAL_COPIES, path, len(cal)))
        factors[counter] = CAL_BYTES / (float(np.median(cal)) * 1024)
        cal_kib[counter] = cal
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
        "HBM traffic of the decode kernel (gemv_t2_kernel, %s), 100B-class shapes, batch 1" % modes[0],
        "",
        "commands (run from the repository root on one MI355X):",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- python bench.py --counters",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- python bench.py --counters",
        "  python bench.py --counter-summary gpurun_out/pmc_fetch/run_counter_collection.csv "
        "gpurun_out/pmc_write/run_counter_collection.csv",
        "",
        "FETCH_SIZE counts the bytes the L2 caches fetch from the memory fabric; an Infinity Cache (MALL) hit",
        "is such a fetch too, so it measures L2 misses, not HBM reads alone (each weight copy is re-read only",
        "after >= 2x the MALL's capacity of other copies, so the weight fetches miss the MALL as well).",
        "",
        "calibration: 64 MiB device copies (__amd_rocclr_copyBuffer) in the same run, each after a 1 GiB fill",
        "  so that no cache holds its source;",
        "  FETCH_SIZE factor %.5f (the copies read %s KiB for 65536 KiB moved each)"
        % (factors["FETCH_SIZE"], ", ".join("%.1f" % v for v in cal_kib["FETCH_SIZE"])),
        "  WRITE_SIZE factor %.5f (the copies read %s KiB)"
        % (factors["WRITE_SIZE"], ", ".join("%.1f" % v for v in cal_kib["WRITE_SIZE"])),
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


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "model": model, "threads_used": THREADS}


def time_reps(fn, budget, min_reps=3):
    """(reps, seconds, median seconds per call) of repeated fn() calls until
    `budget` seconds have passed and at least min_reps calls were made."""
    ts, t0 = [], time.perf_counter()
    while True:
        t1 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t1)
        el = time.perf_counter() - t0
        if len(ts) >= min_reps and el >= budget:
            return len(ts), el, float(np.median(ts))


def oracle_decode(prepared, threads):
    """One oracle step over BitLinears: quantize, int32 product, dequant."""
    import oracle

    def run():
        for t, beta, xb in prepared:
            q, ds, _ = oracle.quant_act(xb, bf16_bits=True)
            oracle.dequant(oracle.matmul_i32(q, t, threads=threads), ds, beta)
    return run


def oracle_chain(terns, x, threads):
    """The oracle's decode step over the decoder stack (terns: per layer, name ->
    (beta, codes)) from the fp32 residual stream x; returns the new stream."""
    import oracle

    def lin(inp, b_t):
        q, ds, _ = oracle.quant_act(inp)
        return oracle.dequant(oracle.matmul_i32(q, b_t[1], threads=threads), ds, b_t[0])
    for tern in terns:
        xn = oracle.rmsnorm(x)
        q = lin(xn, tern["q"])
        lin(xn, tern["k"])
        lin(xn, tern["v"])
        x = oracle.add_f32(x, lin(q, tern["o"]))
        xn = oracle.rmsnorm(x)
        x = oracle.add_f32(x, lin(oracle.relu2_mul(lin(xn, tern["gate"]), lin(xn, tern["up"])), tern["down"]))
    return x


def host_codes(shapes, seed0):
    """Ternary codes and beta of host-drawn weights (oracle) for (K, N) shapes."""
    import oracle
    out = []
    for i, (K, N) in enumerate(shapes):
        w = workloads.gen_weights(N, K, seed=seed0 + i)
        b = oracle.absmean(w)
        out.append((oracle.ternarize(w, b), b))
        del w
    return out


def cpu_baseline(head_prepared, stash):
    """The CPU oracle as it stands, timed on the host cores on bounded samples of
    each configuration (all cores = THREADS OpenMP threads over outputs; one
    thread where the sample is small): decode in GB/s of packed weights, the
    decoder step in tokens/s, prefill in int8 TOPS (2 M N K per product)."""
    per_w = sum(t.size // 4 for t, _, _ in head_prepared)
    reps, el, med = time_reps(oracle_decode(head_prepared, THREADS), 6.0)
    reps1, el1, med1 = time_reps(oracle_decode(head_prepared, 1), 3.0)
    res = {"value": round(per_w / med / 1e9, 3), "unit": "GB/s", "cores": THREADS, "kind": "oracle",
           "sample": "median of %d decode steps (quantize + int32 product + dequant, both 100B shapes, M=1), "
                     "%.1f s in all" % (reps, el),
           "value_1thread": round(per_w / med1 / 1e9, 3),
           "sample_1thread": "median of %d steps on one thread, %.1f s in all" % (reps1, el1),
           "host": host_cpu()}
    cfg = {}

    def decode_cfg(name, shapes, M, seed, outliers=False, one_thread=False, budget=1.5, codes=None):
        codes = codes or host_codes(shapes, seed)
        prep = [(t, b, workloads.gen_acts_bf16(M, K, seed=seed + 50 + i, outliers=outliers))
                for i, ((t, b), (K, N)) in enumerate(zip(codes, shapes))]
        wbytes = sum(N * K // 4 for K, N in shapes)
        r, e, m = time_reps(oracle_decode(prep, THREADS), budget)
        row = {"GB_s": round(wbytes / m / 1e9, 3), "us_per_step": round(m * 1e6, 1),
               "sample": "median of %d steps of M=%d, %.2f s in all" % (r, M, e)}
        if one_thread:
            r1, e1, m1 = time_reps(oracle_decode(prep, 1), budget)
            row["GB_s_1thread"] = round(wbytes / m1 / 1e9, 3)
            row["us_per_step_1thread"] = round(m1 * 1e6, 1)
        cfg[name] = row

    def prefill_cfg(name, shapes, M, sample_m, seed, codes=None):
        import oracle
        codes = codes or host_codes(shapes, seed)
        ops, secs = 0.0, 0.0
        for i, ((t, b), (K, N)) in enumerate(zip(codes, shapes)):
            xb = workloads.gen_acts_bf16(sample_m, K, seed=seed + 50 + i)
            t0 = time.perf_counter()
            q, ds, _ = oracle.quant_act(xb, bf16_bits=True)
            oracle.dequant(oracle.matmul_i32(q, t, threads=THREADS), ds, b)
            secs += time.perf_counter() - t0
            ops += 2.0 * sample_m * N * K
        cfg[name] = {"TOPS": round(ops / secs / 1e12, 4), "seconds": round(secs, 2),
                     "sample": "%d of the %d tokens of each shape (whole output rows), one pass" % (sample_m, M)}

    decode_cfg("single_4x512x512", ((512, 512),), 4, 9000, one_thread=True, budget=0.5)
    shapes_2b = [(l.K, l.N) for l in workloads.DECODE_2B.linears]
    decode_cfg("decode_gemv_2b_m1", shapes_2b, 1, 9100, outliers=True, one_thread=True)
    if "terns" in stash:
        x0s = stash["x0"]
        for M, one in ((1, True), (8, False)):
            r, e, m = time_reps(lambda: oracle_chain(stash["terns"], x0s[M], THREADS), 1.0)
            row = {"tok_s": round(M / m, 2), "us_per_step": round(m * 1e6, 1),
                   "sample": "median of %d steps of the %d-layer chain, M=%d, %.2f s in all"
                             % (r, len(stash["terns"]), M, e)}
            if one:
                r1, e1, m1 = time_reps(lambda: oracle_chain(stash["terns"], x0s[M], 1), 1.0)
                row["tok_s_1thread"] = round(M / m1, 3)
                row["us_per_step_1thread"] = round(m1 * 1e6, 1)
            cfg["decode_step_2b_30l_m%d" % M] = row
    prefill_cfg("prefill_2b_m2048", shapes_2b, 2048, 256, 9200)
    codes_100b = [(t, b) for t, b, _ in head_prepared]
    for M in (8, 32):
        decode_cfg("decode_100b_m%d" % M, workloads.SHAPES_100B, M, 9300, codes=codes_100b)
    prefill_cfg("prefill_100b_m512", workloads.SHAPES_100B, 512, 64, 9400, codes=codes_100b)
    res["configs"] = cfg
    return res


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
    copies = [copies_of(p, rotation(N * K // 4)) for (p, _), (K, N) in zip(packs, shapes)]
    for M in Ms:
        lins = [Linear(M, K, N, copies[i], packs[i][1], gpu_acts(M, K, 200 + i, dev))
                for i, (K, N) in enumerate(shapes)]
        el, _ = timed(lambda: [L.step() for L in lins], steps, steps // 4)
        durs = [kernel_duration(L, 100) for L in lins]
        res["M%d" % M] = {"mode": lins[0].mode, "GB_s": round(per_step * steps / el / 1e9, 1),
                          "gemv_GB_s": round(sum(L.traffic_bytes() for L in lins) / sum(durs) / 1e9, 1),
                          "us_per_step": round(el / steps * 1e6, 2),
                          "kernel_us": [round(d * 1e6, 2) for d in durs],
                          "frac_hbm": round(sum(L.traffic_bytes() for L in lins) / sum(durs) / 1e9 / HBM_PEAK_GBS, 4)}
        del lins
    del copies, packs
    torch.cuda.empty_cache()
    return res


def decode_step(Ms, dev, steps=50, n_layers=workloads.N_LAYERS, stash=None):
    """One decode step over all BitLinears of the 30-layer stack, for each batch in Ms.

    Latent weights are drawn on the device (torch generator, one seed per
    matrix), packed, and copied to the host where the oracle advances its own
    chain layer by layer from the same bf16 input tokens; after one eager step
    the GPU's residual stream must equal the oracle's bit for bit.  A timed
    step restarts from the input tokens (a 10 KB device copy) and runs the
    210 BitLinears with their glue; `steps` of them form one HIP graph.  The
    oracle's codes and input tokens are left in `stash` for its timing."""
    import oracle
    from bitlinear_matmul_02_amd.decoder import DecoderStack, PackedLinear
    threads = min(16, os.cpu_count() or 1)
    x0 = {M: workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, workloads.D_MODEL, workloads.DECODER_X0_SEED))
          for M in Ms}
    xr = dict(x0)
    layers, wbytes, terns = [], 0, []
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
        terns.append(tern)
    if stash is not None:
        stash["terns"], stash["x0"] = terns, x0
    del terns
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

        def one():
            x.copy_(src)
            stack.step(x)
        el, _ = timed(one, steps, max(steps // 5, 1))
        t = el / steps
        res["M%d" % M] = {"tok_s": round(M / t, 1), "us_per_step": round(t * 1e6, 1),
                          "weight_GB_s": round(wbytes / t / 1e9, 1),
                          "frac_hbm": round(wbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                          "path": "fused" if stack.fused else ("requantizing GEMV epilogues" if stack.requant
                                                               else "quant_act + gemv" if stack.gemv
                                                               else "quant_act + gemm"),
                          "oracle_match": "bit-exact" if exact else "rel %.2g" % rel}
        del stack, x, src
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
    copies = [copies_of(p, rotation(p.numel())) for p, _ in packs]
    ctr = [0] * len(shapes)  # per-matrix copy counters, running on across graphs
    for M in Ms:
        bufs = []
        for i, (K, N) in enumerate(shapes):
            x = gpu_acts(M, K, 600 + i, dev)
            bufs.append((x, torch.empty((M, bl.act_stride(K)), dtype=torch.int8, device=dev),
                         torch.empty((M,), dtype=torch.float32, device=dev),
                         torch.empty((M,), dtype=torch.int32, device=dev),
                         torch.empty((M, N), dtype=torch.float32, device=dev)))

        def step(quant=True):
            for i, ((K, N), (x, xq, xds, rs, y), c, (_, beta)) in enumerate(zip(shapes, bufs, copies, packs)):
                if quant:
                    bl.bitlinear_quant_act(x, xq, xds, rs)
                gemv_fn(xq, xds, rs, K, c[ctr[i] % len(c)], beta, N, y)
                ctr[i] += 1
        el, _ = timed(step, steps, steps // 4)
        elk, _ = timed(lambda: step(quant=False), steps, steps // 4)
        res["M%d" % M] = {"GB_s": round(per_step * steps / el / 1e9, 1),
                          "gemv_GB_s": round(per_step * steps / elk / 1e9, 1),
                          "us_per_step": round(el / steps * 1e6, 2),
                          "weights_per_s_T": round(weights * steps / el / 1e12, 3),
                          "frac_hbm_gemv": round(per_step * steps / elk / 1e9 / HBM_PEAK_GBS, 4)}
        del bufs
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
        ops = {"forward": lambda: bl.bitlinear_train_forward(x, packed, beta, N, y),
               "backward_input": lambda: bl.bitlinear_train_backward_input(dy, packed, beta, K, dx),
               "backward_weight": lambda: bl.bitlinear_train_backward_weight(dy, x, dw)}
        flop = 2.0 * M * N * K
        row = {}
        for name, fn in ops.items():
            el, _ = timed(fn, reps, reps)
            d = el / reps
            row[name] = {"us": round(d * 1e6, 1), "TFLOPS": round(flop / d / 1e12, 1),
                         "frac_mfma_bf16": round(flop / d / 1e12 / BF16_PEAK_TFLOPS, 4)}
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
        el, _ = timed(lambda: bl.bitlinear_gemm_b1(x_q, x_ds, rs, K, packed, beta, N, y), reps, reps)
        d = el / reps
        tops = 2.0 * M * N * K / d / 1e12
        res["%dx%d->%d" % (M, K, N)] = {"gemm_us": round(d * 1e6, 1), "TOPS": round(tops, 1),
                                        "frac_mfma": round(tops / INT8_PEAK_TOPS, 4)}
        del packed, x_q, y
        torch.cuda.empty_cache()
    return res


def prefill_extra(M, shapes, dev, reps=20):
    res = {}
    for i, (K, N) in enumerate(shapes):
        packed, beta = gpu_weights(N, K, 300 + i, dev)
        L = Linear(M, K, N, [packed], beta, gpu_acts(M, K, 400 + i, dev))
        L.quant()
        L.run_product()
        torch.cuda.synchronize()
        d = kernel_duration(L, reps)
        # the quantizer alone, as a graph of back-to-back launches (no host
        # launch cost inside the timing)
        nq = 100
        elq, _ = timed(L.quant, nq, nq // 4)
        tops = 2.0 * M * N * K / d / 1e12
        # context, not this library: the platform's int8 GEMM (torch._int_mm,
        # hipBLASLt) on the same shape with dense int8 weights [N][K] (ternary
        # values, one byte each) read as B^T, int32 out
        g = torch.Generator(device=dev).manual_seed(900 + i)
        a8 = torch.randint(-127, 128, (M, K), generator=g, device=dev, dtype=torch.int8)
        w8 = torch.randint(-1, 2, (N, K), generator=g, device=dev, dtype=torch.int8)
        elv, _ = timed(lambda: torch._int_mm(a8, w8.t()), reps, reps)
        tv = 2.0 * M * N * K / (elv / reps) / 1e12
        res["%dx%d->%d" % (M, K, N)] = {"gemm_us": round(d * 1e6, 1), "TOPS": round(tops, 1),
                                        "frac_mfma": round(tops / INT8_PEAK_TOPS, 4),
                                        "quant_us": round(elq / nq * 1e6, 2),
                                        "platform_int8_gemm": {"us": round(elv / reps * 1e6, 1), "TOPS": round(tv, 1),
                                                               "frac_mfma": round(tv / INT8_PEAK_TOPS, 4),
                                                               "what": "torch._int_mm (hipBLASLt), dense int8 "
                                                                       "weights, int32 out"}}
        del L, packed, a8, w8
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
    wl = HEADLINE
    head, head_prepared = decode_workload(wl, args, dev)
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
        "config": {"workload": wl.name,
                   "shapes": ["%dx%d->%d" % (l.M, l.K, l.N) for l in wl.linears],
                   "step": "per BitLinear: absmax int8 quantization + ternary product + dequant (fp32 out), "
                           + ("one fused launch" if head["mode"] == "fused" else "quantizer + product launches"),
                   "rotation_copies": head["rotation_copies"],
                   "rotation_bytes_per_shape": head["rotation_bytes_per_shape"],
                   "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "kernel_us": head["kernel_us"],
        "single_call_us": head["single_call_us"],
        "unfused_us_per_step": head["unfused_us_per_step"],
    }
    shapes_2b = [(l.K, l.N) for l in workloads.DECODE_2B.linears]
    stash = {}
    extras = {
        "decode_gemv_2b_m1": lambda: decode_workload(workloads.DECODE_2B, args, dev, roofline=False)[0],
        "decode_step_2b_30l": lambda: decode_step(workloads.DECODE_STEP_BATCHES, dev, stash=stash),
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
        result["also"] = {}
        for name in chosen:
            result["also"][name] = extras[name]()
            print("bench: %s done" % name, file=sys.stderr, flush=True)
    result["clocks"] = CLOCKS.summary()
    # The oracle runs last: its host threads can keep the cores busy for a
    # while after it returns, which would delay the graph launches between
    # the timing events of the GPU measurements.
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(head_prepared, stash)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
