"""Host-side logic of bench.py (no GPU): the counter summary's calibration
and traffic arithmetic, the weight-copy rotation, and the one-GPU guard."""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_counters(path, counter, rows):
    """rows: (kernel name, grid size, value in KiB) in dispatch order."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, v) in enumerate(rows, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": v})


def _run(tmp_path, fetch_cal, write_cal, fetch_k, write_k, rotation_kib=57344.0):
    """A counter run as bench.py --counters lays it out: the calibration
    copies, then the weight-rotation copies (another size), then each headline
    shape's kernel COUNTER_LAUNCHES times."""
    n = bench.COUNTER_LAUNCHES
    shapes = len(bench.HEADLINE.linears)
    files = {}
    for counter, cal, per_kernel, rot in (("FETCH_SIZE", fetch_cal, fetch_k, rotation_kib / 2),
                                          ("WRITE_SIZE", write_cal, write_k, rotation_kib)):
        rows = [("__amd_rocclr_copyBuffer", 131072, c) for c in cal]
        rows += [("__amd_rocclr_copyBuffer", 114688, rot)] * 10
        for i in range(shapes):
            rows += [("void bl::gemv_t2_kernel<1, 7, 2>(bl::GemvArgs)", 131072, per_kernel[i])] * n
        p = tmp_path / ("%s.csv" % counter)
        _write_counters(p, counter, rows)
        files[counter] = str(p)
    return files


def test_counter_summary_calibrates_on_the_first_copies_only(tmp_path, monkeypatch):
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    # the 64 MiB copies read half their bytes on FETCH_SIZE and all of them on
    # WRITE_SIZE; the later rotation copies (56 MiB) must not enter the factors
    files = _run(tmp_path, [32768.0, 32768.0, 32768.0], [65536.0] * 3, [28672.0, 28672.0], [112.0, 32.0])
    bench.counter_summary(files["FETCH_SIZE"], files["WRITE_SIZE"])
    kv = dict(l.split(" = ", 1) for l in out.read_text().splitlines() if " = " in l)
    text = out.read_text()
    assert "FETCH_SIZE factor 2.00000" in text and "WRITE_SIZE factor 1.00000" in text
    expect = [28672.0 * 1024 * 2 + w * 1024 for w in (112.0, 32.0)]
    assert float(kv["traffic_bytes_per_launch_mean"]) == pytest.approx(sum(expect) / 2, rel=1e-9)
    assert kv["kernel_source_hash"].strip() == bench.kernel_source_hash()


def test_counter_summary_needs_three_calibration_copies(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    files = _run(tmp_path, [], [], [28672.0, 28672.0], [112.0, 32.0], rotation_kib=0.0)
    # without any copy dispatch the summary refuses to guess a factor
    for p in files.values():
        lines = [l for l in open(p) if "copyBuffer" not in l]
        open(p, "w").writelines(lines)
    with pytest.raises(SystemExit):
        bench.counter_summary(files["FETCH_SIZE"], files["WRITE_SIZE"])


def test_counter_summary_counts_the_kernel_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    files = _run(tmp_path, [32768.0] * 3, [65536.0] * 3, [28672.0, 28672.0], [112.0, 32.0])
    lines = open(files["WRITE_SIZE"]).readlines()
    open(files["WRITE_SIZE"], "w").writelines(lines[:-1])  # one dispatch missing
    with pytest.raises(SystemExit):
        bench.counter_summary(files["FETCH_SIZE"], files["WRITE_SIZE"])


@pytest.mark.parametrize("weight_bytes", [1, 4 << 20, 4456448, 58720256, 256 << 20, 1 << 30])
def test_rotation_spans_twice_the_infinity_cache(weight_bytes):
    r = bench.rotation(weight_bytes)
    assert r >= 2
    if weight_bytes * 512 >= 2 * bench.MALL_BYTES:  # below that the copy count is capped
        assert (r - 1) * weight_bytes >= 2 * bench.MALL_BYTES


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    def tree(extra_comment, code_change):
        d = tmp_path / ("t%d%d" % (extra_comment, code_change))
        for rel in bench.KERNEL_SOURCES:
            src = open(os.path.join(ROOT, rel)).read()
            if extra_comment:
                src = "// a new comment line\n" + src.replace("\n", "\n  /* and a block */ ", 1)
            if code_change:
                src += "\nint added_symbol;\n"
            p = d / rel
            p.parent.mkdir(parents=True, exist_ok=True)
            p.write_text(src)
        monkeypatch.setattr(bench, "ROOT", str(d))
        return bench.kernel_source_hash()
    base = tree(False, False)
    assert tree(True, False) == base
    assert tree(False, True) != base
