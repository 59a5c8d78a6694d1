"""Host logic of bench.py, on the CPU: the one-GPU refusal, the code-only
source hash, that the committed HBM-traffic summary was taken on the kernel
sources as they stand (bench.py reports `traffic` only then), and that the
launch shapes bench.py expects are the library's."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 2" in r.stdout + r.stderr


def test_code_only_ignores_comments_and_layout():
    import bench

    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow */ }\n"
    b = "int f(int x) { return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(b) != bench._code_only(c)


def test_traffic_summary_matches_the_sources():
    import bench

    path = os.path.join(ROOT, "profiles", "fused_kernels_T8192_hbm_traffic.md")
    rows = {}
    for line in open(path, encoding="utf-8"):
        m = re.match(r"^\| (\w+) \| `([0-9a-f]{16})` \|", line)
        if m:
            rows[m.group(1)] = m.group(2)
    assert "silu_mul_quant" in rows and len(rows) >= 4, rows
    stale = {k: (h, bench.source_hash(k)) for k, h in rows.items()
             if k in bench.KERNEL_SOURCES and bench.source_hash(k) != h}
    assert not stale, f"counters taken on other code (re-take them): {stale}"


def test_launch_shapes_match_the_library():
    """bench.py tells a kernel trace's launches apart by the grid and symbol the
    library uses at each T; its switch points must be the library's."""
    import bench

    src = open(os.path.join(ROOT, "rope_residual_add_amd", "csrc", "norm_quant.hip"),
               encoding="utf-8").read()
    lib = {name: int(v) for name, v in
           re.findall(r"constexpr int64_t (kNormSplitMaxT|kDualSplitMaxT) = (\d+);", src)}
    assert lib == {"kNormSplitMaxT": bench.NORM_SPLIT_MAX_T,
                   "kDualSplitMaxT": bench.DUAL_SPLIT_MAX_T}
    # one vector per lane up to the switch, then the four-wave (H > 2048) shape
    T = bench.NORM_SPLIT_MAX_T
    assert bench._norm_shape(T, 4096) == (1, 8)
    assert bench._norm_shape(T + 1, 4096) == (2, 4)
    assert bench._norm_shape(T + 1, 1024) == (2, 1)


def test_trace_summary_columns(tmp_path):
    """summarize_trace: the profiler's average per kernel from the per-dispatch
    trace, with the traced run's own event-timed and back-to-back figures
    beside it (read from the run's JSON line)."""
    import csv
    import json

    import bench

    T = 8192
    symbols = {
        "fused_add_rmsnorm_quant": "void rra::add_rmsnorm_quant_kernel<2, 4, true, 2, 0, true>(x)",
        "silu_mul_quant": "void rra::silu_mul_quant_kernel<3, 128, true>(x)",
        "rope_kv_write": "void rra::rope_kv_write_kernel<128, true, 1, rra::ElemBf16>(x)",
        "dual_rmsnorm_quant": "void rra::dual_rmsnorm_quant_kernel<3, 1, 3, 128, true>(x)",
    }
    durations_ns = {k: [10_000 * (i + 1), 10_000 * (i + 1) + 2_000]
                    for i, k in enumerate(bench.KERNELS)}
    trace = tmp_path / "t_kernel_trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"])
        for k in bench.KERNELS:
            for d in durations_ns[k]:
                w.writerow([symbols[k], bench.grid_threads(k, T), 1000, 1000 + d])
            # a launch of the same kernel at another T is left out
            w.writerow([symbols[k], bench.grid_threads(k, 64), 0, 999_999])
    kern = {k: dict(us=1.5 + i, back_to_back=dict(us=0.5 + i)) for i, k in enumerate(bench.KERNELS)}
    js = tmp_path / "bench.json"
    js.write_text("log line\n" + json.dumps(dict(kernels=kern)) + "\n")
    out = tmp_path / "summary.md"
    bench.summarize_trace(str(tmp_path / "t_kernel_stats.csv"), str(out), "cmd", T, str(js))
    text = out.read_text()
    assert "bench.py events avg us | bench.py back-to-back us |" in text
    for i, k in enumerate(bench.KERNELS):
        row = [ln for ln in text.splitlines() if ln.startswith(f"| {k} |")]
        assert len(row) == 1, (k, text)
        cells = [c.strip() for c in row[0].strip("|").split("|")]
        assert cells[2] == "2"  # calls: the launch at T = 64 is not counted
        assert float(cells[3]) == (10_000 * (i + 1) + 1_000) / 1e3  # average us
        assert float(cells[-2]) == 1.5 + i and float(cells[-1]) == 0.5 + i
