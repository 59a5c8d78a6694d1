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
