"""Host-side checks of the benchmark script: the single-GPU guard and the committed counter
summaries it reads (no GPU needed)."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_covers_the_step_kernels():
    """Every kernel of the timed step has calibrated per-launch bytes in the committed summary;
    when the summary was taken on the current sources, the benchmark reads them back."""
    text = open(os.path.join(ROOT, "profiles", "traffic_layer_1p3b.txt")).read()
    for k in bench.KERNELS:
        m = re.search(rf"^{k}\s+fetch_bytes=(\d+)\s+write_bytes=(\d+)", text, re.M)
        assert m, k
        assert int(m.group(1)) > 0 and int(m.group(2)) > 0
    if re.search(r"source_hash:\s*(\w+)", text).group(1) != bench.source_hash():
        pytest.skip("kernel sources changed since the counters were taken")
    st = bench.step_traffic(bench.B * bench.T * bench.H)
    assert st is not None and st["ratio_to_alg"] > 1.0
