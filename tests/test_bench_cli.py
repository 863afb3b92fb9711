"""The benchmark's contract on the host: one GPU only, and the algorithmic
counts its roofline and bandwidth figures divide by, for the workloads whose
totals are stated with them (update bytes of the 1M- and 33M-point workloads,
the assignment's flop of the headline)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert "{" not in r.stdout  # no benchmark line


def test_update_bytes_headline_and_zipf():
    # N*d*s (rows gathered once) + 4N (labels) + 8N (perm written and read)
    # + 8Kd (old and new centroids) + 4K (counts)
    c3 = workloads.WORKLOADS["gmm-n1m-k8192-d128-f16"]
    n, d, k = 1 << 20, 128, 8192
    assert bench.update_bytes(c3) == n * d * 2 + 12 * n + 8 * k * d + 4 * k
    assert abs(bench.update_bytes(c3) - 2.894e8) < 1e5
    c4 = workloads.WORKLOADS["zipf-n32m-k4096-d128-bf16"]
    assert bench.update_bytes(c4) == 8996798464  # 8.997e9
    # weights add 4 bytes per point
    c5 = workloads.WORKLOADS["rows1d-b4096-n4096-k16-f32"]
    assert bench.update_bytes(c5) - (4096 * 4096 * (4 + 12) + 8 * 4096 * 16 + 4 * 4096 * 16) == 4 * 4096 * 4096


def test_assign_bytes_headline():
    c3 = workloads.WORKLOADS["gmm-n1m-k8192-d128-f16"]
    # points once, labels written, centroids once (fp32)
    assert bench.assign_bytes(c3) == (1 << 20) * (128 * 2 + 4) + 8192 * 128 * 4
    assert abs(bench.assign_bytes(c3) - 2.77e8) < 1e6
    # the flop the roofline divides by: 2 B N K d
    assert 2.0 * c3.B * c3.N * c3.K * c3.d == pytest.approx(2.199e12, rel=1e-3)
