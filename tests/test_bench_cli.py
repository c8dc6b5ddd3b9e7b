"""Host-side behaviour of bench.py (no GPU needed): the refusals and the
counter-derived traffic figure."""

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_bench_refuses_several_gpus():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_bench_rejects_unknown_extra_workload():
    r = run_bench("--extra", "nvfp4,bogus")
    assert r.returncode == 2
    assert "bogus" in r.stderr


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU may be present")
def test_bench_without_gpu_fails_loudly():
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs an MI355X GPU" in r.stderr


def test_roofline_traffic_only_for_the_counted_kernel_and_workload(monkeypatch):
    """Stored counter bytes are reported only for the kernel and token count
    they were taken on, and only while that kernel's sources are unchanged."""
    sys.path.insert(0, ROOT)
    import bench
    src = "block_scaled_fp4_moe_amd/csrc/common.h"
    sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    c = dict(tokens=8, fetch_kib=1000.0, write_kib=10.0, fetch_scale=2.0, write_scale=1.0,
             sources=(src,), sha256=(sha,))
    monkeypatch.setattr(bench, "ROOFLINE_COUNTERS", {"fused": c})
    assert bench.roofline_traffic("fused", 8) == int((1000.0 * 2.0 + 10.0) * 1024)
    assert bench.roofline_traffic("fused", 9) is None
    assert bench.roofline_traffic("stage1", 8) is None
    monkeypatch.setattr(bench, "ROOFLINE_COUNTERS", {"fused": dict(c, sha256=("0" * 64,))})
    assert bench.roofline_traffic("fused", 8) is None
