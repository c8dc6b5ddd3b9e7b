"""Host-side behaviour of bench.py (no GPU needed): the refusals and the
counter-derived traffic figure."""

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


def test_stage1_traffic_only_for_the_counted_workload(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    assert bench.stage1_traffic(bench.STAGE1_COUNTERS["tokens"] + 1) is None
    t = bench.stage1_traffic(bench.STAGE1_COUNTERS["tokens"])
    if t is not None:
        c = bench.STAGE1_COUNTERS
        assert t == int((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024)
    # a changed kernel source makes the stored counters stale
    stale = dict(bench.STAGE1_COUNTERS)
    stale["sha256"] = ("0" * 64,) + tuple(stale["sha256"][1:])
    monkeypatch.setattr(bench, "STAGE1_COUNTERS", stale)
    assert bench.stage1_traffic(stale["tokens"]) is None
