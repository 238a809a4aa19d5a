"""bench.py's contract pieces that need no GPU: one GPU only (--gpus N > 1 and a
multi-rank launch exit with a message before touching a device), the HBM-traffic
figure reported only while the kernel sources match the counters' record, and
the published peaks the roofline fraction uses."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_exits_with_a_message():
    r = run_bench([], {"WORLD_SIZE": "2", "RANK": "1"})
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_profiled_sources(monkeypatch):
    record = open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")).read()
    want = int(record.split("bf16_4096_hbm_bytes_per_launch:")[1].split()[0])
    sha = record.split("kernel_source_sha256:")[1].split()[0]
    # well above the compulsory 134 MB (A and B read once, C written once)
    assert 134_217_728 < want < 2 * 1024**3
    if bench.kernel_source_sha() == sha:
        assert bench.measured_traffic("bf16_4096") == want
    else:  # sources changed since the counters were taken: reported as null
        assert bench.measured_traffic("bf16_4096") is None
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    assert bench.measured_traffic("bf16_4096") == want
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 64)
    assert bench.measured_traffic("bf16_4096") is None


def test_published_peaks():
    assert bench.PEAK_TFLOPS == {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
