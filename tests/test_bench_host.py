"""Host logic of bench.py (no GPU): rotating-set sizing, the counter-traffic
lookup and its invalidation, the source hash, and the one-GPU refusal."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_rotating_sets_cover_twice_the_infinity_cache():
    for set_bytes in (1 << 20, 42_000_000, 184_565_760, 369_115_136, 1 << 30):
        s = bench.n_rotating_sets(set_bytes, 0)
        assert s >= 3 and s * set_bytes >= 2 * bench.MALL_BYTES
        assert (s - 1) * set_bytes < 2 * bench.MALL_BYTES or s == 3
    assert bench.n_rotating_sets(10, 7) == 7


def test_hash_ignores_comments_and_whitespace():
    a = "int f(){ return 1; } // note\n/* block */"
    b = "int f() {\n  return 1;  // other note\n}"
    assert bench._strip_comments(a) == bench._strip_comments(b)
    assert bench._strip_comments("int f(){return 2;}") != bench._strip_comments(a)
    assert len(bench.kernel_source_hash()) == 16


def test_counter_traffic_requires_matching_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    path = tmp_path / "fused_demo_counters.md"
    path.write_text("traffic_bytes_per_launch: 123456\nkernel_source_sha256: 0000\n")
    assert bench.counter_traffic("demo") is None          # stale hash
    path.write_text(f"traffic_bytes_per_launch: 123456\nkernel_source_sha256: "
                    f"{bench.kernel_source_hash()}\n")
    assert bench.counter_traffic("demo") == 123456.0
    assert bench.counter_traffic("missing") is None


def test_committed_counter_profile_parses():
    text = open(os.path.join(ROOT, "profiles", "fused_shard70b_counters.md")).read()
    assert "traffic_bytes_per_launch:" in text and "kernel_source_sha256:" in text


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_batch_distribution_percentiles():
    d = bench.batch_distribution([float(v) for v in range(1, 12)], 3)   # 1..11
    assert d == {"batches": 11, "calls_per_batch": 3, "median_us": 6.0, "p10_us": 2.0,
                 "p90_us": 10.0}
    assert bench.batch_distribution([], 3) is None


def test_steps_keep_measurements_near_the_target_time():
    assert bench._steps_for(30.0) == 666          # 20 ms of 30 us calls
    assert bench._steps_for(800.0) == 30          # at least 30 steps
    assert bench._steps_for(1.0) == 2000          # at most 2000 steps
