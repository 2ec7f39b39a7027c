"""bench.py's command line on the CPU: it refuses more than one GPU before
touching a device, and the committed HBM-traffic summary matches the current
attention source (otherwise the bench would report its traffic as null)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert r.stdout == ""
    assert "exactly one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_traffic_summary_matches_the_attention_source():
    sys.path.insert(0, ROOT)
    import bench
    v = bench.traffic_record("attn_d40_L4096_m3")
    assert v is not None and v > 0
