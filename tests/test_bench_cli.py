"""bench.py's command line on the CPU: it refuses more than one GPU before
touching a device, and the committed HBM-traffic summary is well formed (the
bench reports its traffic as null when the attention source no longer matches
the hash the counters were taken on)."""

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


def test_traffic_summary_is_well_formed():
    """The committed counter summary parses: every attention row names a source
    hash and a positive byte count, and the bench reads it back (or reports
    null when the attention source has changed since the counters were taken)."""
    import re
    sys.path.insert(0, ROOT)
    import bench
    path = os.path.join(ROOT, "profiles", "refbank_attn_full_round_m3_hbm_traffic.md")
    rows = [[c.strip() for c in line.strip().strip("|").split("|")] for line in open(path, encoding="utf-8")
            if line.startswith("| attn_") or line.startswith("| short_ctx_")]
    assert any(r[0] == "attn_d40_L4096_m3" for r in rows)
    for r in rows:
        assert re.fullmatch(r"[0-9a-f]{16}", r[1]), r
        assert float(r[2]) > 0, r
    v = bench.traffic_record("attn_d40_L4096_m3")
    assert v is None or v > 0
