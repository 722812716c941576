"""bench.py's command-line contract on the host: more than one GPU, and flag combinations it does not time,
are refused with a message and a non-zero exit before any GPU work, and the counter record it reads matches the
kernel sources it covers."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_fused_with_plan_reuse_is_refused():
    """--fused times plain steps through one call; combined with the layer-reuse mode it is refused before any
    GPU work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--fused", "--plan-reuse"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--fused" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_record_is_well_formed():
    """profiles/attn_traffic.json lists existing sources and, for every workload, read and write bytes."""
    with open(os.path.join(ROOT, "profiles", "attn_traffic.json")) as f:
        rec = json.load(f)
    for src in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, src)), src
    assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0
    for name, w in rec["workloads"].items():
        assert w["read_bytes"] > 0 and w["write_bytes"] >= 0, name
