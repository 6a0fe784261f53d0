"""CPU checks of bench.py's host-side contract: it refuses more than one GPU
before touching any device, and its counter lookup only returns bytes for the
kernel source the counters were taken on."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "not sharded" in r.stderr
    assert r.stdout == ""


def test_traffic_lookup_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "device.hip"
    src.write_bytes(b"kernel source A")
    import hashlib
    sha = hashlib.sha256(b"kernel source A").hexdigest()
    rec = {"kernel_source_sha256": sha, "decode": {"read_bytes": 600, "write_bytes": 24}}
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    assert bench.measured_traffic("decode") == 624
    assert bench.measured_traffic("prefill_append") is None      # no entry
    src.write_bytes(b"kernel source B")                           # the kernel changed
    assert bench.measured_traffic("decode") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("decode") is None


def test_committed_traffic_entries_are_whole():
    """Every committed per-call entry has positive read and write bytes."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    assert len(rec["kernel_source_sha256"]) == 64
    calls = {k: v for k, v in rec.items() if isinstance(v, dict) and "read_bytes" in v}
    for name in ("decode", "decode_int8", "prefill_append", "copy_pages", "rewind_append", "spec_rollback"):
        assert name in calls, name
    for name, v in calls.items():
        assert v["read_bytes"] > 0 and v["write_bytes"] > 0, name
