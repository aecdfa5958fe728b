"""Host-side behaviour of bench.py that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_stored_traffic_counters_go_stale_on_any_source_change(monkeypatch):
    """bench.py reports a stored counter figure only while the hash of the kernel sources and build
    script matches the one recorded with it; otherwise the traffic is unknown (null)."""
    import json

    sys.path.insert(0, ROOT)
    import bench

    for op in bench.KERNEL_SOURCES:
        path = os.path.join(ROOT, "profiles", f"traffic_{op}.json")
        if not os.path.exists(path):
            continue
        with open(path) as f:
            rec = json.load(f)
        monkeypatch.setattr(bench, "source_hash", lambda _op, h=rec["source_sha256"]: h)
        assert bench.load_traffic(op) == rec["traffic_bytes_per_launch"] > 0
        monkeypatch.setattr(bench, "source_hash", lambda _op: "0" * 64)
        assert bench.load_traffic(op) is None
    # every layer's hash covers its kernel source, the shared device header and the build script
    for files in bench.KERNEL_SOURCES.values():
        assert "test_sequence_layers_amd/build.py" in files
        assert "test_sequence_layers_amd/csrc/device.hpp" in files
