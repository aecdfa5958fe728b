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


def test_stored_traffic_counters_are_current_and_go_stale_on_change(monkeypatch):
    """The committed counter summaries match the current kernel sources and build flags; any change
    to those makes bench.py report the traffic as unknown (null) instead of a stale figure."""
    sys.path.insert(0, ROOT)
    import bench

    for op in bench.KERNEL_SOURCES:
        assert bench.load_traffic(op) > 0, op
    monkeypatch.setattr(bench, "source_hash", lambda op: "0" * 64)
    for op in bench.KERNEL_SOURCES:
        assert bench.load_traffic(op) is None
