"""Host-only checks of bench.py's helpers (no GPU): the power average used for energy per
token, and the kernel-source hash that invalidates stored HBM traffic figures."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


class _Run:
    def __init__(self):
        self.calls = 0

    def __call__(self):
        self.calls += 1

    def sync(self):
        pass


def test_average_power_reads_microwatts(tmp_path):
    p = tmp_path / "power1_input"
    p.write_text("750000000\n")  # 750 W in microwatts
    run = _Run()
    w, calls, elapsed = bench.average_power(str(p), run, 0.1)
    assert abs(w - 750.0) < 1e-9
    assert calls == run.calls and calls % 20 == 0 and calls > 0
    assert elapsed >= 0.1


def test_kernel_source_hash_is_stable():
    h1 = bench.kernel_source_hash()
    h2 = bench.kernel_source_hash()
    assert h1 == h2 and len(h1) == 16


def test_power_sensor_absent_or_readable():
    p = bench.power_sensor()
    if p is not None:
        with open(p) as f:
            int(f.read())


def test_traffic_counters_name_their_sources():
    """Stored HBM traffic figures carry the hash of exactly the sources of their kernel."""
    import json
    tc = json.load(open(os.path.join(ROOT, "profiles", "traffic_counters.json")))
    for name, ent in tc.items():
        assert name in bench.KERNEL_SOURCES, name
        assert tuple(ent["sources"]) == bench.KERNEL_SOURCES[name]
        assert len(ent["source_hash"]) == 16
        assert abs(ent["bytes_per_launch"] - ent["fetch_bytes"] - ent["write_bytes"]) <= 1
