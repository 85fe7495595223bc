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


def test_down_roofline_method_work():
    """The down kernel's roofline counts one multiply-add per stored main slot and output
    column plus K x D per backup entry, and reads TwELL + backup + W_down once + writes y."""
    st = {"slots_used": 1000, "overflow_tile_rows": 3, "bytes_main": 5000, "bytes_backup": 800}
    T, D, F, K = 64, 256, 1024, 128
    r = bench.down_roofline(st, T, D, F, K, 2, 0.01, "mfma")
    assert r["algorithmic_flops"] == 2.0 * 1000 * 256 + 2.0 * 128 * 256 * 3
    assert r["algorithmic_bytes"] == 5000 + 800 + F * D * 2 + T * D * 2
    assert abs(r["tflops"] - r["algorithmic_flops"] / 1e-5 / 1e12) < 1e-3
    assert abs(r["hbm_frac"] - r["algorithmic_bytes"] / 1e-5 / 8e12) < 1e-5
    # bytes dominate at 2500 TFLOP/s: the HBM floor binds
    assert r["bound"] == "hbm"
    v = bench.down_roofline(st, T, D, F, K, 2, 0.01, "alu")
    assert "alu_frac" in v and v["floor_us"]["alu"] > r["floor_us"]["mfma"]


def test_parity_metrics_and_spread():
    import numpy as np
    ref = np.array([[1.0, -2.0], [0.0, 4.0]])
    y = ref + np.array([[0.02, 0.0], [0.0, -0.05]])
    m = bench.parity_metrics(y, ref)
    assert abs(m["max_rel_elem"] - max(0.02 / 2.0, 0.05 / 5.0)) < 1e-12
    assert abs(m["rel_frobenius"] - np.linalg.norm([0.02, 0.05]) / np.linalg.norm(ref)) < 1e-12
    s = bench.spread([3.0, 1.0, 2.0, 4.0, 5.0])
    assert s["median"] == 3.0 and s["n"] == 5 and s["p10"] < s["median"] < s["p90"]
