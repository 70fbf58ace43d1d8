"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte and flop counts behind the roofline fractions, and the rule that
counter-based traffic is reported only for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from convolution_nhwc_amd import synth  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_bytes_are_dy_plus_w_plus_dx():
    # pointwise dgrad N=32, 56x56, K=256 -> C=64, fp16: dY 32*56*56*256, W 256*64, dX 32*56*56*64
    m = bench.metrics("c2_pointwise")
    assert m["bytes"] == 2 * (32 * 56 * 56 * 256 + 256 * 64 + 32 * 56 * 56 * 64) == 64258048
    assert m["nominal_flops"] == 2.0 * 32 * 56 * 56 * 256 * 64
    assert m["valid_flops"] == m["nominal_flops"]          # 1x1, no padding: every tap valid
    assert m["bound"] == "hbm"


def test_strided_3x3_counts():
    # N=32, 56x56 -> 28x28 (stride 2, pad 1), C=K=256: output extents and flops
    m = bench.metrics("c3b_3x3_s2")
    assert m["nominal_flops"] == 2.0 * 32 * 28 * 28 * 256 * 256 * 9
    assert m["bytes"] == 2 * (32 * 56 * 56 * 256 + 32 * 28 * 28 * 256 + 256 * 9 * 256)
    # output row 0 meets the top padding with one tap row: 28*3 - 1 valid rows per axis
    assert m["valid_flops"] == 2.0 * 32 * 256 * 256 * (28 * 3 - 1) ** 2
    assert m["bound"] == "mfma"


def test_depthwise_valid_flops_count_only_taps_inside_the_image():
    # 51x5 filter, pads 25/2, on 32x32: per axis sum over outputs of taps inside
    m = bench.metrics("c5_dw51x5")
    def taps(size, f, pad):
        return sum(1 for o in range(size) for t in range(f) if 0 <= o - pad + t < size)
    assert m["valid_flops"] == 2.0 * 8 * 256 * taps(32, 51, 25) * taps(32, 5, 2)
    assert m["nominal_flops"] == 2.0 * 8 * 32 * 32 * 256 * 51 * 5
    assert m["bound"] == "alu"


def test_every_workload_has_a_binding_roof():
    for name in synth.WORKLOADS:
        m = bench.metrics(name)
        assert m["bound"] in ("hbm", "mfma", "alu"), name
        assert m["bytes"] > 0 and m["t_ideal_s"] > 0, name


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    ent = rec["c2_pointwise"]
    # the figure is reported only while the recorded kernel sources are unchanged
    fresh = bench.source_hash(ent["sources"]) == ent["sources_sha256"]
    assert bench.recorded_traffic("c2_pointwise") == (ent["hbm_bytes_per_launch"] if fresh else None)
    # scaled counters: fetch x 2.0 and write x 1.0 of the KiB per dispatch
    assert abs(ent["fetch_kib_per_dispatch"] * 1024 * ent["fetch_scale"] +
               ent["write_kib_per_dispatch"] * 1024 * ent["write_scale"] -
               ent["hbm_bytes_per_launch"]) < 2048
    # a changed source hash makes the figure stale: null, not a number
    stale = dict(rec)
    stale["c2_pointwise"] = dict(ent, sources_sha256="0" * 64)
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.recorded_traffic("c2_pointwise") is None
    assert bench.recorded_traffic("no_such_workload") is None


def test_settle_runs_steps_for_the_requested_time(monkeypatch):
    """The settle phase keeps stepping until the host clock passes its time."""
    import types
    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: None))
    monkeypatch.setitem(sys.modules, "torch", fake_torch)
    clock = {"t": 0.0}
    monkeypatch.setattr(bench.time, "time", lambda: clock["t"])

    class Wk:
        steps = 0

        def step(self):
            Wk.steps += 1
            clock["t"] += 0.001

    bench.settle(Wk(), seconds=0.06)
    assert Wk.steps >= 60
