"""Host-side checks of bench.py's bookkeeping (no GPU): the algorithmic byte counts behind the
roofline, the traffic figure's source-hash guard, the refusal of more than one GPU, and the
shapes of the sweep modes."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_config3():
    # q4_K weights 11008 x 16 x 144 B, q8_1 512 x 4096 x (1 + 4/32) B, f32 output 512 x 11008 x 4 B
    assert bench.algorithmic_bytes(512, 11008, 4096, 144) == 25_362_432 + 2_359_296 + 22_544_384
    # per-weight bytes of each q6_K form: raw 210, prepared 256, expanded 548 per 256 weights
    for b, per_weight in ((210, 0.8203125), (256, 1.0), (548, 2.140625)):
        w = bench.algorithmic_bytes(1, 256, 256, b) - (256 + 4 * 8) - 4 * 256
        assert w == 256 * 256 * per_weight


def test_traffic_guarded_by_kernel_hash(tmp_path, monkeypatch):
    t = json.load(open(bench.TRAFFIC_FILE))
    # the figure is reported only for the kernel source the counters were taken on
    if t["kernel_hash"] == bench.kernel_hash():
        assert bench.load_traffic() == t["hbm_bytes_per_launch"]
    else:
        assert bench.load_traffic() is None
    # any other source hash turns the figure off
    stale = dict(t, kernel_hash="0" * 16)
    f = tmp_path / "traffic.txt"
    f.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.load_traffic() is None


def test_committed_counters_describe_the_committed_kernel():
    """The HBM counters in profiles/ were taken on exactly the q4_K kernel source in the tree
    (mmq_q4k.hip and qpg_common.h), so the bench line carries its traffic figure; any edit of
    those files, comments included, needs the FETCH_SIZE / WRITE_SIZE runs taken again."""
    t = json.load(open(bench.TRAFFIC_FILE))
    assert t["kernel_hash"] == bench.kernel_hash()
    assert bench.load_traffic() == t["hbm_bytes_per_launch"]


def test_traffic_figure_from_counters():
    t = json.load(open(bench.TRAFFIC_FILE))
    cal = t["copy_calibration"]
    # the scale factors are what the counters read for a copy of known size
    assert abs(cal["fetch_scale"] - cal["bytes_copied"] / 1024 / cal["fetch_size_kib"]) < 1e-4
    assert abs(cal["write_scale"] - cal["bytes_copied"] / 1024 / cal["write_size_kib"]) < 1e-4
    hbm = t["fetch_size_kib_per_dispatch"] * 1024 * cal["fetch_scale"] + t["write_size_kib_per_dispatch"] * 1024 * cal["write_scale"]
    assert abs(hbm - t["hbm_bytes_per_launch"]) <= 1
    assert t["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(512, 11008, 4096, 144)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("shapes", [bench.SHARD_SHAPES, bench.MSWEEP_SHAPES])
def test_sweep_shapes_are_valid(shapes):
    for entry in shapes:
        form = entry[0]
        assert form in ("q4K", "q6K", "q6K_prep", "q6K_exp")
        K = entry[-2] if len(entry) == 4 else entry[3]
        assert K % 256 == 0
