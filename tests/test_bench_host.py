"""Host logic of bench.py (no GPU): the HBM-traffic figure it reports.

bench.py reports roofline.traffic from the committed rocprofv3 summary only
while that summary was taken on the current kernel source and the timed
workload; otherwise the figure is null.
"""
import os

import bench


def _write(tmp_path, sha, workload, value="4368000000"):
    p = tmp_path / "traffic.txt"
    p.write_text(f"# summary\nkernel = dec_resident_hd128\nworkload = {workload}\n"
                 f"kernel_sha = {sha}\nhbm_bytes_per_launch = {value}\n")
    return str(p)


def test_committed_traffic_summary_is_read_consistently():
    # the figure of the committed summary while it matches the kernel source,
    # else null (a summary taken on an older kernel is never reported)
    assert os.path.exists(bench.PROFILE_TRAFFIC)
    rec = {}
    for line in open(bench.PROFILE_TRAFFIC):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    current = rec.get("kernel_sha") == bench.kernel_hash() and rec.get("workload") == "dense2b"
    expected = float(rec["hbm_bytes_per_launch"]) if current else None
    assert bench.read_traffic("dense2b") == expected


def test_traffic_only_for_the_same_source_and_workload(tmp_path, monkeypatch):
    sha = bench.kernel_hash()
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", _write(tmp_path, sha, "dense2b"))
    assert bench.read_traffic("dense2b") == 4368000000.0
    assert bench.read_traffic("dense2b_b8") is None          # another workload
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", _write(tmp_path, "0" * 16, "dense2b"))
    assert bench.read_traffic("dense2b") is None             # another kernel source
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", _write(tmp_path, sha, "dense2b", value="n/a"))
    assert bench.read_traffic("dense2b") is None             # unreadable figure
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "missing.txt"))
    assert bench.read_traffic("dense2b") is None


def test_lane_slices_of_drawn_tensors_equal_the_lane_draw():
    # bench.py slices one lane's tensors from the full model it already drew;
    # they must be the arrays synth's own lane generator draws
    import numpy as np
    import synth
    full = synth.shape_for("tiny")
    lane = full.with_(n_heads=1, d_ffn=128, lm_vocab=512)
    a = synth.lane_slice_weights(lane, full, seed=3)
    b = synth.lane_from_full(lane, synth.make_weights(full, seed=3), full)
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x.shape == y.shape and np.array_equal(x, y)
