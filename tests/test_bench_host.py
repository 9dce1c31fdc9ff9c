"""Host logic of bench.py (no GPU): the HBM-traffic figure it reports.

bench.py reports roofline.traffic from the committed rocprofv3 summary of
the timed kernel and workload only while that summary was taken on the
current kernel source; otherwise the figure is null.
"""
import os

import bench


def _write(d, kernel, workload, sha, value="4368000000"):
    p = d / f"traffic_{kernel}_{workload}.txt"
    p.write_text(f"# summary\nkernel = {kernel}\nworkload = {workload}\n"
                 f"kernel_sha = {sha}\nhbm_bytes_per_launch = {value}\n")
    return str(p)


def _record(path):
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    return rec


def test_committed_traffic_summaries_are_read_consistently():
    # the figure of each committed summary while it matches the kernel source,
    # else null (a summary taken on an older kernel is never reported)
    for kernel, workload in (("dec_resident_hd128", "dense2b"), ("dec_resident_batch_hd128", "dense2b_b8")):
        path = os.path.join(bench.PROFILES, f"traffic_{kernel}_{workload}.txt")
        assert os.path.exists(path), path
        rec = _record(path)
        assert rec["workload"] == workload and rec["kernel"] == kernel
        current = rec.get("kernel_sha") == bench.kernel_hash()
        expected = float(rec["hbm_bytes_per_launch"]) if current else None
        assert bench.read_traffic(kernel, workload) == expected


def test_traffic_only_for_the_same_source_kernel_and_workload(tmp_path, monkeypatch):
    sha = bench.kernel_hash()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    _write(tmp_path, "dec_resident_hd128", "dense2b", sha)
    assert bench.read_traffic("dec_resident_hd128", "dense2b") == 4368000000.0
    assert bench.read_traffic("dec_resident_hd128", "dense2b_b8") is None        # another workload
    assert bench.read_traffic("dec_resident_batch_hd128", "dense2b") is None     # another kernel
    _write(tmp_path, "dec_resident_hd128", "dense2b", "0" * 16)
    assert bench.read_traffic("dec_resident_hd128", "dense2b") is None           # another kernel source
    _write(tmp_path, "dec_resident_hd128", "dense2b", sha, value="n/a")
    assert bench.read_traffic("dec_resident_hd128", "dense2b") is None           # unreadable figure
    # a summary whose workload line names another workload than its file name
    p = tmp_path / "traffic_dec_resident_hd128_lane2b.txt"
    p.write_text(f"kernel = dec_resident_hd128\nworkload = dense2b\nkernel_sha = {sha}\nhbm_bytes_per_launch = 1\n")
    assert bench.read_traffic("dec_resident_hd128", "lane2b") is None


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


def test_prefill_flops_counts_every_product_once():
    """The matrix prefill's algorithmic flops, against an explicit count over
    positions, heads and keys on a small shape."""
    import synth
    from memory_bound_transformer_persistent_amd import roofline as R
    s = synth.shape_for("tiny")
    d, q, f = s.d_model, s.n_heads * s.head_dim, s.d_ffn
    for n in (1, 2, 7):
        count = 0
        for _ in range(s.n_layers):
            for i in range(n):
                count += 2 * (3 * q * d) + 2 * (d * q) + 2 * (2 * f * d) + 2 * (d * f)   # the four products
                for _h in range(s.n_heads):
                    for _j in range(i + 1):
                        count += 2 * s.head_dim + 2 * s.head_dim                   # q.k and p v
        count += 2 * s.lm_vocab * d                                                 # the last row's logits
        assert R.prefill_flops(s, n) == count


def test_moe_step_bytes_count_the_active_experts_only():
    import synth
    from memory_bound_transformer_persistent_amd import roofline as R
    m = synth.shape_for("moe2b")
    d, F, E, k = 2560, 1728, 32, 4
    attn = 2 * (4 * 2560 * 2560)
    want = attn + 2 * E * d + 2 * 2 * d + k * 3 * F * d + 4 * k * (2 * F + d)
    assert R.layer_weight_bytes(m) == want
    # the same attention with dense2b's fp16 MLP reads 2 x 3 x 6912 x 2560 bytes more per
    # layer, the FP8 experts 4 x 3 x 1728 x 2560 (plus their scales and the router)
    dense = R.layer_weight_bytes(synth.shape_for("dense2b"))
    assert dense - want == 2 * 3 * 6912 * d - (k * 3 * F * d + 4 * k * (2 * F + d) + 2 * E * d)
    # every other term of a step is the dense model's
    sb, sd = R.step_bytes(m, 200), R.step_bytes(synth.shape_for("dense2b"), 200)
    assert sb.kv_read == sd.kv_read and sb.act == sd.act
    assert sd.weights - sb.weights == 25 * (dense - want)


def test_mxfp4_experts_count_half_a_byte_per_weight_and_their_block_scales():
    import synth
    from memory_bound_transformer_persistent_amd import roofline as R
    e4 = R.layer_weight_bytes(synth.shape_for("moe2b"))
    mx = R.layer_weight_bytes(synth.shape_for("moe2b_mx"))
    k, F, d = 4, 1728, 2560
    codes = k * 3 * F * d
    assert e4 - mx == (codes + 4 * k * (2 * F + d)) - (codes // 2 + codes // 32)
