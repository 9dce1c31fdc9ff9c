"""Pins for the oracle's mixture-of-experts MLP and FP8 E4M3 weights.

Each check ties the oracle to something other than itself: a library's
E4M3 conversion, the format's defining points, a second bit-level decoding
route, brute force over expert subsets, closed forms, the dense reference
decoder as a special case, and invariances.  CPU only.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth

TINY_MOE = synth.shape_for("tiny").with_(n_layers=2, d_ffn=64, n_experts=6, top_k=2, max_ctx=32)


def _idx(shape, name, layer):
    return synth.tensor_names(shape).index(f"{name}.{layer}")


# ----------------------------------------------------------------------------
# E4M3 decoding
# ----------------------------------------------------------------------------

def test_e4m3_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2                                     # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_defining_points():
    v = O.e4m3_value
    assert v(0x38) == 1.0                 # exponent field 7 = bias
    assert v(0x7E) == 448.0               # largest finite
    assert v(0x08) == 2.0 ** -6           # smallest normal
    assert v(0x01) == 2.0 ** -9           # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9       # largest subnormal
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0xB8) == -1.0 and v(0xFE) == -448.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert not math.isnan(v(0x7E)) and not math.isinf(v(0x78))   # 0x78 = 256: no infinities


def test_e4m3_through_fp16_bit_placement():
    # a second route: an E4M3 code's exponent and mantissa bits, placed in
    # the low bits of an fp16 exponent and the top of its mantissa, give
    # value * 2^-8 for every finite code (normals and subnormals alike)
    codes = np.arange(256, dtype=np.uint16)
    finite = (codes & 0x7F) != 0x7F
    bits = ((codes & 0x80) << 8) | ((codes & 0x7F) << 7)
    via16 = bits.astype(np.uint16).view(np.float16).astype(np.float64) * 256.0
    assert np.array_equal(via16[finite], O.e4m3_decode(codes[finite].astype(np.uint8)))


def test_e4m3_order_and_symmetry():
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))       # 0x00 .. 0x7E
    assert np.all(np.diff(pos) > 0)
    neg = O.e4m3_decode((np.arange(0x7F) | 0x80).astype(np.uint8))
    assert np.array_equal(neg, -pos)


def test_dequant_row_scales():
    codes = np.array([[0x38, 0x40], [0x30, 0xB8]], dtype=np.uint8)   # 1, 2 / 0.5, -1
    got = O.dequant(codes, np.array([3.0, 0.25], dtype=np.float32))
    assert np.array_equal(got, np.array([[3.0, 6.0], [0.125, -0.25]]))


def test_synth_codes_are_finite_and_small():
    t = synth.make_weights(TINY_MOE, seed=3)
    for name in ("Wg8", "Wu8", "Wd8"):
        c = t[_idx(TINY_MOE, name, 1)]
        assert c.dtype == np.uint8
        v = O.e4m3_decode(c)
        assert np.all(np.isfinite(v)) and np.max(np.abs(v)) <= 3.75
        assert np.any((c & 0x78) == 0)                             # subnormals are drawn


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def test_route_is_the_best_subset_by_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(50):
        E, k = 7, 1 + trial % 4
        r = np.round(rng.standard_normal(E), 1)          # rounded: ties happen
        sel, w, margin = O.route(r, k)
        best = max(itertools.combinations(range(E), k), key=lambda c: (sum(r[list(c)]), [-e for e in c]))
        assert sorted(sel) == sorted(best) or np.isclose(sum(r[sel]), sum(r[list(best)]))
        # order: larger logit first, lower index first among equals
        for a, b in zip(sel, sel[1:]):
            assert r[a] > r[b] or (r[a] == r[b] and a < b)
        rest = [e for e in range(E) if e not in sel]
        assert margin == pytest.approx(min(r[sel]) - max(r[rest]))
        assert w.sum() == pytest.approx(1.0)


def test_route_ties_take_the_lower_index():
    sel, w, margin = O.route(np.zeros(6), 3)
    assert list(sel) == [0, 1, 2] and margin == 0.0
    np.testing.assert_allclose(w, [1 / 3] * 3, rtol=0, atol=1e-15)


def test_route_weights_closed_form():
    r = np.array([0.3, 1.7, -2.0, 0.9])
    sel, w, margin = O.route(r, 2)
    assert list(sel) == [1, 3]
    a = 1.0 / (1.0 + math.exp(0.9 - 1.7))
    np.testing.assert_allclose(w, [a, 1 - a], rtol=1e-15)
    assert margin == pytest.approx(0.9 - 0.3)
    assert O.route(r, 4)[2] == math.inf


# ----------------------------------------------------------------------------
# the MoE decoder
# ----------------------------------------------------------------------------

def _single_expert_pair(seed):
    """A one-expert MoE model (k = 1, unit scales) and the dense model whose
    fp16 MLP weights are that expert's values exactly."""
    shp = TINY_MOE.with_(n_experts=1, top_k=1)
    t = synth.make_weights(shp, seed=seed, gain_jitter=0.1)
    dshape = shp.with_(n_experts=0, top_k=0)
    dense = []
    for name, x in zip(synth.tensor_names(shp), t):
        base = name.split(".")[0]
        if base in ("sg", "su", "sd"):
            x[:] = 1.0
        if base == "Wr":
            continue
        if base in ("Wg8", "Wu8", "Wd8"):
            dense.append(O.e4m3_decode(x).astype(np.float16))   # exact: E4M3 values are fp16 values
        elif base not in ("sg", "su", "sd"):
            dense.append(x)
    assert len(dense) == len(synth.tensor_names(dshape))
    return shp, t, dshape, dense


def test_single_expert_moe_equals_dense_decoder():
    shp, t, dshape, dense = _single_expert_pair(21)
    a, b = O.OracleMoEDecoder(shp, t), O.OracleDecoder(dshape, dense)
    for tok in (5, 77, 3000, 12):
        la, lb = a.step(tok), b.step(tok)
        np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-12)
        assert a.last_routes.shape == (shp.n_layers, 1) and np.all(a.last_weights == 1.0)
    np.testing.assert_array_equal(a.Kc, b.Kc)


def test_zero_router_averages_the_lowest_experts():
    t = synth.make_weights(TINY_MOE, seed=22)
    w = O.MoEWeights(TINY_MOE, t)
    w.layers[0]["Wr"] = np.zeros_like(w.layers[0]["Wr"])
    xn = np.random.default_rng(1).standard_normal(TINY_MOE.d_model)
    out, sel, wts, margin, _ = O.moe_ffn(w, 0, xn, TINY_MOE.top_k)
    assert list(sel) == [0, 1] and margin == 0.0
    want = 0.5 * (O.expert_ffn(*w.expert(0, 0), xn) + O.expert_ffn(*w.expert(0, 1), xn))
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)


def test_expert_slices_follow_the_row_blocks():
    # expert e's gate row j is row e*F + j of Wg8 with scale sg[e*F + j];
    # its down row i is row e*d + i of Wd8
    t = synth.make_weights(TINY_MOE, seed=23)
    w = O.MoEWeights(TINY_MOE, t)
    F, d = TINY_MOE.d_ffn, TINY_MOE.d_model
    g, u, dn = w.expert(1, 4)
    lw = w.layers[1]
    assert g.shape == (F, d) and dn.shape == (d, F)
    assert g[5, 7] == O.e4m3_value(lw["Wg8"][4 * F + 5, 7]) * float(lw["sg"][4 * F + 5])
    assert u[0, 0] == O.e4m3_value(lw["Wu8"][4 * F, 0]) * float(lw["su"][4 * F])
    assert dn[9, 3] == O.e4m3_value(lw["Wd8"][4 * d + 9, 3]) * float(lw["sd"][4 * d + 9])


def test_expert_permutation_invariance():
    t = synth.make_weights(TINY_MOE, seed=24, gain_jitter=0.1)
    perm = np.random.default_rng(2).permutation(TINY_MOE.n_experts)
    F, d = TINY_MOE.d_ffn, TINY_MOE.d_model
    tp = list(t)
    for l in range(TINY_MOE.n_layers):
        i = _idx(TINY_MOE, "Wr", l)
        tp[i] = t[i][perm]
        for name, n in (("Wg8", F), ("sg", F), ("Wu8", F), ("su", F), ("Wd8", d), ("sd", d)):
            j = _idx(TINY_MOE, name, l)
            tp[j] = np.concatenate([t[j][e * n:(e + 1) * n] for e in perm])
    a, b = O.OracleMoEDecoder(TINY_MOE, t), O.OracleMoEDecoder(TINY_MOE, tp)
    inv = np.argsort(perm)
    for tok in (1, 2, 900):
        np.testing.assert_allclose(a.step(tok), b.step(tok), rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(a.last_routes, perm[b.last_routes])
        np.testing.assert_array_equal(inv[a.last_routes], b.last_routes)


def test_forced_routes_change_only_where_they_differ():
    t = synth.make_weights(TINY_MOE, seed=25)
    a, b = O.OracleMoEDecoder(TINY_MOE, t), O.OracleMoEDecoder(TINY_MOE, t)
    la = a.step(7)
    same = [list(r) for r in a.last_routes]
    lb = b.step(7, force_routes=same)
    np.testing.assert_array_equal(la, lb)
    other = [list(same[0]), [e for e in range(TINY_MOE.n_experts) if e not in same[1]][:2]]
    a2 = O.OracleMoEDecoder(TINY_MOE, t)
    lc = a2.step(7, force_routes=other)
    assert np.max(np.abs(lc - la)) > 1e-3
    np.testing.assert_array_equal(a2.Kc[0], a.Kc[0])             # layer 0's K/V come before its MLP


def test_step_and_matrix_prefill_agree():
    t = synth.make_weights(TINY_MOE, seed=26, gain_jitter=0.1)
    toks = synth.make_prompt(TINY_MOE.vocab, 12, seed=5)[0]
    lg, K16, V16, routes, margins = O.prefill_matrix_moe(TINY_MOE, t, toks)
    dec = O.OracleMoEDecoder(TINY_MOE, t)
    for i, tok in enumerate(toks):
        li = dec.step(int(tok))
        np.testing.assert_allclose(li, lg[i], rtol=1e-10, atol=1e-11)
        np.testing.assert_array_equal(dec.last_routes, routes[i])
        np.testing.assert_allclose(dec.last_margins, margins[i], rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(dec.Kc[:, :, :12], K16)
    np.testing.assert_array_equal(dec.Vc[:, :, :12], V16)


def test_greedy_decode_moe_feeds_its_argmax():
    t = synth.make_weights(TINY_MOE, seed=27)
    prompt = synth.make_prompt(TINY_MOE.vocab, 5, seed=6)[0]
    fed, outs, pre, routes, margins = O.greedy_decode_moe(TINY_MOE, t, prompt, 4)
    assert fed[0] == O.greedy(pre[-1])
    for i in range(1, 4):
        assert fed[i] == O.greedy(outs[i - 1])
    assert routes.shape == (9, TINY_MOE.n_layers, TINY_MOE.top_k) and margins.shape == (9, TINY_MOE.n_layers)


def test_matrix_prefill_with_forced_routes_equals_forced_steps():
    t = synth.make_weights(TINY_MOE, seed=28, gain_jitter=0.1)
    toks = synth.make_prompt(TINY_MOE.vocab, 6, seed=7)[0]
    rng = np.random.default_rng(3)
    force = np.array([[rng.choice(TINY_MOE.n_experts, TINY_MOE.top_k, replace=False)
                       for _ in range(TINY_MOE.n_layers)] for _ in range(6)])
    lg, K16, V16, routes, gaps = O.prefill_matrix_moe(TINY_MOE, t, toks, force_routes=force)
    dec = O.OracleMoEDecoder(TINY_MOE, t)
    for i, tok in enumerate(toks):
        li = dec.step(int(tok), force_routes=[list(r) for r in force[i]])
        np.testing.assert_allclose(li, lg[i], rtol=1e-10, atol=1e-11)
        # the returned routes are the router's own choice on the forced path
        np.testing.assert_array_equal(dec.last_natural, routes[i])
    np.testing.assert_array_equal(dec.Kc[:, :, :6], K16)


# ----------------------------------------------------------------------------
# MXFP4 (OCP microscaling: E2M1 elements, an E8M0 scale per 32)
# ----------------------------------------------------------------------------

TINY_MX = TINY_MOE.with_(mxfp4=True)


def test_e2m1_values_are_the_format_table():
    # the eight magnitudes the OCP MX specification lists for E2M1, then the
    # same with the sign bit set (negative zero included)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [O.e2m1_value(n) for n in range(8)] == mags
    assert [O.e2m1_value(n | 8) for n in range(8)] == [-m for m in mags]
    assert math.copysign(1.0, O.e2m1_value(8)) == -1.0


def test_e2m1_through_e4m3_bit_placement():
    # a second route: an E2M1 code's bits placed in an E4M3 code (exponent
    # field + 6, the mantissa bit at the top of the mantissa) give the same
    # value for every normal code; the subnormal one is 0.5 = E4M3 0x30
    for n in range(16):
        e, m, s = (n >> 1) & 3, n & 1, (n >> 3) & 1
        if e == 0:
            code = (s << 7) | (0x30 if m else 0)
        else:
            code = (s << 7) | ((e + 6) << 3) | (m << 2)
        assert O.e4m3_value(code) == O.e2m1_value(n), n


def test_e8m0_matches_torch_float8_e8m0fnu():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([O.e8m0_value(x) for x in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    # torch reads code 0 as 2^-127 as the format defines; every code's value
    assert np.array_equal(got[:255], ref[:255])
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(120) == 2.0 ** -7


def test_mx_dequant_nibble_order_and_block_scales():
    # row 0: bytes 0x21 -> elements 0.5 (low nibble 1), 1.0 (high nibble 2);
    # block 0 (elements 0..31) scaled by 2^1, block 1 (32..63) by 2^-2
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 16] = 0xF7          # elements 32, 33: 6.0 and -6.0
    scales = np.array([[128, 125]], dtype=np.uint8)
    w = O.mx_dequant(codes, scales)
    assert w.shape == (1, 64)
    assert w[0, 0] == 1.0 and w[0, 1] == 2.0 and w[0, 32] == 1.5 and w[0, 33] == -1.5
    assert np.count_nonzero(w) == 4


def test_single_mx_expert_equals_dense_decoder():
    # MXFP4 values with these scales are exact in fp16
    shp = TINY_MX.with_(n_experts=1, top_k=1)
    t = synth.make_weights(shp, seed=31, gain_jitter=0.1)
    dshape = shp.with_(n_experts=0, top_k=0, mxfp4=False)
    names = synth.tensor_names(shp)
    dense = []
    for i, (name, x) in enumerate(zip(names, t)):
        base = name.split(".")[0]
        if base in ("Wg8", "Wu8", "Wd8"):
            sc = t[i + 1]
            dense.append(O.mx_dequant(x, sc).astype(np.float16))
        elif base not in ("sg", "su", "sd", "Wr"):
            dense.append(x)
    a, b = O.OracleMoEDecoder(shp, t), O.OracleDecoder(dshape, dense)
    for tok in (3, 900, 17):
        np.testing.assert_allclose(a.step(tok), b.step(tok), rtol=1e-12, atol=1e-12)


def test_mx_model_step_and_matrix_forms_agree():
    t = synth.make_weights(TINY_MX, seed=32, gain_jitter=0.1)
    toks = synth.make_prompt(TINY_MX.vocab, 7, seed=8)[0]
    lg, K16, V16, routes, gaps = O.prefill_matrix_moe(TINY_MX, t, toks)
    dec = O.OracleMoEDecoder(TINY_MX, t)
    for i, tok in enumerate(toks):
        np.testing.assert_allclose(dec.step(int(tok)), lg[i], rtol=1e-10, atol=1e-11)
        np.testing.assert_array_equal(dec.last_routes, routes[i])
