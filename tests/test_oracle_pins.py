"""Pins for the CPU oracle: closed forms, invariants, special cases, brute force.

Each test checks the oracle against something other than itself, chosen so a
plausible slip (dropped term, wrong sign or index, transposed operand, wrong
scale) fails at least one of them.  CPU only.
"""
import math

import numpy as np
import pytest

import oracle as O
import synth

TINY = synth.shape_for("tiny")


def _zeros_like_model(shape):
    return [np.zeros(s, dtype=np.float16) for s in synth.tensor_shapes(shape)]


def _idx(shape, name, layer=None):
    names = synth.tensor_names(shape)
    return names.index(name if layer is None else f"{name}.{layer}")


# ----------------------------------------------------------------------------
# fp16 rounding
# ----------------------------------------------------------------------------

def test_f16_round_ties_to_even_and_keeps_subnormals():
    one = 1.0
    ulp = 2.0 ** -10
    assert O.f16_round(one + ulp / 2) == one                  # tie -> even (1.0)
    assert O.f16_round(one + 3 * ulp / 2) == one + 2 * ulp    # tie -> even mantissa
    assert O.f16_round(one + ulp / 2 + 1e-12) == one + ulp    # above the tie rounds up
    tiny = 2.0 ** -24                                         # smallest fp16 subnormal
    assert O.f16_round(tiny) == tiny
    assert O.f16_round(3 * tiny) == 3 * tiny
    assert O.f16_round(70000.0) == math.inf


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

def test_rmsnorm_constant_magnitude_closed_form():
    d, c, eps = 64, 0.5, 1e-5
    signs = np.where(np.arange(d) % 3 == 0, -1.0, 1.0)
    x = c * signs
    # mean(x^2) = c^2 exactly, so the result is signs * c / sqrt(c^2 + eps)
    want = signs * (0.5 / math.sqrt(0.25 + 1e-5))
    np.testing.assert_allclose(O.rmsnorm(x, np.ones(d), eps), want, rtol=0, atol=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(40)
    g = rng.standard_normal(40)
    y = O.rmsnorm(x, np.ones(40), 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14          # unit RMS at eps = 0
    np.testing.assert_allclose(O.rmsnorm(7.5 * x, np.ones(40), 0.0), y, atol=1e-14)  # scale-free
    np.testing.assert_allclose(O.rmsnorm(x, g, 0.0), g * y, atol=1e-14)              # gain is elementwise
    # eps shrinks the output: |rmsnorm(x, eps>0)| < |rmsnorm(x, 0)|
    assert np.all(np.abs(O.rmsnorm(x, np.ones(40), 1.0)) < np.abs(y))


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def test_rope_basis_vectors_closed_form():
    # hd = 4, base = 100: theta = (1, 0.1)
    e = np.eye(4)
    r = O.rope(e[0], 1, 100.0)
    np.testing.assert_allclose(r, [0.5403023058681398, 0.8414709848078965, 0, 0], atol=1e-15)
    r = O.rope(e[1], 1, 100.0)
    np.testing.assert_allclose(r, [-0.8414709848078965, 0.5403023058681398, 0, 0], atol=1e-15)
    r = O.rope(e[2], 3, 100.0)   # angle 0.3 on the second pair
    np.testing.assert_allclose(r, [0, 0, 0.955336489125606, 0.29552020666133955], atol=1e-15)
    r = O.rope(e[3], 3, 100.0)
    np.testing.assert_allclose(r, [0, 0, -0.29552020666133955, 0.955336489125606], atol=1e-15)
    # position 0 is the identity
    v = np.arange(1.0, 5.0)
    np.testing.assert_array_equal(O.rope(v, 0, 100.0), v)


def test_rope_equals_block_rotation_matrix():
    hd, base = 16, 10000.0
    rng = np.random.default_rng(5)
    u = rng.standard_normal(hd)
    for p in (0, 1, 7, 4095):
        R = np.zeros((hd, hd))
        for i in range(hd // 2):
            ang = p * (base ** (-(2 * i) / hd))
            R[2 * i:2 * i + 2, 2 * i:2 * i + 2] = [[math.cos(ang), -math.sin(ang)],
                                                   [math.sin(ang), math.cos(ang)]]
        np.testing.assert_allclose(O.rope(u, p, base), R @ u, atol=1e-12)
        assert abs(np.linalg.norm(O.rope(u, p, base)) - np.linalg.norm(u)) < 1e-12


def test_rope_relative_position_invariance():
    hd, base = 64, 10000.0
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    for m, n in ((5, 2), (100, 37), (4095, 4000)):
        lhs = O.rope(q, m, base) @ O.rope(k, n, base)
        rhs = O.rope(q, m - n, base) @ k
        assert abs(lhs - rhs) < 1e-10


# ----------------------------------------------------------------------------
# softmax / attention / silu / greedy
# ----------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((7, 33)) * 30.0
    w = O.softmax(s)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(O.softmax(s + 123.0), w, atol=1e-12)
    assert np.all(w >= 0)


def test_attention_single_position_returns_v():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(64)
    K = rng.standard_normal((1, 64))
    V = rng.standard_normal((1, 64))
    o, w = O.attend(q, K, V)
    assert w.shape == (1,) and w[0] == 1.0
    np.testing.assert_array_equal(o, V[0])


def test_attention_two_positions_logistic_closed_form():
    hd = 16
    q = np.zeros(hd); q[0] = 2.0
    K = np.zeros((2, hd)); K[0, 0] = 1.0; K[1, 0] = 3.0      # scores 2/4, 6/4
    V = np.zeros((2, hd)); V[0, 1] = 1.0; V[1, 2] = 1.0
    o, w = O.attend(q, K, V)
    # w1 = sigmoid(s1 - s0) with s1 - s0 = (6 - 2) / sqrt(16) = 1
    w1 = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(w, [1 - w1, w1], atol=1e-15)
    np.testing.assert_allclose(o[1:3], [1 - w1, w1], atol=1e-15)


def test_silu_identities():
    z = np.linspace(-20, 20, 101)
    s = O.silu(z)
    np.testing.assert_allclose(s - O.silu(-z), z, atol=1e-12)                 # silu(z) - silu(-z) = z
    np.testing.assert_allclose(s, z * (1 + np.tanh(z / 2)) / 2, atol=1e-12)   # z * sigmoid(z), tanh form
    assert O.silu(0.0) == 0.0


def test_greedy_lowest_index_on_tie_and_margin():
    assert O.greedy([0.0, 3.0, 1.0, 3.0]) == 1
    assert O.top2_margin([0.0, 3.0, 1.0, 2.5]) == pytest.approx(0.5)


# ----------------------------------------------------------------------------
# whole-model special cases
# ----------------------------------------------------------------------------

def _echo_model(perm):
    """V = V_lm = d = 256, E = 16 I, Wo = Wd = 0, W_lm a permutation matrix."""
    shape = TINY.with_(vocab=256, lm_vocab=256)
    t = synth.make_weights(shape, seed=11)
    t[0] = (16.0 * np.eye(256)).astype(np.float16)
    for l in range(shape.n_layers):
        t[_idx(shape, "Wo", l)][:] = 0
        t[_idx(shape, "Wd", l)][:] = 0
    W = np.zeros((256, 256), dtype=np.float16)
    W[np.arange(256), perm] = 1.0          # logits[i] = xn[perm[i]]
    t[-1] = W
    return shape, t


def test_identity_weight_model_reproduces_input_embedding():
    rng = np.random.default_rng(4)
    perm = rng.permutation(256)
    inv = np.argsort(perm)
    shape, t = _echo_model(perm)
    dec = O.OracleDecoder(shape, t)
    peak = 16.0 / math.sqrt(1.0 + shape.rms_eps)
    tok = 17
    for _ in range(6):
        lg = dec.step(tok)
        np.testing.assert_array_equal(dec.last_hidden, 16.0 * np.eye(256)[tok])
        want = np.zeros(256); want[inv[tok]] = peak
        np.testing.assert_allclose(lg, want, atol=1e-12)
        tok = O.greedy(lg)


def _averaging_model(shift):
    """One layer: Wq = Wk = 0 (uniform attention), Wv = cyclic shift, Wo = I, no MLP."""
    shape = TINY.with_(n_layers=1)
    d = shape.d_model
    t = synth.make_weights(shape, seed=12)
    t[_idx(shape, "Wq", 0)][:] = 0
    t[_idx(shape, "Wk", 0)][:] = 0
    S = np.zeros((d, d), dtype=np.float16)
    S[np.arange(d), (np.arange(d) + shift) % d] = 1.0          # (S x)[i] = x[i + shift]
    t[_idx(shape, "Wv", 0)][:] = S
    t[_idx(shape, "Wo", 0)][:] = np.eye(d, dtype=np.float16)
    for name in ("Wg", "Wu", "Wd"):
        t[_idx(shape, name, 0)][:] = 0
    return shape, t


def test_zero_qk_model_averages_cached_values():
    shape, t = _averaging_model(shift=3)
    dec = O.OracleDecoder(shape, t)
    toks = [5, 900, 17, 4000, 5, 256]
    E = t[0].astype(np.float64)
    cached = []
    for p, tok in enumerate(toks):
        dec.step(tok)
        x = E[tok]
        xn = x / np.sqrt(np.mean(x * x) + shape.rms_eps)      # gains are 1
        cached.append(np.roll(xn, -3).astype(np.float16).astype(np.float64))
        want = x + np.mean(cached, axis=0)
        np.testing.assert_allclose(dec.last_hidden, want, rtol=0, atol=1e-12)
        w = dec.last_attn_weights[0]
        for h in range(shape.n_heads):
            np.testing.assert_allclose(w[h], np.full(p + 1, 1.0 / (p + 1)), atol=1e-15)


def test_position_zero_attention_is_cached_value_exactly():
    shape = TINY.with_(n_layers=1)
    d = shape.d_model
    t = synth.make_weights(shape, seed=13)               # random Wq, Wk
    t[_idx(shape, "Wv", 0)][:] = np.eye(d, dtype=np.float16)
    t[_idx(shape, "Wo", 0)][:] = np.eye(d, dtype=np.float16)
    for name in ("Wg", "Wu", "Wd"):
        t[_idx(shape, name, 0)][:] = 0
    dec = O.OracleDecoder(shape, t)
    dec.step(99)
    x = t[0][99].astype(np.float64)
    xn = x / np.sqrt(np.mean(x * x) + shape.rms_eps)
    np.testing.assert_array_equal(dec.last_hidden, x + xn.astype(np.float16).astype(np.float64))
    # and the key cached at position 0 is the un-rotated key
    k = t[_idx(shape, "Wk", 0)].astype(np.float64) @ xn
    np.testing.assert_array_equal(dec.Kc[0, :, 0, :], k.reshape(shape.n_heads, -1).astype(np.float16))


def test_swiglu_closed_form():
    shape = TINY.with_(n_layers=1, d_ffn=TINY.d_model)
    d = shape.d_model
    a = 1.7
    t = synth.make_weights(shape, seed=14)
    for name in ("Wq", "Wk", "Wv", "Wo"):
        t[_idx(shape, name, 0)][:] = 0
    t[_idx(shape, "Wg", 0)][:] = (a * np.eye(d)).astype(np.float16)
    t[_idx(shape, "Wu", 0)][:] = np.eye(d, dtype=np.float16)
    t[_idx(shape, "Wd", 0)][:] = np.eye(d, dtype=np.float16)
    signs = np.where(np.arange(d) % 5 == 1, -1.0, 1.0)
    t[0][7] = (0.5 * signs).astype(np.float16)            # constant-magnitude row
    dec = O.OracleDecoder(shape, t)
    dec.step(7)
    xn = signs * (0.5 / math.sqrt(0.25 + shape.rms_eps))
    ag = np.float64(np.float16(a)) * xn
    want = 0.5 * signs + ag * (1 + np.tanh(ag / 2)) / 2 * xn
    np.testing.assert_allclose(dec.last_hidden, want, rtol=0, atol=1e-12)


def test_head_permutation_invariance():
    shape = TINY
    t = synth.make_weights(shape, seed=15)
    perm = [2, 0, 3, 1]
    hd = shape.head_dim
    t2 = [x.copy() for x in t]
    for l in range(shape.n_layers):
        for name in ("Wq", "Wk", "Wv"):
            src = t[_idx(shape, name, l)].reshape(shape.n_heads, hd, -1)
            t2[_idx(shape, name, l)] = np.ascontiguousarray(src[perm].reshape(shape.n_heads * hd, -1))
        src = t[_idx(shape, "Wo", l)].reshape(shape.d_model, shape.n_heads, hd)
        t2[_idx(shape, "Wo", l)] = np.ascontiguousarray(src[:, perm, :].reshape(shape.d_model, -1))
    a = O.OracleDecoder(shape, t)
    b = O.OracleDecoder(shape, t2)
    for tok in (1, 2000, 3, 4095, 77):
        np.testing.assert_allclose(a.step(tok), b.step(tok), rtol=0, atol=1e-10)
    np.testing.assert_array_equal(a.Kc[:, perm, :5], b.Kc[:, :, :5])


def test_causal_prefix_property():
    shape = TINY
    t = synth.make_weights(shape, seed=16)
    a, b = O.OracleDecoder(shape, t), O.OracleDecoder(shape, t)
    la = [a.step(x) for x in (3, 1, 4, 1, 5)]
    lb = [b.step(x) for x in (3, 1, 4, 2, 6)]
    for j in range(3):
        np.testing.assert_array_equal(la[j], lb[j])
    assert np.max(np.abs(la[4] - lb[4])) > 1e-3


def test_matrix_prefill_equals_stepwise():
    """Prefill KV after the whole-sequence form == the token-at-a-time form."""
    shape = TINY
    t = synth.make_weights(shape, seed=0, gain_jitter=0.1)
    prompt = synth.make_prompt(shape.vocab, 24)[0]
    lg, K16, V16, X = O.prefill_matrix(shape, t, prompt)
    dec = O.OracleDecoder(shape, t)
    steps = [dec.step(int(x)) for x in prompt]
    n = len(prompt)
    kd = np.abs(K16.astype(np.float64) - dec.Kc[:, :, :n].astype(np.float64))
    vd = np.abs(V16.astype(np.float64) - dec.Vc[:, :, :n].astype(np.float64))
    # identical up to fp64 summation order: at most one fp16 ulp, almost always equal
    ulp = np.abs(np.spacing(dec.Kc[:, :, :n].astype(np.float16))).astype(np.float64)
    assert np.all(kd <= ulp) and np.all(vd <= np.abs(np.spacing(dec.Vc[:, :, :n])).astype(np.float64))
    assert np.mean(kd == 0) > 0.999 and np.mean(vd == 0) > 0.999
    np.testing.assert_allclose(lg, np.array(steps), rtol=0, atol=1e-9)


def test_tiny_greedy_decode_matrix_and_step_prefill_agree():
    w = synth.workload("tiny")
    t = synth.make_weights(w.shape, seed=w.weight_seed)
    prompt = synth.make_prompt(w.shape.vocab, w.prompt_len, seed=w.prompt_seed)[0]
    fa, la, pa, na = O.greedy_decode(w.shape, t, prompt, w.steps, matrix_prefill=True)
    fb, lb, pb, nb = O.greedy_decode(w.shape, t, prompt, w.steps, matrix_prefill=False)
    np.testing.assert_allclose(pa, pb, atol=1e-9)
    np.testing.assert_allclose(la, lb, atol=1e-9)
    assert list(fa) == list(fb) and na == nb
    # logits are O(1) for N(0, 0.02) weights and unit-RMS inputs (the tolerance scale)
    assert 0.2 < float(np.std(la)) < 5.0


def test_errors():
    dec = O.OracleDecoder(TINY, synth.make_weights(TINY))
    with pytest.raises(ValueError):
        dec.step(TINY.vocab)
    dec.pos = TINY.max_ctx
    with pytest.raises(ValueError):
        dec.step(0)
