"""The full-size fixtures (tests/golden/fullsize_*.npz) are the oracle's output.

CPU tests.  They check that each fixture was written by the current oracle
source from the workload's seeds, that its stored values are consistent with
one another, and, for the lane workload (small enough to recompute here),
that the oracle run again on a prefix of the token sequence reproduces the
stored logits and K/V rows.
"""
import ast
import os

import numpy as np
import pytest

import oracle as O
import synth
from fullsize import GOLDEN, Fixture, oracle_sha

NAMES = ("dense2b", "lane2b", "dense2b_long", "dense2b_b8", "dense2b_w4", "lane2b_long", "dense2b_b8_long", "moe2b", "moe2b_mx")


@pytest.mark.parametrize("name", NAMES)
def test_fixture_is_from_the_current_oracle_and_seeds(name):
    fx = Fixture(name)
    assert fx.meta["oracle_sha"] == oracle_sha(), "oracle changed: rerun tests/golden/make_fullsize.py"
    np.testing.assert_array_equal(fx.tokens, fx.regenerate_tokens())
    assert fx.tokens.shape == (fx.batch, fx.n0 + fx.steps)
    np.testing.assert_array_equal(fx.pos, np.arange(fx.n0 - 1, fx.n0 + fx.steps))


@pytest.mark.parametrize("name", NAMES)
def test_fixture_values_are_consistent(name):
    fx = Fixture(name)
    tv = fx.top_val.astype(np.float64)
    assert np.all(tv[..., 0] >= tv[..., 1])
    assert np.all(fx.top_idx[..., 0] != fx.top_idx[..., 1])
    # a sampled logit never exceeds the largest one; where the sample holds the
    # argmax index, it holds the same value
    for q, p in enumerate(fx.samp_pos):
        r = int(p) - (fx.n0 - 1)
        for b in range(fx.batch):
            sv = fx.samp_val[b, q].astype(np.float64)
            assert sv.max() <= tv[b, r, 0]
            hit = np.nonzero(fx.samp_idx == fx.top_idx[b, r, 0])[0]
            if hit.size:
                assert sv[hit[0]] == tv[b, r, 0]
    # logits of random N(0, 0.02) weights on unit-rms inputs are about N(0, 1)
    assert 0.5 < float(np.std(fx.samp_val)) < 2.0


def test_dense2b_greedy_starts_from_the_prefill_argmax():
    fx = Fixture("dense2b")
    assert fx.greedy_tokens[0] == fx.top_idx[0, 0, 0]     # position n0 - 1 is the prefill's
    assert len(fx.greedy_margins) == len(fx.greedy_tokens)


def test_lane2b_prefix_recomputes_to_the_stored_values():
    """The oracle run again on the first 130 tokens reproduces the stored rows for positions <= 129."""
    fx = Fixture("lane2b")
    s = fx.shape
    tensors = synth.workload_weights(fx.workload)
    n = 130
    logits, K16, V16, _ = O.prefill_matrix(s, tensors, fx.tokens[0, :n])
    for p in range(fx.n0 - 1, n):
        r = p - (fx.n0 - 1)
        np.testing.assert_allclose(logits[p, fx.top_idx[0, r]], fx.top_val[0, r], rtol=0, atol=1e-5)
        if p in list(fx.samp_pos):
            q = list(fx.samp_pos).index(p)
            np.testing.assert_allclose(logits[p, fx.samp_idx], fx.samp_val[0, q], rtol=0, atol=1e-5)
    for li, layer in enumerate(fx.kv_layers):
        for qi, p in enumerate(fx.kv_pos):
            if p < n:
                np.testing.assert_array_equal(K16[layer][:, p], fx.kv_K[0, li][:, qi])
                np.testing.assert_array_equal(V16[layer][:, p], fx.kv_V[0, li][:, qi])


def test_fixture_script_uses_only_the_oracle_and_the_generators():
    src = open(os.path.join(GOLDEN, "make_fullsize.py")).read()
    mods = set()
    for node in ast.walk(ast.parse(src)):
        if isinstance(node, ast.Import):
            mods |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom):
            mods.add((node.module or "").split(".")[0])
    assert mods <= {"hashlib", "json", "os", "sys", "time", "numpy", "oracle", "synth"}, mods


@pytest.mark.parametrize("name", ["moe2b", "moe2b_mx"])
def test_moe2b_fixture_is_from_the_current_moe_oracle(name):
    import hashlib
    fx = Fixture(name)
    src = os.path.join(os.path.dirname(GOLDEN), "..", "oracle", "moe.py")
    assert fx.meta["moe_sha"] == hashlib.sha256(open(src, "rb").read()).hexdigest()[:16], \
        f"oracle/moe.py changed: rerun tests/golden/make_fullsize.py {name}"
    s = fx.shape
    n = fx.n0 + fx.steps
    assert fx.routes.shape == (n, s.n_layers, s.top_k) and fx.route_gap.shape == (n, s.n_layers)
    assert fx.routes.min() >= 0 and fx.routes.max() < s.n_experts
    # k distinct experts per position and layer, and a non-negative gap to the next
    assert all(len(set(r)) == s.top_k for r in fx.routes.reshape(-1, s.top_k))
    assert fx.route_gap.min() >= 0.0
