"""GPU parity: the HIP decode path (through the C ABI) against the CPU oracle.

Tolerance (per step, teacher forced): max |logit_gpu - logit_oracle| <= 2e-2,
and the same greedy token wherever the oracle's top-2 margin exceeds 0.05.
Logits are O(1) for N(0, 0.02) weights (their std is ~1), so 2e-2 is about 2%
of one standard deviation; fp32 accumulation-order differences are ~1e-5.
"""
import math
import os

import numpy as np
import pytest

import oracle as O
import synth
from memory_bound_transformer_persistent_amd import binding as B

pytestmark = pytest.mark.gpu

TOL = 2e-2
MARGIN = 0.05


@pytest.fixture(scope="module")
def stream():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.cuda.Stream(device=0)


def make(shape, tensors, stream, batch=1, flags=0, **kw):
    return B.Decoder(B.ModelDesc.from_shape(shape, batch=batch, flags=flags), tensors=tensors, device=0,
                     stream=stream.cuda_stream, **kw)


def check_logits(gpu, ref, what, tol=TOL):
    err = float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)))
    print(f"{what}: max |gpu - oracle| = {err:.3e}", flush=True)
    assert err <= tol, f"{what}: {err}"
    if O.top2_margin(ref) > MARGIN:
        assert int(np.argmax(gpu)) == O.greedy(ref), what
    return err


def teacher_forced(shape, tensors, prompt, n_steps, stream, **kw):
    """Oracle greedy run, then the GPU fed the oracle's tokens; compare every step."""
    fed, ref, ref_pre, _ = O.greedy_decode(shape, tensors, prompt, n_steps)
    with make(shape, tensors, stream, **kw) as dec:
        tok, pre = dec.prefill(prompt, want_logits=True)
        worst = check_logits(pre, ref_pre, "prefill")
        if O.top2_margin(ref_pre) > MARGIN:
            assert tok == O.greedy(ref_pre)
        for i in range(n_steps):
            t, lg = dec.step(force_tok=int(fed[i]), want_logits=True)
            worst = max(worst, check_logits(lg, ref[i], f"step {i}"))
            assert t == int(np.argmax(lg))
    return worst


# ----------------------------------------------------------------------------
# tiny shape: full prompt + decode, several special models
# ----------------------------------------------------------------------------

def test_tiny_teacher_forced(stream):
    w = synth.workload("tiny")
    t = synth.make_weights(w.shape, seed=w.weight_seed)
    prompt = synth.make_prompt(w.shape.vocab, w.prompt_len, seed=w.prompt_seed)[0]
    teacher_forced(w.shape, t, prompt, w.steps, stream)


def test_tiny_gain_jitter(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=5, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 20, seed=9)[0]
    teacher_forced(s, t, prompt, 8, stream)


def test_tiny_free_running_generate_matches_oracle(stream):
    w = synth.workload("tiny")
    t = synth.make_weights(w.shape, seed=w.weight_seed)
    prompt = synth.make_prompt(w.shape.vocab, w.prompt_len, seed=w.prompt_seed)[0]
    fed, ref, ref_pre, nxt = O.greedy_decode(w.shape, t, prompt, w.steps)
    want = list(fed[1:]) + [nxt]
    margins = [O.top2_margin(r) for r in ref]
    with make(w.shape, t, stream) as dec:
        tok, _ = dec.prefill(prompt)
        assert tok == fed[0]
        got = dec.generate(w.steps)
    for i in range(w.steps):
        if margins[i] <= MARGIN:
            break       # beyond a near-tie the two greedy paths may legitimately split
        assert got[i] == want[i], i


def test_generate_equals_repeated_steps_bitwise(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=1)
    prompt = synth.make_prompt(s.vocab, 12, seed=3)[0]
    with make(s, t, stream) as a, make(s, t, stream) as b:
        a.prefill(prompt)
        b.prefill(prompt)
        ga = a.generate(20)
        gb = [b.step()[0] for _ in range(20)]
        assert list(ga) == gb
        assert a.position == b.position == 32


def test_multilaunch_equals_resident_bitwise(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=2)
    prompt = synth.make_prompt(s.vocab, 10, seed=4)[0]
    with make(s, t, stream) as a, make(s, t, stream, debug_flags=B.DEC_DEBUG_MULTILAUNCH) as b:
        ta, la = a.prefill(prompt, want_logits=True)
        tb, lb = b.prefill(prompt, want_logits=True)
        np.testing.assert_array_equal(la, lb)
        for _ in range(6):
            ta, la = a.step(want_logits=True)
            tb, lb = b.step(want_logits=True)
            assert ta == tb
            np.testing.assert_array_equal(la, lb)
        gb = b.generate(5)
        ga = a.generate(5)
        assert list(ga) == list(gb)


def test_run_to_run_determinism(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=6)
    prompt = synth.make_prompt(s.vocab, 16, seed=6)[0]
    outs = []
    for _ in range(2):
        with make(s, t, stream) as d:
            _, lg = d.prefill(prompt, want_logits=True)
            steps = [d.step(want_logits=True)[1] for _ in range(4)]
            outs.append(np.concatenate([lg] + steps))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_kv_cache_after_prefill_matches_oracle(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=7, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 40, seed=8)[0]
    _, K16, V16, _ = O.prefill_matrix(s, t, prompt)
    with make(s, t, stream) as d:
        d.prefill(prompt)
        for l in range(s.n_layers):
            k, v = d.read_kv(l, len(prompt))
            for name, g, r in (("K", k, K16[l]), ("V", v, V16[l])):
                g64, r64 = g.astype(np.float64), r.astype(np.float64)
                ulp = np.abs(np.spacing(r.astype(np.float16))).astype(np.float64)
                diff = np.abs(g64 - r64)
                # Both sides round to fp16 from slightly different pre-rounding
                # values (fp32 vs fp64 arithmetic, and from layer 1 on, inputs
                # that already differ by ~1e-6): allow one fp16 spacing plus the
                # absolute fp32 error carried in, 2e-5 for O(0.3) values.  Near
                # zero that is many ulps, so ulps alone are the wrong yardstick.
                assert np.all(diff <= ulp + 2e-5), f"layer {l} {name}: max {diff.max()}"
                # layer 0 sees identical inputs, so only fp32-vs-fp64 rounding can
                # flip an fp16 value; deeper layers also inherit upstream differences
                same = float(np.mean(diff == 0))
                print(f"layer {l} {name}: {same:.4f} identical, max diff {diff.max():.2e}")
                assert same > (0.99 if l == 0 else 0.95), f"layer {l} {name}: {same}"


def _idx(shape, name, layer=None):
    names = synth.tensor_names(shape)
    return names.index(name if layer is None else f"{name}.{layer}")


def test_identity_embedding_model_echoes(stream):
    shape = synth.shape_for("tiny").with_(vocab=256, lm_vocab=256)
    t = synth.make_weights(shape, seed=11)
    t[0] = (16.0 * np.eye(256)).astype(np.float16)
    for l in range(shape.n_layers):
        t[_idx(shape, "Wo", l)][:] = 0
        t[_idx(shape, "Wd", l)][:] = 0
    perm = np.random.default_rng(4).permutation(256)
    W = np.zeros((256, 256), dtype=np.float16)
    W[np.arange(256), perm] = 1.0
    t[-1] = W
    inv = np.argsort(perm)
    peak = 16.0 / math.sqrt(1.0 + shape.rms_eps)
    with make(shape, t, stream) as d:
        tok, lg = d.prefill([17], want_logits=True)
        want = np.zeros(256); want[inv[17]] = peak
        np.testing.assert_allclose(lg, want, atol=1e-5)
        assert tok == inv[17]
        toks = d.generate(10)
    chain = [inv[17]]
    for _ in range(10):
        chain.append(inv[chain[-1]])
    assert list(toks) == chain[1:]


def test_zero_qk_model_averages_values(stream):
    shape = synth.shape_for("tiny").with_(n_layers=1, vocab=4096, lm_vocab=256)
    d_ = shape.d_model
    t = synth.make_weights(shape, seed=12)
    t[_idx(shape, "Wq", 0)][:] = 0
    t[_idx(shape, "Wk", 0)][:] = 0
    S = np.zeros((d_, d_), dtype=np.float16)
    S[np.arange(d_), (np.arange(d_) + 3) % d_] = 1.0
    t[_idx(shape, "Wv", 0)][:] = S
    t[_idx(shape, "Wo", 0)][:] = np.eye(d_, dtype=np.float16)
    for name in ("Wg", "Wu", "Wd"):
        t[_idx(shape, name, 0)][:] = 0
    t[-1] = np.eye(256, dtype=np.float16)
    toks = [5, 900, 17, 4000, 5, 256, 77, 1024, 3000, 2]
    ref = O.OracleDecoder(shape, t)
    with make(shape, t, stream) as d:
        _, lg = d.prefill(toks[:1], want_logits=True)
        np.testing.assert_allclose(lg, ref.step(toks[0]), atol=1e-5)
        for tk in toks[1:]:
            _, lg = d.step(force_tok=tk, want_logits=True)
            np.testing.assert_allclose(lg, ref.step(tk), atol=1e-5)


def test_head_permutation_invariance_on_gpu(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=15)
    perm = [2, 0, 3, 1]
    hd = s.head_dim
    t2 = [x.copy() for x in t]
    for l in range(s.n_layers):
        for name in ("Wq", "Wk", "Wv"):
            src = t[_idx(s, name, l)].reshape(s.n_heads, hd, -1)
            t2[_idx(s, name, l)] = np.ascontiguousarray(src[perm].reshape(s.n_heads * hd, -1))
        src = t[_idx(s, "Wo", l)].reshape(s.d_model, s.n_heads, hd)
        t2[_idx(s, "Wo", l)] = np.ascontiguousarray(src[:, perm, :].reshape(s.d_model, -1))
    prompt = synth.make_prompt(s.vocab, 9, seed=2)[0]
    with make(s, t, stream) as a, make(s, t2, stream) as b:
        _, la = a.prefill(prompt, want_logits=True)
        _, lb = b.prefill(prompt, want_logits=True)
        assert np.max(np.abs(la - lb)) <= 1e-4
        for _ in range(4):
            _, la = a.step(want_logits=True)
            _, lb = b.step(want_logits=True)
            assert np.max(np.abs(la - lb)) <= 1e-4


def test_edges_single_token_prompt_context_cap_and_reset(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=0)
    ref = O.OracleDecoder(s, t)
    with make(s, t, stream) as d:
        tok, lg = d.prefill([123], want_logits=True)           # one-token prompt
        check_logits(lg, ref.step(123), "one-token prefill")
        with pytest.raises(B.DecError) as e:
            d.prefill([1, 2])                                  # prefill needs position 0
        assert e.value.code == B.DEC_ERR_STATE
        with pytest.raises(B.DecError) as e:
            d.step(force_tok=s.vocab)
        assert e.value.code == B.DEC_ERR_TOKEN_RANGE
        d.generate(s.max_ctx - 1)                              # fill the cache to the cap
        assert d.position == s.max_ctx
        with pytest.raises(B.DecError) as e:
            d.step()
        assert e.value.code == B.DEC_ERR_CONTEXT_FULL
        d.reset()
        prompt = synth.make_prompt(s.vocab, s.max_ctx, seed=5)[0]   # the longest prompt
        _, lg_full = d.prefill(prompt, want_logits=True)
        assert d.position == s.max_ctx
    _, K16, V16, _ = O.prefill_matrix(s, t, prompt)
    lgm = O.prefill_matrix(s, t, prompt)[0][-1]
    check_logits(lg_full, lgm, "max-length prompt")


def test_watchdog_timeout_is_an_error_not_a_hang(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=0)
    with make(s, t, stream, watchdog_us=1) as d:      # every barrier wait expires at once
        with pytest.raises(B.DecError) as e:
            d.prefill(synth.make_prompt(s.vocab, 4)[0])
        assert e.value.code == B.DEC_ERR_TIMEOUT
        with pytest.raises(B.DecError) as e:
            d.step(force_tok=1)
        assert e.value.code == B.DEC_ERR_STATE
        d.reset()
    with make(s, t, stream) as d:                     # a normal handle still works
        prompt = synth.make_prompt(s.vocab, 4)[0]
        _, lg = d.prefill(prompt, want_logits=True)
        check_logits(lg, O.prefill_matrix(s, t, prompt)[0][-1], "after timeout")


def test_asynchronous_step_timeout_surfaces_at_sync(stream):
    """dec_step with neither outputs returns before the step has run; a
    watchdog expiry in it is reported by the next call that waits (dec_sync)."""
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=0)
    with make(s, t, stream, watchdog_us=1) as d:
        tok, lg = d.step(force_tok=1, want_tok=False)       # asynchronous: nothing to wait for
        assert tok is None and lg is None
        with pytest.raises(B.DecError) as e:
            d.sync()
        assert e.value.code == B.DEC_ERR_TIMEOUT
        with pytest.raises(B.DecError) as e:
            d.step(force_tok=1)
        assert e.value.code == B.DEC_ERR_STATE
        d.reset()


def test_weights_file_ingest_matches_host_tensors(stream, tmp_path):
    from memory_bound_transformer_persistent_amd import weights_file as WF
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=21, gain_jitter=0.1)
    p = WF.write(tmp_path / "tiny.decw", B.ModelDesc.from_shape(s), t)
    prompt = synth.make_prompt(s.vocab, 7, seed=1)[0]
    with make(s, t, stream) as a, B.Decoder(B.ModelDesc.from_shape(s), path=p, stream=stream.cuda_stream) as b:
        _, la = a.prefill(prompt, want_logits=True)
        _, lb = b.prefill(prompt, want_logits=True)
        np.testing.assert_array_equal(la, lb)


# ----------------------------------------------------------------------------
# real shapes
# ----------------------------------------------------------------------------

def test_dense2b_run_to_run_bitwise(stream):
    """Run to run at full size: the partial row sums meet in an order that does
    not depend on timing (at most two contributors per row pair), so two fresh
    handles give the same bits."""
    w = synth.workload("dense2b")
    t = synth.workload_weights(w)
    prompt = synth.make_prompt(w.shape.vocab, w.prompt_len, seed=w.prompt_seed)[0]
    runs = []
    for _ in range(2):
        with make(w.shape, t, stream) as d:
            _, pre = d.prefill(prompt[:24], want_logits=True)
            runs.append(np.concatenate([pre] + [d.step(want_logits=True)[1] for _ in range(2)]))
    np.testing.assert_array_equal(runs[0], runs[1])


def test_dense2b_generate_across_the_attention_split_equals_steps(stream):
    """dense2b: 24 tokens in one dec_generate launch equal 24 dec_step calls.

    From a 500-token prompt the launch crosses 512 positions, where each
    head's attention goes from one workgroup to three; tokens and the whole
    KV cache must be bitwise equal to the step-by-step run.
    """
    w = synth.workload("dense2b")
    s = w.shape
    t = synth.workload_weights(w)
    prompt = synth.make_prompt(s.vocab, 500, seed=w.prompt_seed)[0]
    with make(s, t, stream) as a, make(s, t, stream) as b:
        a.prefill(prompt)
        b.prefill(prompt)
        ga = a.generate(24)
        gb = [b.step()[0] for _ in range(24)]
        assert list(ga) == gb
        assert a.position == b.position == 524
        for l in (0, s.n_layers // 2, s.n_layers - 1):
            ka, va = a.read_kv(l, 524)
            kb, vb = b.read_kv(l, 524)
            assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16)), f"K layer {l}"
            assert np.array_equal(va.view(np.uint16), vb.view(np.uint16)), f"V layer {l}"


# ----------------------------------------------------------------------------
# small-batch decode: several independent sequences per step
# ----------------------------------------------------------------------------
#
# Each sequence of a batch must decode exactly as it would alone (the oracle is
# batch 1 and is run once per sequence).  The batched kernel keeps every
# sequence's matrix-product input in LDS as fp16 (eight fp32 vectors of the MLP
# width would not fit), so x*g, the attention output and the SwiGLU output are
# rounded to fp16 before each product (relative error 2^-11 at most) where the
# batch-1 path keeps fp32.  The logit tolerance stays 2e-2.  K/V rows: layer 0
# sees exact inputs (an fp16 embedding row times unit gains); deeper layers
# inherit the roundings of the layers below.  A float64 model of exactly these
# roundings, run against the oracle on the 2.3B shape, moves the K/V rows of
# layers 1..24 by 1.4e-3 up to 5e-3 of the layer's rms beyond one fp16 spacing
# (and the logits by 6e-3), so the batched K/V bound is 1e-2 of the rms.
KV_BATCH = 1e-2

def kv_excess(g, r):
    """Per leading index, the largest |g - r| beyond one fp16 spacing, relative to r's rms."""
    g64 = g.astype(np.float64).reshape(g.shape[0], -1)
    r64 = r.astype(np.float64).reshape(r.shape[0], -1)
    spacing = np.abs(np.spacing(np.maximum(np.abs(g64), np.abs(r64)).astype(np.float16))).astype(np.float64)
    rms = np.sqrt(np.mean(r64 * r64, axis=1, keepdims=True))
    return ((np.abs(g64 - r64) - spacing) / rms).max(axis=1)


# d_model 200 and 5 x 8 heads: the O, down and QKV outputs end in a 16-row
# group holding 8 rows (one 8-row block of the exchange vectors); d_ffn 136;
# an LM head of 4090 rows ends inside a group
RAGGED_BATCH = synth.shape_for("tiny").with_(d_model=200, n_heads=5, head_dim=8, d_ffn=136, lm_vocab=4090)


@pytest.mark.parametrize("nb,ragged", [(8, False), (3, False), (5, True)])
def test_tiny_batch_teacher_forced(stream, nb, ragged):
    s = RAGGED_BATCH if ragged else synth.shape_for("tiny")
    t = synth.make_weights(s, seed=21, gain_jitter=0.1)
    n, steps = 16, 12
    prompts = synth.make_prompt(s.vocab, n, batch=nb, seed=22)
    refs = [O.greedy_decode(s, t, prompts[b], steps) for b in range(nb)]
    with make(s, t, stream, batch=nb) as d:
        tok, pre = d.prefill(prompts, want_logits=True)
        pre = pre.reshape(nb, -1)
        for b in range(nb):
            check_logits(pre[b], refs[b][2], f"seq {b} prefill")
            if O.top2_margin(refs[b][2]) > MARGIN:
                assert tok[b] == O.greedy(refs[b][2]), b
        for b in range(nb):
            _, K16, V16, _ = O.prefill_matrix(s, t, prompts[b])
            for l in range(s.n_layers):
                k, v = d.read_kv(l, n, seq=b)
                ek, ev = kv_excess(k, K16[l]), kv_excess(v, V16[l])
                assert ek.max() <= KV_BATCH and ev.max() <= KV_BATCH, (b, l, ek.max(), ev.max())
        for i in range(steps):
            ft = np.array([refs[b][0][i] for b in range(nb)], dtype=np.int32)
            tk, lg = d.step(force_tok=ft, want_logits=True)
            lg = lg.reshape(nb, -1)
            for b in range(nb):
                check_logits(lg[b], refs[b][1][i], f"seq {b} step {i}")
                assert tk[b] == int(np.argmax(lg[b]))


def test_batch_sequences_do_not_interact(stream):
    """Equal prompts give bitwise-equal results whatever the other sequences hold."""
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=23)
    n = 14
    a = synth.make_prompt(s.vocab, n, seed=24)[0]
    runs = []
    for seed in (25, 26):
        prompts = synth.make_prompt(s.vocab, n, batch=8, seed=seed)
        prompts[0::2] = a
        with make(s, t, stream, batch=8) as d:
            _, pre = d.prefill(prompts, want_logits=True)
            outs = [pre.reshape(8, -1)]
            for _ in range(6):
                outs.append(d.step(want_logits=True)[1].reshape(8, -1))
        runs.append(np.stack(outs, axis=1))      # [8, 7, V]
    for r in runs:
        for b in (2, 4, 6):
            np.testing.assert_array_equal(r[b], r[0])
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    assert not np.array_equal(runs[0][1], runs[1][1])


def test_batch_generate_equals_repeated_steps_bitwise(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=27)
    prompts = synth.make_prompt(s.vocab, 10, batch=8, seed=28)
    with make(s, t, stream, batch=8) as a, make(s, t, stream, batch=8) as b:
        ta, _ = a.prefill(prompts)
        tb, _ = b.prefill(prompts)
        np.testing.assert_array_equal(ta, tb)
        ga = a.generate(16).reshape(16, 8)
        gb = np.stack([b.step()[0] for _ in range(16)])
        np.testing.assert_array_equal(ga, gb)
        assert a.position == b.position == 26


# ----------------------------------------------------------------------------
# batched prefill (DEC_FLAG_BATCHED_PREFILL): 8 prompt positions per step of
# the matrix-core kernel, causal attention over the one sequence's cache.
# Its matrix-product inputs are rounded to fp16 as in batched decode, so the
# cache and logit bounds are the batched ones (KV_BATCH, 2e-2).
# ----------------------------------------------------------------------------

BP = B.DEC_FLAG_BATCHED_PREFILL


@pytest.mark.parametrize("n", [1, 8, 21, 128])
def test_tiny_batched_prefill(stream, n):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=31, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, n, seed=32 + n)[0]
    steps = min(6, s.max_ctx - n)
    fed, ref, ref_pre, _ = O.greedy_decode(s, t, prompt, steps)
    _, K16, V16, _ = O.prefill_matrix(s, t, prompt)
    with make(s, t, stream, flags=BP) as d:
        tok, pre = d.prefill(prompt, want_logits=True)
        check_logits(pre, ref_pre, f"batched prefill of {n}")
        if O.top2_margin(ref_pre) > MARGIN:
            assert tok == O.greedy(ref_pre)
        assert d.position == n
        for l in range(s.n_layers):
            k, v = d.read_kv(l, n)
            ek, ev = kv_excess(k, K16[l]), kv_excess(v, V16[l])
            assert ek.max() <= KV_BATCH and ev.max() <= KV_BATCH, (l, ek.max(), ev.max())
        for i in range(steps):
            tk, lg = d.step(force_tok=int(fed[i]), want_logits=True)
            check_logits(lg, ref[i], f"step {i} after batched prefill of {n}")
            assert tk == int(np.argmax(lg))
        if n == s.max_ctx:
            with pytest.raises(B.DecError) as ei:
                d.step()
            assert ei.value.code == B.DEC_ERR_CONTEXT_FULL


def test_batched_prefill_then_generate_matches_steps(stream):
    """After a batched prefill the device-side next token feeds decode."""
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=33)
    prompt = synth.make_prompt(s.vocab, 13, seed=34)[0]
    with make(s, t, stream, flags=BP) as a, make(s, t, stream, flags=BP) as b:
        ta, _ = a.prefill(prompt)
        tb, _ = b.prefill(prompt)
        assert ta == tb
        ga = a.generate(10)
        gb = [b.step()[0] for _ in range(10)]
        assert list(ga) == gb


# ----------------------------------------------------------------------------
# matrix prefill (DEC_FLAG_MATRIX_PREFILL): every prompt position as a row of
# matrix products on the matrix cores, causal attention on the matrix cores.
# The products' inputs, the rotated queries and the softmax weights are fp16,
# so the cache bound is the batched one (KV_BATCH); logits keep the 2e-2 bound.
# Tiny shapes run every product with split K (partials summed in order); the
# full-size tests run the unsplit tiles.
# ----------------------------------------------------------------------------

MP = B.DEC_FLAG_MATRIX_PREFILL


def check_prefill_kv(d, s, K16, V16, n, what):
    for l in range(s.n_layers):
        k, v = d.read_kv(l, n)
        ek, ev = kv_excess(k, K16[l]), kv_excess(v, V16[l])
        print(f"{what} layer {l}: cache excess k {ek.max():.2e} v {ev.max():.2e}", flush=True)
        assert ek.max() <= KV_BATCH and ev.max() <= KV_BATCH, (l, ek.max(), ev.max())


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 33, 100, 128])
def test_tiny_matrix_prefill(stream, n):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=35, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, n, seed=36 + n)[0]
    steps = min(6, s.max_ctx - n)
    fed, ref, ref_pre, _ = O.greedy_decode(s, t, prompt, steps)
    _, K16, V16, _ = O.prefill_matrix(s, t, prompt)
    with make(s, t, stream, flags=MP) as d:
        tok, pre = d.prefill(prompt, want_logits=True)
        check_logits(pre, ref_pre, f"matrix prefill of {n}")
        assert tok == int(np.argmax(pre))
        assert d.position == n
        check_prefill_kv(d, s, K16, V16, n, f"matrix prefill of {n}")
        for i in range(steps):
            tk, lg = d.step(force_tok=int(fed[i]), want_logits=True)
            check_logits(lg, ref[i], f"step {i} after matrix prefill of {n}")
            assert tk == int(np.argmax(lg))
        if n == s.max_ctx:
            with pytest.raises(B.DecError) as ei:
                d.step()
            assert ei.value.code == B.DEC_ERR_CONTEXT_FULL


def test_matrix_prefill_then_generate_matches_steps(stream):
    """After a matrix prefill the device-side next token feeds decode; a reset
    handle prefills again to the same tokens (no state kept between prompts)."""
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=37)
    prompt = synth.make_prompt(s.vocab, 19, seed=38)[0]
    other = synth.make_prompt(s.vocab, 40, seed=39)[0]
    with make(s, t, stream, flags=MP) as a, make(s, t, stream, flags=MP) as b:
        ta, pa = a.prefill(prompt, want_logits=True)
        b.prefill(other)
        b.generate(5)
        b.reset()
        tb, pb = b.prefill(prompt, want_logits=True)
        assert ta == tb
        np.testing.assert_array_equal(pa, pb)
        ga = a.generate(10)
        gb = [b.step()[0] for _ in range(10)]
        assert list(ga) == gb


@pytest.mark.parametrize("hd,H", [(32, 8), (128, 2)])
def test_matrix_prefill_other_head_dims(stream, hd, H):
    """The attention kernel is built per head dimension: 32 and 128 as well as
    tiny's 64, with the same 256-wide Q/K/V."""
    s = synth.shape_for("tiny").with_(head_dim=hd, n_heads=H)
    t = synth.make_weights(s, seed=61 + hd, gain_jitter=0.1)
    n = 45
    prompt = synth.make_prompt(s.vocab, n, seed=62 + hd)[0]
    fed, ref, ref_pre, _ = O.greedy_decode(s, t, prompt, 3)
    _, K16, V16, _ = O.prefill_matrix(s, t, prompt)
    with make(s, t, stream, flags=MP) as d:
        tok, pre = d.prefill(prompt, want_logits=True)
        check_logits(pre, ref_pre, f"matrix prefill, head dim {hd}")
        check_prefill_kv(d, s, K16, V16, n, f"matrix prefill, head dim {hd}")
        for i in range(3):
            _, lg = d.step(force_tok=int(fed[i]), want_logits=True)
            check_logits(lg, ref[i], f"step {i} after matrix prefill, head dim {hd}")


def test_matrix_prefill_spans_two_chunks(stream):
    """2100 prompt positions: 2048 in the first pass over the weights and 52 in
    the second, whose attention reads the first pass's cache entries."""
    n = 2100
    s = synth.shape_for("tiny").with_(max_ctx=2112)
    t = synth.make_weights(s, seed=47, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, n, seed=48)[0]
    lg, K16, V16, _ = O.prefill_matrix(s, t, prompt)
    ref = O.OracleDecoder(s, t)
    ref.load_cache(K16, V16, n)
    with make(s, t, stream, flags=MP) as d:
        tok, pre = d.prefill(prompt, want_logits=True)
        check_logits(pre, lg[-1], f"matrix prefill of {n}")
        check_prefill_kv(d, s, K16, V16, n, f"matrix prefill of {n}")
        nxt = O.greedy(lg[-1])
        for i in range(3):
            want = ref.step(nxt)
            _, got = d.step(force_tok=int(nxt), want_logits=True)
            check_logits(got, want, f"step {i} after matrix prefill of {n}")
            nxt = O.greedy(want)


# ----------------------------------------------------------------------------
# other grid sizes: fewer workgroups than barrier groups, odd splits
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid", [7, 100])
def test_tiny_other_grids(stream, grid):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=41, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 40, seed=42)[0]
    teacher_forced(s, t, prompt, 6, stream, grid=grid)


def test_tiny_batch_and_batched_prefill_grid_64(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=43)
    prompts = synth.make_prompt(s.vocab, 11, batch=8, seed=44)
    refs = [O.greedy_decode(s, t, prompts[b], 3) for b in range(8)]
    with make(s, t, stream, batch=8, grid=64) as d:
        _, pre = d.prefill(prompts, want_logits=True)
        pre = pre.reshape(8, -1)
        for b in range(8):
            check_logits(pre[b], refs[b][2], f"grid 64 seq {b} prefill")
        for i in range(3):
            ft = np.array([refs[b][0][i] for b in range(8)], dtype=np.int32)
            _, lg = d.step(force_tok=ft, want_logits=True)
            lg = lg.reshape(8, -1)
            for b in range(8):
                check_logits(lg[b], refs[b][1][i], f"grid 64 seq {b} step {i}")
    fed, ref, ref_pre, _ = refs[0]
    with make(s, t, stream, flags=BP, grid=64) as d:
        _, pre = d.prefill(prompts[0], want_logits=True)
        check_logits(pre, ref_pre, "grid 64 batched prefill")
        _, lg = d.step(force_tok=int(fed[0]), want_logits=True)
        check_logits(lg, ref[0], "grid 64 step after batched prefill")


def test_grid_smaller_than_head_pairs_is_unsupported(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=45)
    with pytest.raises(B.DecError) as ei:
        make(s, t, stream, batch=8, grid=16)      # 8 x 4 pairs > 16 workgroups
    assert ei.value.code == B.DEC_ERR_UNSUPPORTED
    with make(s, t, stream, batch=4, grid=16) as d:   # 16 pairs: allowed
        d.prefill(synth.make_prompt(s.vocab, 5, batch=4, seed=46))


@pytest.mark.gpu
def test_stream_ceiling_is_a_plausible_hbm_rate():
    """The plain-stream probe reads 1 GiB three times at a rate an MI355X can reach (below its 8 TB/s peak)."""
    g = B.stream_ceiling(1 << 30, 3)
    assert 1000.0 < g < 8500.0, g
