"""GPU: the decode server against one kernel launch per step.

A decode-server handle (serve_idle_us > 0) runs a run of dec_step calls in one
resident launch that takes each step from a host-pinned mailbox.  Its kernel
arithmetic is the per-step launch's, so every output here must be bitwise the
same as a plain handle's for the same calls: greedy tokens, logits and the KV
cache.  The plain path is compared with the oracle in the other GPU tests; one
teacher-forced run below also compares the server path with the oracle
directly.  The server handles run on their own library-owned stream, after the
plain handle has finished: a running server holds every compute unit, so
work of another handle would wait for its idle end.
"""
import time

import numpy as np
import pytest

import oracle as O
import synth
from memory_bound_transformer_persistent_amd import binding as B

pytestmark = pytest.mark.gpu

IDLE_US = 300000   # 0.3 s: no test pauses this long between steps unless it means to


@pytest.fixture(scope="module")
def stream():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.cuda.Stream(device=0)


def run(shape, tensors, prompt, script, batch=1, stream=None, serve=0, flags=0, **kw):
    """Apply `script` to a fresh handle; returns every output in order."""
    out = []
    dec = B.Decoder(B.ModelDesc.from_shape(shape, batch=batch, flags=flags), tensors=tensors, device=0,
                    stream=None if stream is None else stream.cuda_stream, serve_idle_us=serve, **kw)
    try:
        out.append(dec.prefill(prompt, want_logits=True))
        for op in script:
            kind = op[0]
            if kind == "step":
                _, force, want_tok, want_lg = op
                out.append(dec.step(force_tok=force, want_tok=want_tok, want_logits=want_lg))
            elif kind == "generate":
                out.append(dec.generate(op[1]))
            elif kind == "sync":
                dec.sync()
            elif kind == "sleep":
                time.sleep(op[1])
            elif kind == "kv":
                out.append(dec.read_kv(op[1], dec.position))
            elif kind == "restart":
                dec.reset()
                out.append(dec.prefill(op[1], want_logits=True))
            else:
                raise ValueError(kind)
            out.append(dec.position)
        dec.sync()
        out.append(dec.position)
    finally:
        dec.close()
    return out


def same(a, b, what=""):
    assert len(a) == len(b), what
    for i, (x, y) in enumerate(zip(a, b)):
        if isinstance(x, tuple):
            for xx, yy in zip(x, y):
                if xx is None or yy is None:
                    assert xx is None and yy is None, (what, i)
                else:
                    np.testing.assert_array_equal(np.asarray(xx), np.asarray(yy), err_msg=f"{what} output {i}")
        else:
            np.testing.assert_array_equal(np.asarray(x), np.asarray(y), err_msg=f"{what} output {i}")


def compare(shape, tensors, prompt, script, stream, batch=1, serve=IDLE_US, flags=0):
    ref = run(shape, tensors, prompt, script, batch=batch, stream=stream, flags=flags)
    got = run(shape, tensors, prompt, script, batch=batch, serve=serve, flags=flags)
    same(ref, got, "server vs one launch per step")
    return got


def tiny():
    s = synth.shape_for("tiny")
    return s, synth.make_weights(s, seed=31, gain_jitter=0.1)


def test_server_steps_bitwise(stream):
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 14, seed=2)[0]
    rng = np.random.default_rng(5)
    script = []
    for i in range(40):
        force = int(rng.integers(0, s.vocab)) if i % 7 == 3 else None
        script.append(("step", force, i % 2 == 0, i % 3 == 0))
    script += [("kv", l) for l in range(s.n_layers)]
    compare(s, t, prompt, script, stream)


def test_server_after_matrix_prefill(stream):
    """The matrix prefill (its own kernels on the handle's stream) hands its
    cache and next token to the decode server as to a per-step launch; a
    reset and a second matrix prefill follow a running server launch."""
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 23, seed=6)[0]
    other = synth.make_prompt(s.vocab, 9, seed=7)[0]
    script = [("step", None, True, i % 4 == 0) for i in range(12)]
    script += [("restart", other)] + [("step", None, True, True) for _ in range(6)]
    script += [("kv", l) for l in range(s.n_layers)]
    compare(s, t, prompt, script, stream, flags=B.DEC_FLAG_MATRIX_PREFILL)


def test_server_async_steps_past_the_ring(stream):
    # 110 steps posted without waiting: the host wraps the 64-slot request ring
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 9, seed=4)[0]
    script = [("step", None, False, False)] * 110 + [("step", None, True, True)]
    script += [("kv", l) for l in range(s.n_layers)]
    compare(s, t, prompt, script, stream)


def test_server_mixed_with_other_calls(stream):
    # every other call ends the server launch first; the next step starts another
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 11, seed=6)[0]
    script = ([("step", None, True, False)] * 5 + [("generate", 6)] + [("step", 3, True, True)] +
              [("step", None, False, False)] * 4 + [("sync",), ("kv", 0)] + [("step", None, True, False)] * 3 +
              [("restart", synth.make_prompt(s.vocab, 5, seed=7)[0])] + [("step", None, True, True)] * 4 +
              [("kv", 1)])
    compare(s, t, prompt, script, stream)


def test_server_idle_end_and_restart(stream):
    # a 2 ms idle bound: each pause lets the launch close its mailbox and end;
    # the next step starts a new launch
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 8, seed=8)[0]
    script = []
    for j in range(4):
        script += [("step", None, True, j % 2 == 1)] * 3 + [("sleep", 0.05)]
    script += [("step", None, False, False)] * 3 + [("sleep", 0.05), ("step", None, True, True)]
    compare(s, t, prompt, script, stream, serve=2000)


def test_server_batch(stream):
    s, t = tiny()
    nb = 3
    prompt = synth.make_prompt(s.vocab, 10, batch=nb, seed=9)
    script = [("step", None, True, True)] * 6 + [("step", [1, 2, 3], True, True)] + [("step", None, True, False)] * 5
    compare(s, t, prompt, script, stream, batch=nb)


def test_server_dense2b(stream):
    # the 2.3B shape (the head-dim-128 kernel the benchmark times), across the
    # request ring and with logits on some steps
    s = synth.shape_for("dense2b")
    t = synth.make_weights(s, seed=0)
    prompt = synth.make_prompt(s.vocab, 128, seed=1)[0]
    script = ([("step", None, True, True)] * 3 + [("step", None, False, False)] * 70 + [("step", 17, True, True)] +
              [("step", None, True, False)] * 4 + [("kv", 0), ("kv", s.n_layers - 1)])
    compare(s, t, prompt, script, stream)


def test_server_teacher_forced_matches_oracle():
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 12, seed=10)[0]
    n = 12
    fed, ref, ref_pre, _ = O.greedy_decode(s, t, prompt, n)
    with B.Decoder(B.ModelDesc.from_shape(s), tensors=t, device=0, serve_idle_us=IDLE_US) as dec:
        _, pre = dec.prefill(prompt, want_logits=True)
        assert float(np.max(np.abs(pre - ref_pre))) <= 2e-2
        for i in range(n):
            tok, lg = dec.step(force_tok=int(fed[i]), want_logits=True)
            err = float(np.max(np.abs(np.asarray(lg, np.float64) - ref[i])))
            assert err <= 2e-2, (i, err)
            assert tok == int(np.argmax(lg))


def test_server_watchdog_is_an_error_not_a_hang():
    s, t = tiny()
    prompt = synth.make_prompt(s.vocab, 4, seed=1)[0]
    with B.Decoder(B.ModelDesc.from_shape(s), tensors=t, device=0, serve_idle_us=IDLE_US) as dec:
        dec.prefill(prompt)
    # every barrier wait of the server launch expires at once
    with B.Decoder(B.ModelDesc.from_shape(s), tensors=t, device=0, serve_idle_us=IDLE_US, watchdog_us=1) as dec:
        with pytest.raises(B.DecError) as e:
            dec.prefill(prompt)
        assert e.value.code == B.DEC_ERR_TIMEOUT
        dec.reset()
        with pytest.raises(B.DecError) as e:
            dec.step(force_tok=1)
        assert e.value.code == B.DEC_ERR_TIMEOUT
        dec.reset()
