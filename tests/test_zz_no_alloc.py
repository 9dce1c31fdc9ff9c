"""The no-allocation entry point (dec_init_noalloc) against dec_init.

A no-allocation handle runs the same kernels with their scratch in the
library's fixed per-device array instead of the arena, so its tokens and
logits must equal a dec_init handle's bit for bit.  Two handles are made in a
row, the second with a smaller input, so the second starts on an array the
first left dirty (barrier counters past zero, stale exchange vectors).
"""
import numpy as np
import pytest

import synth
from memory_bound_transformer_persistent_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stream():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.cuda.Stream(device=0)


def run(dec, prompt, steps, gen):
    tok, pre = dec.prefill(prompt, want_logits=True)
    logits, toks = [pre], [tok]
    for _ in range(steps):
        t, lg = dec.step(want_logits=True)
        logits.append(lg)
        toks.append(t)
    toks.append(dec.generate(gen))
    return np.stack(logits), np.concatenate([np.atleast_1d(np.asarray(x)).ravel() for x in toks])


def arena_for(desc):
    import torch
    n = B.arena_bytes(desc)
    return torch.empty(n, dtype=torch.uint8, device="cuda:0"), n


def test_noalloc_equals_dec_init_on_two_calls_in_a_row(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=51, gain_jitter=0.1)
    desc = B.ModelDesc.from_shape(s)
    arena, n = arena_for(desc)
    for plen, steps, gen in ((40, 12, 10), (9, 4, 3)):          # the second call's input is smaller
        prompt = synth.make_prompt(s.vocab, plen, seed=52 + plen)[0]
        with B.Decoder(desc, tensors=t, stream=stream.cuda_stream) as ref:
            want = run(ref, prompt, steps, gen)
        with B.Decoder(desc, tensors=t, stream=stream.cuda_stream, arena=arena.data_ptr(), arena_bytes=n,
                       noalloc=True) as d:
            got = run(d, prompt, steps, gen)
        np.testing.assert_array_equal(got[0], want[0])
        np.testing.assert_array_equal(got[1], want[1])
        print(f"prompt {plen} + {steps} steps + {gen} generated: no-allocation handle equals dec_init bitwise",
              flush=True)


def test_noalloc_matrix_prefill_equals_dec_init(stream):
    """With DEC_FLAG_MATRIX_PREFILL the prefill's workspace sits in the caller's
    arena; two handles in a row, the second with a smaller prompt, equal
    dec_init bitwise."""
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=55, gain_jitter=0.1)
    desc = B.ModelDesc.from_shape(s, flags=B.DEC_FLAG_MATRIX_PREFILL)
    arena, n = arena_for(desc)
    for plen, steps, gen in ((70, 8, 6), (12, 3, 2)):
        prompt = synth.make_prompt(s.vocab, plen, seed=56 + plen)[0]
        with B.Decoder(desc, tensors=t, stream=stream.cuda_stream) as ref:
            want = run(ref, prompt, steps, gen)
        with B.Decoder(desc, tensors=t, stream=stream.cuda_stream, arena=arena.data_ptr(), arena_bytes=n,
                       noalloc=True) as d:
            got = run(d, prompt, steps, gen)
        np.testing.assert_array_equal(got[0], want[0])
        np.testing.assert_array_equal(got[1], want[1])
        print(f"matrix prefill {plen} + {steps} steps + {gen} generated: no-allocation handle equals dec_init bitwise",
              flush=True)


def test_noalloc_batch8_and_dense2b_equal_dec_init(stream):
    # batch 8 on the tiny shape (batched kernel, larger scratch) ...
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=53)
    desc = B.ModelDesc.from_shape(s, batch=8)
    prompts = synth.make_prompt(s.vocab, 11, batch=8, seed=54)
    arena, n = arena_for(desc)
    with B.Decoder(desc, tensors=t, stream=stream.cuda_stream) as ref:
        want = run(ref, prompts, 3, 2)
    with B.Decoder(desc, tensors=t, stream=stream.cuda_stream, arena=arena.data_ptr(), arena_bytes=n,
                   noalloc=True) as d:
        got = run(d, prompts, 3, 2)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    del arena
    # ... then the 2.3B shape at batch 1 (smaller scratch than batch 8's)
    w = synth.workload("dense2b")
    t = synth.workload_weights(w)
    desc = B.ModelDesc.from_shape(w.shape)
    prompt = synth.make_prompt(w.shape.vocab, 16, seed=w.prompt_seed)[0]
    arena, n = arena_for(desc)
    with B.Decoder(desc, tensors=t, stream=stream.cuda_stream) as ref:
        want = run(ref, prompt, 3, 2)
    with B.Decoder(desc, tensors=t, stream=stream.cuda_stream, arena=arena.data_ptr(), arena_bytes=n,
                   noalloc=True) as d:
        got = run(d, prompt, 3, 2)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


def test_noalloc_rules(stream):
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=55)
    desc = B.ModelDesc.from_shape(s)
    arena, n = arena_for(desc)
    kw = dict(tensors=t, stream=stream.cuda_stream, noalloc=True)
    # arena and stream are required
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc, tensors=t, stream=stream.cuda_stream, noalloc=True)
    assert e.value.code == B.DEC_ERR_INVALID_ARG
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc, tensors=t, arena=arena.data_ptr(), arena_bytes=n, noalloc=True)
    assert e.value.code == B.DEC_ERR_INVALID_ARG
    # one no-allocation handle per device at a time
    with B.Decoder(desc, arena=arena.data_ptr(), arena_bytes=n, **kw) as d:
        other, m = arena_for(desc)
        with pytest.raises(B.DecError) as e:
            B.Decoder(desc, arena=other.data_ptr(), arena_bytes=m, **kw)
        assert e.value.code == B.DEC_ERR_STATE
        d.prefill([1, 2, 3])
    with B.Decoder(desc, arena=arena.data_ptr(), arena_bytes=n, **kw) as d:   # released by dec_free
        d.prefill([4, 5])
    # a description whose scratch passes the fixed array's size, rejected
    # before any upload: 8 sequences at a 65536-position cap with the trace on
    # (trace 8 MiB, token buffers 4 MiB, attention partials 4 MiB, logits 2 MiB)
    big = s.with_(n_layers=1, d_model=2560, n_heads=32, head_dim=128, d_ffn=6912, vocab=65536, lm_vocab=65536,
                  max_ctx=65536)
    dummy = [np.zeros(1, np.float16)] * len(synth.tensor_names(big))
    with pytest.raises(B.DecError) as e:
        B.Decoder(B.ModelDesc.from_shape(big, batch=8), tensors=dummy, stream=stream.cuda_stream,
                  arena=arena.data_ptr(), arena_bytes=n, noalloc=True, debug_flags=B.DEC_DEBUG_TRACE)
    assert e.value.code == B.DEC_ERR_UNSUPPORTED
    assert "scratch" in str(e.value)
