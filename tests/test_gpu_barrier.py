"""The grid barrier under its debug modes (GPU).

DEC_DEBUG_FENCED adds agent-scope release/acquire fences around every
barrier; DEC_DEBUG_STRESS delays each workgroup's arrival by a pseudo-random
0-2 us and fills every exchange buffer with NaN between its last read and its
next write.  Neither changes any arithmetic, so both must reproduce the
default path's logits and tokens bit for bit.  A read that raced a write
(a stale or poisoned value reaching a phase's input) would show as NaN or as
a difference; each test stops at the first differing step.
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


def make(shape, t, stream, batch=1, flags=0, debug=0):
    return B.Decoder(B.ModelDesc.from_shape(shape, batch=batch, flags=flags), tensors=t, device=0,
                     stream=stream.cuda_stream, debug_flags=debug)


def compare(shape, t, prompt, steps, gen, stream, debug, batch=1, flags=0, what=""):
    with make(shape, t, stream, batch, flags) as ref, make(shape, t, stream, batch, flags, debug) as d:
        _, la = ref.prefill(prompt, want_logits=True)
        _, lb = d.prefill(prompt, want_logits=True)
        assert not np.isnan(lb).any(), f"{what}: NaN in the prefill logits"
        np.testing.assert_array_equal(la, lb, err_msg=f"{what}: prefill")
        for i in range(steps):
            ta, la = ref.step(want_logits=True)
            tb, lb = d.step(want_logits=True)
            assert not np.isnan(lb).any(), f"{what}: NaN in step {i}'s logits"
            np.testing.assert_array_equal(la, lb, err_msg=f"{what}: step {i}")
            np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(ref.generate(gen), d.generate(gen), err_msg=f"{what}: generate")
    print(f"{what}: prefill + {steps} steps + {gen} generated, bitwise equal to the default path", flush=True)


@pytest.mark.parametrize("mode", ["fenced", "stress"])
def test_tiny_debug_mode_is_bitwise_default(stream, mode):
    debug = B.DEC_DEBUG_FENCED if mode == "fenced" else B.DEC_DEBUG_STRESS
    s = synth.shape_for("tiny")
    t = synth.make_weights(s, seed=61, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 40, seed=62)[0]
    compare(s, t, prompt, 24, 16, stream, debug, what=f"tiny {mode}")
    prompts = synth.make_prompt(s.vocab, 12, batch=8, seed=63)
    compare(s, t, prompts, 8, 4, stream, debug, batch=8, what=f"tiny batch 8 {mode}")
    compare(s, t, prompt, 6, 4, stream, debug, flags=B.DEC_FLAG_BATCHED_PREFILL, what=f"tiny batched prefill {mode}")


@pytest.mark.parametrize("mode", ["fenced", "stress"])
def test_dense2b_debug_mode_is_bitwise_default(stream, mode):
    """dense2b from a 500-token prompt through 516 positions: attention on one,
    then three workgroups per head (partials through memory, last-arriver merge)."""
    debug = B.DEC_DEBUG_FENCED if mode == "fenced" else B.DEC_DEBUG_STRESS
    w = synth.workload("dense2b")
    t = synth.workload_weights(w)
    prompt = synth.make_prompt(w.shape.vocab, 500, seed=w.prompt_seed)[0]
    compare(w.shape, t, prompt, 16, 8, stream, debug, what=f"dense2b {mode}")
