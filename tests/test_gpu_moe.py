"""GPU parity of the mixture-of-experts path (router, FP8 E4M3 expert GEMVs)
through the C ABI against the float64 oracle (oracle.moe).

Tolerance: the dense bar, max |logit_gpu - logit_oracle| <= 2e-2 per
teacher-forced step, the same greedy token wherever the oracle's top-2
margin exceeds 0.05, and K/V rows within 2e-3.

Routing.  The router's top-k choice is an integer decided by floating
point: two experts whose logits differ by less than the accumulated rounding
may be ordered either way, and both choices are correct.  The routes are
compared at every position and layer (dec_read_routes); where the library's
set differs from the oracle's own, the oracle's gap between its k-th and
(k+1)-th logit there must be below ROUTE_TIE, and the oracle then
recomputes that position with the library's choice, so that what follows is
compared on the same path.  The tests print how often that happened.
"""
import numpy as np
import pytest

import oracle as O
import synth
from memory_bound_transformer_persistent_amd import binding as B

pytestmark = pytest.mark.gpu

TOL = 2e-2
MARGIN = 0.05
KV_TOL = 2e-3
ROUTE_TIE = 5e-3

TINY_MOE = synth.shape_for("tiny").with_(d_ffn=256, n_experts=8, top_k=2)


@pytest.fixture(scope="module")
def stream():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.cuda.Stream(device=0)


def make(shape, tensors, stream, **kw):
    return B.Decoder(B.ModelDesc.from_shape(shape), tensors=tensors, device=0, stream=stream.cuda_stream, **kw)


def check_logits(gpu, ref, what, tol=TOL):
    err = float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)))
    assert err <= tol, f"{what}: {err}"
    if O.top2_margin(ref) > MARGIN:
        assert int(np.argmax(gpu)) == O.greedy(ref), what
    return err


def oracle_step(orc, tok, gpu_routes):
    """One oracle step that follows the library's routing where it differs
    from the oracle's own only at near-ties.  Returns (logits, layers that
    were forced)."""
    p = orc.pos
    lg = orc.step(int(tok))
    same = [set(a) == set(b) for a, b in zip(orc.last_routes, gpu_routes)]
    if all(same):
        return lg, 0
    orc.pos = p
    lg = orc.step(int(tok), force_routes=[list(r) for r in gpu_routes])
    forced = 0
    for l in range(orc.s.n_layers):
        if set(orc.last_natural[l]) != set(gpu_routes[l]):
            forced += 1
            assert orc.last_margins[l] < ROUTE_TIE, \
                f"position {p} layer {l}: routes {list(gpu_routes[l])} vs {list(orc.last_natural[l])}, " \
                f"oracle gap {orc.last_margins[l]:.3e}"
    return lg, forced


def moe_teacher_forced(shape, tensors, prompt, n_steps, stream, **kw):
    """GPU prefill (one launch) then n_steps steps fed the oracle's greedy
    tokens; routes, K/V and logits compared as the module says."""
    orc = O.OracleMoEDecoder(shape, tensors)
    n = len(prompt)
    worst, forced = 0.0, 0
    with make(shape, tensors, stream, **kw) as dec:
        tok, pre = dec.prefill(prompt, want_logits=True)
        routes = dec.read_routes(0, n)
        assert routes.min() >= 0 and routes.max() < shape.n_experts
        for i in range(n):
            ref, f = oracle_step(orc, prompt[i], routes[i])
            forced += f
        worst = max(worst, check_logits(pre, ref, "prefill"))
        if O.top2_margin(ref) > MARGIN:
            assert tok == O.greedy(ref)
        for l in range(shape.n_layers):
            k16, v16 = dec.read_kv(l, n)
            for got, want, what in ((k16, orc.Kc[l, :, :n], "K"), (v16, orc.Vc[l, :, :n], "V")):
                err = float(np.max(np.abs(got.astype(np.float64) - want.astype(np.float64))))
                assert err <= KV_TOL, f"layer {l} {what}: {err}"
        nxt = O.greedy(ref)
        for i in range(n_steps):
            t, lg = dec.step(force_tok=nxt, want_logits=True)
            r = dec.read_routes(n + i, 1)[0]
            ref, f = oracle_step(orc, nxt, r)
            forced += f
            worst = max(worst, check_logits(lg, ref, f"step {i}"))
            assert t == int(np.argmax(lg))
            nxt = O.greedy(ref)
        assert dec.read_routes(n + n_steps, 1).min() == -1 if n + n_steps < shape.max_ctx else True
    print(f"max |gpu - oracle| = {worst:.3e}; {forced} near-tie routing choices followed", flush=True)
    return worst, forced


def test_moe_tiny_teacher_forced(stream):
    t = synth.make_weights(TINY_MOE, seed=41, gain_jitter=0.1)
    prompt = synth.make_prompt(TINY_MOE.vocab, 16, seed=42)[0]
    worst, forced = moe_teacher_forced(TINY_MOE, t, prompt, 24, stream)
    assert forced == 0


def test_moe_ragged_pieces(stream):
    # d 384 and expert width 160: every expert row ends inside a 1 KB piece
    # (24 and 10 lanes with codes), 3 of 10 experts, three layers
    s = synth.shape_for("tiny").with_(n_layers=3, d_model=384, n_heads=6, head_dim=64, d_ffn=160,
                                      n_experts=10, top_k=3, max_ctx=64)
    t = synth.make_weights(s, seed=43, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 9, seed=44)[0]
    moe_teacher_forced(s, t, prompt, 8, stream)


def test_moe_two_pieces_and_one_expert(stream):
    # expert width 1040: down rows of one full piece plus one lane; top-1 of 2
    s = synth.shape_for("tiny").with_(n_layers=2, d_ffn=1040, n_experts=2, top_k=1, max_ctx=48)
    t = synth.make_weights(s, seed=45)
    prompt = synth.make_prompt(s.vocab, 6, seed=46)[0]
    moe_teacher_forced(s, t, prompt, 6, stream)


def test_moe_most_experts(stream):
    # the limits: 64 experts, 8 per token (the down input is 8 x 64 wide)
    s = synth.shape_for("tiny").with_(n_layers=2, d_ffn=64, n_experts=64, top_k=8, max_ctx=48)
    t = synth.make_weights(s, seed=47, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 7, seed=48)[0]
    moe_teacher_forced(s, t, prompt, 6, stream)


def test_moe_generate_equals_steps_and_stress_bitwise(stream):
    t = synth.make_weights(TINY_MOE, seed=49)
    prompt = synth.make_prompt(TINY_MOE.vocab, 10, seed=50)[0]
    with make(TINY_MOE, t, stream) as a, make(TINY_MOE, t, stream) as b, \
            make(TINY_MOE, t, stream, debug_flags=B.DEC_DEBUG_STRESS) as c:
        ta, _ = a.prefill(prompt)
        tb, _ = b.prefill(prompt)
        tc, _ = c.prefill(prompt)
        assert ta == tb == tc
        ga = a.generate(12)
        gb = [b.step()[0] for _ in range(12)]
        gc = c.generate(12)
        assert list(ga) == gb == list(gc)
        ra, rb, rc = a.read_routes(0, 22), b.read_routes(0, 22), c.read_routes(0, 22)
        assert np.array_equal(ra, rb) and np.array_equal(ra, rc)
        for l in range(TINY_MOE.n_layers):
            assert np.array_equal(a.read_kv(l, 22)[0].view(np.uint16), c.read_kv(l, 22)[0].view(np.uint16))
        a.reset()
        assert a.read_routes(0, 1).min() == -1


def test_moe_rejections(stream):
    t = synth.make_weights(TINY_MOE, seed=51)
    with pytest.raises(B.DecError, match="UNSUPPORTED"):
        make(TINY_MOE, t, stream, debug_flags=B.DEC_DEBUG_MULTILAUNCH)
    with make(TINY_MOE.with_(n_experts=0, top_k=0), synth.make_weights(synth.shape_for("tiny").with_(d_ffn=256),
                                                                        seed=52), stream) as dense:
        with pytest.raises(B.DecError, match="STATE"):
            dense.read_routes(0, 1)


# ----------------------------------------------------------------------------
# MXFP4 experts (DEC_FLAG_EXPERTS_MXFP4)
# ----------------------------------------------------------------------------

def test_moe_mxfp4_tiny_teacher_forced(stream):
    s = TINY_MOE.with_(mxfp4=True)
    t = synth.make_weights(s, seed=61, gain_jitter=0.1)
    prompt = synth.make_prompt(s.vocab, 16, seed=62)[0]
    worst, forced = moe_teacher_forced(s, t, prompt, 16, stream)
    assert forced == 0


def test_moe_mxfp4_ragged_pieces(stream):
    # d 384 and expert width 160: rows of 192 and 80 bytes of code pairs end
    # inside a 1 KB piece (12 and 5 lanes); expert width 2080 (second test):
    # down rows of a full piece plus one lane
    s = synth.shape_for("tiny").with_(n_layers=3, d_model=384, n_heads=6, head_dim=64, d_ffn=160,
                                      n_experts=10, top_k=3, max_ctx=64, mxfp4=True)
    t = synth.make_weights(s, seed=63, gain_jitter=0.1)
    moe_teacher_forced(s, t, synth.make_prompt(s.vocab, 9, seed=64)[0], 8, stream)
    s2 = synth.shape_for("tiny").with_(n_layers=2, d_ffn=2080, n_experts=4, top_k=2, max_ctx=48, mxfp4=True)
    t2 = synth.make_weights(s2, seed=65)
    moe_teacher_forced(s2, t2, synth.make_prompt(s2.vocab, 6, seed=66)[0], 6, stream)


def test_moe_mxfp4_rules(stream):
    s = TINY_MOE.with_(mxfp4=True)
    assert B.check_desc(B.ModelDesc.from_shape(s)) == B.DEC_OK
    assert B.check_desc(B.ModelDesc.from_shape(s, d_ffn=272)) == B.DEC_ERR_UNSUPPORTED      # not a multiple of 32
    dense = synth.shape_for("tiny")
    assert B.check_desc(B.ModelDesc.from_shape(dense, flags=B.DEC_FLAG_EXPERTS_MXFP4)) == B.DEC_ERR_BAD_DESC
