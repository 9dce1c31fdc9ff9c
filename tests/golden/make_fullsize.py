"""Write the full-size parity fixtures from the CPU oracle alone.

Test infrastructure.  This script imports only `oracle/` (the float64 CPU
reference decoder) and `synth/` (the seeded input generators); nothing here
comes from the HIP library.  The GPU parity tests compare the library's
logits and K/V rows with what this script stores, so the full-size checks do
not depend on any state the GPU produced.

Each fixture is one workload run under teacher forcing: the prompt of the
workload, then `steps` decode steps whose input tokens are drawn from their
own seed (uniform over the vocabulary, like the prompt).  The oracle's matrix
form (`prefill_matrix`, explicit causal mask, K/V rounded to fp16 before any
query reads them) over prompt + forced tokens yields the logits of every
position at once: row p is what the decoder predicts after reading token p,
i.e. the prefill's logits for p = prompt_len - 1 and decode step i's logits
for p = prompt_len + i.  The step form and the matrix form are the same
function (pinned in tests/test_oracle_pins.py).

Stored per fixture (npz, float32 values of float64 results):
  tokens      [batch, n]       prompt + forced tokens (int32)
  pos         [P]              checked positions prompt_len-1 .. n-1
  top_idx     [batch, P, 2]    index of the largest and second-largest logit
  top_val     [batch, P, 2]    their values
  samp_idx    [S]              fixed sample of logit indices (seeded)
  samp_pos    [Q]              positions whose sampled logits are stored
  samp_val    [batch, Q, S]    logits at samp_idx for those positions
  kv_layers, kv_pos            where K/V rows are stored
  kv_K, kv_V  [batch, layers, H, positions, hd] fp16 cache rows
  greedy_*    (dense2b only)   the oracle's free-running greedy decode
  routes      [n, L, k]        (mixture of experts) the experts the oracle's
                               router chose at every position and layer
  route_gap   [n, L]           its gap between the k-th and (k+1)-th logit there

Usage: python tests/golden/make_fullsize.py [name ...]   (default: all)
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

ORACLE_SRC = os.path.join(ROOT, "oracle", "decoder.py")
MOE_SRC = os.path.join(ROOT, "oracle", "moe.py")
N_SAMPLES = 1024
FORCED_SEED = 7          # seed of the forced decode tokens (the prompt uses the workload's prompt seed)
SAMPLE_SEED = 12345      # seed of the sampled logit indices

# name -> (workload, prompt_len, forced steps, positions whose sampled logits are
# stored (beyond every `every`-th), every, kv layers, kv positions, sequences
# of a batch whose K/V rows are stored)
FIXTURES = {
    # the metric's workload: 128 + 512, across the switch from one to three
    # attention workgroups per head at 512 positions
    "dense2b": dict(workload="dense2b", prompt_len=128, steps=512, every=8,
                    extra=[126, 127, 128, 129, 508, 509, 510, 511, 512, 513, 514, 515, 516, 639],
                    kv_layers=[0, 1, 12, 24], kv_pos=[0, 5, 127, 128, 511, 512, 639]),
    # one lane of the 8-way split at its real shape: 128 + 1024
    "lane2b": dict(workload="lane2b", prompt_len=128, steps=1024, every=16,
                   extra=[127, 128, 511, 512, 513, 1150, 1151],
                   kv_layers=[0, 12, 24], kv_pos=[0, 127, 128, 640, 1151]),
    # long context: a 3968-token prompt, then decode to the 4096 cap
    "dense2b_long": dict(workload="dense2b_long", prompt_len=3968, steps=128, every=8,
                         extra=[3967, 3968, 3969, 4094, 4095],
                         kv_layers=[0, 1, 12, 24], kv_pos=[0, 5, 1983, 3967, 3968, 4095]),
    # eight sequences of 256-token prompts, then 256 steps together
    "dense2b_b8": dict(workload="dense2b_b8", prompt_len=256, steps=256, every=16,
                       extra=[255, 256, 257, 510, 511],
                       kv_layers=[0, 12, 24], kv_pos=[0, 255, 256, 511], kv_seqs=[0, 7]),
    # dense2b from a 700-token prompt: each head's attention on three, then
    # (past 768 positions) four workgroups
    "dense2b_w4": dict(workload="dense2b", prompt_len=700, steps=152, every=8,
                       extra=[699, 700, 701, 766, 767, 768, 769, 850, 851],
                       kv_layers=[0, 12, 24], kv_pos=[0, 699, 700, 767, 768, 851]),
    # one lane after a 2000-token prompt: 3 heads, each on 8 workgroups
    "lane2b_long": dict(workload="lane2b", prompt_len=2000, steps=16, every=4,
                        extra=[1999, 2000, 2015],
                        kv_layers=[0, 12, 24], kv_pos=[0, 1000, 1999, 2000, 2015]),
    # batch 8 after 3968-token prompts: every (sequence, head) pair's attention
    # over nearly the whole 4096-position cache
    "dense2b_b8_long": dict(workload="dense2b_b8", prompt_len=3968, steps=8, every=1,
                            extra=[], kv_layers=[0, 12, 24], kv_pos=[0, 1983, 3967, 3975], kv_seqs=[0, 7]),
    # dense2b's attention with 32 FP8 experts, top-4: 128 + 64
    "moe2b": dict(workload="moe2b", prompt_len=128, steps=64, every=4, extra=[127, 128, 129, 190, 191],
                  kv_layers=[0, 1, 12, 24], kv_pos=[0, 5, 127, 128, 191]),
    # the same with MXFP4 experts
    "moe2b_mx": dict(workload="moe2b_mx", prompt_len=128, steps=64, every=4, extra=[127, 128, 129, 190, 191],
                     kv_layers=[0, 1, 12, 24], kv_pos=[0, 5, 127, 128, 191]),
}
GREEDY_STEPS = 16        # dense2b: free-running greedy steps after the 128-token prompt


def oracle_sha(path=ORACLE_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def forced_tokens(vocab, steps, batch):
    """The teacher-forced decode inputs: uniform token ids from their own seed."""
    return synth.make_prompt(vocab, steps, batch=batch, seed=FORCED_SEED)


def top2(logits):
    """(indices, values) of the two largest logits per row; ties: lowest index first."""
    order = np.argsort(-logits, axis=-1, kind="stable")[..., :2]
    return order.astype(np.int32), np.take_along_axis(logits, order, axis=-1)


def make(name):
    cfg = FIXTURES[name]
    w = synth.workload(cfg["workload"])
    s = w.shape
    n0, steps, nb = cfg["prompt_len"], cfg["steps"], w.batch
    t0 = time.time()
    tensors = synth.workload_weights(w)
    prompt = synth.make_prompt(s.vocab, n0, batch=nb, seed=w.prompt_seed)
    forced = forced_tokens(s.vocab, steps, nb)
    tokens = np.concatenate([prompt, forced], axis=1).astype(np.int32)   # [batch, n]
    n = tokens.shape[1]
    assert n <= s.max_ctx
    pos = np.arange(n0 - 1, n, dtype=np.int32)
    samp_pos = sorted(set(range(n0 - 1, n, cfg["every"])) | {p for p in cfg["extra"] if n0 - 1 <= p < n})
    samp_pos = np.array(samp_pos, dtype=np.int32)
    rng = np.random.default_rng(SAMPLE_SEED)
    samp_idx = np.sort(rng.choice(s.lm_vocab, size=min(N_SAMPLES, s.lm_vocab), replace=False)).astype(np.int32)
    kv_layers = np.array(cfg["kv_layers"], dtype=np.int32)
    kv_pos = np.array(cfg["kv_pos"], dtype=np.int32)
    kv_seqs = cfg.get("kv_seqs", [0])
    top_idx = np.zeros((nb, len(pos), 2), np.int32)
    top_val = np.zeros((nb, len(pos), 2), np.float32)
    samp_val = np.zeros((nb, len(samp_pos), len(samp_idx)), np.float32)
    kv_K = np.zeros((len(kv_seqs), len(kv_layers), s.n_heads, len(kv_pos), s.head_dim), np.float16)
    kv_V = np.zeros_like(kv_K)
    extra = {}
    for b in range(nb):
        if s.moe:
            logits, K16, V16, routes, gaps = O.prefill_matrix_moe(s, tensors, tokens[b])
            extra = dict(routes=routes.astype(np.int8), route_gap=gaps.astype(np.float32))
        else:
            logits, K16, V16, _ = O.prefill_matrix(s, tensors, tokens[b])
        ti, tv = top2(logits[pos])
        top_idx[b], top_val[b] = ti, tv.astype(np.float32)
        samp_val[b] = logits[samp_pos][:, samp_idx].astype(np.float32)
        if b in kv_seqs:
            j = kv_seqs.index(b)
            kv_K[j] = K16[kv_layers][:, :, kv_pos]
            kv_V[j] = V16[kv_layers][:, :, kv_pos]
        print(f"{name}: sequence {b} done ({time.time() - t0:.0f} s)", flush=True)
    out = dict(tokens=tokens, pos=pos, top_idx=top_idx, top_val=top_val, samp_idx=samp_idx,
               samp_pos=samp_pos, samp_val=samp_val, kv_layers=kv_layers, kv_pos=kv_pos,
               kv_seqs=np.array(kv_seqs, dtype=np.int32), kv_K=kv_K, kv_V=kv_V, **extra)
    if name == "dense2b":
        # free-running greedy decode of the oracle from the same prompt
        fed, lg, pre, nxt = O.greedy_decode(s, tensors, prompt[0], GREEDY_STEPS)
        margins = [O.top2_margin(pre)] + [O.top2_margin(r) for r in lg]
        out["greedy_tokens"] = np.array(list(fed) + [nxt], dtype=np.int32)   # prefill's token, then each step's
        out["greedy_margins"] = np.array(margins, dtype=np.float64)
        print(f"{name}: greedy decode of {GREEDY_STEPS} steps done ({time.time() - t0:.0f} s)", flush=True)
    meta = dict(fixture=name, workload=w.name, prompt_len=n0, steps=steps, batch=nb,
                weight_seed=w.weight_seed, prompt_seed=w.prompt_seed, forced_seed=FORCED_SEED,
                sample_seed=SAMPLE_SEED, oracle_sha=oracle_sha(), script="tests/golden/make_fullsize.py")
    if s.moe:
        meta["moe_sha"] = oracle_sha(MOE_SRC)
    out["meta"] = np.array(json.dumps(meta))
    path = os.path.join(HERE, f"fullsize_{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: wrote {path} ({os.path.getsize(path) / 1e6:.2f} MB, {time.time() - t0:.0f} s)", flush=True)
    return path


def main(argv):
    names = argv or list(FIXTURES)
    for n in names:
        make(n)


if __name__ == "__main__":
    main(sys.argv[1:])
