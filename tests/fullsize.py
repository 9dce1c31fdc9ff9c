"""Loading and checking the full-size parity fixtures (tests/golden/fullsize_*.npz).

The fixtures hold what the CPU oracle computes for each workload at its real
size under teacher forcing (tests/golden/make_fullsize.py writes them from
`oracle/` and `synth/` alone).  The GPU tests feed the library the same
tokens and compare, position by position:

  * the logits at the oracle's two largest indices (every checked position)
    and at a fixed sample of 1024 indices (every stored position), max-abs
    against the logit bound;
  * the greedy token, wherever the oracle's top-2 margin exceeds 0.05;
  * the fp16 K/V cache rows stored for a few layers and positions.
"""
import hashlib
import json
import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GOLDEN = os.path.join(HERE, "golden")
ORACLE_SRC = os.path.join(ROOT, "oracle", "decoder.py")
FORCED_SEED = 7

TOL = 2e-2
MARGIN = 0.05


def oracle_sha():
    return hashlib.sha256(open(ORACLE_SRC, "rb").read()).hexdigest()[:16]


class Fixture:
    def __init__(self, name):
        self.path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
        f = np.load(self.path, allow_pickle=False)
        self.meta = json.loads(str(f["meta"]))
        for k in f.files:
            if k != "meta":
                setattr(self, k, f[k])
        self.workload = synth.workload(self.meta["workload"])
        self.shape = self.workload.shape
        self.n0 = self.meta["prompt_len"]
        self.steps = self.meta["steps"]
        self.batch = self.meta["batch"]
        self._row = {int(p): i for i, p in enumerate(self.pos)}
        self._samp = {int(p): i for i, p in enumerate(self.samp_pos)}

    def regenerate_tokens(self):
        """The token matrix from the seeds: the workload's prompt, then the forced tokens."""
        s = self.shape
        prompt = synth.make_prompt(s.vocab, self.n0, batch=self.batch, seed=self.workload.prompt_seed)
        forced = synth.make_prompt(s.vocab, self.steps, batch=self.batch, seed=self.meta["forced_seed"])
        return np.concatenate([prompt, forced], axis=1).astype(np.int32)

    @property
    def prompt(self):
        return self.tokens[:, :self.n0]

    def forced(self, i):
        """Input tokens of decode step i (one per sequence)."""
        return self.tokens[:, self.n0 + i]


class Tracker:
    """Running parity record of one GPU run against a fixture."""

    def __init__(self, fx, what, tol=TOL):
        self.fx, self.what, self.tol = fx, what, tol
        self.err = 0.0
        self.n_pos = 0
        self.n_tok = 0
        self.n_samp = 0

    def check(self, p, logits, token=None, seq=0):
        """GPU logits (and greedy token) of sequence seq after reading position p."""
        fx = self.fx
        lg = np.asarray(logits, dtype=np.float64)
        r = fx._row[p]
        ti, tv = fx.top_idx[seq, r], fx.top_val[seq, r].astype(np.float64)
        e = float(np.max(np.abs(lg[ti] - tv)))
        if p in fx._samp:
            q = fx._samp[p]
            e = max(e, float(np.max(np.abs(lg[fx.samp_idx] - fx.samp_val[seq, q]))))
            self.n_samp += 1
        assert e <= self.tol, f"{self.what}: sequence {seq} position {p}: max |gpu - oracle| = {e}"
        self.err = max(self.err, e)
        g = int(np.argmax(lg))
        if token is not None:
            assert int(token) == g, f"{self.what}: returned token {token} is not the argmax {g} of its logits"
        if tv[0] - tv[1] > MARGIN:
            assert g == int(ti[0]), f"{self.what}: sequence {seq} position {p}: greedy {g} vs oracle {ti[0]}"
            self.n_tok += 1
        self.n_pos += 1

    def report(self):
        print(f"{self.what}: {self.n_pos} positions ({self.n_samp} with 1024 sampled logits), "
              f"max |gpu - oracle| = {self.err:.3e} (bound {self.tol}); "
              f"greedy token equal at all {self.n_tok} positions with top-2 margin > {MARGIN}", flush=True)
        return self.err


def kv_excess(g, r):
    """Per leading index: the largest |g - r| beyond one fp16 spacing, relative to r's rms."""
    g64 = g.astype(np.float64).reshape(g.shape[0], -1)
    r64 = r.astype(np.float64).reshape(r.shape[0], -1)
    spacing = np.abs(np.spacing(np.maximum(np.abs(g64), np.abs(r64)).astype(np.float16))).astype(np.float64)
    rms = np.sqrt(np.mean(r64 * r64, axis=1, keepdims=True))
    return ((np.abs(g64 - r64) - spacing) / rms).max(axis=1)
