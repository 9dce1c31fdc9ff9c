"""Plain CPU reference decoder.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import, call or run anything in this package.  The product path (the HIP
library and its Python binding) never touches it, and this package imports
nothing from the product.

What it computes
----------------
Batch-1 greedy autoregressive decode of a dense decoder-only transformer
whose weights are stored in fp16.  At batch size 1 every token is a chain of
matrix-vector products over all active weights (hakusoku.com/story/7519,
section GPU推論の速度制限要因：メモリ帯域幅); the ops inside a decode step are
"MatMul, attention, normalization, sampling" (same page, section
Kog Inference Engineの特徴とイノベーション).  Weights are fp16 with no
quantisation, pruning or KV-cache compression (aether-echoes operator view,
section どう出したか; studioglobal.ai article, table under "Laneformer 2B").
Decoding is greedy (studioglobal.ai table: HumanEval+/MBPP+ "greedy").

The pages name no normalisation, position encoding or activation.  The
readings taken here (each is listed with its reason in the design notes):
  * pre-norm RMSNorm before attention and before the MLP, a final RMSNorm,
    residual adds, eps from the model shape;
  * rotary position embedding on q and k, adjacent pairs (2i, 2i+1),
    theta_i = base^(-2i/hd), positions counted from 0 at the first prompt token;
  * multi-head attention, scale 1/sqrt(hd), no biases, causal by construction;
  * SwiGLU MLP: down( silu(gate(x)) * up(x) );
  * untied embedding and LM head, no embedding scale, no logit soft-cap;
  * the KV cache holds fp16 values (round to nearest even on write) and every
    position, including the one just written, is read back from it.

Arithmetic is float64 throughout; the fp16 weights are converted exactly.
"""
import numpy as np


# ----------------------------------------------------------------------------
# element-wise pieces
# ----------------------------------------------------------------------------

def f64(a):
    """Exact float64 copy of an fp16 (or any float) array."""
    return np.asarray(a).astype(np.float64)


def f16_round(a):
    """Round to the nearest fp16 value (ties to even) and return it as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(g)


def rope_angles(pos, head_dim, base):
    """Angles pos * theta_i, theta_i = base^(-2i/hd), i = 0 .. hd/2-1."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / head_dim)
    return np.float64(pos) * theta


def rope(u, pos, base):
    """Rotate each adjacent pair (u[2i], u[2i+1]) of the last axis by pos*theta_i."""
    u = np.asarray(u, dtype=np.float64)
    hd = u.shape[-1]
    ang = rope_angles(pos, hd, base)
    c, s = np.cos(ang), np.sin(ang)
    a = u[..., 0::2]
    b = u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def softmax(s):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q, K, V):
    """One query over positions 0..n-1 of one head.

    q [hd], K [n, hd], V [n, hd] -> (o [hd], weights [n]).
    scores s_j = q.K_j / sqrt(hd); weights = softmax(s); o = sum_j w_j V_j.
    """
    hd = q.shape[-1]
    s = (K @ q) / np.sqrt(np.float64(hd))
    w = softmax(s)
    return w @ V, w


def greedy(logits):
    """First index of the maximum (lowest index wins a tie)."""
    return int(np.argmax(np.asarray(logits)))


def top2_margin(logits):
    """max - second max; decides whether a token comparison is meaningful."""
    v = np.sort(np.asarray(logits, dtype=np.float64))
    return float(v[-1] - v[-2]) if v.size > 1 else float("inf")


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

LAYER_TENSORS = ("g_attn", "Wq", "Wk", "Wv", "Wo", "g_ffn", "Wg", "Wu", "Wd")


class Weights:
    """Named view of the canonical fp16 tensor list.

    Order: E, per layer (g_attn, Wq, Wk, Wv, Wo, g_ffn, Wg, Wu, Wd),
    g_final, W_lm.  Matrices are [out, in].
    """

    def __init__(self, shape, tensors):
        n = 1 + len(LAYER_TENSORS) * shape.n_layers + 2
        if len(tensors) != n:
            raise ValueError(f"expected {n} tensors, got {len(tensors)}")
        self.shape = shape
        self.E = tensors[0]
        self.layers = []
        for l in range(shape.n_layers):
            blk = tensors[1 + l * len(LAYER_TENSORS): 1 + (l + 1) * len(LAYER_TENSORS)]
            self.layers.append(dict(zip(LAYER_TENSORS, blk)))
        self.g_final = tensors[-2]
        self.W_lm = tensors[-1]


def matvec(W, x):
    """W [out, in] (fp16) times x [in] in float64."""
    return f64(W) @ x


# ----------------------------------------------------------------------------
# incremental decoder: one token per call
# ----------------------------------------------------------------------------

class OracleDecoder:
    """Token-at-a-time decoder with an fp16 KV cache, batch 1."""

    def __init__(self, shape, tensors):
        self.s = shape
        self.w = Weights(shape, tensors)
        L, H, hd, C = shape.n_layers, shape.n_heads, shape.head_dim, shape.max_ctx
        self.Kc = np.zeros((L, H, C, hd), dtype=np.float16)
        self.Vc = np.zeros((L, H, C, hd), dtype=np.float16)
        self.pos = 0
        self.last_hidden = None
        self.last_attn_weights = None

    def reset(self):
        self.pos = 0

    def step(self, tok):
        """Run token `tok` at the current position; return float64 logits."""
        s, w = self.s, self.w
        p = self.pos
        if p >= s.max_ctx:
            raise ValueError("context full")
        if not 0 <= int(tok) < s.vocab:
            raise ValueError("token out of range")
        H, hd = s.n_heads, s.head_dim
        x = f64(w.E[int(tok)])
        attn_w = []
        for l, lw in enumerate(w.layers):
            # attention block
            xn = rmsnorm(x, lw["g_attn"], s.rms_eps)
            q = matvec(lw["Wq"], xn).reshape(H, hd)
            k = matvec(lw["Wk"], xn).reshape(H, hd)
            v = matvec(lw["Wv"], xn).reshape(H, hd)
            q = rope(q, p, s.rope_base)
            k = rope(k, p, s.rope_base)
            self.Kc[l, :, p, :] = k.astype(np.float16)
            self.Vc[l, :, p, :] = v.astype(np.float16)
            o = np.empty((H, hd))
            ws = []
            for h in range(H):
                o[h], wh = attend(q[h], f64(self.Kc[l, h, :p + 1]), f64(self.Vc[l, h, :p + 1]))
                ws.append(wh)
            attn_w.append(ws)
            x = x + matvec(lw["Wo"], o.reshape(H * hd))
            # MLP block
            xn = rmsnorm(x, lw["g_ffn"], s.rms_eps)
            a = silu(matvec(lw["Wg"], xn)) * matvec(lw["Wu"], xn)
            x = x + matvec(lw["Wd"], a)
        self.last_hidden = x
        self.last_attn_weights = attn_w
        logits = matvec(w.W_lm, rmsnorm(x, w.g_final, s.rms_eps))
        self.pos = p + 1
        return logits

    def prefill(self, tokens):
        """step() over every prompt token; returns the last position's logits."""
        logits = None
        for t in tokens:
            logits = self.step(int(t))
        return logits

    def load_cache(self, K16, V16, pos):
        """Adopt an externally produced fp16 cache for positions 0..pos-1."""
        n = K16.shape[2]
        self.Kc[:, :, :n] = K16
        self.Vc[:, :, :n] = V16
        self.pos = pos


# ----------------------------------------------------------------------------
# whole-sequence matrix form with an explicit causal mask
# ----------------------------------------------------------------------------

def prefill_matrix(shape, tensors, tokens):
    """All prompt positions at once.

    Returns (logits [n, lm_vocab], K16 [L, H, n, hd], V16 [L, H, n, hd],
    hidden [n, d]).  Position j's keys and values are rounded to fp16 before
    any query reads them, as in the incremental form.  The causal mask is an
    explicit n x n matrix: query i may read key j iff j <= i.
    """
    s = shape
    w = Weights(shape, tensors)
    H, hd = s.n_heads, s.head_dim
    toks = np.asarray(tokens, dtype=np.int64)
    n = toks.shape[0]
    X = f64(w.E[toks])                                   # [n, d]
    allowed = np.tril(np.ones((n, n), dtype=bool))       # [query, key]
    Ks, Vs = [], []
    for lw in w.layers:
        Xn = rmsnorm(X, lw["g_attn"], s.rms_eps)
        Q = (Xn @ f64(lw["Wq"]).T).reshape(n, H, hd)
        K = (Xn @ f64(lw["Wk"]).T).reshape(n, H, hd)
        V = (Xn @ f64(lw["Wv"]).T).reshape(n, H, hd)
        for i in range(n):
            Q[i] = rope(Q[i], i, s.rope_base)
            K[i] = rope(K[i], i, s.rope_base)
        K16 = f16_round(K)
        V16 = f16_round(V)
        O = np.empty((n, H, hd))
        for h in range(H):
            S = (Q[:, h, :] @ K16[:, h, :].T) / np.sqrt(np.float64(hd))   # [n, n]
            S = np.where(allowed, S, -np.inf)
            O[:, h, :] = softmax(S) @ V16[:, h, :]
        X = X + O.reshape(n, H * hd) @ f64(lw["Wo"]).T
        Xn = rmsnorm(X, lw["g_ffn"], s.rms_eps)
        A = silu(Xn @ f64(lw["Wg"]).T) * (Xn @ f64(lw["Wu"]).T)
        X = X + A @ f64(lw["Wd"]).T
        Ks.append(K16.transpose(1, 0, 2))
        Vs.append(V16.transpose(1, 0, 2))
    logits = rmsnorm(X, w.g_final, s.rms_eps) @ f64(w.W_lm).T
    return logits, np.stack(Ks).astype(np.float16), np.stack(Vs).astype(np.float16), X


# ----------------------------------------------------------------------------
# greedy decode drivers
# ----------------------------------------------------------------------------

def greedy_decode(shape, tensors, prompt, n_steps, matrix_prefill=True):
    """Prefill `prompt`, then n_steps greedy steps.

    The prefill's greedy token is the first step's input.  Returns
    (tokens [n_steps] fed to each step, logits [n_steps, lm_vocab],
    prefill logits [lm_vocab], next token after the last step).
    """
    dec = OracleDecoder(shape, tensors)
    prompt = np.asarray(prompt, dtype=np.int64)
    if matrix_prefill and len(prompt) > 1:
        lg, K16, V16, _ = prefill_matrix(shape, tensors, prompt)
        dec.load_cache(K16, V16, len(prompt))
        pre = lg[-1]
    else:
        pre = dec.prefill(prompt)
    tok = greedy(pre)
    fed, outs = [], []
    for _ in range(n_steps):
        fed.append(tok)
        lg = dec.step(tok)
        outs.append(lg)
        tok = greedy(lg)
    return np.array(fed, dtype=np.int32), np.array(outs), pre, tok
