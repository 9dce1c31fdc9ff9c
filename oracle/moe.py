"""Mixture-of-experts decoder for the CPU reference.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import, call or run anything in this package.  The product path never
touches it, and this module imports nothing from the product.

What it computes
----------------
The pages' next milestone is large mixture-of-experts models at batch 1,
whose speed is set by the *active* parameters read per token, with the
expert weights in FP8 or FP4 (hakusoku.com/story/7519, section
Hackerたちの意見: GPT-OSS-120B with 5.1B active parameters in FP8, DeepSeek V4
Flash in FP4/FP8; studioglobal.ai article, section 今後のマイルストーンと課題).
The pages fix no router or expert detail; the readings taken here:
  * every layer's MLP is replaced by E SwiGLU experts of width F (the dense
    SwiGLU MLP of the reference decoder, one per expert);
  * the router is a bias-free fp16 linear map [E, d] of the same normed
    vector the MLP reads (RMSNorm with g_ffn);
  * the k experts with the largest router logits are taken (the lower
    expert index first on equal logits), and their weights are the softmax
    of those k logits;
  * the layer adds sum_s w_s * expert_{e_s}(xn) to the residual stream;
  * expert matrices are FP8 E4M3 codes (the OCP 8-bit floating-point
    format: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, exponent
    field 0 subnormal, S.1111.111 NaN, no infinities) with one float32 scale
    per output row: W[r, c] = value(code[r, c]) * scale[r];
  * or, with the MXFP4 format, OCP microscaling blocks: FP4 E2M1 codes (1
    sign, 2 exponent bits with bias 1, 1 mantissa bit, exponent field 0
    subnormal) two to a byte, element 2i in the low nibble, and one E8M0
    scale (2^(s - 127), 0xFF NaN) per 32 consecutive elements of a row;
  * no shared expert, no expert bias, no capacity limit (one token).
Attention, norms, rotary embedding, KV cache and LM head are those of the
dense reference decoder (oracle.decoder).  Arithmetic is float64.
"""
import numpy as np

from .decoder import f64, rmsnorm, rope, silu, softmax, attend, greedy, f16_round

MOE_LAYER_TENSORS = ("g_attn", "Wq", "Wk", "Wv", "Wo", "g_ffn", "Wr", "Wg8", "sg", "Wu8", "su", "Wd8", "sd")


# ----------------------------------------------------------------------------
# FP8 E4M3
# ----------------------------------------------------------------------------

def e4m3_value(code):
    """The value of one E4M3 code (an int 0..255) as a Python float."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# every code's value, evaluated once code by code
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """Values (float64) of an array of E4M3 codes (uint8)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequant(codes, scales):
    """W[r, c] = value(code[r, c]) * scale[r], float64."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# ----------------------------------------------------------------------------
# MXFP4: E2M1 elements, E8M0 block scales
# ----------------------------------------------------------------------------

MX_BLOCK = 32


def e2m1_value(nibble):
    """The value of one E2M1 code (an int 0..15)."""
    n = int(nibble)
    sign = -1.0 if n & 8 else 1.0
    e = (n >> 1) & 3
    m = n & 1
    if e == 0:
        return sign * 0.5 * m
    return sign * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


def e8m0_value(byte):
    """The value of one E8M0 scale (an int 0..255): 2^(byte - 127), 0xFF NaN."""
    b = int(byte)
    return float("nan") if b == 0xFF else 2.0 ** (b - 127)


E2M1_TABLE = np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def mx_dequant(codes, scales):
    """W [R, K] (float64) from packed codes [R, K/2] (element 2i in the low
    nibble of byte i) and E8M0 scales [R, K/32]."""
    c = np.asarray(codes, dtype=np.uint8)
    vals = np.empty((c.shape[0], 2 * c.shape[1]))
    vals[:, 0::2] = E2M1_TABLE[c & 0x0F]
    vals[:, 1::2] = E2M1_TABLE[c >> 4]
    sc = E8M0_TABLE[np.asarray(scales, dtype=np.uint8)]
    return vals * np.repeat(sc, MX_BLOCK, axis=1)


# ----------------------------------------------------------------------------
# router and experts
# ----------------------------------------------------------------------------

def route(logits, k):
    """Top-k experts of one token.

    Returns (sel [k] expert indices, largest logit first, lower index first
    among equal logits; weights [k] = softmax of the selected logits;
    margin = k-th largest logit minus the (k+1)-th, inf when k == E).
    """
    r = np.asarray(logits, dtype=np.float64)
    E = r.shape[0]
    order = sorted(range(E), key=lambda e: (-r[e], e))
    sel = np.array(order[:k], dtype=np.int64)
    margin = float(r[order[k - 1]] - r[order[k]]) if k < E else float("inf")
    return sel, softmax(r[sel]), margin


class MoEWeights:
    """Named view of the canonical MoE tensor list (see synth.gen)."""

    def __init__(self, shape, tensors):
        n = 1 + len(MOE_LAYER_TENSORS) * shape.n_layers + 2
        if len(tensors) != n:
            raise ValueError(f"expected {n} tensors, got {len(tensors)}")
        self.shape = shape
        self.E = tensors[0]
        self.layers = []
        for l in range(shape.n_layers):
            blk = tensors[1 + l * len(MOE_LAYER_TENSORS): 1 + (l + 1) * len(MOE_LAYER_TENSORS)]
            self.layers.append(dict(zip(MOE_LAYER_TENSORS, blk)))
        self.g_final = tensors[-2]
        self.W_lm = tensors[-1]

    def expert(self, l, e):
        """Expert e of layer l as float64 (Wg [F, d], Wu [F, d], Wd [d, F])."""
        lw = self.layers[l]
        F, d = self.shape.d_ffn, self.shape.d_model
        deq = mx_dequant if getattr(self.shape, "mxfp4", False) else dequant
        g = deq(lw["Wg8"][e * F:(e + 1) * F], lw["sg"][e * F:(e + 1) * F])
        u = deq(lw["Wu8"][e * F:(e + 1) * F], lw["su"][e * F:(e + 1) * F])
        dn = deq(lw["Wd8"][e * d:(e + 1) * d], lw["sd"][e * d:(e + 1) * d])
        return g, u, dn


def expert_ffn(Wg, Wu, Wd, xn):
    """One SwiGLU expert: Wd (silu(Wg xn) * (Wu xn))."""
    return Wd @ (silu(Wg @ xn) * (Wu @ xn))


def moe_ffn(w, l, xn, k, force=None):
    """The MoE MLP of layer l on one normed vector xn.

    Returns (output [d], sel, weights, margin, router logits).  `force`, if
    given, is the expert list to use instead of the router's choice (the
    weights are still the softmax of those experts' logits).
    """
    lw = w.layers[l]
    r = f64(lw["Wr"]) @ xn
    sel, wts, margin = route(r, k)
    if force is not None:
        sel = np.asarray(force, dtype=np.int64)
        wts = softmax(r[sel])
    out = np.zeros(w.shape.d_model)
    for s in range(k):
        out = out + wts[s] * expert_ffn(*w.expert(l, int(sel[s])), xn)
    return out, sel, wts, margin, r


# ----------------------------------------------------------------------------
# incremental decoder
# ----------------------------------------------------------------------------

class OracleMoEDecoder:
    """Token-at-a-time MoE decoder with an fp16 KV cache, batch 1.

    After each step: last_routes [L, k] (the experts used), last_weights
    [L, k], last_margins [L] and last_natural [L, k] (the router's own choice,
    which differs from last_routes only where routes were forced).
    """

    def __init__(self, shape, tensors):
        self.s = shape
        self.w = MoEWeights(shape, tensors)
        L, H, hd, C = shape.n_layers, shape.n_heads, shape.head_dim, shape.max_ctx
        self.Kc = np.zeros((L, H, C, hd), dtype=np.float16)
        self.Vc = np.zeros((L, H, C, hd), dtype=np.float16)
        self.pos = 0

    def step(self, tok, force_routes=None):
        """Run token `tok` at the current position; return float64 logits.

        force_routes: optional [L] list whose entry l (None or k experts)
        replaces layer l's choice.
        """
        s, w = self.s, self.w
        p = self.pos
        if p >= s.max_ctx:
            raise ValueError("context full")
        if not 0 <= int(tok) < s.vocab:
            raise ValueError("token out of range")
        H, hd, k = s.n_heads, s.head_dim, s.top_k
        x = f64(w.E[int(tok)])
        routes, wts, margins, natural = [], [], [], []
        for l, lw in enumerate(w.layers):
            xn = rmsnorm(x, lw["g_attn"], s.rms_eps)
            q = (f64(lw["Wq"]) @ xn).reshape(H, hd)
            kk = (f64(lw["Wk"]) @ xn).reshape(H, hd)
            v = (f64(lw["Wv"]) @ xn).reshape(H, hd)
            q = rope(q, p, s.rope_base)
            kk = rope(kk, p, s.rope_base)
            self.Kc[l, :, p, :] = kk.astype(np.float16)
            self.Vc[l, :, p, :] = v.astype(np.float16)
            o = np.empty((H, hd))
            for h in range(H):
                o[h], _ = attend(q[h], f64(self.Kc[l, h, :p + 1]), f64(self.Vc[l, h, :p + 1]))
            x = x + f64(lw["Wo"]) @ o.reshape(H * hd)
            xn = rmsnorm(x, lw["g_ffn"], s.rms_eps)
            force = None if force_routes is None else force_routes[l]
            y, sel, ws, margin, r = moe_ffn(w, l, xn, k, force)
            x = x + y
            routes.append(sel)
            wts.append(ws)
            margins.append(margin)
            natural.append(route(r, k)[0])
        self.last_routes = np.array(routes)
        self.last_weights = np.array(wts)
        self.last_margins = np.array(margins)
        self.last_natural = np.array(natural)
        self.pos = p + 1
        return f64(w.W_lm) @ rmsnorm(x, w.g_final, s.rms_eps)


# ----------------------------------------------------------------------------
# whole-prompt matrix form
# ----------------------------------------------------------------------------

def prefill_matrix_moe(shape, tensors, tokens, force_routes=None, progress=None):
    """All prompt positions at once (explicit causal mask, experts applied
    to the rows routed to them).

    Returns (logits [n, lm_vocab], K16 [L, H, n, hd], V16 [L, H, n, hd],
    routes [n, L, k], margins [n, L]): the router's own choice at every
    position and layer and its gap between the k-th and (k+1)-th logit.
    force_routes [n, L, k], if given, are the experts used instead (the
    returned routes stay the router's own choice, so the two can be
    compared); progress(l), if given, is called after each layer.
    """
    s = shape
    w = MoEWeights(shape, tensors)
    H, hd, k = s.n_heads, s.head_dim, s.top_k
    toks = np.asarray(tokens, dtype=np.int64)
    n = toks.shape[0]
    X = f64(w.E[toks])
    allowed = np.tril(np.ones((n, n), dtype=bool))
    Ks, Vs = [], []
    routes = np.zeros((n, s.n_layers, k), dtype=np.int64)
    margins = np.zeros((n, s.n_layers))
    for l, lw in enumerate(w.layers):
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
            S = (Q[:, h, :] @ K16[:, h, :].T) / np.sqrt(np.float64(hd))
            S = np.where(allowed, S, -np.inf)
            O[:, h, :] = softmax(S) @ V16[:, h, :]
        X = X + O.reshape(n, H * hd) @ f64(lw["Wo"]).T
        Xn = rmsnorm(X, lw["g_ffn"], s.rms_eps)
        R = Xn @ f64(lw["Wr"]).T                              # [n, E]
        wts = np.zeros((n, s.n_experts))                       # routing weight of (row, expert)
        for i in range(n):
            sel, ws, margins[i, l] = route(R[i], k)
            routes[i, l] = sel
            if force_routes is not None:
                sel = np.asarray(force_routes[i][l], dtype=np.int64)
                ws = softmax(R[i, sel])
            wts[i, sel] = ws
        Y = np.zeros_like(X)
        for e in range(s.n_experts):
            rows = np.nonzero(wts[:, e])[0]
            if rows.size == 0:
                continue
            Wg, Wu, Wd = w.expert(l, e)
            Hm = silu(Xn[rows] @ Wg.T) * (Xn[rows] @ Wu.T)
            Y[rows] += wts[rows, e][:, None] * (Hm @ Wd.T)
        X = X + Y
        Ks.append(K16.transpose(1, 0, 2))
        Vs.append(V16.transpose(1, 0, 2))
        if progress is not None:
            progress(l)
    logits = rmsnorm(X, w.g_final, s.rms_eps) @ f64(w.W_lm).T
    return logits, np.stack(Ks).astype(np.float16), np.stack(Vs).astype(np.float16), routes, margins


def greedy_decode_moe(shape, tensors, prompt, n_steps):
    """Prefill `prompt` (matrix form), then n_steps greedy steps.

    Returns (fed tokens [n_steps], logits [n_steps, lm_vocab], prefill
    logits [n_prompt, lm_vocab], routes [n_prompt + n_steps, L, k],
    margins [n_prompt + n_steps, L]).
    """
    prompt = np.asarray(prompt, dtype=np.int64)
    lg, K16, V16, routes, margins = prefill_matrix_moe(shape, tensors, prompt)
    dec = OracleMoEDecoder(shape, tensors)
    n = len(prompt)
    dec.Kc[:, :, :n] = K16
    dec.Vc[:, :, :n] = V16
    dec.pos = n
    tok = greedy(lg[-1])
    fed, outs, rs, ms = [], [], [routes], [margins]
    for _ in range(n_steps):
        fed.append(tok)
        out = dec.step(tok)
        outs.append(out)
        rs.append(dec.last_routes[None])
        ms.append(dec.last_margins[None])
        tok = greedy(out)
    return (np.array(fed, dtype=np.int32), np.array(outs), lg, np.concatenate(rs), np.concatenate(ms))
