"""Bandwidth roofline for batch-1 decode.

The pages bound single-request decode as
    tokens/s <= effective bandwidth / (beta * active weight bytes + KV-cache bytes)
(hakusoku.com/story/7519, section GPU推論の速度制限要因：メモリ帯域幅).  beta is
not defined there; its worked example (about 30.7 TB/s and 33.6 TB/s, a 2B
fp16 model, 7,700 to 8,400 tokens/s) reproduces with beta = 1 and no KV term,
so beta = 1 here.  The launch-overhead model (4.5 us x 10 kernels x 25 layers)
is from the same page, section 標準推論スタックのボトルネックとKogの工夫.
"""
from dataclasses import dataclass

MI355X_HBM_PEAK = 8.0e12   # bytes/s, published HBM3E peak of one MI355X
MI355X_FP16_PEAK = 2.5e15  # flop/s, published dense fp16 matrix peak of one MI355X


def bound_tokens_per_s(bw_bytes_per_s, weight_bytes, kv_bytes=0.0, beta=1.0):
    return bw_bytes_per_s / (beta * weight_bytes + kv_bytes)


def launch_overhead(launch_us, kernels_per_layer, layers):
    """(microseconds of launch overhead per token, the tokens/s cap it implies)."""
    us = launch_us * kernels_per_layer * layers
    return us, 1e6 / us


@dataclass(frozen=True)
class StepBytes:
    weights: int      # weight bytes streamed once per step (read)
    kv_read: int      # KV-cache bytes read by attention
    kv_write: int     # KV-cache bytes appended
    act: int          # embedding row(s) read

    @property
    def total(self) -> int:
        return self.weights + self.kv_read + self.kv_write + self.act


def layer_weight_bytes(shape) -> int:
    """Weight bytes one token reads in one layer.  A mixture of experts reads
    its fp16 router and only the top_k chosen experts: one byte per E4M3 code
    and a 4-byte scale per row (page 標準GPUによるリアルタイムLLM推論, section
    Hackerたちの意見: batch-1 speed follows the active parameters)."""
    d, q, f = shape.d_model, shape.n_heads * shape.head_dim, shape.d_ffn
    if getattr(shape, "n_experts", 0):
        k = shape.top_k
        fp16 = 3 * q * d + d * q + shape.n_experts * d
        if getattr(shape, "mxfp4", False):
            # MXFP4: half a byte per weight and a 1-byte scale per 32 weights
            return 2 * (fp16 + 2 * d) + k * (3 * f * d) // 2 + k * (3 * f * d) // 32
        return 2 * (fp16 + 2 * d) + k * (3 * f * d) + 4 * k * (2 * f + d)
    mats = 3 * q * d + d * q + 2 * f * d + d * f
    return 2 * (mats + 2 * d)            # fp16 matrices + the two norm gains


def weight_bytes(shape) -> int:
    """Layer weights + norms + final norm + the full LM head (fp16)."""
    return shape.n_layers * layer_weight_bytes(shape) + 2 * shape.d_model + \
        2 * shape.lm_vocab * shape.d_model


def step_bytes(shape, pos: int, batch: int = 1) -> StepBytes:
    """Algorithmic HBM bytes of one decode step writing position `pos`.

    Attention reads pos+1 cached positions (the new one included) of K and V
    for every layer and head; each sequence of the batch has its own cache.
    Weights are read once per step whatever the batch.
    """
    kv_row = 2 * shape.n_layers * shape.n_heads * shape.head_dim * 2   # K and V, fp16
    return StepBytes(weights=weight_bytes(shape),
                     kv_read=batch * kv_row * (pos + 1),
                     kv_write=batch * kv_row,
                     act=batch * 2 * shape.d_model)


def mean_step_bytes(shape, first_pos: int, n_steps: int, batch: int = 1) -> float:
    tot = 0
    for i in range(n_steps):
        tot += step_bytes(shape, first_pos + i, batch).total
    return tot / n_steps


def roofline_tokens_per_s(shape, first_pos: int, n_steps: int, batch: int = 1,
                          bw=MI355X_HBM_PEAK) -> float:
    """Per-request tokens/s bound over a run of n_steps starting at first_pos."""
    return bw / mean_step_bytes(shape, first_pos, n_steps, batch)


def prefill_flops(shape, n: int) -> int:
    """Algorithmic flops of a whole-prompt prefill of n positions (one sequence).

    Every position goes through every layer's matrices (2 flops per weight),
    causal attention scores and weighted sums for query i over keys 0..i
    (2 hd flops each, twice), and the LM head for the last position only.
    """
    d, q, f = shape.d_model, shape.n_heads * shape.head_dim, shape.d_ffn
    mats = 3 * q * d + d * q + 2 * f * d + d * f
    attn = 2 * shape.n_heads * shape.head_dim * n * (n + 1)     # sum over i of 2 * 2 hd (i + 1)
    return shape.n_layers * (2 * n * mats + attn) + 2 * shape.lm_vocab * d
