"""Seeded weight and prompt generators.

Every matrix is drawn as float32 standard normals times 0.02 and rounded once
to fp16 (round to nearest even); norm gains are 1.0.  Each tensor has its own
generator, seeded with (seed, tensor index), so tensors can be drawn one at a
time and a lane's tensors are row/column slices of the full model's.

Canonical tensor order (also the order of the C ABI's host tensor list):
  E [vocab, d]
  per layer: g_attn [d], Wq [H*hd, d], Wk [H*hd, d], Wv [H*hd, d],
             Wo [d, H*hd], g_ffn [d], Wg [F, d], Wu [F, d], Wd [d, F]
  g_final [d], W_lm [lm_vocab, d]
All matrices are stored [out, in], row-major.

Mixture-of-experts shapes (n_experts E > 0, expert width F = d_ffn) replace
Wg, Wu, Wd by a router and E experts per layer:
  per layer: g_attn, Wq, Wk, Wv, Wo, g_ffn, Wr [E, d] (fp16),
             Wg8 [E*F, d] (uint8 FP8 E4M3 codes), sg [E*F] (float32 row scales),
             Wu8 [E*F, d], su [E*F], Wd8 [E*d, F], sd [E*d]
Expert e owns rows e*F .. e*F+F-1 of Wg8/Wu8 and rows e*d .. e*d+d-1 of Wd8.
The expert weights are drawn as codes, never as values: sign and mantissa
bits uniform, the exponent field from a fixed 16-entry table that roughly
follows the magnitudes of a standard normal (1/16 of the codes subnormal,
none with the all-ones exponent, so no NaN and no value above 3.75), and
every row's scale is 0.01 * (0.75 + 0.5 u), u uniform.  The router is drawn
like the other fp16 matrices.

MXFP4 experts (shape.mxfp4) fill the same slots with OCP microscaling
blocks: Wg8 / Wu8 [E*F, d/2] and Wd8 [E*d, F/2] hold two E2M1 codes per
byte (uniform random bytes), sg / su [E*F, d/32] and sd [E*d, F/32] one E8M0
scale per 32 weights of a row (118, 119 or 120 uniformly, i.e. 2^-9 .. 2^-7).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .shapes import ModelShape, Workload, DENSE_2B

_THREADS = min(16, os.cpu_count() or 1)

LAYER_TENSORS = ("g_attn", "Wq", "Wk", "Wv", "Wo", "g_ffn", "Wg", "Wu", "Wd")
N_TENSORS_PER_LAYER = len(LAYER_TENSORS)
MOE_LAYER_TENSORS = ("g_attn", "Wq", "Wk", "Wv", "Wo", "g_ffn", "Wr", "Wg8", "sg", "Wu8", "su", "Wd8", "sd")

# exponent field of a drawn FP8 code, indexed by 4 random bits
_EXP_FIELD = np.array([8, 7, 7, 7, 7, 6, 6, 6, 6, 6, 5, 5, 5, 4, 3, 0], dtype=np.uint8)


def layer_tensors(shape: ModelShape):
    return MOE_LAYER_TENSORS if shape.moe else LAYER_TENSORS


def tensor_names(shape: ModelShape):
    names = ["E"]
    for l in range(shape.n_layers):
        names += [f"{t}.{l}" for t in layer_tensors(shape)]
    names += ["g_final", "W_lm"]
    return names


def tensor_shapes(shape: ModelShape):
    d, q, f, E = shape.d_model, shape.qkv_width, shape.d_ffn, shape.n_experts
    per = {"g_attn": (d,), "Wq": (q, d), "Wk": (q, d), "Wv": (q, d), "Wo": (d, q),
           "g_ffn": (d,), "Wg": (f, d), "Wu": (f, d), "Wd": (d, f),
           "Wr": (E, d), "Wg8": (E * f, d), "sg": (E * f,), "Wu8": (E * f, d), "su": (E * f,),
           "Wd8": (E * d, f), "sd": (E * d,)}
    if getattr(shape, "mxfp4", False):
        per.update({"Wg8": (E * f, d // 2), "sg": (E * f, d // 32), "Wu8": (E * f, d // 2), "su": (E * f, d // 32),
                    "Wd8": (E * d, f // 2), "sd": (E * d, f // 32)})
    shapes = [(shape.vocab, d)]
    for _ in range(shape.n_layers):
        shapes += [per[t] for t in layer_tensors(shape)]
    shapes += [(d,), (shape.lm_vocab, d)]
    return shapes


def _draw_codes(shp, seed, index):
    """FP8 E4M3 codes (uint8): sign and mantissa bits uniform, exponent field from _EXP_FIELD."""
    rng = np.random.default_rng([seed, index])
    u = rng.integers(0, 256, size=shp, dtype=np.uint8)
    e = _EXP_FIELD[rng.integers(0, 16, size=shp, dtype=np.uint8)]
    return (u & np.uint8(0x87)) | (e << np.uint8(3))


def _draw_mx_codes(shp, seed, index):
    """Two E2M1 codes per byte, every byte value equally likely."""
    return np.random.default_rng([seed, index]).integers(0, 256, size=shp, dtype=np.uint8)


def _draw_mx_scales(shp, seed, index):
    """E8M0 block scales 118, 119 or 120."""
    return np.random.default_rng([seed, index]).integers(118, 121, size=shp, dtype=np.uint8)


def _draw_scales(shp, seed, index):
    rng = np.random.default_rng([seed, index])
    return (0.01 * (0.75 + 0.5 * rng.random(shp))).astype(np.float32)


def _draw(shp, seed, index, scale=0.02):
    rng = np.random.default_rng([seed, index])
    a = rng.standard_normal(shp, dtype=np.float32)
    a *= np.float32(scale)
    return a.astype(np.float16)


def make_weights(shape: ModelShape, seed: int = 0, gain_jitter: float = 0.0):
    """List of fp16 arrays in canonical order.

    gain_jitter > 0 draws every gain as 1 + N(0, gain_jitter) (rounded to
    fp16) instead of 1.0, so that a consumer that ignores gains is caught.
    """
    def one(item):
        idx, (name, shp) = item
        if name.startswith("g_"):
            if gain_jitter > 0.0:
                rng = np.random.default_rng([seed, idx, 7])
                return (1.0 + gain_jitter * rng.standard_normal(shp)).astype(np.float16)
            return np.ones(shp, dtype=np.float16)
        base = name.split(".")[0]
        mx = getattr(shape, "mxfp4", False)
        if base in ("Wg8", "Wu8", "Wd8"):
            return _draw_mx_codes(shp, seed, idx) if mx else _draw_codes(shp, seed, idx)
        if base in ("sg", "su", "sd"):
            return _draw_mx_scales(shp, seed, idx) if mx else _draw_scales(shp, seed, idx)
        return _draw(shp, seed, idx)

    items = list(enumerate(zip(tensor_names(shape), tensor_shapes(shape))))
    # every tensor has its own generator, so drawing them concurrently
    # yields exactly the same arrays as drawing them in order
    with ThreadPoolExecutor(_THREADS) as ex:
        return list(ex.map(one, items))


def lane_slice_weights(lane_shape: ModelShape, full_shape: ModelShape = DENSE_2B, seed: int = 0):
    """Lane 0's tensors: the first heads, FFN columns and LM rows of the full model.

    Heads 0..n_heads-1 are Q/K/V rows [0, n_heads*hd) and Wo columns
    [0, n_heads*hd); FFN columns [0, d_ffn) are rows of Wg/Wu and columns of
    Wd; the LM head keeps rows [0, lm_vocab); the embedding is whole.
    """
    q, f = lane_shape.qkv_width, lane_shape.d_ffn
    names = tensor_names(full_shape)
    shapes = tensor_shapes(full_shape)

    def one(item):
        idx, (name, shp) = item
        base = name.split(".")[0]
        if base.startswith("g_"):
            return np.ones(shp, dtype=np.float16)
        full = _draw(shp, seed, idx)
        if base == "E":
            return full
        if base == "W_lm":
            # rows are drawn row-major, so the first lm_vocab rows of the full
            # table are exactly the lane's shard
            return np.ascontiguousarray(full[:lane_shape.lm_vocab])
        if base in ("Wq", "Wk", "Wv"):
            return np.ascontiguousarray(full[:q])
        if base == "Wo":
            return np.ascontiguousarray(full[:, :q])
        if base in ("Wg", "Wu"):
            return np.ascontiguousarray(full[:f])
        if base == "Wd":
            return np.ascontiguousarray(full[:, :f])
        raise AssertionError(name)

    with ThreadPoolExecutor(_THREADS) as ex:
        out = list(ex.map(one, list(enumerate(zip(names, shapes)))))
    assert len(out) == len(names)
    return out


def lane_from_full(lane_shape: ModelShape, full_tensors, full_shape: ModelShape = DENSE_2B):
    """Lane 0's tensors sliced from an already drawn full model (the same
    arrays lane_slice_weights draws, without drawing the full model again)."""
    q, f = lane_shape.qkv_width, lane_shape.d_ffn
    out = []
    for name, t in zip(tensor_names(full_shape), full_tensors):
        base = name.split(".")[0]
        if base.startswith("g_"):
            out.append(np.ones(t.shape, dtype=np.float16))
        elif base == "E":
            out.append(t)
        elif base == "W_lm":
            out.append(np.ascontiguousarray(t[:lane_shape.lm_vocab]))
        elif base in ("Wq", "Wk", "Wv", "Wg", "Wu"):
            out.append(np.ascontiguousarray(t[:q if base in ("Wq", "Wk", "Wv") else f]))
        elif base in ("Wo", "Wd"):
            out.append(np.ascontiguousarray(t[:, :q if base == "Wo" else f]))
        else:
            raise AssertionError(name)
    return out


def make_prompt(vocab: int, n: int, batch: int = 1, seed: int = 1):
    """Uniform random token ids, int32, shape [batch, n]."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=(batch, n)).astype(np.int32)


def workload_weights(w: Workload):
    if w.lane:
        return lane_slice_weights(w.shape, DENSE_2B, seed=w.weight_seed)
    return make_weights(w.shape, seed=w.weight_seed)
