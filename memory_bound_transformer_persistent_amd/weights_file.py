"""Writer for the DECW weight file that dec_init ingests (layout in include/dec.h).

Header (72 bytes): "DECW", version 1, tensor count, reserved, the model
description (10 int32, rms_eps, rope_base, flags, 4 pad bytes); then one
40-byte entry per tensor (index, dtype=1 fp16, ndim, reserved, dim0, dim1,
offset, nbytes); then each tensor's row-major fp16 payload at a 256-byte
aligned offset.  Tensors are in the canonical order of the C ABI.
"""
import struct

import numpy as np

MAGIC = b"DECW"
VERSION = 1
HDR = 72
ENTRY = 40
ALIGN = 256


def _desc_bytes(desc):
    return struct.pack("<10i2fI4x", desc.n_layers, desc.d_model, desc.n_heads, desc.n_kv_heads,
                       desc.head_dim, desc.d_ffn, desc.vocab, desc.lm_vocab, desc.max_ctx, desc.batch,
                       desc.rms_eps, desc.rope_base, desc.flags)


def write(path, desc, tensors):
    """Write `tensors` (fp16 arrays, canonical order) and `desc` to `path`."""
    n = len(tensors)
    entries = []
    off = HDR + ENTRY * n
    off = (off + ALIGN - 1) // ALIGN * ALIGN
    for i, t in enumerate(tensors):
        t = np.asarray(t)
        if t.dtype != np.float16:
            raise TypeError(f"tensor {i} is {t.dtype}, expected float16")
        if t.ndim == 1:
            ndim, d0, d1 = 1, t.shape[0], 1
        elif t.ndim == 2:
            ndim, d0, d1 = 2, t.shape[0], t.shape[1]
        else:
            raise ValueError(f"tensor {i} has {t.ndim} dimensions")
        entries.append((i, 1, ndim, 0, d0, d1, off, t.nbytes))
        off = (off + t.nbytes + ALIGN - 1) // ALIGN * ALIGN
    with open(path, "wb") as f:
        f.write(MAGIC + struct.pack("<3I", VERSION, n, 0) + _desc_bytes(desc))
        for e in entries:
            f.write(struct.pack("<6IQQ", *e))
        for (i, _, _, _, _, _, o, nb), t in zip(entries, tensors):
            f.seek(o)
            f.write(np.ascontiguousarray(t).tobytes())
        f.truncate(entries[-1][6] + entries[-1][7] if entries else f.tell())
    return path
