"""ctypes binding of libdecmono.so (include/dec.h).

Argument marshalling only: every step of decode runs in the HIP library.
Loading fails loudly (DecLibraryMissing) when the library has not been built;
there is no fallback path.
"""
import ctypes
import os
import re

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libdecmono.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dec.h")

DEC_OK = 0
DEC_ERR_INVALID_ARG = -1
DEC_ERR_BAD_DESC = -2
DEC_ERR_WEIGHTS = -3
DEC_ERR_NO_DEVICE = -4
DEC_ERR_OOM = -5
DEC_ERR_CONTEXT_FULL = -6
DEC_ERR_STATE = -7
DEC_ERR_TOKEN_RANGE = -8
DEC_ERR_DEVICE = -9
DEC_ERR_TIMEOUT = -10
DEC_ERR_UNSUPPORTED = -11
DEC_DEBUG_MULTILAUNCH = 0x1
DEC_DEBUG_TRACE = 0x2
DEC_DEBUG_FENCED = 0x4
DEC_DEBUG_STRESS = 0x8
DEC_FLAG_BATCHED_PREFILL = 0x2
DEC_FLAG_MATRIX_PREFILL = 0x4
DEC_FLAG_EXPERTS_MXFP4 = 0x8

ERR_NAMES = {v: k for k, v in globals().items() if k.startswith("DEC_ERR_")}


class DecLibraryMissing(RuntimeError):
    pass


class DecError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("lm_vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]

    @classmethod
    def from_shape(cls, s, batch=1, **override):
        """From any object with the model-shape attributes."""
        kw = dict(n_layers=s.n_layers, d_model=s.d_model, n_heads=s.n_heads, n_kv_heads=s.n_heads,
                  head_dim=s.head_dim, d_ffn=s.d_ffn, vocab=s.vocab, lm_vocab=s.lm_vocab,
                  max_ctx=s.max_ctx, batch=batch, rms_eps=s.rms_eps, rope_base=s.rope_base,
                  flags=DEC_FLAG_EXPERTS_MXFP4 if getattr(s, "mxfp4", False) else 0,
                  n_experts=getattr(s, "n_experts", 0), top_k=getattr(s, "top_k", 0))
        kw.update(override)
        if getattr(s, "mxfp4", False):
            # the experts' tensors have MXFP4 shapes whatever other flags are asked for
            kw["flags"] |= DEC_FLAG_EXPERTS_MXFP4
        return cls(**kw)


class WeightsSrc(ctypes.Structure):
    _fields_ = [("path", ctypes.c_char_p), ("host_tensors", ctypes.POINTER(ctypes.POINTER(ctypes.c_uint16))),
                ("n_tensors", ctypes.c_int32)]


class InitOpts(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("grid", ctypes.c_int32), ("stream", ctypes.c_void_p),
                ("arena", ctypes.c_void_p), ("arena_bytes", ctypes.c_size_t), ("debug_flags", ctypes.c_uint32),
                ("watchdog_us", ctypes.c_int32), ("serve_idle_us", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


_lib = None

_P = ctypes.POINTER
_i32p = _P(ctypes.c_int32)
_f32p = _P(ctypes.c_float)
_u16p = _P(ctypes.c_uint16)

SIGNATURES = {
    "dec_abi_version": (ctypes.c_int32, []),
    "dec_arena_bytes": (ctypes.c_int, [_P(ModelDesc), ctypes.c_int32, _P(ctypes.c_size_t)]),
    "dec_check_desc": (ctypes.c_int, [_P(ModelDesc)]),
    "dec_weights_file_check": (ctypes.c_int, [ctypes.c_char_p, _P(ModelDesc)]),
    "dec_init": (ctypes.c_int, [_P(ModelDesc), _P(WeightsSrc), _P(InitOpts), _P(ctypes.c_void_p)]),
    "dec_init_noalloc": (ctypes.c_int, [_P(ModelDesc), _P(WeightsSrc), _P(InitOpts), _P(ctypes.c_void_p)]),
    "dec_prefill": (ctypes.c_int, [ctypes.c_void_p, _i32p, ctypes.c_int32, _i32p, _f32p]),
    "dec_step": (ctypes.c_int, [ctypes.c_void_p, _i32p, _i32p, _f32p]),
    "dec_generate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, _i32p]),
    "dec_sync": (ctypes.c_int, [ctypes.c_void_p]),
    "dec_reset": (ctypes.c_int, [ctypes.c_void_p]),
    "dec_position": (ctypes.c_int32, [ctypes.c_void_p]),
    "dec_read_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _u16p, _u16p]),
    "dec_read_routes": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _i32p]),
    "dec_free": (None, [ctypes.c_void_p]),
    "dec_last_error": (ctypes.c_char_p, [ctypes.c_void_p]),
    "dec_read_trace": (ctypes.c_int, [ctypes.c_void_p, _P(ctypes.c_uint64), _i32p, _i32p, _P(ctypes.c_double)]),
    "dec_stream_ceiling": (ctypes.c_int, [ctypes.c_int32, ctypes.c_uint64, ctypes.c_int32, _P(ctypes.c_double)]),
    "dec_packed_bytes": (ctypes.c_int, [_P(ModelDesc), _P(ctypes.c_size_t)]),
    "dec_pack": (ctypes.c_int, [_P(ModelDesc), _P(_u16p), ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]),
}


def header_functions(path=HEADER):
    """Names of the functions include/dec.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dec_[a-z_]+)\s*\(", text)))


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise DecLibraryMissing(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error(handle=None):
    msg = load().dec_last_error(handle)
    return msg.decode() if msg else ""


def _check(rc, handle=None):
    if rc != DEC_OK:
        raise DecError(rc, last_error(handle))


def _tensor_ptrs(tensors):
    """float16 tensors; a mixture of experts' expert codes are uint8 and
    their row scales float32 (the library reads each pointer as its tensor's
    own element type)."""
    arrs = [np.ascontiguousarray(t) for t in tensors]
    for a in arrs:
        if a.dtype not in (np.float16, np.uint8, np.float32):
            raise TypeError("weights must be float16 arrays (expert codes uint8, their scales float32)")
    ptrs = (_u16p * len(arrs))(*[a.ctypes.data_as(_u16p) for a in arrs])
    return arrs, ptrs


def check_desc(desc):
    return load().dec_check_desc(ctypes.byref(desc))


def arena_bytes(desc, grid=0):
    n = ctypes.c_size_t()
    _check(load().dec_arena_bytes(ctypes.byref(desc), grid, ctypes.byref(n)))
    return n.value


def packed_bytes(desc):
    n = ctypes.c_size_t()
    _check(load().dec_packed_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def pack(desc, tensors):
    """Host packer: the fp16 device image as a uint16 numpy array."""
    arrs, ptrs = _tensor_ptrs(tensors)
    out = np.zeros(packed_bytes(desc) // 2, dtype=np.uint16)
    _check(load().dec_pack(ctypes.byref(desc), ptrs, len(arrs), out.ctypes.data, out.nbytes))
    return out


def stream_ceiling(nbytes=1 << 32, reps=5, device=0):
    """Sustained HBM read rate (GB/s) of a plain 16-byte non-temporal stream (dec_stream_ceiling)."""
    g = ctypes.c_double()
    _check(load().dec_stream_ceiling(device, nbytes, reps, ctypes.byref(g)))
    return g.value


def weights_file_check(path):
    d = ModelDesc()
    rc = load().dec_weights_file_check(str(path).encode(), ctypes.byref(d))
    return rc, d


class Decoder:
    """One handle of the decode library (one device, one stream)."""

    def __init__(self, desc, tensors=None, path=None, device=0, stream=None, grid=0,
                 debug_flags=0, watchdog_us=0, arena=None, arena_bytes=0, noalloc=False, serve_idle_us=0):
        """noalloc: dec_init_noalloc (needs arena, arena_bytes and stream; the
        library allocates no device memory for this handle).  serve_idle_us > 0:
        decode server (dec_step posts to one resident launch; sync() ends it)."""
        lib = load()
        self.desc = desc
        src = WeightsSrc()
        keep = None
        if tensors is not None:
            keep, ptrs = _tensor_ptrs(tensors)
            src.host_tensors = ptrs
            src.n_tensors = len(keep)
        if path is not None:
            src.path = str(path).encode()
        opts = InitOpts(device=device, grid=grid, stream=stream, arena=arena, arena_bytes=arena_bytes,
                        debug_flags=debug_flags, watchdog_us=watchdog_us, serve_idle_us=serve_idle_us)
        h = ctypes.c_void_p()
        init = lib.dec_init_noalloc if noalloc else lib.dec_init
        rc = init(ctypes.byref(desc), ctypes.byref(src), ctypes.byref(opts), ctypes.byref(h))
        del keep
        _check(rc)
        self._h = h
        self._lib = lib

    def close(self):
        if getattr(self, "_h", None):
            self._lib.dec_free(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def _rc(self, rc):
        _check(rc, self._h)

    @property
    def position(self):
        return self._lib.dec_position(self._h)

    def prefill(self, tokens, want_logits=False):
        """tokens: [batch, n] (or n tokens at batch 1), sequence-major."""
        t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        if t.size == 0 or t.size % self.desc.batch:
            raise ValueError(f"{t.size} prompt tokens do not split into {self.desc.batch} equal sequences")
        n = t.size // self.desc.batch
        out = np.zeros(self.desc.batch, dtype=np.int32)
        lg = np.zeros(self.desc.batch * self.desc.lm_vocab, dtype=np.float32) if want_logits else None
        self._rc(self._lib.dec_prefill(self._h, t.ctypes.data_as(_i32p), n, out.ctypes.data_as(_i32p),
                                       lg.ctypes.data_as(_f32p) if lg is not None else None))
        return (int(out[0]) if self.desc.batch == 1 else out), lg

    def step(self, force_tok=None, want_tok=True, want_logits=False):
        ft = None
        if force_tok is not None:
            ft = np.ascontiguousarray(np.atleast_1d(force_tok), dtype=np.int32).reshape(-1)
            if ft.size != self.desc.batch:
                raise ValueError(f"force_tok holds {ft.size} tokens; the batch is {self.desc.batch}")
        out = np.zeros(self.desc.batch, dtype=np.int32) if want_tok else None
        lg = np.zeros(self.desc.batch * self.desc.lm_vocab, dtype=np.float32) if want_logits else None
        self._rc(self._lib.dec_step(self._h, ft.ctypes.data_as(_i32p) if ft is not None else None,
                                    out.ctypes.data_as(_i32p) if out is not None else None,
                                    lg.ctypes.data_as(_f32p) if lg is not None else None))
        tok = None if out is None else (int(out[0]) if self.desc.batch == 1 else out)
        return tok, lg

    def generate(self, n_steps):
        out = np.zeros(n_steps * self.desc.batch, dtype=np.int32)
        self._rc(self._lib.dec_generate(self._h, n_steps, out.ctypes.data_as(_i32p)))
        return out

    def sync(self):
        self._rc(self._lib.dec_sync(self._h))

    def reset(self):
        self._rc(self._lib.dec_reset(self._h))

    def read_trace(self):
        """(stamps [grid, stride] uint64, clock Hz) of the most recent launch."""
        g, st, hz = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_double()
        self._rc(self._lib.dec_read_trace(self._h, None, ctypes.byref(g), ctypes.byref(st), ctypes.byref(hz)))
        out = np.zeros((g.value, st.value), dtype=np.uint64)
        self._rc(self._lib.dec_read_trace(self._h, out.ctypes.data_as(_P(ctypes.c_uint64)), None, None, None))
        return out, hz.value

    def read_routes(self, pos0, n_pos):
        """Mixture of experts: the experts chosen at positions [pos0, pos0 + n_pos),
        int32 [n_pos, n_layers, top_k] (-1 where not computed)."""
        out = np.zeros((n_pos, self.desc.n_layers, self.desc.top_k), dtype=np.int32)
        self._rc(self._lib.dec_read_routes(self._h, pos0, n_pos, out.ctypes.data_as(_i32p)))
        return out

    def read_kv(self, layer, n_pos, seq=0):
        H, hd = self.desc.n_heads, self.desc.head_dim
        k = np.zeros((H, n_pos, hd), dtype=np.uint16)
        v = np.zeros((H, n_pos, hd), dtype=np.uint16)
        self._rc(self._lib.dec_read_kv(self._h, layer, seq, n_pos, k.ctypes.data_as(_u16p), v.ctypes.data_as(_u16p)))
        return k.view(np.float16), v.view(np.float16)
