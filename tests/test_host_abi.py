"""The C ABI on the CPU: exports, descriptor rules, packer, DECW reader, no-device path.

No compute calls: these run without a GPU.
"""
import ctypes
import os

import re

import numpy as np
import pytest

import synth
from memory_bound_transformer_persistent_amd import binding as B
from memory_bound_transformer_persistent_amd import weights_file as WF

TINY = synth.shape_for("tiny")


@pytest.fixture(scope="module")
def lib():
    return B.load()


def desc(**kw):
    return B.ModelDesc.from_shape(TINY, **kw)


def test_exports_every_declared_symbol(lib):
    names = B.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    want = int(re.search(r"#define DEC_ABI_VERSION (\d+)", open(B.HEADER).read()).group(1))
    assert lib.dec_abi_version() == want == 2
    assert set(names) == set(B.SIGNATURES)


@pytest.mark.parametrize("field,value,code", [
    ("n_layers", 0, B.DEC_ERR_BAD_DESC),
    ("d_model", 12, B.DEC_ERR_BAD_DESC),
    ("n_kv_heads", 2, B.DEC_ERR_BAD_DESC),
    ("head_dim", 48, B.DEC_ERR_BAD_DESC),
    ("d_ffn", 1001, B.DEC_ERR_BAD_DESC),
    ("lm_vocab", 4097, B.DEC_ERR_BAD_DESC),
    ("lm_vocab", 3, B.DEC_ERR_BAD_DESC),
    ("max_ctx", 0, B.DEC_ERR_BAD_DESC),
    ("rms_eps", 0.0, B.DEC_ERR_BAD_DESC),
    ("rope_base", 1.0, B.DEC_ERR_BAD_DESC),
    ("flags", 1, B.DEC_ERR_BAD_DESC),
    ("batch", 0, B.DEC_ERR_BAD_DESC),
    ("batch", 9, B.DEC_ERR_UNSUPPORTED),
    ("d_ffn", 8200, B.DEC_ERR_UNSUPPORTED),
])
def test_desc_rules(lib, field, value, code):
    d = desc(**{field: value})
    assert B.check_desc(d) == code
    assert B.last_error()  # reason recorded for handle-less calls


def test_batch_rules(lib):
    # batched decode keeps every sequence's GEMV inputs in LDS: d_model <= 2560,
    # d_ffn and n_heads*head_dim <= 7680 (padded to 512)
    for b in (1, 2, 8):
        assert B.check_desc(desc(batch=b)) == B.DEC_OK, B.last_error()
    assert B.check_desc(B.ModelDesc.from_shape(synth.shape_for("dense2b"), batch=8)) == B.DEC_OK, B.last_error()
    assert B.check_desc(desc(batch=2, d_model=3072)) == B.DEC_ERR_UNSUPPORTED
    assert B.check_desc(desc(batch=2, d_ffn=8192)) == B.DEC_ERR_UNSUPPORTED
    assert B.check_desc(desc(batch=1, d_model=3072)) == B.DEC_OK
    # per-sequence buffers grow with the batch
    assert B.arena_bytes(desc(batch=8), 256) > B.arena_bytes(desc(batch=1), 256)


def test_batched_prefill_flag_rules(lib):
    f = B.DEC_FLAG_BATCHED_PREFILL
    assert B.check_desc(desc(flags=f)) == B.DEC_OK, B.last_error()
    assert B.check_desc(desc(flags=f, batch=2)) == B.DEC_ERR_BAD_DESC       # batch-1 handles only
    assert B.check_desc(desc(flags=f | 1)) == B.DEC_ERR_BAD_DESC            # unknown bit
    assert B.check_desc(desc(flags=f, d_model=3072)) == B.DEC_ERR_UNSUPPORTED   # inputs must fit in LDS
    d2 = synth.shape_for("dense2b")
    plain = B.arena_bytes(B.ModelDesc.from_shape(d2))
    withf = B.arena_bytes(B.ModelDesc.from_shape(d2, flags=f))
    # a second, tiled copy of the weights (about 4.6 GB) plus 8-column buffers
    assert 4.5e9 < withf - plain < 4.8e9


def test_matrix_prefill_flag_rules(lib):
    f = B.DEC_FLAG_MATRIX_PREFILL
    assert B.check_desc(desc(flags=f)) == B.DEC_OK, B.last_error()
    assert B.check_desc(desc(flags=f, batch=2)) == B.DEC_ERR_BAD_DESC       # batch-1 handles only
    assert B.check_desc(desc(flags=f | B.DEC_FLAG_BATCHED_PREFILL)) == B.DEC_ERR_BAD_DESC   # one prefill form
    assert B.check_desc(desc(flags=f | 1)) == B.DEC_ERR_BAD_DESC            # unknown bit
    # matrix-product K dimensions and head_dim in whole 32-wide K steps
    assert B.check_desc(desc(flags=f, head_dim=16)) == B.DEC_ERR_UNSUPPORTED
    assert B.check_desc(desc(flags=f, d_model=264)) == B.DEC_ERR_UNSUPPORTED
    assert B.check_desc(desc(flags=f, d_ffn=1000)) == B.DEC_ERR_UNSUPPORTED
    assert B.check_desc(desc(head_dim=16)) == B.DEC_OK                     # no flag: no such limit
    for name in ("dense2b", "lane2b"):
        assert B.check_desc(B.ModelDesc.from_shape(synth.shape_for(name), flags=f)) == B.DEC_OK, B.last_error()
    d2 = synth.shape_for("dense2b")
    plain = B.arena_bytes(B.ModelDesc.from_shape(d2))
    withf = B.arena_bytes(B.ModelDesc.from_shape(d2, flags=f))
    # workspace for 2048 positions (per position: fp32 residual 10 KB, fp16 product input
    # 5 KB, fp16 q 5 KB, fp16 SwiGLU output 13.8 KB, one scale), about 70 MB, plus 32 MB of
    # split-K partial sums
    per_pos = 4 * 2560 + 2 * 2560 + 2 * 2560 + 2 * 6912 + 4
    assert 2048 * per_pos + 32 * 2**20 <= withf - plain < 2048 * per_pos + 32 * 2**20 + 4096


def test_moe_desc_rules(lib):
    m = synth.shape_for("moe2b")
    ok = B.ModelDesc.from_shape(m)
    assert (ok.n_experts, ok.top_k) == (32, 4)
    assert B.check_desc(ok) == B.DEC_OK, B.last_error()
    assert B.check_desc(desc(top_k=2)) == B.DEC_ERR_BAD_DESC                       # dense with top_k
    tiny = synth.shape_for("tiny")
    for E, k in ((1, 1), (7, 2), (66, 2), (8, 0), (8, 9), (4, 5), (16, 9)):
        assert B.check_desc(B.ModelDesc.from_shape(tiny, n_experts=E, top_k=k, d_ffn=256)) == B.DEC_ERR_BAD_DESC, (E, k)
    for kw in (dict(batch=2), dict(flags=B.DEC_FLAG_MATRIX_PREFILL), dict(flags=B.DEC_FLAG_BATCHED_PREFILL),
               dict(d_ffn=264), dict(d_model=264), dict(d_ffn=2048)):   # 4 x 2048 > 7168
        assert B.check_desc(B.ModelDesc.from_shape(m, **kw)) == B.DEC_ERR_UNSUPPORTED, kw
    assert B.check_desc(B.ModelDesc.from_shape(m, d_ffn=1792)) == B.DEC_OK       # 4 x 1792 = 7168
    with pytest.raises(B.DecError, match="UNSUPPORTED"):
        B.packed_bytes(ok)
    # the arena holds the dense parts, the experts' codes and row scales and
    # the routing record on top of what a dense model of the same attention needs
    dense = B.arena_bytes(B.ModelDesc.from_shape(synth.shape_for("dense2b")))
    moe = B.arena_bytes(ok)
    L, d, F, E, k, C = 25, 2560, 1728, 32, 4, 4096
    fp16_mlp = L * (3 * 6912 * d) * 2                     # dense2b's gate, up and down
    experts = L * (E * 3 * F * d + 4 * E * (2 * F + d)) + C * L * k * 4 + L * E * d * 2
    assert abs((moe - dense) - (experts - fp16_mlp)) < 2e6, (moe - dense, experts - fp16_mlp)


def test_valid_descs_and_arena(lib):
    for name in ("tiny", "dense2b", "lane2b"):
        d = B.ModelDesc.from_shape(synth.shape_for(name))
        assert B.check_desc(d) == B.DEC_OK, B.last_error()
    d2 = B.ModelDesc.from_shape(synth.shape_for("dense2b"))
    n = B.arena_bytes(d2)
    # weights (with the whole embedding) + a 4096-position fp16 KV cache
    assert 4.63e9 + 1.04e9 < n < 4.63e9 + 1.04e9 + 64e6


def test_packer_layout_round_trip(lib):
    s = TINY.with_(n_layers=2)
    t = synth.make_weights(s, seed=3, gain_jitter=0.1)
    d = B.ModelDesc.from_shape(s)
    img = B.pack(d, t)
    assert img.nbytes == B.packed_bytes(d)
    al = lambda n: (n + 127) // 128 * 128
    D, q, F = s.d_model, s.qkv_width, s.d_ffn
    off_o = al(3 * q * D)
    off_gu = al(off_o + D * q)
    off_d = al(off_gu + 2 * F * D)
    stride = al(off_d + D * F)
    names = synth.tensor_names(s)
    bits = lambda a: np.ascontiguousarray(a).view(np.uint16)
    for l in range(s.n_layers):
        base = l * stride
        get = lambda n: t[names.index(f"{n}.{l}")]
        qkv = img[base:base + 3 * q * D].reshape(3 * q, D)
        np.testing.assert_array_equal(qkv, np.concatenate([bits(get("Wq")), bits(get("Wk")), bits(get("Wv"))]))
        np.testing.assert_array_equal(img[base + off_o: base + off_o + D * q].reshape(D, q), bits(get("Wo")))
        gu = img[base + off_gu: base + off_gu + 2 * F * D].reshape(2 * F, D)
        np.testing.assert_array_equal(gu[0::2], bits(get("Wg")))
        np.testing.assert_array_equal(gu[1::2], bits(get("Wu")))
        np.testing.assert_array_equal(img[base + off_d: base + off_d + D * F].reshape(D, F), bits(get("Wd")))
    off_E = stride * s.n_layers
    np.testing.assert_array_equal(img[off_E: off_E + s.vocab * D].reshape(s.vocab, D), bits(t[0]))
    off_lm = al(off_E + s.vocab * D)
    np.testing.assert_array_equal(img[off_lm: off_lm + s.lm_vocab * D].reshape(s.lm_vocab, D), bits(t[-1]))


def _untile(region, rows, cols):
    """Inverse of the tiled layout documented in dec.h (16 x 32 tiles, lane-major inside)."""
    rg, kt = -(-rows // 16), -(-cols // 32)
    t = region[:rg * kt * 512].reshape(rg, kt, 4, 16, 8)        # [g, j, l // 16, l % 16, element]
    return t.transpose(0, 3, 1, 2, 4).reshape(rg * 16, kt * 32), rg * kt * 512


def test_packer_tiled_layout_for_batch(lib):
    # rows and row lengths that are not multiples of 16 / 32 exercise the zero padding
    s = TINY.with_(n_layers=2, n_heads=3, head_dim=8, d_ffn=40, vocab=64, lm_vocab=50)
    t = synth.make_weights(s, seed=4)
    d = B.ModelDesc.from_shape(s, batch=2)
    assert B.check_desc(d) == B.DEC_OK, B.last_error()
    img = B.pack(d, t)
    assert img.nbytes == B.packed_bytes(d)
    names = synth.tensor_names(s)
    bits = lambda a: np.ascontiguousarray(a).view(np.uint16)
    al = lambda n: (n + 127) // 128 * 128
    D, q, F = s.d_model, s.qkv_width, s.d_ffn
    off = 0
    for l in range(s.n_layers):
        get = lambda n: bits(t[names.index(f"{n}.{l}")])
        gu = np.empty((2 * F, D), np.uint16)
        gu[0::2], gu[1::2] = get("Wg"), get("Wu")
        for mat in (np.concatenate([get("Wq"), get("Wk"), get("Wv")]), get("Wo"), gu, get("Wd")):
            R, C = mat.shape
            full, n = _untile(img[off:], R, C)
            np.testing.assert_array_equal(full[:R, :C], mat)
            assert not full[R:].any() and not full[:, C:].any()
            off = al(off + n)
    np.testing.assert_array_equal(img[off: off + s.vocab * D].reshape(s.vocab, D), bits(t[0]))   # E stays row-major
    off = al(off + s.vocab * D)
    full, n = _untile(img[off:], s.lm_vocab, D)
    np.testing.assert_array_equal(full[:s.lm_vocab, :D], bits(t[-1]))
    assert not full[s.lm_vocab:].any()
    assert off + n <= img.size


def test_pack_rejects_wrong_count(lib):
    d = desc()
    t = synth.make_weights(TINY)
    arrs, ptrs = B._tensor_ptrs(t[:-1])
    out = np.zeros(B.packed_bytes(d) // 2, dtype=np.uint16)
    assert lib.dec_pack(ctypes.byref(d), ptrs, len(arrs), out.ctypes.data, out.nbytes) == B.DEC_ERR_WEIGHTS


@pytest.fixture(scope="module")
def good_file(tmp_path_factory):
    p = tmp_path_factory.mktemp("w") / "tiny.decw"
    WF.write(p, desc(), synth.make_weights(TINY))
    return p


def test_weights_file_round_trip(lib, good_file):
    rc, d = B.weights_file_check(good_file)
    assert rc == B.DEC_OK, B.last_error()
    assert (d.n_layers, d.d_model, d.vocab, d.max_ctx) == (2, 256, 4096, 128)
    assert abs(d.rms_eps - 1e-5) < 1e-12


def _corrupt(src, dst, offset, data):
    b = bytearray(open(src, "rb").read())
    b[offset:offset + len(data)] = data
    open(dst, "wb").write(bytes(b))


@pytest.mark.parametrize("what", ["magic", "version", "count", "dtype", "shape", "offset", "nbytes", "truncated", "empty"])
def test_weights_file_defects(lib, good_file, tmp_path, what):
    import struct
    p = tmp_path / f"{what}.decw"
    if what == "magic":
        _corrupt(good_file, p, 0, b"XECW")
    elif what == "version":
        _corrupt(good_file, p, 4, struct.pack("<I", 2))
    elif what == "count":
        _corrupt(good_file, p, 8, struct.pack("<I", 20))
    elif what == "dtype":
        _corrupt(good_file, p, 72 + 40 * 3 + 4, struct.pack("<I", 2))
    elif what == "shape":
        _corrupt(good_file, p, 72 + 40 * 2 + 16, struct.pack("<I", 255))
    elif what == "offset":
        _corrupt(good_file, p, 72 + 40 * 5 + 24, struct.pack("<Q", 1 << 40))
    elif what == "nbytes":
        _corrupt(good_file, p, 72 + 40 * 5 + 32, struct.pack("<Q", 12))
    elif what == "truncated":
        b = open(good_file, "rb").read()
        open(p, "wb").write(b[:len(b) - 1000])
    elif what == "empty":
        open(p, "wb").write(b"")
    rc, _ = B.weights_file_check(p)
    assert rc == B.DEC_ERR_WEIGHTS, what
    assert B.last_error()


def test_init_errors_before_any_device_work(lib, good_file, tmp_path):
    t = synth.make_weights(TINY)
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc(head_dim=48), tensors=t)
    assert e.value.code == B.DEC_ERR_BAD_DESC
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc(), tensors=t[:-1])
    assert e.value.code == B.DEC_ERR_WEIGHTS
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc(), path=tmp_path / "missing.decw")
    assert e.value.code == B.DEC_ERR_WEIGHTS
    with pytest.raises(B.DecError) as e:   # file shapes differ from the description
        B.Decoder(desc(d_ffn=512), path=good_file)
    assert e.value.code == B.DEC_ERR_WEIGHTS
    with pytest.raises(B.DecError) as e:   # unknown debug flag
        B.Decoder(desc(), tensors=t, debug_flags=0x100)
    assert e.value.code == B.DEC_ERR_INVALID_ARG
    with pytest.raises(B.DecError) as e:   # the stress mode runs on the resident kernel only
        B.Decoder(desc(), tensors=t, debug_flags=B.DEC_DEBUG_STRESS | B.DEC_DEBUG_MULTILAUNCH)
    assert e.value.code == B.DEC_ERR_INVALID_ARG
    with pytest.raises(B.DecError) as e:   # the no-allocation handle needs a caller arena and stream
        B.Decoder(desc(), tensors=t, noalloc=True)
    assert e.value.code == B.DEC_ERR_INVALID_ARG
    # the decode server: idle bound in [0, 10 s]; one resident launch with
    # host-pinned memory, so neither with one launch per phase nor without allocation
    for kw in (dict(serve_idle_us=-1), dict(serve_idle_us=10_000_001),
               dict(serve_idle_us=1000, debug_flags=B.DEC_DEBUG_MULTILAUNCH),
               dict(serve_idle_us=1000, noalloc=True)):
        with pytest.raises(B.DecError) as e:
            B.Decoder(desc(), tensors=t, **kw)
        assert e.value.code == B.DEC_ERR_INVALID_ARG, kw


def test_init_without_gpu_reports_no_device(lib, good_file):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc(), tensors=synth.make_weights(TINY))
    assert e.value.code == B.DEC_ERR_NO_DEVICE
    with pytest.raises(B.DecError) as e:
        B.Decoder(desc(), path=good_file)
    assert e.value.code == B.DEC_ERR_NO_DEVICE


def test_null_handle_calls(lib):
    assert lib.dec_step(None, None, None, None) == B.DEC_ERR_INVALID_ARG
    assert lib.dec_prefill(None, None, 1, None, None) == B.DEC_ERR_INVALID_ARG
    assert lib.dec_generate(None, 1, None) == B.DEC_ERR_INVALID_ARG
    assert lib.dec_reset(None) == B.DEC_ERR_INVALID_ARG
    assert lib.dec_sync(None) == B.DEC_ERR_INVALID_ARG
    assert lib.dec_position(None) == -1
    lib.dec_free(None)
    assert isinstance(lib.dec_last_error(None), bytes)


def test_stream_ceiling_argument_checks(lib):
    """dec_stream_ceiling rejects bad arguments before it touches a device."""
    g = ctypes.c_double()
    assert lib.dec_stream_ceiling(0, 1 << 20, 3, ctypes.byref(g)) == B.DEC_ERR_INVALID_ARG      # below 64 MiB
    assert lib.dec_stream_ceiling(0, 1 << 40, 3, ctypes.byref(g)) == B.DEC_ERR_INVALID_ARG      # above 64 GiB
    assert lib.dec_stream_ceiling(0, 1 << 30, 0, ctypes.byref(g)) == B.DEC_ERR_INVALID_ARG      # reps
    assert lib.dec_stream_ceiling(0, 1 << 30, 3, None) == B.DEC_ERR_INVALID_ARG


def test_library_missing_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libdecmono.so")
    with pytest.raises(B.DecLibraryMissing):
        B.load()
