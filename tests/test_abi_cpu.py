"""The C-ABI library loads without a GPU, exports every entry point that
include/rd.h declares, and rejects bad input on the host before touching a
device.  No compute calls here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rd_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def rd():
    import request_decode_amd as rd
    rd.lib()
    return rd


def test_every_declared_symbol_is_exported(rd):
    names = declared_functions()
    assert len(names) >= 20
    lib = C.CDLL(rd.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding knows every one of them
    bound = {s[0] for s in rd.SIGNATURES}
    assert set(names) <= bound, set(names) - bound


def test_options_defaults(rd):
    o = rd.rd_options()
    rd.lib().rd_options_init(C.byref(o))
    assert o.struct_size == C.sizeof(rd.rd_options)
    assert (o.device, o.max_context, o.max_batch, o.kv_format, o.executor, o.attn_splits) == (0, 4096, 1, 0, 0, 0)


def _create(rd, blob, **kw):
    o = rd.rd_options()
    rd.lib().rd_options_init(C.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    h = C.c_void_p()
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    st = rd.lib().rd_model_create(b.ctypes.data, b.size, C.byref(o), C.byref(h))
    return st, h


def test_blob_validation_on_host(rd):
    shape = synth.SHAPES["tiny"]
    blob = synth.make_blob(shape, seed=1)
    st, h = _create(rd, blob[:100])
    assert st == rd.RD_ERR_BAD_BLOB and not h.value
    st, _ = _create(rd, blob[:-2])
    assert st == rd.RD_ERR_BAD_BLOB and "implies" in rd.last_error()
    bad = blob.copy()
    bad[0:4] = np.frombuffer(b"XXXX", np.uint8)
    assert _create(rd, bad)[0] == rd.RD_ERR_BAD_BLOB
    bad = blob.copy()
    bad[12] = 2                                   # dtype field
    assert _create(rd, bad)[0] == rd.RD_ERR_BAD_BLOB
    # a shape the kernels do not cover (head_dim 96)
    odd = synth.ModelShape(1, 192, 2, 2, 96, 256, 64)
    assert _create(rd, synth.make_blob(odd, seed=1))[0] == rd.RD_ERR_UNSUPPORTED


def test_option_validation_on_host(rd):
    blob = synth.make_blob(synth.SHAPES["tiny"], seed=1)
    assert _create(rd, blob, max_context=0)[0] == rd.RD_ERR_INVALID_ARG
    assert _create(rd, blob, max_batch=9)[0] == rd.RD_ERR_UNSUPPORTED
    assert _create(rd, blob, max_batch=0)[0] == rd.RD_ERR_UNSUPPORTED
    assert _create(rd, blob, max_batch=8, executor=3)[0] == rd.RD_ERR_UNSUPPORTED   # persistent: batch 1
    assert _create(rd, blob, kv_format=7)[0] == rd.RD_ERR_INVALID_ARG
    assert _create(rd, blob, executor=9)[0] == rd.RD_ERR_INVALID_ARG
    assert _create(rd, blob, attn_splits=1000)[0] == rd.RD_ERR_INVALID_ARG
    # paged cache: fp16 or E5M2 rows, the batch step, a pool below 2 GiB per layer
    assert _create(rd, blob, max_batch=2, kv_pages=-1)[0] == rd.RD_ERR_INVALID_ARG
    assert _create(rd, blob, max_batch=2, kv_pages=8, kv_format=2)[0] == rd.RD_ERR_UNSUPPORTED
    assert _create(rd, blob, max_batch=1, kv_pages=8)[0] == rd.RD_ERR_UNSUPPORTED
    assert _create(rd, blob, max_batch=2, kv_pages=1 << 20)[0] == rd.RD_ERR_INVALID_ARG
    assert _create(rd, blob, max_batch=2, kv_pages=8, max_context=(1 << 22) - 1)[0] == rd.RD_ERR_INVALID_ARG
    # INT8: the open segment is a split of its own, so one split is too few
    assert _create(rd, blob, kv_format=2, attn_splits=1)[0] == rd.RD_ERR_INVALID_ARG
    # 4 kv heads x 64 dims x 2 bytes: at 2^22 positions one layer's K is 2 GiB,
    # past the attention's 32-bit row offsets
    assert _create(rd, blob, max_context=1 << 22)[0] == rd.RD_ERR_INVALID_ARG
    assert "2 GiB" in rd.last_error()
    o = rd.rd_options()
    rd.lib().rd_options_init(C.byref(o))
    o.struct_size = 3
    h = C.c_void_p()
    assert rd.lib().rd_model_create(blob.ctypes.data, blob.size, C.byref(o), C.byref(h)) == rd.RD_ERR_INVALID_ARG


def test_null_arguments(rd):
    L = rd.lib()
    assert L.rd_model_get_info(None, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_reset(None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_decode_step(None, None, 1, None, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_generate(None, None, 1, 1, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_gemv_f16(None, None, None, 1, 8, 1, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_attention_f16(None, None, None, None, 1, 1, 64, 1, 1, 1.0, 1, None) == rd.RD_ERR_INVALID_ARG
    # argument checks before any device work (the addresses are never read):
    # INT8 with one split, and a cache past 2 GiB
    a = 256
    assert L.rd_attention(a, a, a, a, a, a, a, a, 2, 1, 64, 1, 1, 2, 1.0, 1, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_attention(a, a, a, a, a, a, a, a, 16, 8, 128, 1, 1 << 20, 0, 1.0, 8, None) == rd.RD_ERR_INVALID_ARG
    assert "2 GiB" in rd.last_error()
    assert L.rd_seg_quant(None, 1, 8, None, None, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_argmax_f32(None, 1, None, None) == rd.RD_ERR_INVALID_ARG
    L.rd_model_destroy(None)   # NULL-safe


def test_gemv_argument_checks(rd):
    # Rejected before anything touches a device: fake aligned pointers.
    L, p = rd.lib(), C.c_void_p(256)
    assert L.rd_gemv_f16(p, p, p, 16, 64, 3, None) == rd.RD_ERR_UNSUPPORTED
    assert L.rd_gemv_f16(p, p, p, 16, 72, 8, None) == rd.RD_ERR_INVALID_ARG      # K % 64
    assert L.rd_gemv_f16(p, p, p, 16, 8256, 8, None) == rd.RD_ERR_INVALID_ARG    # K > 8192
    assert L.rd_gemv_f16(p, p, p, 0, 64, 8, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_gemv_f16(p, p, p, 16, 12, 1, None) == rd.RD_ERR_INVALID_ARG      # K % 8
    assert L.rd_gemv_f16(p, C.c_void_p(258), p, 16, 64, 1, None) == rd.RD_ERR_INVALID_ARG  # alignment


def test_blob_layout_matches_shapes():
    s = synth.SHAPES["2b"]
    lay, total = synth.blob_layout(s)
    params = sum(int(np.prod(shp)) for _, shp, _, _ in lay)
    assert params == 1_263_634_432
    assert all(off % 256 == 0 for *_, off in lay)
    assert total >= 256 + 2 * params


def test_q4_argument_checks(rd):
    # rejected before anything touches a device: fake aligned pointers
    L, p = rd.lib(), C.c_void_p(256)
    assert L.rd_gemv_q4(p, p, p, p, 16, 100, None) == rd.RD_ERR_INVALID_ARG     # K % 128
    assert L.rd_gemv_q4(p, p, p, p, 16, 8320, None) == rd.RD_ERR_INVALID_ARG    # K > 8192
    assert L.rd_gemv_q4(p, p, p, p, 0, 128, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_gemv_q4(C.c_void_p(258), p, p, p, 16, 128, None) == rd.RD_ERR_INVALID_ARG   # alignment
    assert L.rd_q4_quantize(p, 16, 64, p, p, None) == rd.RD_ERR_INVALID_ARG
    assert L.rd_q4_quantize(None, 16, 128, p, p, None) == rd.RD_ERR_INVALID_ARG

