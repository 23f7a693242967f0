"""Python binding of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the HIP library and
its binding never do.  The binding only marshals arguments (ctypes); all
arithmetic is in oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_FORMATS = {"fp16": 0, "e5m2": 1, "int8": 2, "exact": 3}
SEG = 128


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (always recompiles).

    No fast-math and no contraction: every binary64/binary32 operation is the
    IEEE operation written in the source."""
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", LIB_PATH + ".tmp", os.path.join(_HERE, "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        u16p, u8p, dp, fp, i32p = (C.POINTER(C.c_uint16), C.POINTER(C.c_uint8), C.POINTER(C.c_double),
                                   C.POINTER(C.c_float), C.POINTER(C.c_int32))
        L.orc_h2d.restype = C.c_double
        L.orc_h2d.argtypes = [C.c_uint16]
        L.orc_d2h.restype = C.c_uint16
        L.orc_d2h.argtypes = [C.c_double]
        L.orc_h2d_n.argtypes = [u16p, C.c_size_t, dp]
        L.orc_d2h_n.argtypes = [dp, C.c_size_t, u16p]
        L.orc_e5m2_from_h_n.argtypes = [u16p, C.c_size_t, u8p]
        L.orc_h_from_e5m2_n.argtypes = [u8p, C.c_size_t, u16p]
        L.orc_seg_quant.argtypes = [u16p, C.c_int, u8p, fp, fp]
        L.orc_seg_dequant.restype = C.c_float
        L.orc_seg_dequant.argtypes = [C.c_uint8, C.c_float, C.c_float]
        L.orc_seg_dequant_n.argtypes = [u8p, C.c_size_t, C.c_float, C.c_float, fp]
        L.orc_delta_seal.argtypes = [u16p, C.c_int, C.c_int, u16p, u8p, fp, fp]
        L.orc_delta_restore.argtypes = [u16p, u8p, C.c_int, C.c_int, C.c_float, C.c_float, fp]
        L.orc_q4_quant.argtypes = [u16p, C.c_int, C.c_int, u8p, fp]
        L.orc_q4_dequant.argtypes = [u8p, fp, C.c_int, C.c_int, u16p]
        L.orc_q4_code.restype = C.c_int
        L.orc_q4_code.argtypes = [u8p, C.c_size_t]
        L.orc_rmsnorm.argtypes = [dp, u16p, C.c_int, C.c_double, dp]
        L.orc_rope.argtypes = [dp, C.c_int, C.c_int, C.c_double]
        L.orc_gemv.argtypes = [u16p, dp, C.c_int, C.c_int, dp]
        L.orc_attention.argtypes = [dp, dp, dp, C.c_int, C.c_int, dp]
        L.orc_silu.restype = C.c_double
        L.orc_silu.argtypes = [C.c_double]
        L.orc_argmax.restype = C.c_int
        L.orc_argmax.argtypes = [dp, C.c_int]
        L.orc_create.restype = C.c_void_p
        L.orc_create.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_int]
        L.orc_destroy.argtypes = [C.c_void_p]
        L.orc_last_error.restype = C.c_char_p
        L.orc_reset.argtypes = [C.c_void_p]
        L.orc_pos.restype = C.c_int
        L.orc_pos.argtypes = [C.c_void_p, C.c_int]
        L.orc_dims.argtypes = [C.c_void_p, C.POINTER(C.c_int)]
        L.orc_step.restype = C.c_int
        L.orc_step.argtypes = [C.c_void_p, i32p, dp, i32p]
        L.orc_layer0_kv.argtypes = [C.c_void_p, C.c_int32, C.c_int, dp, dp]
        L.orc_prefill.restype = C.c_int
        L.orc_prefill.argtypes = [C.c_void_p, i32p, C.c_int]
        for f in (L.orc_get_rows, L.orc_set_rows):
            f.restype = C.c_int
            f.argtypes = [C.c_void_p] + [C.c_int] * 6 + [C.c_void_p]
        L.orc_seg_meta.restype = C.c_int
        L.orc_seg_meta.argtypes = [C.c_void_p] + [C.c_int] * 5 + [fp, fp, C.c_int]
        L.orc_read_row.restype = C.c_int
        L.orc_read_row.argtypes = [C.c_void_p] + [C.c_int] * 5 + [dp]
        L.orc_set_store.argtypes = [C.c_void_p, C.c_int]
        L.orc_record_rows.restype = C.c_int
        L.orc_record_rows.argtypes = [C.c_void_p, C.c_int]
        L.orc_get_computed.restype = C.c_int
        L.orc_get_computed.argtypes = [C.c_void_p] + [C.c_int] * 6 + [dp]
        L.orc_set_pos.restype = C.c_int
        L.orc_set_pos.argtypes = [C.c_void_p, C.c_int, C.c_int]
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(C.POINTER(t))


# ---- number formats -------------------------------------------------------

def h2d(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_h2d_n(_p(h, C.c_uint16), h.size, _p(out, C.c_double))
    return out


def d2h(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_d2h_n(_p(x, C.c_double), x.size, _p(out, C.c_uint16))
    return out


def e5m2_from_h(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.uint8)
    lib().orc_e5m2_from_h_n(_p(h, C.c_uint16), h.size, _p(out, C.c_uint8))
    return out


def h_from_e5m2(e: np.ndarray) -> np.ndarray:
    e = np.ascontiguousarray(e, dtype=np.uint8)
    out = np.empty(e.shape, np.uint16)
    lib().orc_h_from_e5m2_n(_p(e, C.c_uint8), e.size, _p(out, C.c_uint16))
    return out


def seg_quant(h: np.ndarray):
    """binary16 bits (any shape) -> (uint8 codes, float32 scale, float32 zp)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    codes = np.empty(h.shape, np.uint8)
    s, z = C.c_float(), C.c_float()
    lib().orc_seg_quant(_p(h, C.c_uint16), h.size, _p(codes, C.c_uint8), C.byref(s), C.byref(z))
    return codes, np.float32(s.value), np.float32(z.value)


def delta_seal(x: np.ndarray):
    """Delta quantization of one segment (orc_delta_seal): binary16 bits
    [n, hd] -> (anchor uint16 [hd], codes uint8 [n-1, hd], float32 scale,
    float32 zp)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n, hd = x.shape
    anchor = np.empty(hd, np.uint16)
    codes = np.empty((max(n - 1, 0), hd), np.uint8)
    s, z = C.c_float(), C.c_float()
    lib().orc_delta_seal(_p(x, C.c_uint16), n, hd, _p(anchor, C.c_uint16), _p(codes, C.c_uint8), C.byref(s),
                         C.byref(z))
    return anchor, codes, np.float32(s.value), np.float32(z.value)


def delta_restore(anchor: np.ndarray, codes: np.ndarray, scale, zp) -> np.ndarray:
    """The segment's rows restored from a delta seal (orc_delta_restore):
    float32 [n, hd]."""
    a = np.ascontiguousarray(anchor, dtype=np.uint16)
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    hd = a.size
    n = c.shape[0] + 1
    y = np.empty((n, hd), np.float32)
    lib().orc_delta_restore(_p(a, C.c_uint16), _p(c, C.c_uint8), n, hd, float(scale), float(zp), _p(y, C.c_float))
    return y


def seg_dequant(codes: np.ndarray, scale, zp) -> np.ndarray:
    """(code - zp) * scale in binary32, element-wise (orc_seg_dequant)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().orc_seg_dequant_n(_p(c, C.c_uint8), c.size, float(scale), float(zp), _p(out, C.c_float))
    return out


def q4_quant(W_f16):
    """fp16 [n][k] (k % 128 == 0) -> (codes uint8 [n][k/2], scales float32 [n][k/128])."""
    W = np.ascontiguousarray(np.asarray(W_f16, dtype=np.float16).view(np.uint16))
    n, k = W.shape
    codes = np.empty((n, k // 2), np.uint8)
    scales = np.empty((n, k // 128), np.float32)
    lib().orc_q4_quant(_p(W, C.c_uint16), n, k, _p(codes, C.c_uint8), _p(scales, C.c_float))
    return codes, scales


def q4_dequant(codes, scales) -> np.ndarray:
    """-> fp16 [n][k]: fp16(float(code) * scale)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    n, k = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, k), np.uint16)
    lib().orc_q4_dequant(_p(codes, C.c_uint8), _p(scales, C.c_float), n, k, _p(out, C.c_uint16))
    return out.view(np.float16)


# ---- building blocks ---------------------------------------------------------

def rmsnorm(x, gain_f16, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(np.asarray(gain_f16, dtype=np.float16).view(np.uint16))
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x, C.c_double), _p(g, C.c_uint16), x.size, eps, _p(out, C.c_double))
    return out


def rope(v, pos: int, base: float = 10000.0) -> np.ndarray:
    v = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_p(v, C.c_double), v.size, pos, base)
    return v


def gemv(W_f16, x) -> np.ndarray:
    W = np.ascontiguousarray(np.asarray(W_f16, dtype=np.float16).view(np.uint16))
    x = np.ascontiguousarray(x, dtype=np.float64)
    n, k = W.shape
    y = np.empty(n, np.float64)
    lib().orc_gemv(_p(W, C.c_uint16), _p(x, C.c_double), n, k, _p(y, C.c_double))
    return y


def attention(q, K, V) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    L, hd = K.shape
    out = np.empty(hd, np.float64)
    lib().orc_attention(_p(q, C.c_double), _p(K, C.c_double), _p(V, C.c_double), L, hd, _p(out, C.c_double))
    return out


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def argmax(v) -> int:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return lib().orc_argmax(_p(v, C.c_double), v.size)


# ---- the model --------------------------------------------------------------

class OracleModel:
    """Decode-step oracle over a weight blob (uint8 array in the RDW1 layout)."""

    def __init__(self, blob: np.ndarray, max_ctx: int, batch: int = 1, kv_format: str = "fp16"):
        L = lib()
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        self.kv_format = kv_format
        self._h = L.orc_create(blob.ctypes.data, blob.size, max_ctx, batch, KV_FORMATS[kv_format])
        if not self._h:
            raise ValueError("oracle: " + L.orc_last_error().decode())
        d = (C.c_int * 7)()
        L.orc_dims(self._h, d)
        (self.n_layers, self.d_model, self.n_heads, self.n_kv_heads, self.head_dim, self.d_ff,
         self.vocab) = list(d)
        self.batch = batch
        self.max_ctx = max_ctx

    def close(self):
        if getattr(self, "_h", None):
            lib().orc_destroy(self._h)
            self._h = None

    __del__ = close

    def reset(self):
        lib().orc_reset(self._h)

    def pos(self, b: int = 0) -> int:
        return lib().orc_pos(self._h, b)

    def set_pos(self, pos: int, b: int = 0):
        if lib().orc_set_pos(self._h, b, pos) != 0:
            raise ValueError("bad position")

    def set_store(self, store: bool):
        """False: steps keep the rows already at their position (orc_set_store)."""
        lib().orc_set_store(self._h, 1 if store else 0)

    def record_rows(self, on: bool = True):
        """Keep the K/V rows every later step computes (orc_record_rows)."""
        if lib().orc_record_rows(self._h, 1 if on else 0) != 0:
            raise MemoryError("oracle: no memory for the row record")

    def computed_rows(self, layer, which, head, pos0, n, b=0) -> np.ndarray:
        out = np.empty((n, self.head_dim), np.float64)
        if lib().orc_get_computed(self._h, b, layer, which, head, pos0, n, _p(out, C.c_double)) != 0:
            raise ValueError("no record, or bad row region")
        return out

    def step(self, tokens):
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(self.batch))
        logits = np.empty((self.batch, self.vocab), np.float64)
        nxt = np.empty(self.batch, np.int32)
        rc = lib().orc_step(self._h, _p(t, C.c_int32), _p(logits, C.c_double), _p(nxt, C.c_int32))
        if rc != 0:
            raise ValueError("oracle: " + lib().orc_last_error().decode())
        return logits, nxt

    def prefill(self, tokens):
        """Teacher-forced prompt steps, loop-interchanged (orc_prefill)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        if lib().orc_prefill(self._h, _p(t, C.c_int32), t.size) != 0:
            raise ValueError("oracle: " + lib().orc_last_error().decode())

    def layer0_kv(self, token: int, pos: int):
        n = self.n_kv_heads * self.head_dim
        k = np.empty(n, np.float64)
        v = np.empty(n, np.float64)
        lib().orc_layer0_kv(self._h, int(token), int(pos), _p(k, C.c_double), _p(v, C.c_double))
        return k.reshape(self.n_kv_heads, self.head_dim), v.reshape(self.n_kv_heads, self.head_dim)

    def _row_dtype(self, pos0: int, b: int):
        if self.kv_format == "fp16":
            return np.uint16
        if self.kv_format == "e5m2":
            return np.uint8
        if self.kv_format == "exact":
            return np.float64
        return np.uint8 if pos0 < self.pos(b) // SEG * SEG else np.uint16

    def get_rows(self, layer, which, head, pos0, n, b=0):
        out = np.empty((n, self.head_dim), self._row_dtype(pos0, b))
        if lib().orc_get_rows(self._h, b, layer, which, head, pos0, n, out.ctypes.data) != 0:
            raise ValueError("bad row region")
        return out

    def set_rows(self, layer, which, head, pos0, src, b=0):
        src = np.ascontiguousarray(src, dtype=self._row_dtype(pos0, b))
        n = src.shape[0]
        if lib().orc_set_rows(self._h, b, layer, which, head, pos0, n, src.ctypes.data) != 0:
            raise ValueError("bad row region")

    def seg_meta(self, layer, which, head, seg, b=0, set_to=None):
        s, z = C.c_float(), C.c_float()
        if set_to is not None:
            s.value, z.value = float(set_to[0]), float(set_to[1])
        if lib().orc_seg_meta(self._h, b, layer, which, head, seg, C.byref(s), C.byref(z),
                              1 if set_to is not None else 0) != 0:
            raise ValueError("bad segment")
        return np.float32(s.value), np.float32(z.value)

    def read_row(self, layer, which, head, pos, b=0) -> np.ndarray:
        out = np.empty(self.head_dim, np.float64)
        if lib().orc_read_row(self._h, b, layer, which, head, pos, _p(out, C.c_double)) != 0:
            raise ValueError("bad row")
        return out
