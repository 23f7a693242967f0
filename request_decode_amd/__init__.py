"""Python binding of librd.so (include/rd.h): argument marshalling only.

Every computation of the decode step runs in the HIP kernels of librd.so.
There is no fallback: importing this package without the built library
raises.  Device pointers are plain integers (e.g. torch's `data_ptr()`);
streams are `hipStream_t` handles as integers (torch's `cuda_stream`) or 0.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librd.so")

RD_OK = 0
RD_ERR_INVALID_ARG = -1
RD_ERR_BAD_BLOB = -2
RD_ERR_OUT_OF_MEMORY = -3
RD_ERR_CONTEXT_FULL = -4
RD_ERR_UNSUPPORTED = -5
RD_ERR_DEVICE = -6
RD_ERR_NUMERIC = -7
_NAMES = {0: "RD_OK", -1: "RD_ERR_INVALID_ARG", -2: "RD_ERR_BAD_BLOB", -3: "RD_ERR_OUT_OF_MEMORY",
          -4: "RD_ERR_CONTEXT_FULL", -5: "RD_ERR_UNSUPPORTED", -6: "RD_ERR_DEVICE", -7: "RD_ERR_NUMERIC"}

RD_KV_FP16, RD_KV_FP8_E5M2, RD_KV_INT8_SEG128 = 0, 1, 2
KV_FORMATS = {"fp16": RD_KV_FP16, "e5m2": RD_KV_FP8_E5M2, "int8": RD_KV_INT8_SEG128}
RD_EXEC_AUTO, RD_EXEC_EAGER, RD_EXEC_GRAPH, RD_EXEC_PERSISTENT = 0, 1, 2, 3
EXECUTORS = {"auto": RD_EXEC_AUTO, "eager": RD_EXEC_EAGER, "graph": RD_EXEC_GRAPH, "persistent": RD_EXEC_PERSISTENT}
SEG = 128


class rd_options(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("device", C.c_int32), ("stream", C.c_void_p),
                ("max_context", C.c_int32), ("max_batch", C.c_int32), ("kv_format", C.c_int32),
                ("executor", C.c_int32), ("attn_splits", C.c_int32), ("kv_pages", C.c_int32)]


class rd_model_info(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ff", C.c_int32), ("vocab", C.c_int32),
                ("rope_base", C.c_float), ("norm_eps", C.c_float), ("max_context", C.c_int32),
                ("max_batch", C.c_int32), ("kv_format", C.c_int32), ("executor", C.c_int32),
                ("attn_splits", C.c_int32), ("weight_bytes", C.c_uint64), ("streamed_bytes", C.c_uint64),
                ("kv_bytes", C.c_uint64), ("kv_pages", C.c_int32), ("page_rows", C.c_int32)]


class RdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_NAMES.get(status, status)}: {msg}")
        self.status = status


# (name, restype, argtypes) of every exported entry point of include/rd.h
_VP, _I32, _SZ, _I32P, _FP = C.c_void_p, C.c_int32, C.c_size_t, C.POINTER(C.c_int32), C.POINTER(C.c_float)
SIGNATURES = [
    ("rd_options_init", None, [C.POINTER(rd_options)]),
    ("rd_model_create", _I32, [_VP, _SZ, C.POINTER(rd_options), C.POINTER(_VP)]),
    ("rd_model_destroy", None, [_VP]),
    ("rd_model_get_info", _I32, [_VP, C.POINTER(rd_model_info)]),
    ("rd_reset", _I32, [_VP]),
    ("rd_get_position", _I32, [_VP, _I32P]),
    ("rd_seq_reset", _I32, [_VP, _I32]),
    ("rd_seq_fork", _I32, [_VP, _I32, _I32]),
    ("rd_seq_position", _I32, [_VP, _I32, _I32P]),
    ("rd_kv_page_stats", _I32, [_VP, _I32P, _I32P, _I32P]),
    ("rd_decode_step", _I32, [_VP, _I32P, _I32, _FP, _I32P]),
    ("rd_generate", _I32, [_VP, _I32P, _I32, _I32, _I32P]),
    ("rd_generate_async", _I32, [_VP, _I32P, _I32, _I32, _VP]),
    ("rd_synchronize", _I32, [_VP]),
    ("rd_debug_export_kv", _I32, [_VP, _I32, _I32, _I32, _VP, _SZ, C.POINTER(_SZ)]),
    ("rd_debug_import_kv", _I32, [_VP, _I32, _I32, _I32, _VP, _SZ, _I32]),
    ("rd_set_position", _I32, [_VP, _I32]),
    ("rd_set_executor", _I32, [_VP, _I32]),
    ("rd_debug_run_phase", _I32, [_VP, _I32, _I32, _I32]),
    ("rd_debug_trace_step", _I32, [_VP, _I32, C.POINTER(C.c_uint64), _I32, _I32P]),
    ("rd_debug_trace_step_all", _I32, [_VP, _I32, C.POINTER(C.c_uint64), _I32, _I32P]),
    ("rd_last_error", C.c_char_p, []),
    ("rd_prefill", _I32, [_VP, _I32P, _I32, _I32]),
    ("rd_prefill_batched", _I32, [_VP, _I32P, _I32]),
    ("rd_gemv_f16", _I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    ("rd_attention_f16", _I32, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, C.c_float, _I32, _VP]),
    ("rd_attention", _I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, C.c_float,
                            _I32, _VP]),
    ("rd_attention_noalloc", _I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32,
                                    C.c_float, _I32, _VP]),
    ("rd_q4_quantize", _I32, [_VP, _I32, _I32, _VP, _VP, _VP]),
    ("rd_gemv_q4", _I32, [_VP, _VP, _VP, _VP, _I32, _I32, _VP]),
    ("rd_e5m2_encode", _I32, [_VP, _VP, _SZ, _VP]),
    ("rd_seg_quant", _I32, [_VP, _I32, _I32, _VP, _VP, _VP]),
    ("rd_delta_seal", _I32, [_VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP]),
    ("rd_delta_restore", _I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP]),
    ("rd_argmax_f32", _I32, [_VP, _I32, _VP, _VP]),
    ("rd_release_scratch", _I32, []),
]

_lib = None


def lib():
    """The loaded librd.so.  Raises if it has not been built: no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with request_decode_amd/build.py "
                              "(or __graft_entry__.build()); there is no non-HIP path")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().rd_last_error().decode()


def check(status: int):
    if status != RD_OK:
        raise RdError(status, last_error())
    return status


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_I32P)


# ---- model ----------------------------------------------------------------------

class Model:
    """A decode-step model on one GPU (rd_model_create and friends)."""

    def __init__(self, blob: np.ndarray, max_context: int = 4096, kv_format: str = "fp16",
                 executor: str = "auto", device: int = 0, stream: int = 0, attn_splits: int = 0, batch: int = 1,
                 kv_pages: int = 0):
        L = lib()
        o = rd_options()
        L.rd_options_init(C.byref(o))
        o.device = device
        o.stream = stream or None
        o.max_context = max_context
        o.max_batch = batch
        o.kv_format = KV_FORMATS[kv_format]
        o.executor = EXECUTORS[executor]
        o.attn_splits = attn_splits
        o.kv_pages = kv_pages
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        h = _VP()
        self._destroy = L.rd_model_destroy
        check(L.rd_model_create(blob.ctypes.data, blob.size, C.byref(o), C.byref(h)))
        self._h = h
        self.info = self.get_info()
        self.vocab = self.info.vocab
        self.kv_format = kv_format
        self.batch = batch

    def close(self):
        h = getattr(self, "_h", None)
        if h:
            self._h = None
            self._destroy(h)   # held on the instance: usable during interpreter shutdown

    __del__ = close

    def get_info(self) -> rd_model_info:
        i = rd_model_info()
        check(lib().rd_model_get_info(self._h, C.byref(i)))
        return i

    def reset(self):
        check(lib().rd_reset(self._h))

    def position(self) -> int:
        p = C.c_int32()
        check(lib().rd_get_position(self._h, C.byref(p)))
        return p.value

    def set_position(self, pos: int):
        check(lib().rd_set_position(self._h, pos))

    # paged cache: per-sequence positions and prefix sharing
    def seq_reset(self, seq: int):
        check(lib().rd_seq_reset(self._h, seq))

    def seq_fork(self, src: int, dst: int):
        check(lib().rd_seq_fork(self._h, src, dst))

    def seq_position(self, seq: int) -> int:
        p = C.c_int32()
        check(lib().rd_seq_position(self._h, seq, C.byref(p)))
        return p.value

    def page_stats(self):
        """(free, used, shared) page groups of a paged cache."""
        f, u, sh = C.c_int32(), C.c_int32(), C.c_int32()
        check(lib().rd_kv_page_stats(self._h, C.byref(f), C.byref(u), C.byref(sh)))
        return f.value, u.value, sh.value

    def set_executor(self, executor: str):
        check(lib().rd_set_executor(self._h, EXECUTORS[executor]))
        self.info = self.get_info()

    def run_phase(self, phase: int, layer: int, iters: int):
        check(lib().rd_debug_run_phase(self._h, phase, layer, iters))

    def trace_step(self, token: int, max_events: int = 4096):
        """Event trace of one persistent step: (codes, clocks in 10 ns ticks)."""
        cap = 1 + 2 * max_events
        ts = np.zeros(cap, np.uint64)
        n = C.c_int32()
        check(lib().rd_debug_trace_step(self._h, token, ts.ctypes.data_as(C.POINTER(C.c_uint64)), cap, C.byref(n)))
        ev = ts[1:1 + 2 * n.value].reshape(-1, 2).astype(np.int64)
        return ev[:, 0], ev[:, 1]

    def trace_step_all(self, token: int, n_wg: int = 1024, max_events: int = 1024):
        """Event traces of every workgroup of one persistent step: a list, per
        workgroup, of (codes, clocks in 10 ns ticks); n_wg: at least the
        device's CU count (the buffer is sized for it)."""
        cap = 1 + 2 * max_events
        ts = np.zeros(cap * n_wg, np.uint64)
        n = C.c_int32()
        check(lib().rd_debug_trace_step_all(self._h, token, ts.ctypes.data_as(C.POINTER(C.c_uint64)), cap,
                                            C.byref(n)))
        out = []
        for w in range(n.value):
            r = ts[w * cap:(w + 1) * cap]
            ev = r[1:1 + 2 * int(r[0])].reshape(-1, 2).astype(np.int64)
            out.append((ev[:, 0], ev[:, 1]))
        return out

    def _tokens(self, tokens):
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        if t.size != self.batch:
            raise ValueError(f"need {self.batch} token(s), one per sequence")
        return t, t.ctypes.data_as(_I32P)

    def decode_step(self, token, want_logits: bool = True, allow_numeric: bool = False):
        """One step.  Batch 1: token int -> (logits [V], next int); batch B:
        tokens [B] -> (logits [B][V], next [B])."""
        t, tp = self._tokens(token)
        nxt = np.zeros(self.batch, np.int32)
        logits = np.empty((self.batch, self.vocab), np.float32) if want_logits else None
        lp = logits.ctypes.data_as(_FP) if want_logits else None
        st = lib().rd_decode_step(self._h, tp, self.batch, lp, nxt.ctypes.data_as(_I32P))
        if not (allow_numeric and st == RD_ERR_NUMERIC):
            check(st)
        if self.batch == 1:
            return (logits[0] if want_logits else None), int(nxt[0])
        return logits, nxt

    def prefill(self, tokens):
        """Teacher-forced steps over `tokens` ([n] at batch 1, [n][B] at batch B,
        step-major), no logits, one sync at the end."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        if t.size % self.batch:
            raise ValueError("token count must be a multiple of the batch")
        check(lib().rd_prefill(self._h, t.ctypes.data_as(_I32P), self.batch, int(t.size // self.batch)))

    def prefill_batched(self, tokens):
        """The prompt `tokens` ([n], batch-1 models) through the batched
        prefill (matrix products per layer, chunked), one sync."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        check(lib().rd_prefill_batched(self._h, t.ctypes.data_as(_I32P), int(t.size)))

    def generate(self, first, n_steps: int) -> np.ndarray:
        """n_steps greedy steps from `first` (int, or [B]): tokens [n_steps]
        (batch 1) or [n_steps][B]."""
        f, fp = self._tokens(first)
        out = np.zeros(n_steps * self.batch, np.int32)
        check(lib().rd_generate(self._h, fp, self.batch, n_steps, out.ctypes.data_as(_I32P)))
        return out if self.batch == 1 else out.reshape(n_steps, self.batch)

    def generate_async(self, first, n_steps: int, out_dev_ptr: int):
        f, fp = self._tokens(first)
        check(lib().rd_generate_async(self._h, fp, self.batch, n_steps, out_dev_ptr))

    def synchronize(self):
        check(lib().rd_synchronize(self._h))

    def kv_region_bytes(self):
        i = self.info
        es = 2 if i.kv_format == RD_KV_FP16 else 1
        main = i.n_kv_heads * i.max_context * i.head_dim * es   # a paged cache exports this layout too
        if i.kv_format != RD_KV_INT8_SEG128:
            return main, 0, 0
        nseg = (i.max_context + SEG - 1) // SEG
        return main, i.n_kv_heads * SEG * i.head_dim * 2, i.n_kv_heads * nseg * 8

    def export_kv(self, layer: int, which: int, seq: int = 0):
        """Raw cache of (sequence, layer, K=0|V=1): dict of numpy arrays in the ABI layout."""
        i = self.info
        main, st, meta = self.kv_region_bytes()
        buf = np.empty(main + st + meta, np.uint8)
        w = C.c_size_t()
        check(lib().rd_debug_export_kv(self._h, seq, layer, which, buf.ctypes.data, buf.size, C.byref(w)))
        Hk, ctx, hd = i.n_kv_heads, i.max_context, i.head_dim
        if i.kv_format == RD_KV_FP16:
            return {"rows": buf.view(np.uint16).reshape(Hk, ctx, hd)}
        if i.kv_format == RD_KV_FP8_E5M2:
            return {"rows": buf.reshape(Hk, ctx, hd)}
        nseg = (ctx + SEG - 1) // SEG
        return {"rows": buf[:main].reshape(Hk, ctx, hd),
                "stage": buf[main:main + st].view(np.uint16).reshape(Hk, SEG, hd),
                "meta": buf[main + st:].view(np.float32).reshape(Hk, nseg, 2)}

    def import_kv(self, layer: int, which: int, parts: dict, pos: int, seq: int = 0):
        i = self.info
        if i.kv_format == RD_KV_INT8_SEG128:
            raw = np.concatenate([np.ascontiguousarray(parts["rows"]).view(np.uint8).reshape(-1),
                                  np.ascontiguousarray(parts["stage"]).view(np.uint8).reshape(-1),
                                  np.ascontiguousarray(parts["meta"]).view(np.uint8).reshape(-1)])
        else:
            raw = np.ascontiguousarray(parts["rows"]).view(np.uint8).reshape(-1)
        check(lib().rd_debug_import_kv(self._h, seq, layer, which, raw.ctypes.data, raw.size, pos))


# ---- standalone kernels (device pointers as ints) -------------------------------------

def rd_gemv_f16(W: int, x: int, y: int, N: int, K: int, batch: int = 1, stream: int = 0):
    check(lib().rd_gemv_f16(W, x, y, N, K, batch, stream or None))


def rd_attention_f16(q: int, K: int, V: int, out: int, n_heads: int, n_kv_heads: int, hd: int, L: int, ld: int,
                     scale: float, splits: int, stream: int = 0):
    check(lib().rd_attention_f16(q, K, V, out, n_heads, n_kv_heads, hd, L, ld, scale, splits, stream or None))


def rd_attention(q: int, K: int, V: int, out: int, n_heads: int, n_kv_heads: int, hd: int, L: int, ld: int,
                 kv_format: str, scale: float, splits: int, k_stage: int = 0, v_stage: int = 0, k_meta: int = 0,
                 v_meta: int = 0, stream: int = 0):
    check(lib().rd_attention(q, K, V, k_stage or None, v_stage or None, k_meta or None, v_meta or None, out, n_heads,
                             n_kv_heads, hd, L, ld, KV_FORMATS[kv_format], scale, splits, stream or None))


def rd_attention_noalloc(q: int, K: int, V: int, out: int, n_heads: int, n_kv_heads: int, hd: int, L: int,
                         ld: int, kv_format: str, scale: float, splits: int, k_stage: int = 0, v_stage: int = 0,
                         k_meta: int = 0, v_meta: int = 0, stream: int = 0):
    check(lib().rd_attention_noalloc(q, K, V, k_stage or None, v_stage or None, k_meta or None, v_meta or None, out,
                                     n_heads, n_kv_heads, hd, L, ld, KV_FORMATS[kv_format], scale, splits,
                                     stream or None))


def rd_q4_quantize(W: int, N: int, K: int, codes: int, scales: int, stream: int = 0):
    check(lib().rd_q4_quantize(W, N, K, codes, scales, stream or None))


def rd_gemv_q4(codes: int, scales: int, x: int, y: int, N: int, K: int, stream: int = 0):
    check(lib().rd_gemv_q4(codes, scales, x, y, N, K, stream or None))


def rd_e5m2_encode(inp: int, out: int, n: int, stream: int = 0):
    check(lib().rd_e5m2_encode(inp, out, n, stream or None))


def rd_delta_seal(inp: int, n_seg: int, n: int, hd: int, anchor: int, codes: int, meta: int, stream: int = 0):
    check(lib().rd_delta_seal(inp, n_seg, n, hd, anchor, codes or None, meta, stream or None))


def rd_delta_restore(anchor: int, codes: int, meta: int, n_seg: int, n: int, hd: int, out: int, stream: int = 0):
    check(lib().rd_delta_restore(anchor, codes or None, meta, n_seg, n, hd, out, stream or None))


def rd_seg_quant(inp: int, n_seg: int, seg_elems: int, codes: int, meta: int, stream: int = 0):
    check(lib().rd_seg_quant(inp, n_seg, seg_elems, codes, meta, stream or None))


def rd_argmax_f32(v: int, n: int, out: int, stream: int = 0):
    check(lib().rd_argmax_f32(v, n, out, stream or None))


def release_scratch():
    check(lib().rd_release_scratch())
