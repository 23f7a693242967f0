"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side tests.

This module holds no arithmetic of the decode method.  It only draws random
numbers and lays them out in the weight-blob container format, so that the
CPU oracle and the HIP library can be fed byte-identical inputs.

Weight blob ("RDW1", little-endian), the container both sides parse on their
own:

    offset  size  field
    0       4     magic b"RDW1"
    4       4     u32 version = 1
    8       4     u32 header_bytes = 256
    12      4     u32 dtype = 1 (IEEE binary16 tensors)
    16      4     i32 n_layers
    20      4     i32 d_model
    24      4     i32 n_heads
    28      4     i32 n_kv_heads
    32      4     i32 head_dim
    36      4     i32 d_ff
    40      4     i32 vocab
    44      4     f32 rope_base
    48      4     f32 norm_eps
    52      4     u32 flags = 0
    56..255       zero

then fp16 row-major tensors [out, in], each starting on a 256-byte boundary:
embed[V,D]; per layer: attn_norm[D], wq[H*hd,D], wk[Hk*hd,D], wv[Hk*hd,D],
wo[D,H*hd], ffn_norm[D], w_gate[F,D], w_up[F,D], w_down[D,F]; then
final_norm[D], lm_head[V,D].  The blob ends right after lm_head.

Workloads (the shapes of the decode configurations):
  * tiny: 1 layer, d_model 256, 4 heads x 64 (MHA), SwiGLU 1024, vocab 4096;
  * 2b:   24 layers, d_model 2048, 16 q-heads x 128, 8 KV heads, SwiGLU 5632,
          vocab 32000, untied LM head.
Linear and embedding weights are N(0, 0.02) rounded to fp16; RMSNorm gains
are 1.0.  Prompts are uniform token ids.
"""
from __future__ import annotations

import dataclasses
import os
import struct
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MAGIC = b"RDW1"
HEADER_BYTES = 256
ALIGN = 256


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    rope_base: float = 10000.0
    norm_eps: float = 1e-6


SHAPES = {
    "tiny": ModelShape(1, 256, 4, 4, 64, 1024, 4096),
    "2b": ModelShape(24, 2048, 16, 8, 128, 5632, 32000),
}


def tensor_list(s: ModelShape):
    """(name, shape, is_norm_gain) in blob order."""
    D, H, Hk, hd, F, V = s.d_model, s.n_heads, s.n_kv_heads, s.head_dim, s.d_ff, s.vocab
    out = [("embed", (V, D), False)]
    for l in range(s.n_layers):
        out += [
            (f"l{l}.attn_norm", (D,), True),
            (f"l{l}.wq", (H * hd, D), False),
            (f"l{l}.wk", (Hk * hd, D), False),
            (f"l{l}.wv", (Hk * hd, D), False),
            (f"l{l}.wo", (D, H * hd), False),
            (f"l{l}.ffn_norm", (D,), True),
            (f"l{l}.w_gate", (F, D), False),
            (f"l{l}.w_up", (F, D), False),
            (f"l{l}.w_down", (D, F), False),
        ]
    out += [("final_norm", (D,), True), ("lm_head", (V, D), False)]
    return out


def blob_layout(s: ModelShape):
    """List of (name, shape, is_gain, byte_offset) and the total blob size."""
    off = HEADER_BYTES
    lay = []
    for name, shp, gain in tensor_list(s):
        off = (off + ALIGN - 1) // ALIGN * ALIGN
        lay.append((name, shp, gain, off))
        off += int(np.prod(shp)) * 2
    return lay, off


def header_bytes(s: ModelShape) -> bytes:
    h = struct.pack("<4sIII7iffI", MAGIC, 1, HEADER_BYTES, 1, s.n_layers, s.d_model,
                    s.n_heads, s.n_kv_heads, s.head_dim, s.d_ff, s.vocab,
                    float(s.rope_base), float(s.norm_eps), 0)
    return h + b"\0" * (HEADER_BYTES - len(h))


_CHUNK = 1 << 22


def _fill_normal_f16(dst: np.ndarray, seq: np.random.SeedSequence, std: float, workers: int):
    """dst (flat fp16 view) <- N(0, std) drawn in fixed 4 Mi-element chunks,
    chunk i from child i of `seq`, so the bytes do not depend on `workers`."""
    n = dst.size
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = seq.spawn(nch)

    def one(i):
        a = i * _CHUNK
        b = min(n, a + _CHUNK)
        r = np.random.default_rng(kids[i]).standard_normal(b - a, dtype=np.float32)
        r *= np.float32(std)
        dst[a:b] = r

    if nch == 1 or workers <= 1:
        for i in range(nch):
            one(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(nch)))


def make_blob(s: ModelShape, seed: int, std: float = 0.02, gain: float | np.ndarray | None = None,
              workers: int | None = None) -> np.ndarray:
    """The weight blob as a uint8 array.  Tensor t (blob order) draws from
    child t of SeedSequence(seed).  `gain` overrides the RMSNorm gains (1.0)."""
    lay, total = blob_layout(s)
    buf = np.zeros(total, dtype=np.uint8)
    buf[:HEADER_BYTES] = np.frombuffer(header_bytes(s), dtype=np.uint8)
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    kids = np.random.SeedSequence(seed).spawn(len(lay))
    for (name, shp, is_gain, off), kid in zip(lay, kids):
        n = int(np.prod(shp))
        view = buf[off:off + 2 * n].view(np.float16)
        if is_gain:
            view[:] = np.float16(1.0) if gain is None else np.asarray(gain, dtype=np.float16)
        else:
            _fill_normal_f16(view, kid, std, workers)
    return buf


def tensor_view(blob: np.ndarray, s: ModelShape, name: str) -> np.ndarray:
    """fp16 view of one tensor of a blob (no copy)."""
    lay, _ = blob_layout(s)
    for n, shp, _, off in lay:
        if n == name:
            return blob[off:off + 2 * int(np.prod(shp))].view(np.float16).reshape(shp)
    raise KeyError(name)


def prompt(seed: int, n: int, vocab: int) -> np.ndarray:
    """n token ids uniform in [0, vocab)."""
    return np.random.default_rng(seed).integers(0, vocab, n).astype(np.int32)


def prompts(seed: int, n: int, vocab: int, batch: int) -> np.ndarray:
    """[batch, n] token ids from one generator (row b = the b-th draw)."""
    g = np.random.default_rng(seed)
    return np.stack([g.integers(0, vocab, n) for _ in range(batch)]).astype(np.int32)


def normal_f16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    g = np.random.default_rng(seed)
    return (g.standard_normal(int(np.prod(shape)), dtype=np.float32) * np.float32(std)).astype(
        np.float16).reshape(shape)


def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    g = np.random.default_rng(seed)
    return (g.standard_normal(int(np.prod(shape)), dtype=np.float64) * std).astype(np.float32).reshape(shape)


def gemv_inputs(N: int, K: int, batch: int = 1, seed_w: int = 2, seed_x: int = 3):
    """GEMV microbench operands: W [N,K] fp16 ~N(0,0.02), X [batch,K] fp16 ~N(0,1)."""
    W = np.empty((N, K), dtype=np.float16)
    _fill_normal_f16(W.reshape(-1), np.random.SeedSequence(seed_w), 0.02,
                     min(16, len(os.sched_getaffinity(0))))
    X = normal_f16(seed_x, (batch, K))
    return W, X
