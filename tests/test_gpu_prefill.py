"""GPU parity of the batched prefill (rd_prefill_batched) against the oracle.

The batched prefill computes, for every prompt position, what the decode
step computes there (the position's K/V rows; its attention over positions
0..p as stored), with the layer products as matrix products on the matrix
cores.  So its cache rows must agree with the oracle's (orc_prefill, pinned
bit-identical to single decode steps) within rounding, and the decode step
that follows must pass the per-step rule.

Row tolerances: layer 0's rows depend on the token alone and carry only the
fp16 operand rounding (2e-3 absolute and relative, as for the decode step's
rows); deeper rows carry the roundings of every layer before them and are
held to the per-logit rule's 2e-2 + 1e-2 |x|.  E5M2 values add one step of
the format, INT8 sealed values one quantization step of either side's
segment (each side's codes come from its own fp16 rows).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

ATOL, RTOL, MARGIN = 2e-2, 1e-2, 5e-2
GQA2 = synth.ModelShape(n_layers=2, d_model=512, n_heads=8, n_kv_heads=2, head_dim=64, d_ff=1408, vocab=1000)
HK8 = synth.ModelShape(n_layers=2, d_model=512, n_heads=8, n_kv_heads=8, head_dim=64, d_ff=1024, vocab=2048)


@pytest.fixture(scope="module")
def rd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import request_decode_amd as rd
    rd.lib()
    return rd


def compare_step(g_logits, o_logits, g_next, tag):
    o = o_logits.astype(np.float64)
    g = g_logits.astype(np.float64)
    err = np.abs(g - o)
    assert np.all(err <= ATOL + RTOL * np.abs(o)), (tag, float(err.max()), int(np.argmax(err)))
    top2 = np.sort(o)[-2:]
    if top2[1] - top2[0] > MARGIN:
        assert g_next == int(np.argmax(o)), tag
    return float(err.max())


def e5m2_step(a):
    a = np.abs(a)
    return np.where(a < 2.0 ** -14, 2.0 ** -16, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 2))


def gpu_rows(orc, gm, kv, layer, which, n):
    """The GPU's rows 0..n-1 of (layer, K/V) as attended values [Hk][n][hd],
    plus for INT8 the quantization step of each row's segment."""
    parts = gm.export_kv(layer, which)
    step = None
    if kv == "fp16":
        vals = parts["rows"][:, :n].view(np.float16).astype(np.float64)
    elif kv == "e5m2":
        vals = orc.h2d(orc.h_from_e5m2(parts["rows"][:, :n]))
    else:
        Hk, _, hd = parts["rows"].shape
        vals = np.empty((Hk, n, hd))
        step = np.zeros((Hk, n, 1))
        open0 = n // 128 * 128
        for g in range(Hk):
            for s in range(open0 // 128):
                sc, zp = parts["meta"][g, s]
                vals[g, s * 128:(s + 1) * 128] = orc.seg_dequant(parts["rows"][g, s * 128:(s + 1) * 128], sc, zp)
                step[g, s * 128:(s + 1) * 128] = sc
            for p in range(open0, n):
                vals[g, p] = parts["stage"][g, p % 128].view(np.float16).astype(np.float64)
    return vals, step


def oracle_rows(orc, om, kv, layer, which, n, Hk):
    out = np.empty((Hk, n, om.head_dim))
    step = np.zeros((Hk, n, 1)) if kv == "int8" else None
    for g in range(Hk):
        for p in range(n):
            out[g, p] = om.read_row(layer, which, g, p)
        if kv == "int8":
            for s in range(n // 128):
                step[g, s * 128:(s + 1) * 128] = om.seg_meta(layer, which, g, s)[0]
    return out, step


def check_cache(orc, gm, om, shape, kv, n, tag, layers=None):
    worst = 0.0
    for l in (range(shape.n_layers) if layers is None else layers):
        for w in (0, 1):
            g, gs = gpu_rows(orc, gm, kv, l, w, n)
            o, os_ = oracle_rows(orc, om, kv, l, w, n, shape.n_kv_heads)
            tol = (2e-3 + 2e-3 * np.abs(o)) if l == 0 else (ATOL + RTOL * np.abs(o))
            if kv == "e5m2":
                tol = tol + e5m2_step(np.maximum(np.abs(g), np.abs(o)))
            elif kv == "int8":
                tol = tol + np.maximum(gs, os_)
            err = np.abs(g - o)
            bad = err > tol
            assert not bad.any(), (tag, l, w, np.argwhere(bad)[:3].tolist(), float(err.max()))
            worst = max(worst, float(err.max()))
    return worst


# (start, n, model): the 2500-token prompt (two chunks of 2048) on the tiny
# model only, the shorter ones on every small model
PREFILL_CASES = [(s0, n, m) for s0, n in ((0, 1), (0, 37), (0, 300), (50, 200)) for m in ("tiny", "gqa2", "hk8")]
PREFILL_CASES += [(0, 2500, "tiny")]


@pytest.mark.parametrize("kv", ["fp16", "e5m2", "int8"])
@pytest.mark.parametrize("start,n,shape_name", PREFILL_CASES)
def test_prefill_small_models(rd, orc, shape_name, kv, start, n):
    """Small models: prompts of 1 to 2500 tokens (two chunks of 2048),
    from position 0 or after 50 single decode steps (the chunk starts inside
    a segment and inside a 64-position attention block), every cache row
    against the oracle's, then 3 decode steps teacher-forced."""
    shape = {"tiny": synth.SHAPES["tiny"], "gqa2": GQA2, "hk8": HK8}[shape_name]
    print(f"prefill {shape_name} {kv} start={start} n={n}", flush=True)
    blob = synth.make_blob(shape, seed=21)
    toks = synth.prompt(22, start + n + 3, shape.vocab)
    ctx = start + n + 8
    gm = rd.Model(blob, max_context=ctx, kv_format=kv, executor="graph")
    om = orc.OracleModel(blob, ctx, kv_format=kv)
    for t in toks[:start]:
        gm.decode_step(int(t), want_logits=False)
        om.step([t])
    gm.prefill_batched(toks[start:start + n])
    om.prefill(toks[start:start + n])
    assert gm.position() == om.pos() == start + n
    worst_row = check_cache(orc, gm, om, shape, kv, start + n, (shape_name, kv, start, n))
    worst = 0.0
    for t in toks[start + n:]:
        gl, gn = gm.decode_step(int(t))
        ol, on = om.step([t])
        worst = max(worst, compare_step(gl, ol[0], gn, (shape_name, kv, start, n)))
    print(f"  rows max|d| {worst_row:.3e}, next steps max|dlogit| {worst:.3e}")
    gm.close()
    om.close()


@pytest.fixture(scope="module")
def blob2b():
    return synth.make_blob(synth.SHAPES["2b"], seed=2)


# the 2B-class model's widths (head_dim 128, two query heads per kv head)
# with two layers
WIDE2 = synth.ModelShape(n_layers=2, d_model=2048, n_heads=16, n_kv_heads=8, head_dim=128, d_ff=5632, vocab=32000)


def check_e5m2_against_record(orc, gm, blob, shape, toks, n, tag):
    """E5M2 prefill, every layer: the oracle is given the GPU's stored bytes
    of every position, runs its own prefill over them storing nothing and
    recording the rows it computes (orc_record_rows); the GPU's row of every
    layer and position must be within the row tolerance of that record plus
    one E5M2 step.  Returns the oracle, positioned after the prompt, holding
    the GPU's cache."""
    om = orc.OracleModel(blob, n + 8, kv_format="e5m2")
    for l in range(shape.n_layers):
        for w in (0, 1):
            rows = gm.export_kv(l, w)["rows"]
            for g in range(shape.n_kv_heads):
                om.set_rows(l, w, g, 0, rows[g, :n])
    om.set_store(False)
    om.record_rows(True)
    om.prefill(toks[:n])
    worst = 0.0
    for l in range(shape.n_layers):
        for w in (0, 1):
            got = orc.h2d(orc.h_from_e5m2(gm.export_kv(l, w)["rows"][:, :n]))
            ref = np.stack([om.computed_rows(l, w, g, 0, n) for g in range(shape.n_kv_heads)])
            tol = (2e-3 + 2e-3 * np.abs(ref)) if l == 0 else (ATOL + RTOL * np.abs(ref))
            tol = tol + e5m2_step(np.maximum(np.abs(got), np.abs(ref)))
            err = np.abs(got - ref)
            assert np.all(err <= tol), (tag, l, w, np.argwhere(err > tol)[:3].tolist(), float(err.max()))
            worst = max(worst, float(err.max()))
    om.record_rows(False)
    return om, worst


@pytest.mark.parametrize("kv", ["e5m2", "int8"])
def test_prefill_8bit_2b_widths_vs_oracle(rd, orc, kv):
    """The 8-bit caches at the 2B-class widths (head_dim 128, G = 2), two
    layers, 300 tokens (two INT8 seals): every row of both layers against
    the oracle's prefill, then 3 decode steps."""
    print(f"prefill wide2 {kv}", flush=True)
    blob = synth.make_blob(WIDE2, seed=23)
    n = 300
    toks = synth.prompt(24, n + 3, WIDE2.vocab)
    gm = rd.Model(blob, max_context=n + 8, kv_format=kv, executor="graph")
    om = orc.OracleModel(blob, n + 8, kv_format=kv)
    gm.prefill_batched(toks[:n])
    if kv == "e5m2":
        om.close()
        om, worst_row = check_e5m2_against_record(orc, gm, blob, WIDE2, toks, n, ("wide2", kv))
    else:
        om.prefill(toks[:n])
        worst_row = check_cache(orc, gm, om, WIDE2, kv, n, ("wide2", kv))
    worst = 0.0
    for t in toks[n:]:
        gl, gn = gm.decode_step(int(t))
        if kv == "e5m2":    # the oracle attends the GPU's rows of this position too (store still off)
            p = gm.position() - 1
            for l in range(WIDE2.n_layers):
                for w in (0, 1):
                    rows = gm.export_kv(l, w)["rows"]
                    for g in range(WIDE2.n_kv_heads):
                        om.set_rows(l, w, g, p, rows[g, p:p + 1])
        ol, on = om.step([t])
        worst = max(worst, compare_step(gl, ol[0], gn, ("wide2", kv)))
    print(f"  rows max|d| {worst_row:.3e}, next steps max|dlogit| {worst:.3e}")
    gm.close()
    om.close()


@pytest.mark.parametrize("kv,n", [("fp16", 300), ("int8", 300), ("e5m2", 140)])
def test_prefill_2b_vs_oracle(rd, orc, blob2b, kv, n):
    """The 2B-class model: a prompt (seed 103) through the batched prefill
    against the oracle; then the next decode step.  fp16: every row of every
    layer against the oracle's prefill.  E5M2: every row of every layer
    against the rows the oracle computes from the GPU's cache
    (check_e5m2_against_record).  INT8: the layer-0 rows (those depend on the
    token alone); below them each side's rows follow from its own quantized
    segments, whose codes differ by whole steps in places, compounded over 24
    layers (the two-layer check above covers the rows themselves).  8-bit
    formats: the oracle is then given the GPU's cache bytes and the next
    step is compared on that cache."""
    shape = synth.SHAPES["2b"]
    print(f"prefill 2b {kv} n={n}", flush=True)
    toks = synth.prompt(103, n + 1, shape.vocab)
    ctx = n + 8
    gm = rd.Model(blob2b, max_context=ctx, kv_format=kv)
    om = orc.OracleModel(blob2b, ctx, kv_format=kv)
    gm.prefill_batched(toks[:n])
    if kv == "e5m2":
        om.close()
        om, worst_row = check_e5m2_against_record(orc, gm, blob2b, shape, toks, n, ("2b", kv, n))
    else:
        om.prefill(toks[:n])
        worst_row = check_cache(orc, gm, om, shape, kv, n, ("2b", kv, n), layers=None if kv == "fp16" else [0])
    if kv != "fp16":
        for l in range(shape.n_layers):
            for w in (0, 1):
                parts = gm.export_kv(l, w)
                for g in range(shape.n_kv_heads):
                    if kv == "e5m2":
                        om.set_rows(l, w, g, 0, parts["rows"][g, :n])
                    else:
                        sealed = n // 128 * 128
                        if sealed:
                            om.set_rows(l, w, g, 0, parts["rows"][g, :sealed])
                            for s in range(sealed // 128):
                                om.seg_meta(l, w, g, s, set_to=parts["meta"][g, s])
                        om.set_rows(l, w, g, sealed, parts["stage"][g, :n - sealed])
    gl, gn = gm.decode_step(int(toks[n]))
    if kv == "e5m2":    # store still off: the oracle attends the GPU's row n too
        for l in range(shape.n_layers):
            for w in (0, 1):
                rows = gm.export_kv(l, w)["rows"]
                for g in range(shape.n_kv_heads):
                    om.set_rows(l, w, g, n, rows[g, n:n + 1])
    ol, on = om.step([toks[n]])
    e = compare_step(gl, ol[0], gn, ("2b", kv, n))
    print(f"  rows max|d| {worst_row:.3e}, next step max|dlogit| {e:.3e}")
    gm.close()
    om.close()


def test_prefill_2b_long_matches_steps(rd, blob2b):
    """A 4608-token prompt (three chunks: at positions 0, 2048 and 4096)
    through the batched prefill and through single decode steps (rd_prefill)
    on the GPU: cache rows of every layer within the row tolerance of each
    other (layer 0: both sides' rounding, twice the decode-row tolerance),
    and the next decode step's logits by the per-step rule."""
    shape = synth.SHAPES["2b"]
    n = 4608
    toks = synth.prompt(104, n + 1, shape.vocab)
    a = rd.Model(blob2b, max_context=n + 4, executor="graph")
    b = rd.Model(blob2b, max_context=n + 4, executor="graph")
    a.prefill_batched(toks[:n])
    b.prefill(toks[:n])
    worst = 0.0
    for l in range(shape.n_layers):
        for w in (0, 1):
            x = a.export_kv(l, w)["rows"][:, :n].view(np.float16).astype(np.float64)
            y = b.export_kv(l, w)["rows"][:, :n].view(np.float16).astype(np.float64)
            err = np.abs(x - y)
            tol = (4e-3 + 4e-3 * np.abs(y)) if l == 0 else (ATOL + RTOL * np.abs(y))
            assert np.all(err <= tol), (l, w, float(err.max()))
            worst = max(worst, float(err.max()))
    la, na = a.decode_step(int(toks[n]))
    lb, nb = b.decode_step(int(toks[n]))
    e = compare_step(la, lb, na, "long")
    print(f"2b 4608 batched vs steps: rows max|d| {worst:.3e}, next step max|dlogit| {e:.3e}")
    a.close()
    b.close()


def test_prefill_errors(rd):
    shape = synth.SHAPES["tiny"]
    blob = synth.make_blob(shape, seed=1)
    m = rd.Model(blob, max_context=16)
    with pytest.raises(rd.RdError) as e:
        m.prefill_batched(np.arange(17) % shape.vocab)
    assert e.value.status == rd.RD_ERR_CONTEXT_FULL and m.position() == 0
    with pytest.raises(rd.RdError) as e:
        m.prefill_batched([1, shape.vocab])
    assert e.value.status == rd.RD_ERR_INVALID_ARG and m.position() == 0
    m.prefill_batched([])
    assert m.position() == 0
    m.close()
    m8 = rd.Model(blob, max_context=16, batch=8)
    with pytest.raises(rd.RdError) as e:
        m8.prefill_batched([1, 2])
    assert e.value.status == rd.RD_ERR_UNSUPPORTED
    m8.close()
