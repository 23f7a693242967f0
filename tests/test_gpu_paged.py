"""GPU tests of the paged KV cache (rd_options.kv_pages > 0) of the batch step.

The paged cache keeps 4 KiB pages of one (layer, K/V, kv head) in a shared
pool, a page table per sequence, refcounts and prefix sharing ("LLM inference
architecture rebuild", §3.2).  Pinned by equivalence: only where a row lives
changes, so a paged model must reproduce the contiguous cache's logits,
tokens and rows bit for bit on the same token streams.  Ragged sequences
(each at its own position, a token of -1 sitting a step out) are compared with
independent oracle models per sequence by the per-step logit rule.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

ATOL, RTOL, MARGIN = 2e-2, 1e-2, 5e-2
GQA2 = synth.ModelShape(n_layers=2, d_model=512, n_heads=8, n_kv_heads=2, head_dim=64, d_ff=1408, vocab=1000)


@pytest.fixture(scope="module")
def rd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import request_decode_amd as rd
    rd.lib()
    return rd


@pytest.fixture(scope="module")
def blob():
    return synth.make_blob(GQA2, seed=31)


def compare_step(g_logits, o_logits, g_next, tag):
    o = o_logits.astype(np.float64)
    err = np.abs(g_logits.astype(np.float64) - o)
    assert np.all(err <= ATOL + RTOL * np.abs(o)), (tag, float(err.max()))
    top2 = np.sort(o)[-2:]
    if top2[1] - top2[0] > MARGIN:
        assert g_next == int(np.argmax(o)), tag
    return float(err.max())


def caches(m, B):
    return [m.export_kv(l, w, seq=b)["rows"].copy() for b in range(B) for l in range(GQA2.n_layers) for w in (0, 1)]


@pytest.mark.parametrize("kv", ["fp16", "e5m2"])
def test_paged_matches_contiguous_lockstep(rd, blob, kv):
    """Three sequences in lockstep: 60 teacher-forced steps and 20 greedy ones
    on a paged and on a contiguous cache give identical logits, tokens and
    rows (exported through the page table)."""
    B, ctx = 3, 200
    toks = synth.prompt(32, 60 * B, GQA2.vocab).reshape(60, B)
    a = rd.Model(blob, max_context=ctx, kv_format=kv, batch=B, executor="graph")
    p = rd.Model(blob, max_context=ctx, kv_format=kv, batch=B, executor="graph", kv_pages=32)
    info = p.get_info()
    assert info.kv_pages == 32 and info.page_rows == 4096 // (GQA2.head_dim * (2 if kv == "fp16" else 1))
    for i in range(60):
        la, na = a.decode_step(toks[i])
        lp, npg = p.decode_step(toks[i])
        assert np.array_equal(la, lp) and np.array_equal(na, npg), i
    ga = a.generate(na, 20)
    gp = p.generate(npg, 20)
    assert np.array_equal(ga, gp)
    assert [p.seq_position(b) for b in range(B)] == [80] * B
    for x, y in zip(caches(a, B), caches(p, B)):
        assert np.array_equal(x, y)
    R = info.page_rows
    free, used, shared = p.page_stats()
    assert used == B * -(-80 // R) and shared == 0 and free == 32 - used
    p.reset()
    assert p.page_stats() == (32, 0, 0)
    a.close()
    p.close()


def test_paged_ragged_vs_oracle(rd, orc, blob):
    """Three sequences at their own positions: prompts of 5, 23 and 47 tokens
    starting at steps 0, 3 and 9, sequence 1 sitting out steps 12..16 in the
    middle, then every sequence decodes its own greedy tokens.  Each
    sequence's logits at each of its steps against an oracle model fed only
    that sequence's tokens."""
    B, ctx = 3, 128
    lens, starts = [5, 23, 47], [0, 3, 9]
    prompts = [synth.prompt(40 + b, lens[b], GQA2.vocab) for b in range(B)]
    oms = [orc.OracleModel(blob, ctx) for _ in range(B)]
    p = rd.Model(blob, max_context=ctx, batch=B, executor="graph", kv_pages=24)
    fed = [0] * B           # prompt tokens consumed
    nxt = [None] * B        # greedy token once the prompt is done
    gen = [0] * B
    for i in range(70):
        t = np.full(B, -1, np.int32)
        for b in range(B):
            if i < starts[b] or (b == 1 and 12 <= i < 17) or gen[b] >= 12:
                continue
            t[b] = prompts[b][fed[b]] if fed[b] < lens[b] else nxt[b]
        if (t == -1).all():
            break
        lg, nx = p.decode_step(t)
        for b in range(B):
            if t[b] == -1:
                assert nx[b] == -1
                continue
            ol, on = oms[b].step([int(t[b])])
            compare_step(lg[b], ol[0], int(nx[b]), (b, i))
            if fed[b] < lens[b]:
                fed[b] += 1
            else:
                gen[b] += 1
            nxt[b] = int(nx[b])
    assert fed == lens and all(g == 12 for g in gen)
    assert [p.seq_position(b) for b in range(B)] == [lens[b] + 12 for b in range(B)]
    for om in oms:
        om.close()
    p.close()


def test_paged_prefix_sharing(rd, blob):
    """Sequence 0 takes a 37-token prompt while the others sit out; it is
    forked into sequences 1 and 2 (the prompt's pages shared, refcount 3);
    then the three continue with different tokens.  Their logits equal a
    contiguous cache fed [prompt, own continuation] in lockstep, and the
    pages are counted once: the shared partial page is copied on write by the
    first two writers, the third keeps it."""
    B, ctx, P, N = 3, 128, 37, 10
    prompt = synth.prompt(50, P, GQA2.vocab)
    cont = synth.prompt(51, N * B, GQA2.vocab).reshape(N, B)
    p = rd.Model(blob, max_context=ctx, batch=B, executor="graph", kv_pages=16)
    R = p.get_info().page_rows
    steps = np.full((P, B), -1, np.int32)
    steps[:, 0] = prompt
    p.prefill(steps)
    assert [p.seq_position(b) for b in range(B)] == [P, 0, 0]
    p.seq_fork(0, 1)
    p.seq_fork(0, 2)
    npg = -(-P // R)
    assert p.page_stats() == (16 - npg, npg, npg)
    a = rd.Model(blob, max_context=ctx, batch=B, executor="graph")
    a.prefill(np.repeat(prompt[:, None], B, axis=1))
    for i in range(N):
        la, na = a.decode_step(cont[i])
        lp, npp = p.decode_step(cont[i])
        assert np.array_equal(la, lp) and np.array_equal(na, npp), i
    # P = 37 and N = 10 stay inside the prompt's last page when R >= 48; with
    # R = 32 the rows 37..46 fall in page 1: its owner count was 3, so two
    # copies are made and the third writer keeps it
    last = (P - 1) // R
    grows = -(-(P + N) // R) - npg   # new pages per sequence past the shared ones
    copies = 2 if (P % R) else 0
    exp_used = npg + copies + B * grows
    free, used, shared = p.page_stats()
    assert used == exp_used and free == 16 - exp_used and shared == (last if P % R else npg), (free, used, shared)
    a.close()
    p.close()


def test_paged_pool_exhausted(rd, blob):
    """A pool of 3 page groups: when a step needs a 4th, OUT_OF_MEMORY with
    nothing changed; after a sequence is reset its pages serve the step."""
    B, ctx = 2, 256
    p = rd.Model(blob, max_context=ctx, batch=B, executor="graph", kv_pages=3)
    R = p.get_info().page_rows
    t = synth.prompt(60, 3 * R, GQA2.vocab)
    steps = np.full((2 * R, B), -1, np.int32)
    steps[:, 0] = t[:2 * R]
    steps[:R, 1] = t[2 * R:]
    p.prefill(steps)
    assert p.page_stats() == (0, 3, 0)
    with pytest.raises(rd.RdError) as e:
        p.decode_step(np.array([int(t[0]), -1], np.int32))
    assert e.value.status == rd.RD_ERR_OUT_OF_MEMORY
    assert [p.seq_position(0), p.seq_position(1)] == [2 * R, R]
    p.seq_reset(1)
    assert p.page_stats() == (1, 2, 0)
    p.decode_step(np.array([int(t[0]), -1], np.int32))
    assert p.seq_position(0) == 2 * R + 1 and p.page_stats() == (0, 3, 0)
    p.close()


def test_paged_2b_shape_matches_contiguous(rd):
    """The 2B-class shape (head_dim 128: 16 fp16 positions per page, two
    query heads per kv head), two sequences in lockstep over 40 prompt steps
    (three page boundaries) and 24 greedy steps: paged and contiguous give
    identical logits, tokens and rows."""
    shape = synth.SHAPES["2b"]
    blob = synth.make_blob(shape, seed=2)
    B, ctx = 2, 80
    toks = synth.prompts(106, 40, shape.vocab, B)          # [B][40]
    a = rd.Model(blob, max_context=ctx, batch=B, executor="graph")
    p = rd.Model(blob, max_context=ctx, batch=B, executor="graph", kv_pages=B * 5)
    assert p.get_info().page_rows == 16
    for i in range(40):
        la, na = a.decode_step(toks[:, i])
        lp, npg = p.decode_step(toks[:, i])
        assert np.array_equal(la, lp) and np.array_equal(na, npg), i
    assert np.array_equal(a.generate(na, 24), p.generate(npg, 24))
    for b in range(B):
        for l in (0, shape.n_layers - 1):
            for w in (0, 1):
                assert np.array_equal(a.export_kv(l, w, seq=b)["rows"], p.export_kv(l, w, seq=b)["rows"])
    assert p.page_stats() == (B * 5 - B * 4, B * 4, 0)
    a.close()
    p.close()
