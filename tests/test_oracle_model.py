"""Pins of the oracle's whole decode step.

The decode-with-cache step must reproduce, position by position, a full
causal forward pass over the whole prefix (the KV-cache identity).  The full
forward comes from a library routine: Hugging Face Transformers'
LlamaForCausalLM in float64 on the CPU, which uses the same block (RMSNorm,
half-split RoPE, grouped-query attention with consecutive query groups,
SwiGLU, untied LM head).  Its rotary angles are computed in binary32, which
bounds the agreement at about 1e-6.
"""
import numpy as np
import pytest
import torch

import synth


def hf_logits(blob, shape, tokens):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.d_model, intermediate_size=shape.d_ff,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=float(np.float32(shape.norm_eps)), rope_theta=shape.rope_base,
                      max_position_embeddings=4096, tie_word_embeddings=False, attention_bias=False,
                      mlp_bias=False, hidden_act="silu")
    torch.manual_seed(0)
    model = LlamaForCausalLM(cfg).to(torch.float64).eval()
    model.config._attn_implementation = "eager"

    def t(name):
        return torch.from_numpy(synth.tensor_view(blob, shape, name).astype(np.float64))

    sd = {"model.embed_tokens.weight": t("embed"), "model.norm.weight": t("final_norm"),
          "lm_head.weight": t("lm_head")}
    for l in range(shape.n_layers):
        p = f"model.layers.{l}."
        sd.update({p + "input_layernorm.weight": t(f"l{l}.attn_norm"),
                   p + "self_attn.q_proj.weight": t(f"l{l}.wq"),
                   p + "self_attn.k_proj.weight": t(f"l{l}.wk"),
                   p + "self_attn.v_proj.weight": t(f"l{l}.wv"),
                   p + "self_attn.o_proj.weight": t(f"l{l}.wo"),
                   p + "post_attention_layernorm.weight": t(f"l{l}.ffn_norm"),
                   p + "mlp.gate_proj.weight": t(f"l{l}.w_gate"),
                   p + "mlp.up_proj.weight": t(f"l{l}.w_up"),
                   p + "mlp.down_proj.weight": t(f"l{l}.w_down")})
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in m for m in missing), (missing, unexpected)
    with torch.no_grad():
        out = model(torch.from_numpy(np.asarray(tokens, np.int64))[None], use_cache=False)
    return out.logits[0].numpy()


SMALL_GQA = synth.ModelShape(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, d_ff=256, vocab=512)


@pytest.mark.parametrize("name,shape,gain", [("tiny", synth.SHAPES["tiny"], None),
                                             ("gqa2", SMALL_GQA, None),
                                             ("gqa2-gains", SMALL_GQA, "random")])
def test_step_matches_full_causal_forward(orc, name, shape, gain):
    g = None
    if gain == "random":
        g = np.random.default_rng(9).uniform(0.5, 1.5, shape.d_model).astype(np.float16)
    blob = synth.make_blob(shape, seed=1, gain=g)
    tokens = synth.prompt(101, 40, shape.vocab)
    ref = hf_logits(blob, shape, tokens)
    m = orc.OracleModel(blob, max_ctx=64, kv_format="exact")
    got = np.stack([m.step([t])[0][0] for t in tokens])
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= 2e-6 * scale, (name, err, scale)


def test_fp16_cache_close_to_exact(orc):
    shape = synth.SHAPES["tiny"]
    blob = synth.make_blob(shape, seed=1)
    toks = synth.prompt(101, 48, shape.vocab)
    a = orc.OracleModel(blob, 64, kv_format="exact")
    b = orc.OracleModel(blob, 64, kv_format="fp16")
    la = np.stack([a.step([t])[0][0] for t in toks])
    lb = np.stack([b.step([t])[0][0] for t in toks])
    d = np.abs(la - lb).max()
    assert 0 < d < 5e-3
    # the fp16 cache holds exactly the binary16 rounding of the exact rows
    for p in (0, 17, 47):
        ek = a.get_rows(0, 0, 1, p, 1)[0]
        hk = b.get_rows(0, 0, 1, p, 1)[0]
        assert np.array_equal(hk, orc.d2h(ek))


def test_layer0_kv_matches_cache(orc):
    shape = SMALL_GQA
    blob = synth.make_blob(shape, seed=3)
    toks = synth.prompt(5, 20, shape.vocab)
    m = orc.OracleModel(blob, 32, kv_format="exact")
    for t in toks:
        m.step([t])
    for p in (0, 9, 19):
        k, v = m.layer0_kv(int(toks[p]), p)
        for g in range(shape.n_kv_heads):
            assert np.array_equal(m.get_rows(0, 0, g, p, 1)[0], k[g])
            assert np.array_equal(m.get_rows(0, 1, g, p, 1)[0], v[g])


def test_quantized_caches(orc):
    """E5M2 and INT8 caches store the quantization of the fp16 rows the fp16
    cache stores, and attention reads their dequantized values."""
    shape = synth.ModelShape(1, 128, 2, 2, 64, 256, 256)
    blob = synth.make_blob(shape, seed=4)
    toks = synth.prompt(6, 300, shape.vocab)
    ref = orc.OracleModel(blob, 320, kv_format="fp16")
    e5 = orc.OracleModel(blob, 320, kv_format="e5m2")
    i8 = orc.OracleModel(blob, 320, kv_format="int8")
    for t in toks[:128]:
        ref.step([t]); e5.step([t]); i8.step([t])
    # position 128 reached: segment 0 is sealed in the INT8 cache
    for which in (0, 1):
        for g in range(2):
            # identical prefix tokens give identical fp16 rows only while the caches agree,
            # which holds for the first row (the first step attends to itself only)
            h = ref.get_rows(0, which, g, 0, 1)
            assert np.array_equal(e5.get_rows(0, which, g, 0, 1), orc.e5m2_from_h(h))
            codes = i8.get_rows(0, which, g, 0, 128)
            scale, zp = i8.seg_meta(0, which, g, 0)
            assert codes.dtype == np.uint8
            deq = i8.read_row(0, which, g, 5)
            assert np.array_equal(deq, ((codes[5].astype(np.float32) - zp) * scale).astype(np.float64))
    for t in toks[128:]:
        ref.step([t]); e5.step([t]); i8.step([t])
    assert ref.pos() == e5.pos() == i8.pos() == 300


# ---- in-model KV formats: every row of the cache against an independent path ----------

# head_dim 64 and 128, two kv heads, two layers (the seal runs for every layer)
SEAL64 = synth.ModelShape(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=64, d_ff=256, vocab=512)
SEAL128 = synth.ModelShape(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128, d_ff=256, vocab=512)


@pytest.mark.parametrize("shape", [SEAL64, SEAL128], ids=["hd64", "hd128"])
def test_int8_seal_codes_in_model(orc, shape):
    """The INT8 cache after 256 steps holds two sealed segments per (layer,
    K/V, kv head).  Each one's codes and fp32 (scale, zero point) must be the
    segment quantizer of exactly the 128 x head_dim binary16 rows that segment
    held ("Grok-3 v3.2.4 hot update deep dive", section 3.2):
      * layer 0, both segments: the rows from orc_layer0_kv, which depend on
        (token, position) alone (an independent path to the same rows);
      * every layer, segment 0: the rows of an fp16-cache run on the same
        tokens (until the first seal both runs attend to the same binary16
        rows, so their caches agree bit for bit);
      * every layer, segment 1: the staging rows the run itself held, read
        back by rewinding into that segment.
    A wrong lane, head or segment offset in the seal, or a per-row seal,
    fails one of the three."""
    blob = synth.make_blob(shape, seed=11)
    toks = synth.prompt(12, 256, shape.vocab)
    i8 = orc.OracleModel(blob, 300, kv_format="int8")
    f16 = orc.OracleModel(blob, 300, kv_format="fp16")
    for t in toks[:128]:
        i8.step([t])
        f16.step([t])
    for t in toks[128:]:
        i8.step([t])
    assert i8.pos() == 256
    Hk = shape.n_kv_heads
    sealed = {}
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(Hk):
                for seg in (0, 1):
                    codes = i8.get_rows(l, w, g, seg * 128, 128)
                    assert codes.dtype == np.uint8
                    sealed[l, w, g, seg] = (codes, i8.seg_meta(l, w, g, seg))
    # layer 0 against orc_layer0_kv
    k0 = np.empty((256, Hk, shape.head_dim))
    v0 = np.empty((256, Hk, shape.head_dim))
    for p in range(256):
        k0[p], v0[p] = i8.layer0_kv(int(toks[p]), p)
    for w, rows in ((0, k0), (1, v0)):
        for g in range(Hk):
            for seg in (0, 1):
                h = orc.d2h(rows[seg * 128:(seg + 1) * 128, g])
                codes, scale, zp = orc.seg_quant(h)
                got, (gs, gz) = sealed[0, w, g, seg]
                assert np.array_equal(got, codes) and gs == scale and gz == zp, (w, g, seg)
    # every layer, segment 0, against the fp16-cache run
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(Hk):
                codes, scale, zp = orc.seg_quant(f16.get_rows(l, w, g, 0, 128))
                got, (gs, gz) = sealed[l, w, g, 0]
                assert np.array_equal(got, codes) and gs == scale and gz == zp, (l, w, g)
    # every layer, segment 1, against its own staging rows (rewound into segment 1)
    i8.set_pos(255)
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(Hk):
                st = i8.get_rows(l, w, g, 128, 128)
                assert st.dtype == np.uint16
                codes, scale, zp = orc.seg_quant(st)
                got, (gs, gz) = sealed[l, w, g, 1]
                assert np.array_equal(got, codes) and gs == scale and gz == zp, (l, w, g)
    # the attention reads a sealed row as (code - zp) * scale
    i8.set_pos(256)
    codes, (scale, zp) = sealed[1, 1, 1, 0]
    assert np.array_equal(i8.read_row(1, 1, 1, 77),
                          ((codes[77].astype(np.float32) - zp) * scale).astype(np.float64))


def test_quantized_rows_layer0_every_position(orc):
    """Every layer-0 row of the E5M2 cache is the E5M2 encoding of the
    binary16 rounding of orc_layer0_kv; every row of the INT8 cache's open
    segment is that binary16 value (staging), for all positions and heads."""
    shape = SEAL64
    blob = synth.make_blob(shape, seed=13)
    toks = synth.prompt(14, 200, shape.vocab)
    e5 = orc.OracleModel(blob, 256, kv_format="e5m2")
    i8 = orc.OracleModel(blob, 256, kv_format="int8")
    for t in toks:
        e5.step([t])
        i8.step([t])
    for p in range(200):
        k, v = e5.layer0_kv(int(toks[p]), p)
        for w, rows in ((0, k), (1, v)):
            for g in range(shape.n_kv_heads):
                h = orc.d2h(rows[g])
                assert np.array_equal(e5.get_rows(0, w, g, p, 1)[0], orc.e5m2_from_h(h)), (p, w, g)
                if p >= 128:
                    assert np.array_equal(i8.get_rows(0, w, g, p, 1)[0], h), (p, w, g)
                    assert np.array_equal(i8.read_row(0, w, g, p), orc.h2d(h))
                else:
                    assert np.array_equal(e5.read_row(0, w, g, p), orc.h2d(orc.h_from_e5m2(orc.e5m2_from_h(h))))


@pytest.mark.parametrize("kv,n", [("fp16", 40), ("e5m2", 40), ("int8", 140)])
def test_batch_step_equals_independent_sequences(orc, kv, n):
    """The batch-B step is B independent sequences: its logits and argmax are
    bit-identical to B batch-1 models fed the same token streams (int8: the
    streams cross a segment seal)."""
    shape = SEAL64
    blob = synth.make_blob(shape, seed=15)
    B = 3
    streams = synth.prompts(16, n, shape.vocab, B)
    mb = orc.OracleModel(blob, n + 4, batch=B, kv_format=kv)
    singles = [orc.OracleModel(blob, n + 4, kv_format=kv) for _ in range(B)]
    for i in range(n):
        lb, nb = mb.step(streams[:, i])
        for b in range(B):
            ls, ns = singles[b].step([streams[b, i]])
            assert np.array_equal(lb[b], ls[0]) and nb[b] == ns[0], (kv, i, b)
    for b in range(B):
        assert mb.pos(b) == n
        for w in (0, 1):
            got = mb.get_rows(1, w, 1, 0, n // 128 * 128 or n, b=b)
            ref = singles[b].get_rows(1, w, 1, 0, n // 128 * 128 or n)
            assert np.array_equal(got, ref)


@pytest.mark.parametrize("kv", ["fp16", "e5m2", "int8"])
def test_store_off_step_is_the_same_step(orc, kv):
    """With its store switched off, a step whose position already holds the
    rows the step would store gives bit-identical logits and argmax; it
    stores nothing (no row, no seal), so model B gets A's rows of each
    position before its step and, after a seal, A's codes and tables."""
    shape = SEAL64
    blob = synth.make_blob(shape, seed=17)
    toks = synth.prompt(18, 140, shape.vocab)
    a = orc.OracleModel(blob, 160, kv_format=kv)
    b = orc.OracleModel(blob, 160, kv_format=kv)
    b.set_store(False)
    for i, t in enumerate(toks):
        la, na = a.step([t])
        sealed = kv == "int8" and i % 128 == 127
        b.set_pos(i)
        for l in range(shape.n_layers):
            for w in (0, 1):
                for g in range(shape.n_kv_heads):
                    if sealed:               # A's segment is sealed by now: B gets the staging row A held
                        a.set_pos(i)
                        row = a.get_rows(l, w, g, i, 1)
                        a.set_pos(i + 1)
                    else:
                        row = a.get_rows(l, w, g, i, 1)
                    b.set_rows(l, w, g, i, row)
        lb, nb = b.step([t])
        assert np.array_equal(la, lb) and na[0] == nb[0], (kv, i)
        if sealed:                           # B sealed nothing: its codes and tables come from A
            for l in range(shape.n_layers):
                for w in (0, 1):
                    for g in range(shape.n_kv_heads):
                        b.set_rows(l, w, g, 0, a.get_rows(l, w, g, 0, 128))
                        b.seg_meta(l, w, g, 0, set_to=a.seg_meta(l, w, g, 0))
    n = 128 if kv == "int8" else 140
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(shape.n_kv_heads):
                assert np.array_equal(a.get_rows(l, w, g, 0, n), b.get_rows(l, w, g, 0, n))
    # switched off it stores nothing: a fresh position keeps what it held
    c = orc.OracleModel(blob, 8, kv_format=kv)
    c.set_store(False)
    before = c.get_rows(0, 0, 0, 0, 1).copy()
    c.step([int(toks[0])])
    c.set_pos(0)
    assert np.array_equal(c.get_rows(0, 0, 0, 0, 1), before)


@pytest.mark.parametrize("path", ["steps", "prefill"])
def test_recorded_rows_are_the_stored_rows_unrounded(orc, path):
    """The row record holds each position's K/V rows before rounding: a
    model with the exact cache stores the same binary64 values, one with the
    fp16 cache their binary16 rounding (every layer, head and position, by
    single steps and by the blocked prefill)."""
    shape = SEAL64
    blob = synth.make_blob(shape, seed=25)
    toks = synth.prompt(26, 150, shape.vocab)
    ex = orc.OracleModel(blob, 160, kv_format="exact")
    h = orc.OracleModel(blob, 160, kv_format="fp16")
    for m in (ex, h):
        m.record_rows(True)
        if path == "steps":
            for t in toks:
                m.step([t])
        else:
            m.prefill(toks)
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(shape.n_kv_heads):
                assert np.array_equal(ex.computed_rows(l, w, g, 0, 150), ex.get_rows(l, w, g, 0, 150))
                assert np.array_equal(orc.d2h(h.computed_rows(l, w, g, 0, 150)), h.get_rows(l, w, g, 0, 150))


@pytest.mark.parametrize("kv", ["fp16", "e5m2", "int8", "exact"])
@pytest.mark.parametrize("start", [0, 50])
def test_blocked_prefill_is_the_steps(orc, kv, start):
    """orc_prefill is the decode steps loop-interchanged: after it, the
    cache (every layer, head, row; INT8 codes and tables) and the next
    steps' logits are bit-identical to feeding the tokens one step at a
    time; the prompt crosses two segment boundaries, starting at position 0
    or part-way into a segment (after `start` single steps)."""
    shape = SEAL64
    blob = synth.make_blob(shape, seed=19)
    toks = synth.prompt(20, 300, shape.vocab)
    a = orc.OracleModel(blob, 320, kv_format=kv)
    b = orc.OracleModel(blob, 320, kv_format=kv)
    for t in toks[:start]:
        a.step([t])
        b.step([t])
    for t in toks[start:290]:
        a.step([t])
    b.prefill(toks[start:290])
    assert a.pos() == b.pos() == 290
    for l in range(shape.n_layers):
        for w in (0, 1):
            for g in range(shape.n_kv_heads):
                for p0, n in ((0, 256), (256, 34)):
                    assert np.array_equal(a.get_rows(l, w, g, p0, n), b.get_rows(l, w, g, p0, n)), (l, w, g, p0)
                if kv == "int8":
                    for seg in (0, 1):
                        assert a.seg_meta(l, w, g, seg) == b.seg_meta(l, w, g, seg)
    for t in toks[290:]:
        la, na = a.step([t])
        lb, nb = b.step([t])
        assert np.array_equal(la, lb) and na[0] == nb[0]
