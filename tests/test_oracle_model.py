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
