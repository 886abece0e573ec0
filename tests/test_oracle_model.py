"""Pins of the oracle's composed decode step (CPU only).

The composition is checked against an independent implementation of the
standard Llama decoder (the `transformers` library's LlamaForCausalLM, run in
float64 over the whole token history with no cache), and against invariants
that hold exactly: tied == untied with a copied matrix, GQA == MHA with
duplicated key/value heads, batch == separate sequences, and the cache write
touching exactly the slots of the current position.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import oracle as orc

transformers = pytest.importorskip("transformers")


def _hf_model(shape: si.ModelShape, w):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.ffn,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_theta,
                      tie_word_embeddings=shape.tied, max_position_embeddings=4096,
                      attention_bias=False, mlp_bias=False)
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).double().eval()
    f = lambda t: t.to(torch.float64)
    sd = {"model.embed_tokens.weight": f(w["embed"]), "model.norm.weight": f(w["final_norm"])}
    if not shape.tied:
        sd["lm_head.weight"] = f(w["lm_head"])
    names = {"attn_norm": "input_layernorm.weight", "wq": "self_attn.q_proj.weight",
             "wk": "self_attn.k_proj.weight", "wv": "self_attn.v_proj.weight", "wo": "self_attn.o_proj.weight",
             "mlp_norm": "post_attention_layernorm.weight", "wg": "mlp.gate_proj.weight",
             "wu": "mlp.up_proj.weight", "wd": "mlp.down_proj.weight"}
    for l, ld in enumerate(w["layers"]):
        for k, v in ld.items():
            sd[f"model.layers.{l}.{names[k]}"] = f(v)
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected
    assert all("lm_head" in k for k in missing)  # tied head only
    return m


def _oracle_run(model: orc.Model, tokens, kv_dtype, max_ctx):
    s = model.shape
    if kv_dtype == "f64":
        kv = np.zeros(si.kv_cache_shape(s, 1, max_ctx), dtype=np.float64)
    else:
        kv = np.zeros(si.kv_cache_shape(s, 1, max_ctx), dtype=np.uint16)
    out = []
    for p, t in enumerate(tokens):
        logits, _ = model.step([t], [p], kv, 1, max_ctx)
        out.append(logits[0])
    return np.stack(out)


CASES = [
    # (shape, weight std, gain std): one layer and one head first, then GQA stacks
    (si.ModelShape(1, 8, 1, 1, 8, 16, 32, rope_theta=1e4), 0.5, 0.3),
    (si.ModelShape(2, 32, 4, 2, 8, 48, 64, rms_eps=1e-5, rope_theta=1e4), 0.3, 0.3),
    (si.ModelShape(2, 64, 4, 2, 16, 96, 50, rms_eps=1e-2, rope_theta=100.0, tied=True), 0.25, 0.2),
    (si.ModelShape(3, 48, 6, 3, 16, 64, 40, rope_theta=5e5), 0.3, 0.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_step_matches_library_llama_full_recompute(case):
    """Incremental decode with a float64 cache equals the library's full
    causal forward over the token history (no cache) at every position."""
    shape, std, gstd = CASES[case]
    w = si.make_weights(shape, master=100 + case, std=std, gain_std=gstd)
    tokens = si.uniform_ints(12, 0, shape.vocab, 100 + case, "hf/tokens")
    model = orc.Model(shape, w)
    got = _oracle_run(model, tokens, "f64", 16)
    hf = _hf_model(shape, w)
    with torch.no_grad():
        ref = hf(input_ids=torch.tensor([tokens]), use_cache=False).logits[0].numpy()
    # the library computes RoPE angles in fp32, hence ~1e-6 rather than 1e-15
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err < 2e-5, err
    # the logits are far from trivial, so the comparison has teeth
    assert np.std(ref) > 0.1


def test_bf16_cache_close_to_f64_cache():
    shape, std, gstd = CASES[1]
    w = si.make_weights(shape, master=7, std=std, gain_std=gstd)
    tokens = si.uniform_ints(10, 0, shape.vocab, 7, "t")
    model = orc.Model(shape, w)
    a = _oracle_run(model, tokens, "f64", 16)
    b = _oracle_run(model, tokens, "bf16", 16)
    err = np.max(np.abs(a - b)) / np.max(np.abs(a))
    assert 0 < err < 2e-2


def test_tied_equals_untied_with_copied_matrix():
    s_t = si.ModelShape(2, 32, 4, 2, 8, 48, 64, tied=True)
    s_u = si.ModelShape(2, 32, 4, 2, 8, 48, 64, tied=False)
    w = si.make_weights(s_t, master=3, std=0.3)
    wu = dict(w)
    wu["lm_head"] = w["embed"].clone()
    toks = si.uniform_ints(6, 0, 64, 3, "t")
    a = _oracle_run(orc.Model(s_t, w), toks, "bf16", 8)
    b = _oracle_run(orc.Model(s_u, wu), toks, "bf16", 8)
    assert np.array_equal(a, b)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    d = 8
    s_g = si.ModelShape(2, 32, 4, 2, d, 48, 64)
    s_m = si.ModelShape(2, 32, 4, 4, d, 48, 64)
    w = si.make_weights(s_g, master=4, std=0.3, gain_std=0.2)
    wm = {k: v for k, v in w.items() if k != "layers"}
    wm["layers"] = []
    for ld in w["layers"]:
        nd = dict(ld)
        for name in ("wk", "wv"):
            # MHA kv head h holds GQA kv head h // 2 (q heads 0,1 share group 0)
            nd[name] = torch.cat([ld[name][(h // 2) * d:(h // 2 + 1) * d] for h in range(4)], dim=0)
        wm["layers"].append(nd)
    toks = si.uniform_ints(7, 0, 64, 4, "t")
    a = _oracle_run(orc.Model(s_g, w), toks, "bf16", 8)
    b = _oracle_run(orc.Model(s_m, wm), toks, "bf16", 8)
    assert np.array_equal(a, b)


def test_batch_equals_separate_sequences_and_cache_write_is_exact():
    s = si.ModelShape(2, 32, 4, 2, 8, 48, 64)
    w = si.make_weights(s, master=5, std=0.3)
    model = orc.Model(s, w)
    b_max, max_ctx = 3, 20
    lens = [5, 11, 0]
    kv0 = si.bf16_bits(si.make_kv_cache(s, b_max, max_ctx, lens, master=5)).reshape(
        si.kv_cache_shape(s, b_max, max_ctx)).copy()
    toks = [3, 17, 60]
    kv = kv0.copy()
    logits, nxt = model.step(toks, lens, kv, b_max, max_ctx)
    # exactly the slots [l][plane][b][g][lens[b]][:] changed
    changed = (kv != kv0)
    mask = np.zeros_like(changed)
    for b, p in enumerate(lens):
        mask[:, :, b, :, p, :] = True
    assert not changed[~mask].any()
    assert changed[mask].mean() > 0.9  # fresh values replace the zero slots
    # each sequence alone gives bit-identical logits and cache slots
    for b in range(3):
        one = kv0[:, :, b:b + 1].copy()
        lb, nb = model.step([toks[b]], [lens[b]], one, 1, max_ctx)
        assert np.array_equal(lb[0], logits[b]) and nb[0] == nxt[b]
        assert np.array_equal(one[:, :, 0], kv[:, :, b])
    # the greedy token is the argmax of the fp32-rounded logits
    for b in range(3):
        f = logits[b].astype(np.float32)
        assert nxt[b] == int(np.flatnonzero(f == f.max())[0])


def test_kv_index_layout():
    s = si.ModelShape(2, 32, 4, 2, 8, 48, 64)
    model = orc.Model(s, si.make_weights(s, master=6))
    b_max, max_ctx = 3, 20
    ref = np.arange(np.prod(si.kv_cache_shape(s, b_max, max_ctx))).reshape(si.kv_cache_shape(s, b_max, max_ctx))
    for (l, c, b, g, t) in [(0, 0, 0, 0, 0), (1, 1, 2, 1, 19), (1, 0, 1, 0, 7)]:
        assert model.kv_index(b_max, max_ctx, l, c, b, g, t) == ref[l, c, b, g, t, 0]


def test_step_rejects_bad_inputs():
    s = si.ModelShape(1, 8, 1, 1, 8, 16, 32)
    model = orc.Model(s, si.make_weights(s, master=1))
    kv = np.zeros(si.kv_cache_shape(s, 1, 4), dtype=np.uint16)
    with pytest.raises(ValueError):
        model.step([32], [0], kv, 1, 4)   # token out of range
    with pytest.raises(ValueError):
        model.step([1], [4], kv, 1, 4)    # position beyond the cache


def test_step_probe_is_what_the_cache_receives():
    # the unrounded keys/values the step reports are exactly the values it
    # appends: rounded to bf16 they equal the cache bits at the slot, and the
    # pre-rotation keys rotated at the position give the post-rotation ones
    s = si.TINY
    w = si.make_weights(s, master=3)
    model = orc.Model(s, w)
    max_ctx, B = 16, 2
    kv = np.zeros(si.kv_cache_shape(s, B, max_ctx), dtype=np.uint16)
    pos = [5, 9]
    probe = np.empty((B, s.n_layers, 3, s.n_kv_heads, s.head_dim))
    model.step([7, 11], pos, kv, B, max_ctx, probe=probe)
    for b in range(B):
        for l in range(s.n_layers):
            for g in range(s.n_kv_heads):
                assert np.array_equal(orc.f64_to_bf16(probe[b, l, 1, g]), kv[l, 0, b, g, pos[b]])
                assert np.array_equal(orc.f64_to_bf16(probe[b, l, 2, g]), kv[l, 1, b, g, pos[b]])
                np.testing.assert_allclose(orc.rope(probe[b, l, 0, g], pos[b], s.rope_theta), probe[b, l, 1, g],
                                           rtol=0, atol=1e-15)
