"""Pins of the oracle's decode layer with real attention (``decode_layer``).

The composition is checked against what its parts and the definitions fix: with a context
of one position (the new token only), each Q head's attention output is the V row of its
KV head taken from QKV, so the layer equals O and the MLP applied to those rows; the QKV
stage equals the identity-attention layer's; ``o_projection`` on the Q slice reproduces
the identity-attention layer's h1 and output; the new token's K and V land in the cache
slot its position names and nothing else in the cache changes.
"""

import numpy as np

import oracle as O
from w8a8_quantized_decode_amd import synth

TOY = synth.Config(0, "toy layer", 2, 256, 768, "layer", n_q_heads=2, n_kv_heads=1,
                   head_dim=128)


def _layer(cfg, contexts, seed_layer=0):
    d = synth.layer_inputs(cfg, layer=seed_layer, M=len(contexts))
    a = synth.attention_inputs(cfg, contexts, block_size=4, layer=seed_layer)
    out, st = O.decode_layer(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps, d["w_qkv"],
                             d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"], d["s_gate"],
                             d["w_up"], d["s_up"], d["w_down"], d["s_down"], cfg.n_q_heads,
                             cfg.n_kv_heads, cfg.head_dim, cfg.split_k, a["q_gamma"],
                             a["k_gamma"], cfg.eps, a["cos"], a["sin"], a["positions"],
                             a["context_lens"], a["block_table"], a["k_cache"], a["v_cache"],
                             a["scale"])
    return d, a, out, st


def test_context_of_one_attends_to_its_own_value():
    cfg = TOY
    d, a, out, st = _layer(cfg, [1, 1])
    hd, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    v0 = (nq + nkv) * hd
    for h in range(nq):
        g = h // (nq // nkv)
        want = st["qkv"][:, v0 + g * hd : v0 + (g + 1) * hd]
        assert np.array_equal(st["attn"][:, h * hd : (h + 1) * hd], want)
    h1 = O.o_projection(st["attn"], d["x"], d["w_o"], d["s_o"])
    assert np.array_equal(st["h1"], h1)
    want_out, _ = O.mlp_block_decode(h1, d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                                     d["w_up"], d["s_up"], d["w_down"], d["s_down"], h1,
                                     split_k=cfg.split_k)
    assert np.array_equal(out, want_out)


def test_qkv_and_o_match_the_identity_attention_layer():
    cfg = TOY
    d, a, out, st = _layer(cfg, [9, 6])
    ref_out, ref = O.layer_linears_decode(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps,
                                          d["w_qkv"], d["s_qkv"], d["w_o"], d["s_o"],
                                          d["w_gate"], d["s_gate"], d["w_up"], d["s_up"],
                                          d["w_down"], d["s_down"], cfg.n_q_heads,
                                          cfg.head_dim, cfg.split_k)
    assert np.array_equal(st["qkv"], ref["qkv"])
    h1_identity = O.o_projection(ref["qkv"][:, : cfg.H], d["x"], d["w_o"], d["s_o"])
    assert np.array_equal(h1_identity, ref["h1"])


def test_new_token_written_to_its_slot_only():
    cfg = TOY
    d, a, out, st = _layer(cfg, [9, 6])
    bs = a["k_cache"].shape[1]
    changed = np.argwhere(np.any(st["k_cache"] != a["k_cache"], axis=(2, 3)))
    want = sorted((int(a["block_table"][m, p // bs]), int(p % bs))
                  for m, p in enumerate(a["positions"]))
    assert sorted(map(tuple, changed.tolist())) == want
    for m, p in enumerate(a["positions"]):
        b, o = a["block_table"][m, p // bs], p % bs
        v0 = (cfg.n_q_heads + cfg.n_kv_heads) * cfg.head_dim
        assert np.array_equal(st["v_cache"][b, o, 0], st["qkv"][m, v0 : v0 + cfg.head_dim])
