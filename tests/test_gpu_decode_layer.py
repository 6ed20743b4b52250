"""GPU parity of the decode layer with real attention (``a8w8_decode_layer``).

Compared stage by stage with the oracle, each stage on the GPU's own input to it (the
library returns QKV, the rotated Q, the updated caches, the attention output and h1):
QKV, the rotated Q, the caches, h1 and the layer output are bit-identical to the oracle;
the attention output is held to the BF16 tolerance of decode attention (relative 1e-2,
absolute 1e-2 below 1).  Cases: a toy layer (M=2, 2 Q / 1 KV heads of 128) and the
Qwen3-14B layer at M=1 (fused quantization prologues) and M=16 (separate quantization
kernels), with and without an attention workspace, plus the argument checks that must
fail before anything is enqueued.
"""

import numpy as np
import pytest

import oracle as O
from w8a8_quantized_decode_amd import binding as B
from w8a8_quantized_decode_amd import synth

from gpu_helpers import announce, dev, empty, host, qw, torch, zeros

pytestmark = pytest.mark.gpu

TOY = synth.Config(0, "toy layer", 2, 256, 768, "layer", n_q_heads=2, n_kv_heads=1,
                   head_dim=128)
C2 = synth.CONFIGS[2]


def _attn_ok(got, want):
    g, w = O.bf16_to_f32(got).astype(np.float64), O.bf16_to_f32(want).astype(np.float64)
    err = np.abs(g - w)
    return np.where(np.abs(w) < 1.0, err <= 1e-2, err <= 1e-2 * np.abs(w))


def _run(cfg, contexts, with_ws):
    M = len(contexts)
    print(f"[case] decode layer {cfg.name} M={M} contexts max {max(contexts)} "
          f"workspace={with_ws}", flush=True)
    d = synth.layer_inputs(cfg, layer=0, M=M)
    a = synth.attention_inputs(cfg, contexts, block_size=16)
    lay = B.LAYOUT_TILED
    w = {k: qw(d["w_" + k], d["s_" + k], lay) for k in ("qkv", "o", "gate", "up", "down")}
    H, nq, nkv, hd = cfg.H, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kc, vc = dev(a["k_cache"]), dev(a["v_cache"])
    qkv_out = empty((M, cfg.n_qkv), np.uint16)
    h1_out, out = empty((M, H), np.uint16), empty((M, H), np.uint16)
    q_rot, attn = empty((M, nq * hd), np.uint16), empty((M, nq * hd), np.uint16)
    ws = zeros((B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, H, cfg.I, cfg.n_qkv,
                                       cfg.split_k),), np.uint8)
    aws = None
    if with_ws:
        n = B.a8w8_decode_attention_workspace_bytes(M, nq, nkv, hd, a["block_table"].shape[1] * 16)
        aws = zeros((max(n, 256),), np.uint8)
    B.a8w8_decode_layer(dev(d["x"]), dev(d["gamma_in"]), dev(d["gamma_post"]), cfg.eps,
                        w["qkv"], w["o"], w["gate"], w["up"], w["down"], out, ws, nq, nkv, hd,
                        q_gamma=dev(a["q_gamma"]), k_gamma=dev(a["k_gamma"]), qk_eps=cfg.eps,
                        cos_table=dev(a["cos"]), sin_table=dev(a["sin"]),
                        positions=dev(a["positions"]), context_lens=dev(a["context_lens"]),
                        block_table=dev(a["block_table"]), k_cache=kc, v_cache=vc,
                        scale=a["scale"], q_rot=q_rot, attn=attn, attn_workspace=aws,
                        split_k=cfg.split_k, qkv_out=qkv_out, h1_out=h1_out)
    torch().cuda.synchronize()
    g_qkv, g_q = host(qkv_out, np.uint16), host(q_rot, np.uint16)
    g_kc, g_vc = host(kc, np.uint16), host(vc, np.uint16)
    g_attn, g_h1, g_out = host(attn, np.uint16), host(h1_out, np.uint16), host(out, np.uint16)

    _, st = O.decode_layer(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps, d["w_qkv"],
                           d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"], d["s_gate"], d["w_up"],
                           d["s_up"], d["w_down"], d["s_down"], nq, nkv, hd, cfg.split_k,
                           a["q_gamma"], a["k_gamma"], cfg.eps, a["cos"], a["sin"],
                           a["positions"], a["context_lens"], a["block_table"], a["k_cache"],
                           a["v_cache"], a["scale"])
    np.testing.assert_array_equal(g_qkv, st["qkv"], err_msg="QKV")
    q_w, kc_w, vc_w = O.qk_norm_rope_kv(g_qkv, nq, nkv, hd, a["q_gamma"], a["k_gamma"], cfg.eps,
                                        a["cos"], a["sin"], a["positions"], a["block_table"],
                                        a["k_cache"], a["v_cache"])
    np.testing.assert_array_equal(g_q, q_w, err_msg="rotated Q")
    np.testing.assert_array_equal(g_kc, kc_w, err_msg="K cache")
    np.testing.assert_array_equal(g_vc, vc_w, err_msg="V cache")
    attn_w = O.decode_attention(g_q, nq, nkv, hd, g_kc, g_vc, a["block_table"],
                                a["context_lens"], a["scale"])
    ok = _attn_ok(g_attn, attn_w)
    print(f"[note] decode layer attention: {np.mean(g_attn == attn_w):.4f} bit-identical")
    assert np.all(ok), f"attention: {np.count_nonzero(~ok)} outputs beyond tolerance"
    np.testing.assert_array_equal(g_h1, O.o_projection(g_attn, d["x"], d["w_o"], d["s_o"]),
                                  err_msg="h1")
    out_w, _ = O.mlp_block_decode(g_h1, d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                                  d["w_up"], d["s_up"], d["w_down"], d["s_down"], g_h1,
                                  split_k=cfg.split_k)
    np.testing.assert_array_equal(g_out, out_w, err_msg="layer output")


@pytest.mark.parametrize("with_ws", [True, False], ids=["split", "whole"])
def test_decode_layer_toy(with_ws):
    announce(f"decode layer toy {with_ws}")
    _run(TOY, [37, 130], with_ws)


def test_decode_layer_qwen3_14b_m1():
    announce("decode layer qwen3-14b M=1")
    _run(C2, [777], True)


def test_decode_layer_qwen3_14b_m16():
    announce("decode layer qwen3-14b M=16")
    ctx = np.random.default_rng(11).integers(1, 1024, size=16).tolist()
    _run(C2, ctx, True)


@pytest.mark.parametrize("M", [4, 5])
def test_decode_layer_qwen3_14b_few_rows(M):
    """4 rows: the last row count whose GEMMs quantize their rows in the fused prologue;
    5 rows: the first whose QKV and O read codes quantized by a kernel before them."""
    announce(f"decode layer qwen3-14b M={M}")
    ctx = np.random.default_rng(12 + M).integers(1, 1536, size=M).tolist()
    _run(C2, ctx, True)


@pytest.mark.parametrize("M", [1, 16])
def test_decode_layer_first_token(M):
    """Context 1: attention reads only the slot the QK step has just written in the same
    call, so the output depends on that write being visible to the attention kernel."""
    announce(f"decode layer qwen3-14b first token M={M}")
    _run(C2, [1] * M, True)


@pytest.mark.parametrize("with_ws", [True, False], ids=["split", "whole"])
def test_decode_layer_toy_head_dim_64(with_ws):
    """Head size 64 through the whole layer (4 Q and 2 KV heads, H = 256)."""
    cfg = synth.Config(0, "toy layer d64", 2, 256, 768, "layer", n_q_heads=4, n_kv_heads=2,
                       head_dim=64)
    announce(f"decode layer toy d=64 {with_ws}")
    _run(cfg, [300, 45], with_ws)
