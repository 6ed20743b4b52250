"""HIP-graph capture of the decode calls: replays match the CPU oracle.

The decode GEMMs take their exchange tags from two words at the start of the workspace
that each GEMM advances on the device, so a captured call stays correct when replayed:
no replay can mistake a partial sum left by an earlier replay or call for its own.
Each case captures one call, then replays it several times with eager calls on other
inputs in between (which move the tags and rewrite the exchange words) and two replays
back to back; every replay and every eager call is compared with the oracle.
"""

import numpy as np
import pytest

import oracle as O
from w8a8_quantized_decode_amd import binding as B
from w8a8_quantized_decode_amd import synth

from gpu_helpers import announce, dev, empty, host, qw, torch, zeros

pytestmark = pytest.mark.gpu

C1, C2 = synth.CONFIGS[1], synth.CONFIGS[2]
TOY_LAYER = synth.Config(0, "toy layer", 1, 256, 768, "layer", n_q_heads=2, n_kv_heads=1,
                         head_dim=128)


def _layer_want(cfg, d):
    want, _ = O.layer_linears_decode(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps,
                                     d["w_qkv"], d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"],
                                     d["s_gate"], d["w_up"], d["s_up"], d["w_down"],
                                     d["s_down"], cfg.n_q_heads, cfg.head_dim, cfg.split_k)
    return want


@pytest.mark.parametrize("cfg,M", [(TOY_LAYER, 2), (C2, 1)], ids=["toy-M2", "qwen3-14b-M1"])
def test_layer_graph_replay(cfg, M):
    announce(f"layer graph replay {cfg.name} M={M}")
    t = torch()
    dA = synth.layer_inputs(cfg, layer=0, M=M)
    dB = dict(dA)
    dB["x"] = synth.layer_inputs(cfg, layer=1, M=M)["x"]
    want_a, want_b = _layer_want(cfg, dA), _layer_want(cfg, dB)
    lay = B.LAYOUT_TILED
    w = dict(qkv=qw(dA["w_qkv"], dA["s_qkv"], lay), o=qw(dA["w_o"], dA["s_o"], lay),
             gate=qw(dA["w_gate"], dA["s_gate"], lay), up=qw(dA["w_up"], dA["s_up"], lay),
             down=qw(dA["w_down"], dA["s_down"], lay))
    gin, gpost = dev(dA["gamma_in"]), dev(dA["gamma_post"])
    xa, xb = dev(dA["x"]), dev(dB["x"])
    out_g, out_e = empty((M, cfg.H), np.uint16), empty((M, cfg.H), np.uint16)
    ws = zeros((B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, cfg.H, cfg.I, cfg.n_qkv,
                                       cfg.split_k),), np.uint8)

    def call(x, out):
        B.a8w8_layer_linears(x, gin, gpost, cfg.eps, w["qkv"], w["o"], w["gate"], w["up"],
                             w["down"], out, ws, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                             split_k=cfg.split_k)

    call(xa, out_e)
    t.cuda.synchronize()
    np.testing.assert_array_equal(host(out_e, np.uint16), want_a)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        call(xa, out_g)
    for rep in range(3):
        out_g.zero_()
        g.replay()
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(out_g, np.uint16), want_a, err_msg=f"replay {rep}")
        call(xb, out_e)
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(out_e, np.uint16), want_b, err_msg=f"eager {rep}")
    out_g.zero_()
    g.replay()
    g.replay()
    t.cuda.synchronize()
    np.testing.assert_array_equal(host(out_g, np.uint16), want_a, err_msg="back-to-back")


def test_mlp_graph_replay_qwen3_14b():
    cfg, M = C1, 1
    announce(f"mlp graph replay {cfg.name} M={M}")
    t = torch()
    dA = synth.mlp_inputs(cfg, M=M)
    dB = dict(dA)
    dB["x"] = synth.mlp_inputs(cfg, layer=1, M=M)["x"]

    def want(d):
        return O.mlp_block_decode(d["x"], d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                                  d["w_up"], d["s_up"], d["w_down"], d["s_down"], d["res"],
                                  split_k=cfg.split_k)[0]

    want_a, want_b = want(dA), want(dB)
    lay = B.LAYOUT_TILED
    gate, up, down = (qw(dA["w_gate"], dA["s_gate"], lay), qw(dA["w_up"], dA["s_up"], lay),
                      qw(dA["w_down"], dA["s_down"], lay))
    gam, res = dev(dA["gamma_post"]), dev(dA["res"])
    xa, xb = dev(dA["x"]), dev(dB["x"])
    out_g, out_e = empty((M, cfg.H), np.uint16), empty((M, cfg.H), np.uint16)
    ws = zeros((B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, M, cfg.H, cfg.I, 0, cfg.split_k),),
               np.uint8)

    def call(x, out):
        B.a8w8_mlp_block(x, gam, cfg.eps, gate, up, down, res, out, ws, split_k=cfg.split_k)

    g = t.cuda.CUDAGraph()
    call(xa, out_e)
    t.cuda.synchronize()
    with t.cuda.graph(g):
        call(xa, out_g)
    for rep in range(3):
        g.replay()
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(out_g, np.uint16), want_a, err_msg=f"replay {rep}")
        call(xb, out_e)
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(out_e, np.uint16), want_b, err_msg=f"eager {rep}")
