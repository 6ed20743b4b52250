"""a8w8_layer_linears_static (the library's own per-GPU workspace, no allocation) against
a8w8_layer_linears with a caller workspace: both run the same kernels, so the outputs
must be bit-identical.  Two calls in a row, the second with fewer rows, the way a
serving loop reuses the static workspace; then a call whose workspace would not fit is
refused before anything is enqueued."""

import numpy as np
import pytest

from tests.gpu_helpers import announce, dev, empty, host, qw, zeros
from w8a8_quantized_decode_amd import binding as B
from w8a8_quantized_decode_amd import synth

pytestmark = pytest.mark.gpu

C2 = synth.CONFIGS[2]


def _pair(cfg, M, layer):
    announce(f"static-workspace layer linears {cfg.name} M={M}")
    d = synth.layer_inputs(cfg, layer=layer, M=M)
    w = {k: qw(d["w_" + k], d["s_" + k], B.LAYOUT_TILED) for k in ("qkv", "o", "gate", "up", "down")}
    x, gin, gpost = dev(d["x"]), dev(d["gamma_in"]), dev(d["gamma_post"])
    ws = zeros((B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, cfg.H, cfg.I, cfg.n_qkv,
                                       cfg.split_k),), np.uint8)
    out_ref, qkv_ref = empty((M, cfg.H), np.uint16), empty((M, cfg.n_qkv), np.uint16)
    B.a8w8_layer_linears(x, gin, gpost, cfg.eps, w["qkv"], w["o"], w["gate"], w["up"], w["down"],
                         out_ref, ws, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                         split_k=cfg.split_k, qkv_out=qkv_ref)
    out, qkv = empty((M, cfg.H), np.uint16), empty((M, cfg.n_qkv), np.uint16)
    B.a8w8_layer_linears_static(x, gin, gpost, cfg.eps, w["qkv"], w["o"], w["gate"], w["up"],
                                w["down"], out, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                                split_k=cfg.split_k, qkv_out=qkv)
    np.testing.assert_array_equal(host(qkv, np.uint16), host(qkv_ref, np.uint16))
    np.testing.assert_array_equal(host(out, np.uint16), host(out_ref, np.uint16))


def test_static_workspace_matches_caller_workspace():
    # Qwen3-14B shapes: M = 4, then M = 1 on the same static workspace.
    _pair(C2, 4, layer=11)
    _pair(C2, 1, layer=12)


def test_static_workspace_refuses_oversize():
    announce("static-workspace layer linears: oversize request")
    cfg, M = C2, 256
    need = B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, cfg.H, cfg.I, cfg.n_qkv, cfg.split_k)
    assert need > B.a8w8_layer_linears_static_max_workspace()
    x = empty((M, cfg.H), np.uint16)
    w = (empty((cfg.n_qkv, cfg.H), np.int8), empty((cfg.n_qkv,), np.float32), B.LAYOUT_TILED)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        B.a8w8_layer_linears_static(x, x[0], x[0], cfg.eps, w, w, w, w, w, x, cfg.n_q_heads,
                                    cfg.n_kv_heads, cfg.head_dim, split_k=cfg.split_k)
