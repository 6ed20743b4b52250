"""Host-side checks of the C ABI (no GPU): the library loads, exports every function
that include/a8w8.h declares, and rejects invalid arguments before touching the GPU.

Validation runs on the host before any HIP call, so these calls are safe without a
device: every one of them must return an error status (or OK for an empty batch)
without enqueueing anything.
"""

import ctypes
import os
import re

import pytest

from w8a8_quantized_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "a8w8.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from w8a8_quantized_decode_amd import build
        build.build(verbose=False)
    return B.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(a8w8_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"a8w8_quantize_rows", "a8w8_linear", "a8w8_mlp_block", "a8w8_layer_linears",
            "a8w8_layer_linears_prefill", "a8w8_qk_norm_rope_kv",
            "a8w8_decode_attention", "a8w8_decode_attention_workspace_bytes",
            "a8w8_decode_layer",
            "a8w8_workspace_bytes", "a8w8_status_string", "a8w8_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in B.STATUS_NAMES.items():
        assert B.status_string(code).startswith(name)
    assert B.status_string(99) == "A8W8_ERR_UNKNOWN"
    assert B.a8w8_version() >= 100


def test_workspace_bytes(L):
    ws = B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 1, 5120, 17408, 0, 2)
    # at least q_x, h (FP32), q_h
    assert ws >= 5120 + 17408 * 4 + 17408
    ws_layer = B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 1, 5120, 17408, 7168, 2)
    assert ws_layer > ws
    assert B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 16, 5120, 17408, 0, 2) > ws
    # invalid: split not in {1,2,4,8}, I not a multiple of 64*split, bad op, bad mode
    assert B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 1, 5120, 17408, 0, 3) == 0
    assert B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 1, 5120, 17408 + 64, 0, 2) == 0
    assert B.a8w8_workspace_bytes(7, 1, 5120, 17408, 0, 2) == 0
    assert B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 1, 5120, 17408, 0, 2, 9) == 0
    assert B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 1, 5120, 17408, 7160, 2) == 0


FAKE = 0x10000000  # 16-byte aligned, never dereferenced: validation fails first
MIS = FAKE + 4
QW = B.QWeight(FAKE, FAKE, 0)


def test_quantize_rows_validation(L):
    f = L.a8w8_quantize_rows
    assert f(FAKE, 64, None, 1e-6, 0, 64, FAKE, FAKE, None, None) == 0         # M == 0
    assert f(FAKE, 64, None, 1e-6, 2, 60, FAKE, FAKE, None, None) == 2         # K % 8
    assert f(FAKE, 32, None, 1e-6, 2, 64, FAKE, FAKE, None, None) == 2         # ldx < K
    assert f(FAKE, 64, None, 1e-6, -1, 64, FAKE, FAKE, None, None) == 2        # M < 0
    assert f(None, 64, None, 1e-6, 2, 64, FAKE, FAKE, None, None) == 1         # x NULL
    assert f(FAKE, 64, None, 1e-6, 2, 64, None, FAKE, None, None) == 1         # q NULL
    assert f(MIS, 64, None, 1e-6, 2, 64, FAKE, FAKE, None, None) == 3          # misaligned
    assert f(FAKE, 64, MIS, 1e-6, 2, 64, FAKE, FAKE, None, None) == 3          # gamma misaligned


def test_pack_weight_validation(L):
    f = L.a8w8_pack_weight
    assert f(FAKE, 24, 64, FAKE, None) == 2          # N % 16
    assert f(FAKE, 16, 100, FAKE, None) == 2         # K % 64
    assert f(None, 16, 64, FAKE, None) == 1
    assert f(FAKE, 16, 64, MIS, None) == 3


def test_linear_validation(L):
    f = L.a8w8_linear
    assert f(FAKE, FAKE, B.QWeight(FAKE, FAKE, 7), None, 1, 16, 64, FAKE, None, None) == 2
    assert f(FAKE, FAKE, QW, None, 0, 16, 64, FAKE, None, None) == 0            # M == 0
    assert f(FAKE, FAKE, QW, None, 1, 16, 100, FAKE, None, None) == 2           # K % 64
    assert f(FAKE, FAKE, QW, None, 1, 24, 64, FAKE, None, None) == 2            # N % 16
    assert f(FAKE, FAKE, QW, None, 1, 16, 131072 + 64, FAKE, None, None) == 2   # K too large
    assert f(FAKE, FAKE, QW, None, 65535 * 64 + 1, 16, 64, FAKE, None, None) == 2  # grid rows
    assert f(FAKE, FAKE, B.QWeight(FAKE, None, 0), None, 1, 16, 64, FAKE, None, None) == 1
    assert f(FAKE, FAKE, QW, None, 1, 16, 64, None, None, None) == 1
    assert f(FAKE, FAKE, B.QWeight(MIS, FAKE, 0), None, 1, 16, 64, FAKE, None, None) == 3
    assert f(FAKE, FAKE, QW, MIS, 1, 16, 64, FAKE, None, None) == 3


def test_mlp_block_validation(L):
    f = L.a8w8_mlp_block
    ws = B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 1, 256, 768, 0, 2)

    def call(M=1, H=256, I=768, split=2, mode=0, wsp=FAKE, wsb=ws, x=FAKE, gate=QW):
        return f(x, FAKE, 1e-6, gate, QW, QW, FAKE, FAKE, M, H, I, split, mode, wsp, wsb,
                 None, None)
    assert call(M=0) == 0
    assert call(H=200) == 2
    assert call(I=768 + 64) == 2            # I % (64 * split_k)
    assert call(split=3) == 2
    assert call(M=65535 * 64 + 1) == 2       # more 64-row groups than a grid dimension holds
    assert call(mode=5) == 2
    assert call(x=None) == 1
    assert call(gate=B.QWeight(None, FAKE, 0)) == 1
    assert call(wsp=None) == 4
    assert call(wsb=ws - 1) == 4
    assert call(wsp=FAKE + 16) == 3          # workspace must be 256-byte aligned
    assert call(x=MIS) == 3


def test_layer_static_validation(L):
    """The allocation-free layer entry validates like a8w8_layer_linears and refuses a call
    whose workspace would not fit its static one, all before touching a device."""
    f = L.a8w8_layer_linears_static

    def call(M=1, H=256, I=768, nq=2, nkv=1, hd=128, x=FAKE):
        return f(x, FAKE, FAKE, 1e-6, QW, QW, QW, QW, QW, M, H, I, nq, nkv, hd, 2, None, FAKE,
                 None, None)
    assert B.a8w8_layer_linears_static_max_workspace() == 16 << 20
    assert call(M=0) == 0
    assert call(nq=3) == 2                   # n_q * head_dim != H
    assert call(hd=0) == 2
    assert call(x=None) == 1
    assert call(x=MIS) == 3
    # Qwen3-14B shapes: 8.7 MB of workspace at M = 16 fits, 139 MB at M = 256 does not
    assert B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 16, 5120, 17408, 7168, 2) <= 16 << 20
    assert call(M=256, H=5120, I=17408, nq=40, nkv=8, hd=128) == 4


def test_layer_validation(L):
    f = L.a8w8_layer_linears
    ws = B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 1, 256, 768, 512, 2)

    def call(M=1, H=256, nq=2, nkv=1, hd=128, wsb=ws):
        return f(FAKE, FAKE, FAKE, 1e-6, QW, QW, QW, QW, QW, M, H, 768, nq, nkv, hd, 2, None,
                 FAKE, FAKE, wsb, None, None)
    assert call(M=0) == 0
    assert call(nq=3) == 2                   # n_q * head_dim != H
    assert call(hd=0) == 2
    assert call(wsb=ws - 1) == 4


def test_layer_prefill_validation(L):
    """Shape, workspace and alignment errors are returned before any launch."""
    f = L.a8w8_layer_linears_prefill
    ws = B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 1, 256, 768, 512, 2, B.MODE_PREFILL_W8A16)
    assert ws > B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, 1, 256, 768, 0, 2, B.MODE_PREFILL_W8A16)
    assert B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 1, 256, 768, 512 + 16, 2,
                                  B.MODE_PREFILL_W8A16) == 0   # n_qkv % 128

    def call(M=1, H=256, nq=2, nkv=1, hd=128, wsb=ws, x=FAKE, wsp=FAKE):
        return f(x, FAKE, FAKE, 1e-6, QW, QW, QW, QW, QW, M, H, 768, nq, nkv, hd, None, None,
                 FAKE, wsp, wsb, None)
    assert call(M=0) == 0
    assert call(nq=3) == 2                   # n_q * head_dim != H
    assert call(wsb=ws - 1) == 4
    assert call(x=None) == 1
    assert call(x=MIS) == 3
    assert call(wsp=FAKE + 16) == 3


def test_qk_rope_validation(L):
    """Shape, null and alignment errors are returned before any launch."""
    f = L.a8w8_qk_norm_rope_kv

    def call(M=1, nq=40, nkv=8, d=128, qkv=FAKE, cos=FAKE, bt=FAKE, kc=FAKE, maxp=64, nb=4):
        return f(qkv, M, nq, nkv, d, FAKE, FAKE, 1e-6, cos, FAKE, maxp, FAKE, bt, 2, kc, FAKE,
                 nb, 16, FAKE, None)
    assert call(M=0) == 0
    assert call(d=127) == 2                  # odd head_dim
    assert call(d=1024) == 2                 # above 512
    assert call(nq=0) == 2
    assert call(maxp=0) == 2
    assert call(nb=0) == 2
    assert call(qkv=None) == 1
    assert call(kc=None) == 1
    assert call(cos=FAKE + 2) == 3


def test_attention_validation(L):
    """Shape, null, alignment and workspace errors are returned before any launch."""
    f = L.a8w8_decode_attention

    def call(M=1, nq=40, nkv=8, d=128, q=FAKE, kc=FAKE, bt=FAKE, bps=4, ws=None, wsb=0):
        return f(q, M, nq, nkv, d, kc, FAKE, 16, 16, bt, bps, FAKE, 0.088, FAKE, ws, wsb, None)
    assert call(M=0) == 0
    assert call(nq=41) == 2                  # n_q % n_kv
    assert call(nq=72) == 2                  # group of 9 > 8
    assert call(d=96) == 2                   # d % 64
    assert call(d=256) == 2                  # above 128
    assert call(bps=(1 << 26) + 1) == 2      # blocks_per_seq * block_size > 2^30
    assert call(kc=None) == 1
    assert call(kc=MIS) == 3
    assert call(q=FAKE + 8) == 3
    assert call(bt=FAKE + 2) == 3
    # context 4096 at M=1 is cut into splits: the workspace must fit them and be aligned
    need = B.a8w8_decode_attention_workspace_bytes(1, 40, 8, 128, 256 * 16)
    assert need == 1 * 40 * 64 * (128 + 2) * 4
    assert call(bps=256, ws=FAKE, wsb=need - 1) == 4
    assert call(bps=256, ws=FAKE + 16, wsb=need) == 3


def test_attention_workspace_bytes(L):
    ws = B.a8w8_decode_attention_workspace_bytes
    assert ws(1, 40, 8, 128, 64) == 0            # one split: no workspace
    assert ws(8, 40, 8, 128, 256) == 0           # 64 (row, KV head) pairs of 4 chunks: no split
    assert ws(9, 40, 8, 128, 256) > 0            # more pairs: split
    assert ws(1, 40, 8, 128, 320) > 0            # more chunks: split
    assert ws(1, 40, 8, 128, 4096) == 40 * 64 * 130 * 4
    # many rows: splits grow in whole chunks so the grid stays near 2048 workgroups
    assert ws(16, 40, 8, 128, 4096) == 16 * 40 * 16 * 130 * 4
    assert ws(1, 41, 8, 128, 4096) == 0          # invalid shapes
    assert ws(1, 40, 8, 96, 4096) == 0
    assert ws(1, 40, 8, 128, 0) == 0


def test_decode_layer_validation(L):
    """The attention step's arguments are checked with the layer's, before any launch: a
    missing step, a bad block size (QK step) and a context range the attention step
    rejects all return their status with nothing enqueued."""
    need = B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, 1, 256, 768, 512, 2)

    def call(step=True, bs=16, bps=4, rot=FAKE):
        a = B.AttentionStep()
        for f in ("q_gamma", "k_gamma", "cos_table", "sin_table", "positions", "context_lens",
                  "block_table", "k_cache", "v_cache", "attn"):
            setattr(a, f, FAKE)
        a.q_rot = rot
        a.qk_eps, a.max_pos, a.blocks_per_seq, a.num_blocks = 1e-6, 64, bps, 8
        a.block_size, a.scale = bs, 0.088
        return L.a8w8_decode_layer(FAKE, FAKE, FAKE, 1e-6, QW, QW, QW, QW, QW, 1, 256, 768, 2, 1,
                                   128, 2, ctypes.byref(a) if step else None, None, None, FAKE,
                                   FAKE, need, None)
    assert call(step=False) == 1
    assert call(bs=0) == 2
    assert call(rot=None) == 1
    assert call(bps=(1 << 26) + 1) == 2      # context range above 2^30: attention's check
