"""ctypes binding of liba8w8.so: argument marshalling only.

Each function has the name of the C entry point it calls (see ``include/a8w8.h``),
takes torch tensors that already live on the GPU, passes their raw device pointers and
torch's current HIP stream, and raises :class:`A8W8Error` on a non-OK status.  Nothing
here computes: every step runs in the library's HIP kernels.  If the library has not
been built the first call fails loudly; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liba8w8.so")

A8W8_OK = 0
STATUS_NAMES = {0: "A8W8_OK", 1: "A8W8_ERR_NULL", 2: "A8W8_ERR_SHAPE", 3: "A8W8_ERR_ALIGN",
                4: "A8W8_ERR_WORKSPACE", 5: "A8W8_ERR_UNSUPPORTED", 6: "A8W8_ERR_HIP"}
MODE_DECODE_A8W8 = 0
MODE_PREFILL_W8A16 = 1
OP_MLP_BLOCK = 0
OP_LAYER_LINEARS = 1

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class A8W8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


LAYOUT_ROWMAJOR = 0
LAYOUT_TILED = 1
KERNEL_QUANT_IN, KERNEL_QKV, KERNEL_QUANT_ATTN, KERNEL_O = 0, 1, 2, 3
KERNEL_QUANT_POST, KERNEL_GATE_UP, KERNEL_REQUANT, KERNEL_DOWN, KERNEL_REDUCE = 4, 5, 6, 7, 8


class QWeight(ctypes.Structure):
    _fields_ = [("w", _vp), ("scale", _vp), ("layout", ctypes.c_int)]


class MlpTaps(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("xn", "q_x", "s_x", "acc_gate", "acc_up", "h", "q_h",
                                   "s_h", "acc_down", "p_down", "a_bf16", "g", "u",
                                   "h_bf16", "d", "ev_start", "ev_stop")] + \
               [("ev_kernel", ctypes.c_int)]


class AttentionStep(ctypes.Structure):
    _fields_ = [("q_gamma", _vp), ("k_gamma", _vp), ("qk_eps", ctypes.c_float),
                ("cos_table", _vp), ("sin_table", _vp), ("max_pos", ctypes.c_int64),
                ("positions", _vp), ("context_lens", _vp), ("block_table", _vp),
                ("blocks_per_seq", ctypes.c_int64), ("k_cache", _vp), ("v_cache", _vp),
                ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("scale", ctypes.c_float), ("q_rot", _vp), ("attn", _vp),
                ("attn_workspace", _vp), ("attn_ws_bytes", ctypes.c_size_t)]


class LayerTaps(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("xn_in", "q_in", "s_in", "acc_qkv", "qkv", "q_attn",
                                   "s_attn", "acc_o", "h1")] + [("mlp", MlpTaps)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Loads liba8w8.so once; raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m w8a8_quantized_decode_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.a8w8_status_string.restype = ctypes.c_char_p
        L.a8w8_status_string.argtypes = [ctypes.c_int]
        L.a8w8_version.restype = ctypes.c_int
        L.a8w8_version.argtypes = []
        L.a8w8_pack_weight.restype = ctypes.c_int
        L.a8w8_pack_weight.argtypes = [_vp, _c_i64, _c_i64, _vp, _vp]
        L.a8w8_quantize_rows.restype = ctypes.c_int
        L.a8w8_quantize_rows.argtypes = [_vp, _c_i64, _vp, ctypes.c_float, _c_i64, _c_i64,
                                         _vp, _vp, _vp, _vp]
        L.a8w8_linear.restype = ctypes.c_int
        L.a8w8_linear.argtypes = [_vp, _vp, QWeight, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp,
                                  _vp]
        L.a8w8_workspace_bytes.restype = ctypes.c_size_t
        L.a8w8_workspace_bytes.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64,
                                           ctypes.c_int, ctypes.c_int]
        L.a8w8_mlp_block.restype = ctypes.c_int
        L.a8w8_mlp_block.argtypes = [_vp, _vp, ctypes.c_float, QWeight, QWeight, QWeight, _vp,
                                     _vp, _c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int,
                                     _vp, ctypes.c_size_t, ctypes.POINTER(MlpTaps), _vp]
        L.a8w8_layer_linears.restype = ctypes.c_int
        L.a8w8_layer_linears.argtypes = [_vp, _vp, _vp, ctypes.c_float, QWeight, QWeight,
                                         QWeight, QWeight, QWeight, _c_i64, _c_i64, _c_i64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _vp, _vp, _vp, ctypes.c_size_t,
                                         ctypes.POINTER(LayerTaps), _vp]
        L.a8w8_layer_linears_static.restype = ctypes.c_int
        L.a8w8_layer_linears_static.argtypes = [_vp, _vp, _vp, ctypes.c_float, QWeight,
                                                QWeight, QWeight, QWeight, QWeight, _c_i64,
                                                _c_i64, _c_i64, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, _vp, _vp,
                                                ctypes.POINTER(LayerTaps), _vp]
        L.a8w8_layer_linears_static_max_workspace.restype = ctypes.c_size_t
        L.a8w8_layer_linears_static_max_workspace.argtypes = []
        L.a8w8_layer_linears_prefill.restype = ctypes.c_int
        L.a8w8_layer_linears_prefill.argtypes = [_vp, _vp, _vp, ctypes.c_float, QWeight,
                                                 QWeight, QWeight, QWeight, QWeight, _c_i64,
                                                 _c_i64, _c_i64, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, _vp, _vp, _vp, _vp,
                                                 ctypes.c_size_t, _vp]
        L.a8w8_qk_norm_rope_kv.restype = ctypes.c_int
        L.a8w8_qk_norm_rope_kv.argtypes = [_vp, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           _vp, _vp, ctypes.c_float, _vp, _vp, _c_i64, _vp, _vp,
                                           _c_i64, _vp, _vp, _c_i64, _c_i64, _vp, _vp]
        L.a8w8_decode_attention.restype = ctypes.c_int
        L.a8w8_decode_attention.argtypes = [_vp, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp,
                                            ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]
        L.a8w8_decode_layer.restype = ctypes.c_int
        L.a8w8_decode_layer.argtypes = [_vp, _vp, _vp, ctypes.c_float, QWeight, QWeight, QWeight,
                                        QWeight, QWeight, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(AttentionStep), _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
        L.a8w8_decode_attention_workspace_bytes.restype = ctypes.c_size_t
        L.a8w8_decode_attention_workspace_bytes.argtypes = [_c_i64, ctypes.c_int, ctypes.c_int,
                                                            ctypes.c_int, _c_i64]
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().a8w8_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != A8W8_OK:
        raise A8W8Error(status, where)


def _ptr(t) -> Optional[int]:
    """Raw device pointer of a GPU tensor (None stays NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("liba8w8 takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("liba8w8 takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def qweight(w, scale, layout: int = LAYOUT_ROWMAJOR) -> QWeight:
    return QWeight(_ptr(w), _ptr(scale), int(layout))


def _qw(spec) -> QWeight:
    """(w, scale) or (w, scale, layout) -> QWeight."""
    return qweight(*spec)


def a8w8_pack_weight(w, w_tiled, stream=None) -> None:
    """w: [N, K] INT8 row-major device tensor -> w_tiled (same size) in the tiled layout."""
    N, K = w.shape
    st = lib().a8w8_pack_weight(_ptr(w), N, K, _ptr(w_tiled), _stream(stream))
    _check(st, "a8w8_pack_weight")


def _fill_taps(struct, taps: Optional[dict]):
    if not taps:
        return
    for k, v in taps.items():
        if k == "mlp" and isinstance(struct, LayerTaps):
            _fill_taps(struct.mlp, v)
        elif k == "ev_kernel":
            struct.ev_kernel = int(v)
        elif k in ("ev_start", "ev_stop"):
            setattr(struct, k, v if isinstance(v, int) else v.cuda_event)
        else:
            setattr(struct, k, _ptr(v))


def a8w8_quantize_rows(x, q_out, row_scale_out, gamma=None, eps: float = 1e-6,
                       xn_tap=None, K: Optional[int] = None, stream=None) -> None:
    """x: [M, ldx] BF16 bits (int16/uint16 tensor); quantizes the first K columns."""
    M, ldx = x.shape
    K = ldx if K is None else K
    st = lib().a8w8_quantize_rows(_ptr(x), ldx, _ptr(gamma), float(eps), M, K, _ptr(q_out),
                                  _ptr(row_scale_out), _ptr(xn_tap), _stream(stream))
    _check(st, "a8w8_quantize_rows")


def a8w8_linear(q, row_scale, w, w_scale, y_out, residual=None, acc_tap=None,
                layout: int = LAYOUT_ROWMAJOR, stream=None) -> None:
    """w: [N, K] row-major, or its tiled form (same byte count) with layout=LAYOUT_TILED."""
    M, K = q.shape
    N = y_out.shape[1]
    st = lib().a8w8_linear(_ptr(q), _ptr(row_scale), qweight(w, w_scale, layout),
                           _ptr(residual), M, N, K, _ptr(y_out), _ptr(acc_tap),
                           _stream(stream))
    _check(st, "a8w8_linear")


def a8w8_workspace_bytes(op: int, M: int, H: int, I: int, n_qkv: int = 0, split_k: int = 2,
                         mode: int = MODE_DECODE_A8W8) -> int:
    return int(lib().a8w8_workspace_bytes(op, M, H, I, n_qkv, split_k, mode))


def a8w8_mlp_block(x, gamma, eps, gate, up, down, residual, out, workspace, split_k: int = 2,
                   mode: int = MODE_DECODE_A8W8, taps: Optional[dict] = None,
                   stream=None) -> None:
    """gate/up/down: (w, scale[, layout]) device tensors; workspace: a uint8 device tensor."""
    M, H = x.shape
    I = gate[1].shape[0]
    t = None
    if taps:
        t = MlpTaps()
        t.ev_kernel = -1
        _fill_taps(t, taps)
    st = lib().a8w8_mlp_block(_ptr(x), _ptr(gamma), float(eps), _qw(gate), _qw(up),
                              _qw(down), _ptr(residual), _ptr(out), M, H, I, int(split_k),
                              int(mode), _ptr(workspace), workspace.numel(),
                              ctypes.byref(t) if t is not None else None, _stream(stream))
    _check(st, "a8w8_mlp_block")


def a8w8_layer_linears(x, gamma_in, gamma_post, eps, qkv, o, gate, up, down, out, workspace,
                       n_q_heads: int, n_kv_heads: int, head_dim: int, split_k: int = 2,
                       qkv_out=None, taps: Optional[dict] = None, stream=None) -> None:
    M, H = x.shape
    I = gate[1].shape[0]
    t = None
    if taps:
        t = LayerTaps()
        t.mlp.ev_kernel = -1
        _fill_taps(t, taps)
    st = lib().a8w8_layer_linears(_ptr(x), _ptr(gamma_in), _ptr(gamma_post), float(eps),
                                  _qw(qkv), _qw(o), _qw(gate), _qw(up), _qw(down), M, H, I, int(n_q_heads), int(n_kv_heads),
                                  int(head_dim), int(split_k), _ptr(qkv_out), _ptr(out),
                                  _ptr(workspace), workspace.numel(),
                                  ctypes.byref(t) if t is not None else None, _stream(stream))
    _check(st, "a8w8_layer_linears")


def a8w8_layer_linears_static(x, gamma_in, gamma_post, eps, qkv, o, gate, up, down, out,
                              n_q_heads: int, n_kv_heads: int, head_dim: int, split_k: int = 2,
                              qkv_out=None, taps: Optional[dict] = None, stream=None) -> None:
    """a8w8_layer_linears with the library's own per-GPU workspace (no allocation)."""
    M, H = x.shape
    I = gate[1].shape[0]
    t = None
    if taps:
        t = LayerTaps()
        t.mlp.ev_kernel = -1
        _fill_taps(t, taps)
    st = lib().a8w8_layer_linears_static(_ptr(x), _ptr(gamma_in), _ptr(gamma_post), float(eps),
                                         _qw(qkv), _qw(o), _qw(gate), _qw(up), _qw(down), M, H, I,
                                         int(n_q_heads), int(n_kv_heads), int(head_dim),
                                         int(split_k), _ptr(qkv_out), _ptr(out),
                                         ctypes.byref(t) if t is not None else None,
                                         _stream(stream))
    _check(st, "a8w8_layer_linears_static")


def a8w8_layer_linears_static_max_workspace() -> int:
    return int(lib().a8w8_layer_linears_static_max_workspace())


def a8w8_decode_layer(x, gamma_in, gamma_post, eps, qkv, o, gate, up, down, out, workspace,
                      n_q_heads: int, n_kv_heads: int, head_dim: int, *, q_gamma, k_gamma,
                      qk_eps: float, cos_table, sin_table, positions, context_lens, block_table,
                      k_cache, v_cache, scale: float, q_rot, attn, attn_workspace=None,
                      split_k: int = 2, qkv_out=None, h1_out=None, stream=None) -> None:
    """One decode layer with real attention; the attention-step tensors follow
    a8w8_qk_norm_rope_kv and a8w8_decode_attention (q_rot and attn receive the rotated
    Q and the attention output)."""
    M, H = x.shape
    I = gate[1].shape[0]
    a = AttentionStep()
    a.q_gamma, a.k_gamma, a.qk_eps = _ptr(q_gamma), _ptr(k_gamma), float(qk_eps)
    a.cos_table, a.sin_table, a.max_pos = _ptr(cos_table), _ptr(sin_table), cos_table.shape[0]
    a.positions, a.context_lens = _ptr(positions), _ptr(context_lens)
    a.block_table, a.blocks_per_seq = _ptr(block_table), block_table.shape[1]
    a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
    a.num_blocks, a.block_size = k_cache.shape[0], k_cache.shape[1]
    a.scale, a.q_rot, a.attn = float(scale), _ptr(q_rot), _ptr(attn)
    a.attn_workspace = _ptr(attn_workspace) if attn_workspace is not None else None
    a.attn_ws_bytes = attn_workspace.numel() if attn_workspace is not None else 0
    st = lib().a8w8_decode_layer(_ptr(x), _ptr(gamma_in), _ptr(gamma_post), float(eps), _qw(qkv),
                                 _qw(o), _qw(gate), _qw(up), _qw(down), M, H, I, int(n_q_heads),
                                 int(n_kv_heads), int(head_dim), int(split_k), ctypes.byref(a),
                                 _ptr(qkv_out), _ptr(h1_out), _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check(st, "a8w8_decode_layer")


def a8w8_layer_linears_prefill(x, gamma_in, gamma_post, eps, qkv, o, gate, up, down, out,
                               workspace, n_q_heads: int, n_kv_heads: int, head_dim: int,
                               qkv_out=None, h1_out=None, stream=None) -> None:
    M, H = x.shape
    I = gate[1].shape[0]
    st = lib().a8w8_layer_linears_prefill(_ptr(x), _ptr(gamma_in), _ptr(gamma_post), float(eps),
                                          _qw(qkv), _qw(o), _qw(gate), _qw(up), _qw(down), M, H,
                                          I, int(n_q_heads), int(n_kv_heads), int(head_dim),
                                          _ptr(qkv_out), _ptr(h1_out), _ptr(out), _ptr(workspace),
                                          workspace.numel(), _stream(stream))
    _check(st, "a8w8_layer_linears_prefill")


def a8w8_qk_norm_rope_kv(qkv, n_q_heads: int, n_kv_heads: int, head_dim: int, q_gamma, k_gamma,
                         eps, cos_table, sin_table, positions, block_table, k_cache, v_cache,
                         q_out, stream=None) -> None:
    M = qkv.shape[0]
    st = lib().a8w8_qk_norm_rope_kv(_ptr(qkv), M, int(n_q_heads), int(n_kv_heads), int(head_dim),
                                    _ptr(q_gamma), _ptr(k_gamma), float(eps), _ptr(cos_table),
                                    _ptr(sin_table), cos_table.shape[0], _ptr(positions),
                                    _ptr(block_table), block_table.shape[1], _ptr(k_cache),
                                    _ptr(v_cache), k_cache.shape[0], k_cache.shape[1],
                                    _ptr(q_out), _stream(stream))
    _check(st, "a8w8_qk_norm_rope_kv")


def a8w8_decode_attention_workspace_bytes(M: int, n_q_heads: int, n_kv_heads: int,
                                          head_dim: int, max_context: int) -> int:
    return int(lib().a8w8_decode_attention_workspace_bytes(int(M), int(n_q_heads),
                                                           int(n_kv_heads), int(head_dim),
                                                           int(max_context)))


def a8w8_decode_attention(q, n_q_heads: int, n_kv_heads: int, head_dim: int, k_cache, v_cache,
                          block_table, context_lens, scale: float, out, workspace=None,
                          stream=None) -> None:
    """workspace: None or a uint8 device tensor of at least
    a8w8_decode_attention_workspace_bytes(...) bytes."""
    M = q.shape[0]
    st = lib().a8w8_decode_attention(_ptr(q), M, int(n_q_heads), int(n_kv_heads), int(head_dim),
                                     _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                     k_cache.shape[1], _ptr(block_table), block_table.shape[1],
                                     _ptr(context_lens), float(scale), _ptr(out),
                                     _ptr(workspace) if workspace is not None else None,
                                     workspace.numel() if workspace is not None else 0,
                                     _stream(stream))
    _check(st, "a8w8_decode_attention")


def a8w8_version() -> int:
    return int(lib().a8w8_version())
