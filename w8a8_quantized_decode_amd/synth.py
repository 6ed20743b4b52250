"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers; it holds none of the method's arithmetic.
Every draw comes from numpy's PCG64 seeded with
``seed = 1_000_003 * config + 1_009 * layer + tensor_id``.

Distributions (the workloads of the Qwen3-14B A8W8 decode linears):

* activations ``x`` and residual ``res``: FP32 standard normal, stored as BF16 by
  keeping the top 16 bits of the FP32 pattern (truncation, a sampling choice);
* RMSNorm gains: FP32 uniform on [0.5, 1.5), truncated to BF16 the same way;
* weights: INT8 codes from a discretized normal, rint(32 z) for standard-normal z,
  clipped to [-127, 127], ``[N_out, K_in]`` row-major;
* per-output-channel scales: uniform on [4e-4, 8e-4), stored as FP32.

With these, a dequantized weight has a standard deviation near 0.02 and a layer's
outputs are of order one, as in a trained model's linears.  The ``wide`` variant keeps
the first recipe (codes uniform on [-127, 127], scales uniform on [1e-3, 1e-2)): weights
twenty times larger and block outputs near 2e4, a stress case for the FP32 accumulation
bounds.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {
    "x": 1, "gamma_post": 2,
    "w_gate": 3, "s_gate": 4, "w_up": 5, "s_up": 6, "w_down": 7, "s_down": 8,
    "res": 9, "gamma_in": 10,
    "w_qkv": 11, "s_qkv": 12, "w_o": 13, "s_o": 14,
    "q_gamma": 15, "k_gamma": 16, "k_cache": 17, "v_cache": 18, "block_table": 19,
}


def seed_for(config: int, layer: int, tensor: str) -> int:
    return 1_000_003 * config + 1_009 * layer + TENSOR_IDS[tensor]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _trunc_bf16(x: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def normal_bf16(seed: int, shape) -> np.ndarray:
    return _trunc_bf16(_rng(seed).standard_normal(size=shape, dtype=np.float32))


def uniform_bf16(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    return _trunc_bf16(_rng(seed).uniform(lo, hi, size=shape).astype(np.float32))


def int8_weights(seed: int, shape, wide: bool = False) -> np.ndarray:
    if wide:
        return _rng(seed).integers(-127, 128, size=shape, dtype=np.int8)
    z = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    return np.clip(np.rint(z * np.float32(32.0)), -127, 127).astype(np.int8)


def channel_scales(seed: int, n: int, wide: bool = False) -> np.ndarray:
    lo, hi = (1e-3, 1e-2) if wide else (4e-4, 8e-4)
    return _rng(seed).uniform(lo, hi, size=(n,)).astype(np.float32)


@dataclass(frozen=True)
class Config:
    """One workload: rows ``M``, hidden ``H``, intermediate ``I`` and the layer extras."""
    index: int
    name: str
    M: int
    H: int
    I: int
    kind: str                 # "mlp", "layer", "stack" or "prefill"
    layers: int = 1
    n_q_heads: int = 40
    n_kv_heads: int = 8
    head_dim: int = 128
    split_k: int = 2
    eps: float = 1e-6

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


CONFIGS = [
    Config(0, "toy A8W8 MLP block, M=1, H=256, I=768", 1, 256, 768, "mlp",
           n_q_heads=2, n_kv_heads=1, head_dim=128),
    Config(1, "Qwen3-14B A8W8 MLP block, M=1, H=5120, I=17408", 1, 5120, 17408, "mlp"),
    Config(2, "Qwen3-14B A8W8 layer linears (QKV 5120->7168, O 5120->5120, MLP), M=1",
           1, 5120, 17408, "layer"),
    Config(3, "40-layer stack of Qwen3-14B A8W8 layer linears, M=16", 16, 5120, 17408,
           "stack", layers=40),
    Config(4, "Qwen3-14B W8A16 prefill MLP chunk, M=256", 256, 5120, 17408, "prefill"),
]


def mlp_inputs(cfg: Config, layer: int = 0, M: int | None = None, with_x: bool = True,
               wide: bool = False):
    """Seeded MLP-block tensors as numpy arrays (BF16 as uint16 bits)."""
    c, H, I = cfg.index, cfg.H, cfg.I
    M = cfg.M if M is None else M
    d = {
        "gamma_post": uniform_bf16(seed_for(c, layer, "gamma_post"), (H,), 0.5, 1.5),
        "w_gate": int8_weights(seed_for(c, layer, "w_gate"), (I, H), wide),
        "s_gate": channel_scales(seed_for(c, layer, "s_gate"), I, wide),
        "w_up": int8_weights(seed_for(c, layer, "w_up"), (I, H), wide),
        "s_up": channel_scales(seed_for(c, layer, "s_up"), I, wide),
        "w_down": int8_weights(seed_for(c, layer, "w_down"), (H, I), wide),
        "s_down": channel_scales(seed_for(c, layer, "s_down"), H, wide),
    }
    if with_x:
        d["x"] = normal_bf16(seed_for(c, layer, "x"), (M, H))
        d["res"] = normal_bf16(seed_for(c, layer, "res"), (M, H))
    return d


def layer_inputs(cfg: Config, layer: int = 0, M: int | None = None, with_x: bool = True,
                 wide: bool = False):
    """Seeded tensors of one full layer (QKV, O and the MLP block)."""
    c, H = cfg.index, cfg.H
    d = mlp_inputs(cfg, layer, M, with_x, wide)
    d.pop("res", None)
    d["gamma_in"] = uniform_bf16(seed_for(c, layer, "gamma_in"), (H,), 0.5, 1.5)
    d["w_qkv"] = int8_weights(seed_for(c, layer, "w_qkv"), (cfg.n_qkv, H), wide)
    d["s_qkv"] = channel_scales(seed_for(c, layer, "s_qkv"), cfg.n_qkv, wide)
    d["w_o"] = int8_weights(seed_for(c, layer, "w_o"), (H, cfg.n_q_heads * cfg.head_dim), wide)
    d["s_o"] = channel_scales(seed_for(c, layer, "s_o"), H, wide)
    return d


def rope_tables(max_pos: int, head_dim: int, base: float = 1_000_000.0):
    """Rotary-embedding angle tables, an input of the QK-norm + RoPE step: for position p and
    pair i < head_dim / 2, the angle p * base**(-2i / head_dim) (Qwen3's base 1e6), as FP32
    cos and sin tables [max_pos, head_dim / 2] computed in FP64 and rounded once."""
    inv = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def attention_inputs(cfg: Config, contexts, block_size: int = 16, layer: int = 0):
    """Seeded inputs of the attention step of one decode layer: row m holds its new token
    at position contexts[m] - 1 and attends to contexts[m] positions.  QK-norm gains in
    [0.5, 1.5); K and V caches of standard-normal BF16 values (the earlier positions'
    entries; the step writes the new token's); a block table of disjoint random blocks per
    row with room for the longest context; Qwen3 RoPE tables; scale 1/sqrt(head_dim)."""
    c, d = cfg.index, cfg.head_dim
    contexts = np.asarray(contexts, dtype=np.int32)
    M = contexts.size
    bps = int(-(-int(contexts.max()) // block_size))
    nblocks = M * bps + 2
    cos, sin = rope_tables(bps * block_size, d)
    perm = _rng(seed_for(c, layer, "block_table")).permutation(nblocks)[: M * bps]
    return {
        "q_gamma": uniform_bf16(seed_for(c, layer, "q_gamma"), (d,), 0.5, 1.5),
        "k_gamma": uniform_bf16(seed_for(c, layer, "k_gamma"), (d,), 0.5, 1.5),
        "cos": cos, "sin": sin,
        "positions": contexts - 1, "context_lens": contexts,
        "block_table": perm.reshape(M, bps).astype(np.int32),
        "k_cache": normal_bf16(seed_for(c, layer, "k_cache"),
                               (nblocks, block_size, cfg.n_kv_heads, d)),
        "v_cache": normal_bf16(seed_for(c, layer, "v_cache"),
                               (nblocks, block_size, cfg.n_kv_heads, d)),
        "scale": float(1.0 / np.sqrt(d)),
    }
