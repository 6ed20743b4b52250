"""CPU oracle for the A8W8 decode linears -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path never routes through it.
"""

from .a8w8_oracle import (  # noqa: F401
    bf16_to_f32,
    decode_attention,
    decode_layer,
    dequant,
    dequant_weight_bf16,
    down_split,
    exp_f32,
    int_gemm,
    layer_linears_decode,
    layer_linears_prefill,
    linear_decode,
    mlp_block_decode,
    o_projection,
    prefill_linear,
    prefill_mlp,
    qk_norm_rope_kv,
    quantize_rows,
    reduce_residual_bf16,
    rmsnorm,
    rne_bf16,
    rope_rotate_half,
    silu_mul,
    split_k_ranges,
)
