"""GPU parity of the QK-norm + RoPE + paged BF16 KV-cache write against the oracle.

Bit-exact: the kernel takes the oracle's operations in the same order (FP64 sum of the
BF16 squares of a head, FP32 norm steps, FP32 rotation without contraction, RNE to
BF16), on the same angle tables.  Cases: the Qwen3-14B head counts (40 Q, 8 KV heads of
128) at the decode batches 1 and 16 with a permuted block table, a toy shape with a
small head dimension, and rows with an out-of-range position or block, which must leave
the cache untouched.
"""

import numpy as np
import pytest

import oracle as O
from w8a8_quantized_decode_amd import binding as B
from w8a8_quantized_decode_amd import synth

from gpu_helpers import announce, dev, empty, host, torch

pytestmark = pytest.mark.gpu


def _run(M, nq, nkv, d, nblocks, bs, bps, pos, seed, bad_rows=()):
    rng = np.random.default_rng(seed)
    qkv = O.rne_bf16(rng.normal(size=(M, (nq + 2 * nkv) * d)).astype(np.float32))
    qg = O.rne_bf16(rng.uniform(0.5, 1.5, size=d).astype(np.float32))
    kg = O.rne_bf16(rng.uniform(0.5, 1.5, size=d).astype(np.float32))
    max_pos = bs * bps
    cos, sin = synth.rope_tables(max_pos, d)
    positions = np.asarray(pos, np.int32)
    # disjoint blocks per row (one permutation split up), so no two rows share a slot
    assert nblocks >= M * bps
    bt = rng.permutation(nblocks)[: M * bps].reshape(M, bps).astype(np.int32)
    kc = O.rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    vc = O.rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    good = np.array([m not in bad_rows for m in range(M)])
    q_want, kc_want, vc_want = O.qk_norm_rope_kv(qkv[good], nq, nkv, d, qg, kg, 1e-6, cos, sin,
                                                 positions[good], bt[good], kc, vc)
    for m in bad_rows:          # out of range: the position, or the block index
        if m % 2:
            positions[m] = max_pos + 3
        else:
            bt[m, positions[m] // bs] = nblocks + 5
    kd, vd = dev(kc), dev(vc)
    q_out = torch().zeros((M, nq * d), dtype=torch().int16, device="cuda")
    B.a8w8_qk_norm_rope_kv(dev(qkv), nq, nkv, d, dev(qg), dev(kg), 1e-6, dev(cos), dev(sin),
                           dev(positions), dev(bt), kd, vd, q_out)
    torch().cuda.synchronize()
    q = host(q_out, np.uint16)
    np.testing.assert_array_equal(q[good], q_want)
    assert np.all(q[~good] == 0)
    np.testing.assert_array_equal(host(kd, np.uint16), kc_want)
    np.testing.assert_array_equal(host(vd, np.uint16), vc_want)


@pytest.mark.parametrize("M", [1, 16])
def test_qk_rope_qwen3_14b(M):
    announce(f"qk-norm rope kv qwen3-14b M={M}")
    pos = np.random.default_rng(M).integers(0, 256, size=M)
    _run(M, 40, 8, 128, nblocks=16 * M + 8, bs=16, bps=16, pos=pos, seed=M)


def test_qk_rope_small_head():
    announce("qk-norm rope kv toy d=64")
    _run(5, 3, 1, 64, nblocks=16, bs=4, bps=3, pos=[0, 1, 5, 11, 7], seed=7)


def test_qk_rope_skips_out_of_range_rows():
    announce("qk-norm rope kv out-of-range rows")
    _run(6, 4, 2, 128, nblocks=24, bs=8, bps=4, pos=[3, 9, 17, 30, 0, 12], seed=9,
         bad_rows=(1, 4))
