"""GPU parity of decode attention over the paged BF16 KV cache against the oracle.

The oracle is the exact definition (FP64); the kernel computes in FP32 with an online
softmax, so outputs are held to the stated BF16 tolerance: relative 1e-2, absolute 1e-2
where |y| < 1.  Cases: the Qwen3-14B head counts (40 Q, 8 KV heads of 128) at the decode
batches 1 and 16 with context lengths that cross chunk and block boundaries, a toy shape
with a different group and head size, and a row with an out-of-range length, which must
leave its output untouched.
"""

import math

import numpy as np
import pytest

import oracle as O

from gpu_helpers import announce, dev, host, torch

pytestmark = pytest.mark.gpu


def _run(lens, nq, nkv, d, bs, bps, seed):
    rng = np.random.default_rng(seed)
    M = len(lens)
    nblocks = M * bps + 3
    q = O.rne_bf16(rng.normal(size=(M, nq * d)).astype(np.float32))
    kc = O.rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    vc = O.rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    bt = rng.permutation(nblocks)[: M * bps].reshape(M, bps).astype(np.int32)
    lens = np.asarray(lens, np.int32)
    scale = 1.0 / math.sqrt(d)
    good = (lens >= 1) & (lens <= bs * bps)
    out = torch().full((M, nq * d), 0x7FC0, dtype=torch().int16, device="cuda")  # BF16 NaN
    from w8a8_quantized_decode_amd import binding as B
    B.a8w8_decode_attention(dev(q), nq, nkv, d, dev(kc), dev(vc), dev(bt), dev(lens), scale, out)
    torch().cuda.synchronize()
    got = host(out, np.uint16)
    assert np.all(got[~good] == 0x7FC0)
    want = O.decode_attention(q[good], nq, nkv, d, kc, vc, bt[good], lens[good], scale)
    g, w = O.bf16_to_f32(got[good]).astype(np.float64), O.bf16_to_f32(want).astype(np.float64)
    err = np.abs(g - w)
    ok = np.where(np.abs(w) < 1.0, err <= 1e-2, err <= 1e-2 * np.abs(w))
    print(f"[note] attention: max error {err.max():.3g}, {np.mean(got[good] == want):.4f} of "
          f"outputs bit-identical")
    assert np.all(ok), f"{np.count_nonzero(~ok)} outputs beyond tolerance"


@pytest.mark.parametrize("M", [1, 16])
def test_attention_qwen3_14b(M):
    announce(f"decode attention qwen3-14b M={M}")
    lens = np.random.default_rng(100 + M).integers(1, 1024, size=M)
    lens[0] = 1 if M > 1 else 777
    _run(lens, 40, 8, 128, bs=16, bps=64, seed=M)


def test_attention_toy_group4_d64():
    announce("decode attention toy group 4 d=64")
    _run([1, 63, 64, 65, 129, 200], 8, 2, 64, bs=8, bps=32, seed=3)


def test_attention_skips_out_of_range_rows():
    announce("decode attention out-of-range lengths")
    _run([5, 0, 70, 4096], 4, 1, 128, bs=16, bps=8, seed=4)
