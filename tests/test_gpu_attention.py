"""GPU parity of decode attention over the paged BF16 KV cache against the oracle.

The oracle is the exact definition (FP64); the kernel computes in FP32 with an online
softmax, so outputs are held to the stated BF16 tolerance: relative 1e-2, absolute 1e-2
where |y| < 1.  Each case runs twice: with a workspace (the context cut into splits that
separate workgroups take, then merged) and without one (one workgroup walks the whole
context).  Cases: the Qwen3-14B head counts (40 Q, 8 KV heads of 128) at the decode
batches 1 and 16 with context lengths that cross chunk and block boundaries, a context
of 4096 at batch 1 (64 splits) and of 16384 (256 splits, merged in groups of 64), a toy
shape with a different group and head size, a row
with an out-of-range length, which must leave its output untouched, block tables with
holes (block numbers out of range), whose positions are left out, and the group sizes 1,
3 and 8 at both head sizes (the kernel is compiled per group size and head size).
"""

import math

import numpy as np
import pytest

import oracle as O

from gpu_helpers import announce, dev, host, torch

pytestmark = pytest.mark.gpu

MODES = ["split", "whole"]


def _run(lens, nq, nkv, d, bs, bps, seed, mode, holes=0):
    from w8a8_quantized_decode_amd import binding as B
    rng = np.random.default_rng(seed)
    M = len(lens)
    nblocks = M * bps + 3
    q = O.rne_bf16(rng.normal(size=(M, nq * d)).astype(np.float32))
    kc = O.rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    vc = O.rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    bt = rng.permutation(nblocks)[: M * bps].reshape(M, bps).astype(np.int32)
    for i in range(holes):                      # out-of-range block numbers, both signs
        bt[i % M, rng.integers(0, bps)] = -1 - i if i % 2 == 0 else nblocks + i
    lens = np.asarray(lens, np.int32)
    scale = 1.0 / math.sqrt(d)
    good = (lens >= 1) & (lens <= bs * bps)
    out = torch().full((M, nq * d), 0x7FC0, dtype=torch().int16, device="cuda")  # BF16 NaN
    ws = None
    if mode == "split":
        nbytes = B.a8w8_decode_attention_workspace_bytes(M, nq, nkv, d, bs * bps)
        if nbytes:
            ws = torch().full((nbytes,), 0x7F, dtype=torch().uint8, device="cuda")
    print(f"[case] M={M} nq={nq} nkv={nkv} d={d} bs={bs} bps={bps} mode={mode} "
          f"workspace={0 if ws is None else ws.numel()}", flush=True)
    B.a8w8_decode_attention(dev(q), nq, nkv, d, dev(kc), dev(vc), dev(bt), dev(lens), scale, out,
                            workspace=ws)
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


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [1, 16])
def test_attention_qwen3_14b(M, mode):
    announce(f"decode attention qwen3-14b M={M} {mode}")
    lens = np.random.default_rng(100 + M).integers(1, 1024, size=M)
    lens[0] = 1 if M > 1 else 777
    _run(lens, 40, 8, 128, bs=16, bps=64, seed=M, mode=mode)


def test_attention_qwen3_14b_context_4096():
    announce("decode attention qwen3-14b M=1 context 4096 split")
    _run([4096], 40, 8, 128, bs=16, bps=256, seed=7, mode="split")


@pytest.mark.parametrize("mode", MODES)
def test_attention_toy_group4_d64(mode):
    announce(f"decode attention toy group 4 d=64 {mode}")
    _run([1, 63, 64, 65, 129, 200], 8, 2, 64, bs=8, bps=32, seed=3, mode=mode)


@pytest.mark.parametrize("mode", MODES)
def test_attention_skips_out_of_range_rows(mode):
    announce(f"decode attention out-of-range lengths {mode}")
    _run([5, 0, 70, 4096], 4, 1, 128, bs=16, bps=8, seed=4, mode=mode)


@pytest.mark.parametrize("mode", MODES)
def test_attention_block_table_holes(mode):
    announce(f"decode attention block-table holes {mode}")
    _run([300, 129, 64, 17], 16, 2, 128, bs=16, bps=20, seed=9, mode=mode, holes=6)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("nq,nkv,d", [(4, 4, 128), (6, 2, 64), (16, 2, 128), (24, 3, 64)],
                         ids=["mha-d128", "group3-d64", "group8-d128", "group8-d64"])
def test_attention_group_sizes(nq, nkv, d, mode):
    announce(f"decode attention nq={nq} nkv={nkv} d={d} {mode}")
    _run([1, 64, 100, 257, 700], nq, nkv, d, bs=16, bps=48, seed=nq + d, mode=mode)


def test_attention_long_context_many_splits():
    """Context 16384 at M=2: 256 splits per row, so the merge runs over several groups of
    64 splits; the second row is ragged (a partial last split)."""
    announce("decode attention qwen3-14b M=2 context 16384 split")
    _run([16384, 12345], 40, 8, 128, bs=16, bps=1024, seed=11, mode="split")


@pytest.mark.parametrize("mode", MODES)
def test_attention_many_rows(mode):
    """100 rows with ragged contexts (1 .. 300): a large batch of rows, where the grid's
    row dimension and the split choice for many (row, KV head) pairs are exercised."""
    announce(f"decode attention qwen3-14b M=100 {mode}")
    lens = np.random.default_rng(21).integers(1, 301, size=100)
    _run(lens, 40, 8, 128, bs=16, bps=19, seed=21, mode=mode)
