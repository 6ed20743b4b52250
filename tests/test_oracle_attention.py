"""Pins of the oracle's decode attention over the paged BF16 KV cache.

Checked against what the definition fixes: one position gives that position's value
row; equal keys give the mean of the values; a key far above the others selects its
value; a constant added to every score changes nothing; a brute-force loop over
positions with Python floats agrees; the grouped-query mapping (consecutive Q heads share
a KV head) and the block table are followed.
"""

import math

import numpy as np

from oracle import bf16_to_f32, decode_attention, rne_bf16


def _cache(rng, nblocks, bs, nkv, d):
    return (rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32)),
            rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32)))


def test_single_position_returns_its_value():
    rng = np.random.default_rng(1)
    nq, nkv, d, bs = 4, 2, 16, 4
    kc, vc = _cache(rng, 5, bs, nkv, d)
    q = rne_bf16(rng.normal(size=(1, nq * d)).astype(np.float32))
    bt = np.array([[3, 1]], np.int32)
    out = decode_attention(q, nq, nkv, d, kc, vc, bt, [1], 0.1)
    for h in range(nq):
        assert np.array_equal(out[0, h * d : (h + 1) * d], vc[3, 0, h // 2])


def test_equal_keys_average_values_and_shift_invariance():
    rng = np.random.default_rng(2)
    nq, nkv, d, bs = 2, 1, 8, 4
    kc, vc = _cache(rng, 3, bs, nkv, d)
    kc[:] = kc[0, 0, 0]                               # every key the same
    q = rne_bf16(rng.normal(size=(1, nq * d)).astype(np.float32))
    bt = np.array([[2, 0, 1]], np.int32)
    out = decode_attention(q, nq, nkv, d, kc, vc, bt, [10], 0.3)
    j = np.arange(10)
    mean = bf16_to_f32(vc[bt[0, j // bs], j % bs, 0]).astype(np.float64).mean(axis=0)
    assert np.array_equal(out[0, :d], rne_bf16(mean.astype(np.float32)))
    # a large key on one position selects its value
    kc2 = kc.copy()
    kc2[0, 1, 0] = rne_bf16(np.full(d, 40.0, np.float32) * np.sign(bf16_to_f32(q[0, :d]) + 1e-9))
    out2 = decode_attention(q, nq, nkv, d, kc2, vc, bt, [10], 1.0)
    assert np.array_equal(out2[0, :d], vc[0, 1, 0])


def test_brute_force_small():
    rng = np.random.default_rng(3)
    nq, nkv, d, bs = 6, 2, 8, 2
    kc, vc = _cache(rng, 7, bs, nkv, d)
    q = rne_bf16(rng.normal(size=(2, nq * d)).astype(np.float32))
    bt = np.array([[6, 2, 4, 0], [1, 3, 5, 0]], np.int32)
    lens = [7, 3]
    scale = 1.0 / math.sqrt(d)
    out = decode_attention(q, nq, nkv, d, kc, vc, bt, lens, scale)
    qf, kf, vf = bf16_to_f32(q), bf16_to_f32(kc), bf16_to_f32(vc)
    for m in range(2):
        for h in range(nq):
            g = h // (nq // nkv)
            slots = [(int(bt[m, j // bs]), j % bs) for j in range(lens[m])]
            sc = [scale * sum(float(qf[m, h * d + i]) * float(kf[b, o, g, i]) for i in range(d))
                  for b, o in slots]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for i in range(d):
                o_i = sum(wj * float(vf[b, o, g, i]) for wj, (b, o) in zip(w, slots)) / tot
                want = rne_bf16(np.array([o_i], np.float32))[0]
                assert out[m, h * d + i] == want, (m, h, i)


def test_block_table_holes_are_left_out():
    """A block number outside [0, num_blocks) drops its positions: a table with a hole in
    the middle gives what the table without that block gives over the shorter context,
    and a row with nothing left gives zeros."""
    rng = np.random.default_rng(5)
    nq, nkv, d, bs = 4, 2, 16, 4
    kc, vc = _cache(rng, 4, bs, nkv, d)
    q = rne_bf16(rng.normal(size=(2, nq * d)).astype(np.float32))
    holed = np.array([[2, -1, 0], [7, 4, -3]], np.int32)
    out = decode_attention(q, nq, nkv, d, kc, vc, holed, [10, 9], 0.25)
    compact = decode_attention(q[:1], nq, nkv, d, kc, vc, np.array([[2, 0]], np.int32), [6], 0.25)
    assert np.array_equal(out[0], compact[0])
    assert np.all(out[1] == 0)
