"""Pins of the oracle's QK-norm + RoPE + KV-cache write.

RoPE is checked against independent statements of a rotation (complex multiplication in
FP64), its invariants (angle 0 is the identity, rotations compose, the norm is kept, and
the dot product of a rotated query and key depends only on the position difference),
and the batched application is checked against the per-row one, since the pages blame a
bug that repeated output on a batched Q RoPE that did not match the per-row one.  The KV write
is checked slot by slot against the block table, and everything else in the cache is
left untouched.
"""

import numpy as np

from oracle import qk_norm_rope_kv, rmsnorm, rne_bf16, rope_rotate_half
from w8a8_quantized_decode_amd.synth import rope_tables as tables


def test_rope_is_a_complex_rotation():
    rng = np.random.default_rng(1)
    d = 16
    x = rng.normal(size=(5, d)).astype(np.float32)
    th = rng.uniform(-3, 3, size=(5, d // 2))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    got = rope_rotate_half(x, c, s).astype(np.float64)
    z = (x[:, : d // 2].astype(np.float64) + 1j * x[:, d // 2 :]) * (c.astype(np.float64) + 1j * s)
    want = np.concatenate([z.real, z.imag], axis=1)
    assert np.allclose(got, want, rtol=0, atol=4e-7 * np.abs(x).max())


def test_rope_identity_composition_and_norm():
    rng = np.random.default_rng(2)
    d = 128
    x = rng.normal(size=(3, d)).astype(np.float32)
    one, zero = np.ones((1, d // 2), np.float32), np.zeros((1, d // 2), np.float32)
    assert np.array_equal(rope_rotate_half(x, one, zero), x)
    c, s = tables(64, d)
    twice = rope_rotate_half(rope_rotate_half(x, c[7], s[7]), c[7], s[7])
    assert np.allclose(twice, rope_rotate_half(x, c[14], s[14]), atol=2e-6)
    assert np.allclose(np.linalg.norm(rope_rotate_half(x, c[9], s[9]), axis=1),
                       np.linalg.norm(x, axis=1), rtol=2e-6)


def test_rope_dot_product_depends_on_position_difference():
    rng = np.random.default_rng(3)
    d = 128
    q = rng.normal(size=d).astype(np.float32)
    k = rng.normal(size=d).astype(np.float32)
    c, s = tables(64, d)
    dot = lambda pq, pk: float(np.dot(rope_rotate_half(q, c[pq], s[pq]).astype(np.float64),
                                      rope_rotate_half(k, c[pk], s[pk]).astype(np.float64)))
    assert abs(dot(5, 2) - dot(13, 10)) < 1e-4 * d
    assert abs(dot(5, 2) - dot(5, 5)) > 1e-3          # and it does depend on the difference


def _case(M=4, nq=4, nkv=2, d=128, nblocks=6, bs=4, seed=0):
    rng = np.random.default_rng(seed)
    qkv = rne_bf16(rng.normal(size=(M, (nq + 2 * nkv) * d)).astype(np.float32))
    qg = rne_bf16(rng.uniform(0.5, 1.5, size=d).astype(np.float32))
    kg = rne_bf16(rng.uniform(0.5, 1.5, size=d).astype(np.float32))
    c, s = tables(32, d)
    pos = np.array([0, 5, 9, 3], np.int32)[:M]
    bt = rng.permutation(nblocks).astype(np.int32)[: M * 3].reshape(M, 3) if M * 3 <= nblocks \
        else np.stack([rng.permutation(nblocks)[:3] for _ in range(M)]).astype(np.int32)
    kc = rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    vc = rne_bf16(rng.normal(size=(nblocks, bs, nkv, d)).astype(np.float32))
    return qkv, qg, kg, c, s, pos, bt, kc, vc, nq, nkv, d


def test_qk_norm_rope_kv_slots_and_heads():
    qkv, qg, kg, c, s, pos, bt, kc, vc, nq, nkv, d = _case(M=2, nblocks=6)
    eps = 1e-6
    q, kc2, vc2 = qk_norm_rope_kv(qkv, nq, nkv, d, qg, kg, eps, c, s, pos, bt, kc, vc)
    bs = kc.shape[1]
    touched = np.zeros(kc.shape[:2], bool)
    for m in range(2):
        p = pos[m]
        b, o = bt[m, p // bs], p % bs
        touched[b, o] = True
        for h in range(nkv):
            k0, v0 = (nq + h) * d, (nq + nkv + h) * d
            kn = rmsnorm(qkv[m : m + 1, k0 : k0 + d], kg, eps)
            assert np.array_equal(kc2[b, o, h], rne_bf16(rope_rotate_half(kn, c[p], s[p]))[0])
            assert np.array_equal(vc2[b, o, h], qkv[m, v0 : v0 + d])
        for h in range(nq):
            qn = rmsnorm(qkv[m : m + 1, h * d : (h + 1) * d], qg, eps)
            assert np.array_equal(q[m, h * d : (h + 1) * d], rne_bf16(rope_rotate_half(qn, c[p], s[p]))[0])
    assert np.array_equal(kc2[~touched], kc[~touched])
    assert np.array_equal(vc2[~touched], vc[~touched])
    # position 0 rotates nothing: row 0's Q heads are the normalized heads, rounded
    qn0 = rmsnorm(qkv[0:1, :d], qg, eps)
    assert np.array_equal(q[0, :d], rne_bf16(qn0)[0])


def test_batched_q_rope_equals_per_row():
    """All rows' Q heads rotated in one batched call with each row's own angles equal the
    per-row results; a batched call that takes the first row's angles for every row (a
    batched form that no longer matches the per-row one, the kind of fault the pages
    report) does not."""
    qkv, qg, kg, c, s, pos, bt, kc, vc, nq, nkv, d = _case(M=4, nblocks=12)
    eps = 1e-6
    q, _, _ = qk_norm_rope_kv(qkv, nq, nkv, d, qg, kg, eps, c, s, pos, bt, kc, vc)
    M = qkv.shape[0]
    heads = qkv[:, : nq * d].reshape(M * nq, d)
    qn = rmsnorm(heads, qg, eps).reshape(M, nq, d)
    batched = rne_bf16(rope_rotate_half(qn, c[pos][:, None, :], s[pos][:, None, :]))
    assert np.array_equal(batched.reshape(M, nq * d), q)
    wrong = rne_bf16(rope_rotate_half(qn, c[pos[0]], s[pos[0]]))
    assert not np.array_equal(wrong.reshape(M, nq * d), q)
