"""Pins of the two operation orders the pages fix only in words, by hand-worked vectors.

The vectors in tests/golden/ were derived by hand (the derivations are in the files): each
one is chosen so that the stated order gives one result and every plausible other order
(another association of the partial sums, narrowing the partial sum first, the scales in
the other order, a combined scale, one rounding of the exact product, a truncating INT32
conversion) gives a different one.  The oracle must give the stated result; the wrong
orders are evaluated here too, to show that each of them fails the vector.
"""

import os

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F = np.float32


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _f32(bits_hex):
    return np.array([int(bits_hex, 16)], np.uint32).view(np.float32)


def _bf16_bits(x):
    return int(O.rne_bf16(np.asarray(x, np.float32).reshape(1))[0])


def test_reduce_residual_order_golden():
    rows = _rows("reduce_residual_order.txt")
    assert len(rows) == 2
    for p0h, p1h, rh, outh in rows:
        p0, p1 = _f32(p0h), _f32(p1h)
        res = np.array([int(rh, 16)], np.uint16)
        want = int(outh, 16)
        got = O.reduce_residual_bf16([p0, p1], res)
        assert int(got[0]) == want, (p0h, p1h, rh, hex(int(got[0])), outh)
        r = O.bf16_to_f32(res)
        # each plausible mistake gives a different BF16 result on this vector
        wrong = {
            "(p0+res)+p1": _bf16_bits(F(F(p0[0] + r[0]) + p1[0])),
            "p0+(p1+res)": _bf16_bits(F(p0[0] + F(p1[0] + r[0]))),
            "bf16(p0+p1)+res": _bf16_bits(
                F(O.bf16_to_f32(O.rne_bf16(F(p0[0] + p1[0]).reshape(1)))[0] + r[0])),
            "exact sum": _bf16_bits(F(float(p0[0]) + float(p1[0]) + float(r[0]))),
        }
        for name, v in wrong.items():
            assert v != want, f"vector {p0h} {p1h} {rh} does not separate {name}"


def test_dequant_order_golden():
    rows = _rows("dequant_order.txt")
    assert len(rows) == 3
    for acch, sxh, swh, yh in rows:
        acc = np.array([[int(acch)]], np.int64)
        sx, sw = _f32(sxh), _f32(swh)
        want = int(yh, 16)
        got = O.dequant(acc, sx, sw)
        assert int(got.view(np.uint32)[0, 0]) == want, (acch, sxh, swh, hex(int(got.view(np.uint32)[0, 0])), yh)
        a = F(acc[0, 0])
        wrong = [
            F(F(a * sw[0]) * sx[0]),                              # weight scale first
            F(a * F(sx[0] * sw[0])),                               # combined scale
            F(float(acc[0, 0]) * float(sx[0]) * float(sw[0])),     # exact product, one rounding
        ]
        if abs(int(acc[0, 0])) > 2**24:
            # truncating INT32 -> FP32 conversion (towards zero)
            t = int(acc[0, 0])
            mag = abs(t)
            shift = mag.bit_length() - 24
            trunc = F(np.sign(t) * ((mag >> shift) << shift))
            wrong.append(F(F(trunc * sx[0]) * sw[0]))
        else:
            assert all(int(np.asarray(v).view(np.uint32)) != want for v in wrong), (acch, sxh, swh)
        assert int(np.asarray(wrong[-1]).view(np.uint32)) != want
