"""The arithmetic behind the float32 split products, checked on the host with
an emulated bf16 (round to nearest even on the float32 bit pattern).

Each float32 a is written as a1 + a2 + a3 with a1 = bf16(a), a2 = bf16(a - a1),
a3 = bf16(a - a1 - a2). The split must be exact, and the sum of the six part
products a_i * b_j with i + j <= 4 must be within about 2^-23 of a * b
(the two largest dropped terms, a2*b3 and a3*b2, are at most 2^-24 |a b| each).
This pins the scheme the kernels implement; the kernels themselves are checked
against the oracle by the GPU tests.
"""
import numpy as np


def bf16_rne(x):
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split3(a):
    a = np.asarray(a, np.float32)
    a1 = bf16_rne(a)
    r = (a - a1).astype(np.float32)
    a2 = bf16_rne(r)
    a3 = bf16_rne((r - a2).astype(np.float32))
    return a1, a2, a3


def _values(rng, n):
    return np.concatenate([
        rng.standard_normal(n).astype(np.float32),
        (rng.standard_normal(n // 8) * 1e-20).astype(np.float32),
        (rng.standard_normal(n // 8) * 1e20).astype(np.float32),
        (rng.uniform(1.0, 2.0, n // 8)).astype(np.float32),  # full mantissas near powers of two
    ])


def test_split_is_exact():
    a = _values(np.random.default_rng(0), 400_000)
    a1, a2, a3 = split3(a)
    for p in (a1, a2, a3):
        assert np.array_equal(bf16_rne(p), p)  # every part is a bf16 number
    assert np.array_equal(a1.astype(np.float64) + a2 + a3, a.astype(np.float64))


def test_six_products_error_bound():
    rng = np.random.default_rng(1)
    a = _values(rng, 400_000)
    b = rng.permutation(_values(rng, 400_000))[: a.size]
    A, B = split3(a), split3(b)
    six = sum(A[i].astype(np.float64) * B[j] for i in range(3) for j in range(3) if i + j <= 2)
    exact = a.astype(np.float64) * b
    nz = exact != 0
    rel = np.abs(six[nz] - exact[nz]) / np.abs(exact[nz])
    assert rel.max() <= 2.0 ** -23
    # dropping one more term (the (2,2) product) is far less accurate: the
    # sixth product is needed
    five = six - A[1].astype(np.float64) * B[1]
    rel5 = np.abs(five[nz] - exact[nz]) / np.abs(exact[nz])
    assert rel5.max() > 2.0 ** -20
