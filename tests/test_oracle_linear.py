"""Pins of the projection oracle: brute force, identity, linearity, the bank
projection's per-token independence."""

import numpy as np

from oracle import linear


def test_linear_brute_force():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7)).astype(np.float16)
    w = rng.standard_normal((3, 7)).astype(np.float16)
    b = rng.standard_normal(3)
    y = linear(x, w, b)
    for m in range(5):
        for n in range(3):
            acc = b[n]
            for k in range(7):
                acc += float(x[m, k]) * float(w[n, k])
            assert abs(y[m, n] - acc) < 1e-12


def test_linear_identity_and_linearity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 16))
    assert np.array_equal(linear(x, np.eye(16)), x)
    w = rng.standard_normal((4, 16))
    a, c = 2.5, -0.75
    x2 = rng.standard_normal((9, 16))
    assert np.allclose(linear(a * x + c * x2, w), a * linear(x, w) + c * linear(x2, w), atol=1e-12)


def test_projecting_the_bank_once_equals_projecting_the_joined_sequence():
    # the reading behind projecting the bank when it is written: rows are independent
    rng = np.random.default_rng(2)
    own, bank = rng.standard_normal((6, 8)), rng.standard_normal((4, 8))
    w = rng.standard_normal((8, 8))
    joined = linear(np.concatenate([own, bank]), w)
    assert np.allclose(joined, np.concatenate([linear(own, w), linear(bank, w)]), atol=1e-12)
