"""Pins of the oracle's projections (P1 linear, P2 grouped_linear) to
definitions computed another way: brute-force sums on tiny inputs, the grouped
product as one dense product with a block-diagonal weight, and special cases
(identity weight, one group)."""
import numpy as np

import oracle as O


def test_linear_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = O.linear(x, w)
    for m in range(3):
        for n in range(4):
            s = 0.0
            for k in range(5):
                s += x[m, k] * w[n, k]
            assert abs(y[m, n] - s) < 1e-12


def test_linear_identity_and_batch_dims():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 3, 6))
    assert np.array_equal(O.linear(x, np.eye(6)), x)
    w = rng.standard_normal((7, 6))
    y = O.linear(x, w)
    assert y.shape == (2, 3, 7)
    assert np.allclose(y[1, 2], [sum(x[1, 2, k] * w[n, k] for k in range(6)) for n in range(7)], atol=1e-12)


def test_grouped_is_block_diagonal():
    """G products side by side = one product with the block-diagonal weight."""
    rng = np.random.default_rng(3)
    G, N, K, M = 4, 3, 5, 6
    x = rng.standard_normal((M, G * K))
    w = rng.standard_normal((G, N, K))
    dense = np.zeros((G * N, G * K))
    for g in range(G):
        dense[g * N:(g + 1) * N, g * K:(g + 1) * K] = w[g]
    y = O.grouped_linear(x, w)
    ref = np.array([[sum(dense[n, k] * x[m, k] for k in range(G * K)) for n in range(G * N)] for m in range(M)])
    assert np.allclose(y, ref, atol=1e-12)


def test_grouped_one_group_and_locality():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 8))
    w = rng.standard_normal((1, 3, 8))
    assert np.allclose(O.grouped_linear(x, w), O.linear(x, w[0]), atol=1e-12)
    # changing group 1's inputs leaves group 0's outputs alone
    w2 = rng.standard_normal((2, 3, 4))
    x2 = rng.standard_normal((5, 8))
    y = O.grouped_linear(x2, w2)
    x3 = x2.copy()
    x3[:, 4:] += 1.0
    y3 = O.grouped_linear(x3, w2)
    assert np.array_equal(y[:, :3], y3[:, :3]) and not np.allclose(y[:, 3:], y3[:, 3:])
