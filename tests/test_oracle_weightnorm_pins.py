"""Pins of the oracle's weight normalisation ("MLP Megakernel" README, "Key
ideas": W = g * v / ||v||, all layers normalised in one launch) and its
backward, to things other than the oracle itself (CPU only).

Reading: the norm is per output unit -- each column of the x @ W matrix, the
per-output-row norm of torch's weight_norm on a Linear weight -- with one gain
per output unit.  Pinned by: values worked out by hand (a 3-4-5 column, signed
and one-hot columns), the defining invariants (every column of W has norm |g|,
W is invariant to positive rescaling of v and odd in v), the column-wise
formula against numpy's norm, and for the backward central differences of the
forward, the orthogonality of dv to v per column and a hand-worked case.
"""
import numpy as np
import pytest

import oracle


def test_by_hand():
    v = np.array([[3.0, 1.0, 0.0], [4.0, 0.0, -2.0]])
    g = np.array([2.0, -1.0, 0.5])
    W = oracle.weight_norm(v, g)
    # column 0: (3, 4) / 5 * 2; column 1: (1, 0) * -1; column 2: (0, -1) * 0.5
    assert np.array_equal(W, np.array([[1.2, -1.0, 0.0], [1.6, 0.0, -0.5]]))


def test_invariants_and_numpy_formula():
    rng = np.random.default_rng(4)
    for din, dout in ((7, 5), (128, 128), (64, 96), (1, 3)):
        v = rng.standard_normal((din, dout))
        g = rng.standard_normal(dout)
        W = oracle.weight_norm(v, g)
        np.testing.assert_allclose(np.linalg.norm(W, axis=0), np.abs(g), rtol=1e-13)
        np.testing.assert_allclose(W, g * v / np.linalg.norm(v, axis=0), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(oracle.weight_norm(3.7 * v, g), W, rtol=1e-13, atol=1e-15)
        assert np.array_equal(oracle.weight_norm(-v, g), -W)


def test_zero_column_is_nan():
    v = np.array([[0.0, 1.0], [0.0, 1.0]])
    W = oracle.weight_norm(v, [1.0, 1.0])
    assert np.isnan(W[:, 0]).all() and np.all(np.isfinite(W[:, 1]))


@pytest.mark.parametrize("din,dout", [(4, 3), (6, 6), (1, 2)])
def test_backward_central_differences(din, dout):
    rng = np.random.default_rng(din * 10 + dout)
    v = rng.standard_normal((din, dout))
    g = rng.standard_normal(dout)
    dW = rng.standard_normal((din, dout))
    dv, dg = oracle.weight_norm_backward(v, g, dW)

    def loss(vv, gg):
        return float(np.sum(dW * oracle.weight_norm(vv, gg)))

    eps = 1e-6
    for k in range(din):
        for n in range(dout):
            vp, vm = v.copy(), v.copy()
            vp[k, n] += eps
            vm[k, n] -= eps
            fd = (loss(vp, g) - loss(vm, g)) / (2 * eps)
            assert abs(fd - dv[k, n]) <= 1e-7 * (1 + abs(fd)), (k, n, fd, dv[k, n])
    for n in range(dout):
        gp, gm = g.copy(), g.copy()
        gp[n] += eps
        gm[n] -= eps
        fd = (loss(v, gp) - loss(v, gm)) / (2 * eps)
        assert abs(fd - dg[n]) <= 1e-7 * (1 + abs(fd)), (n, fd, dg[n])


def test_backward_properties_and_by_hand():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((32, 16))
    g = rng.standard_normal(16)
    dW = rng.standard_normal((32, 16))
    dv, dg = oracle.weight_norm_backward(v, g, dW)
    # dv is orthogonal to v in every column (W does not change along v)
    np.testing.assert_allclose(np.sum(dv * v, axis=0), 0.0, atol=1e-12)
    # dg = <dW, v / ||v||> per column
    np.testing.assert_allclose(dg, np.sum(dW * v, axis=0) / np.linalg.norm(v, axis=0), rtol=1e-13)
    # by hand: v = (3, 4), g = 2, dW = (1, 0): ||v|| = 5, <v, dW> = 3,
    # dg = 3/5, dv = 2/5 * ((1, 0) - (3, 4) * 3/25) = (0.256, -0.192)
    dv1, dg1 = oracle.weight_norm_backward(np.array([[3.0], [4.0]]), [2.0], np.array([[1.0], [0.0]]))
    np.testing.assert_allclose(dg1, [0.6], rtol=1e-15)
    np.testing.assert_allclose(dv1.ravel(), [0.256, -0.192], rtol=1e-14)
