"""Pins of the oracle's training pair (forward with stored activations, and
the backward) to things other than itself (CPU only).

The backward is the chain rule applied to the forward chain of the "MLP
Megakernel" README ("Key ideas": the training forward keeps the hidden
activations and the backward multiplies by the derivative of softplus).  It
is tied here to:
  * central finite differences of the oracle's own forward (pinned on its
    own elsewhere): the backward must be the derivative of the forward, which
    fails a transposed operand, a dropped or extra activation derivative, a
    wrong sign or a layer off by one;
  * gradients worked out by hand (tests/golden/mlp_backward_by_hand.txt);
  * closed forms: a single layer (dW = x^T dout, dx = dout W^T, the textbook
    product), identity weights (dx = dout times a product of sigmoids),
    signed-permutation linear chains (dx exactly known element by element);
  * the properties the GPU checks at full size rely on: rows add
    (dW of a row set = sum over its parts), periodic rows scale dW;
  * the sigmoid identities: sigmoid(z) = 1 - exp(-softplus(z)), the reading
    by which a backward that holds only the stored activation a = softplus(z)
    recovers the derivative.
"""
import os

import numpy as np
import pytest
import scipy.special

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mlp_backward_by_hand.txt")


def _loss(x, Ws, g, act):
    return float(np.sum(oracle.mlp_forward(x, Ws, hidden_act=act) * g))


def _random_chain(seed, dims, M, scale=0.6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, dims[0]))
    Ws = [rng.standard_normal((dims[l], dims[l + 1])) * scale for l in range(len(dims) - 1)]
    g = rng.standard_normal((M, dims[-1]))
    return x, Ws, g


@pytest.mark.parametrize("act", ["softplus", "relu", "none"])
@pytest.mark.parametrize("dims", [(6, 7, 5, 4), (5, 3), (4, 6, 6, 5, 3, 4), (3, 4, 2, 3, 4, 3, 2, 4, 3, 3, 2, 4, 3)])
def test_backward_matches_central_differences(act, dims):
    M = 5
    x, Ws, g = _random_chain(1000 + len(dims), dims, M)
    dWs, dx = oracle.mlp_backward(x, Ws, g, hidden_act=act)
    eps = 1e-6
    for l, W in enumerate(Ws):
        for k in range(W.shape[0]):
            for n in range(W.shape[1]):
                Wp = [w.copy() for w in Ws]
                Wm = [w.copy() for w in Ws]
                Wp[l][k, n] += eps
                Wm[l][k, n] -= eps
                fd = (_loss(x, Wp, g, act) - _loss(x, Wm, g, act)) / (2 * eps)
                assert abs(fd - dWs[l][k, n]) <= 1e-6 * (1 + abs(fd)), (act, l, k, n, fd, dWs[l][k, n])
    for r in range(M):
        for k in range(dims[0]):
            xp = x.copy()
            xm = x.copy()
            xp[r, k] += eps
            xm[r, k] -= eps
            fd = (_loss(xp, Ws, g, act) - _loss(xm, Ws, g, act)) / (2 * eps)
            assert abs(fd - dx[r, k]) <= 1e-6 * (1 + abs(fd)), (act, r, k)


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        cur = None
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "act": tok[2], "dims": [int(v) for v in tok[3].split(",")], "M": int(tok[4])}
            elif tok[0] == "end":
                cases.append(cur)
                cur = None
            else:
                cur[tok[0]] = np.array([float(v) for v in tok[1:]])
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_backward_by_hand(case):
    dims, M, L = case["dims"], case["M"], len(case["dims"]) - 1
    x = case["x"].reshape(M, dims[0])
    Ws = [case["W%d" % (l + 1)].reshape(dims[l], dims[l + 1]) for l in range(L)]
    g = case["dout"].reshape(M, dims[L])
    dWs, dx = oracle.mlp_backward(x, Ws, g, hidden_act=case["act"])
    for l in range(L):
        want = case["dW%d" % (l + 1)].reshape(dims[l], dims[l + 1])
        np.testing.assert_allclose(dWs[l], want, rtol=1e-15, atol=1e-15, err_msg="dW%d" % (l + 1))
    np.testing.assert_allclose(dx, case["dx"].reshape(M, dims[0]), rtol=1e-15, atol=1e-15, err_msg="dx")


def test_single_layer_is_the_textbook_product():
    rng = np.random.default_rng(7)
    x = rng.integers(-4, 5, (9, 6)).astype(np.float64)
    W = rng.integers(-4, 5, (6, 5)).astype(np.float64)
    g = rng.integers(-4, 5, (9, 5)).astype(np.float64)
    for act in ("softplus", "relu", "none"):  # one layer: no hidden activation
        dWs, dx = oracle.mlp_backward(x, [W], g, hidden_act=act)
        assert np.array_equal(dWs[0], x.T @ g)
        assert np.array_equal(dx, g @ W.T)


@pytest.mark.parametrize("L", [2, 3, 5, 12, 16])
def test_identity_weights_product_of_sigmoids(L):
    # W_l = I: out = softplus^(L-1)(x) elementwise, so dx = dout * prod_j sigmoid(z_j)
    # with z_1 = x, z_{j+1} = softplus(z_j); and dW_L = h_{L-1}^T dout.
    D, M = 4, 7
    rng = np.random.default_rng(L)
    x = rng.uniform(-6, 6, (M, D))
    g = rng.standard_normal((M, D))
    Ws = [np.eye(D) for _ in range(L)]
    dWs, dx = oracle.mlp_backward(x, Ws, g)
    z = x.copy()
    prod = np.ones_like(x)
    for _ in range(L - 1):
        prod *= scipy.special.expit(z)
        z = np.logaddexp(0.0, z)
    np.testing.assert_allclose(dx, g * prod, rtol=1e-13, atol=0)
    np.testing.assert_allclose(dWs[-1], z.T @ g, rtol=1e-12, atol=1e-12)


def test_signed_permutation_linear_chain_exact():
    # linear chain of signed permutations: dx = dout P_L^T ... P_1^T exactly,
    # i.e. each dx element is +-1 times one dout element of the same row.
    D, L, M = 8, 3, 6
    rng = np.random.default_rng(3)
    perms, signs, Ws = [], [], []
    for _ in range(L):
        p = rng.permutation(D)
        s = rng.choice([-1.0, 1.0], D)
        P = np.zeros((D, D))
        P[np.arange(D), p] = s
        perms.append(p)
        signs.append(s)
        Ws.append(P)
    x = rng.integers(-9, 10, (M, D)).astype(np.float64)
    g = rng.integers(-9, 10, (M, D)).astype(np.float64)
    dWs, dx = oracle.mlp_backward(x, Ws, g, hidden_act="none")
    # forward: y[:, p[k]] = s[k] x[:, k]; backward: dx[:, k] = s[k] dy[:, p[k]]
    want = g.copy()
    for p, s in zip(reversed(perms), reversed(signs)):
        want = want[:, p] * s
    assert np.array_equal(dx, want)
    # dW_1 = x^T dz_1 with dz_1 the gradient at layer 1's output
    dz1 = g.copy()
    for p, s in zip(reversed(perms[1:]), reversed(signs[1:])):
        dz1 = dz1[:, p] * s
    assert np.array_equal(dWs[0], x.T @ dz1)


def test_rows_add_and_periodic_rows_scale():
    dims = (6, 5, 5, 4)
    x, Ws, g = _random_chain(11, dims, 40)
    dW_all, dx_all = oracle.mlp_backward(x, Ws, g)
    dW_a, dx_a = oracle.mlp_backward(x[:17], Ws, g[:17])
    dW_b, dx_b = oracle.mlp_backward(x[17:], Ws, g[17:])
    for l in range(3):
        np.testing.assert_allclose(dW_all[l], dW_a[l] + dW_b[l], rtol=1e-13, atol=1e-13)
    assert np.array_equal(dx_all, np.vstack([dx_a, dx_b]))  # each dx row depends on its own row only
    # rows repeated 4 times: every dW is 4 times the block's
    dW_rep, _ = oracle.mlp_backward(np.tile(x, (4, 1)), Ws, np.tile(g, (4, 1)))
    for l in range(3):
        np.testing.assert_allclose(dW_rep[l], 4 * dW_all[l], rtol=1e-13, atol=1e-13)


def test_backward_is_thread_count_independent():
    dims = (16, 16, 16, 16)
    x, Ws, g = _random_chain(5, dims, 3000)
    a, dxa = oracle.mlp_backward(x, Ws, g, nthreads=1)
    b, dxb = oracle.mlp_backward(x, Ws, g, nthreads=max(2, oracle.max_threads()))
    for l in range(3):
        assert np.array_equal(a[l], b[l])
    assert np.array_equal(dxa, dxb)


def test_forward_train_activations_and_output():
    dims = (6, 7, 5, 4)
    x, Ws, _ = _random_chain(21, dims, 9)
    for act in ("softplus", "relu", "none"):
        out, acts = oracle.mlp_forward_train(x, Ws, hidden_act=act)
        assert np.array_equal(out, oracle.mlp_forward(x, Ws, hidden_act=act))
        assert len(acts) == 2
        # h_1 = act(x W_1), h_2 = act(h_1 W_2), out = h_2 W_3 (numpy products)
        f = {"softplus": lambda z: np.logaddexp(0.0, z), "relu": lambda z: np.maximum(z, 0.0),
             "none": lambda z: z}[act]
        np.testing.assert_allclose(acts[0], f(x @ Ws[0]), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(acts[1], f(acts[0] @ Ws[1]), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(out, acts[1] @ Ws[2], rtol=1e-12, atol=1e-13)


def test_sigmoid_derivative_and_its_recovery_from_the_activation():
    z = np.concatenate([np.linspace(-40, 40, 161), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    d = oracle.act_deriv(z, "softplus")
    np.testing.assert_allclose(d, scipy.special.expit(z), rtol=1e-15, atol=0)
    assert oracle.act_deriv(0.0, "softplus") == 0.5
    np.testing.assert_allclose(d + oracle.act_deriv(-z, "softplus"), 1.0, rtol=0, atol=4.5e-16)
    # the derivative recovered from a = softplus(z): 1 - exp(-a) = -expm1(-a)
    a = oracle.softplus(z)
    np.testing.assert_allclose(-np.expm1(-a), d, rtol=1e-14, atol=0)
    assert np.array_equal(oracle.act_deriv(np.array([-1.0, 0.0, 2.0]), "relu"), [0.0, 0.0, 1.0])
    assert np.array_equal(oracle.act_deriv(np.array([-1.0, 0.0, 2.0]), "none"), [1.0, 1.0, 1.0])


def test_backward_rejects_bad_arguments():
    x, Ws, g = _random_chain(1, (4, 4), 3)
    with pytest.raises(ValueError):
        oracle.mlp_backward(x, Ws, g[:, :3])
    with pytest.raises(ValueError):  # at most 16 layers
        oracle.mlp_backward(x, [np.eye(4)] * 17, g)
    with pytest.raises(ValueError):
        oracle.mlp_backward(x, [np.ones((5, 4))], g)
    dWs, dx = oracle.mlp_backward(x[:0], Ws, g[:0])
    assert dx.shape == (0, 4) and np.array_equal(dWs[0], np.zeros((4, 4)))
