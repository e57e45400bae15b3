"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties the oracle to mathematics or to the pages: tabulated closed
forms, an independent high-precision series, library routines that compute
the same special function by a different method, exact integer arithmetic,
invariants, and the pages' own test recipes ("Coalesce" README, "Notes for
future sessions": the ((i*7)%13)*0.1 / ((i*3)%11)*0.1 fills and the B = 1/N
trick that puts the accumulator at 1.0).  A plausible slip in the oracle -- a
dropped bias, a transposed operand, a bias indexed by row, a wrong GELU
constant, a naive softplus, an activation on the last MLP layer, the MLP
layers applied in the wrong order -- fails at least one of them.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "activation_closed_forms.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            fn, z, v, tol = line.split()
            rows.append((fn, float(z), float(v), float(tol)))
    return rows


@pytest.mark.parametrize("fn,z,value,tol", _golden_rows())
def test_activation_closed_forms(fn, z, value, tol):
    got = float((oracle.gelu if fn == "gelu" else oracle.softplus)(z))
    if value == 0.0:
        assert got == 0.0
    else:
        assert abs(got - value) <= tol * abs(value) + 1e-300, (fn, z, got, value)


def _erf_series(x: Decimal) -> Decimal:
    """erf by its Maclaurin series at 60 digits (independent of libm)."""
    getcontext().prec = 60
    s, n, fact = Decimal(0), 0, Decimal(1)
    while True:
        t = ((-1) ** n) * x ** (2 * n + 1) / (fact * (2 * n + 1))
        s += t
        if abs(t) < Decimal(10) ** -45:
            break
        n += 1
        fact *= n
    pi = Decimal("3.14159265358979323846264338327950288419716939937510582097494")
    return 2 / pi.sqrt() * s


@pytest.mark.parametrize("z", [-4.0, -2.5, -0.75, -0.1, 0.1, 0.3, 1.7, 2.9, 4.0])
def test_gelu_matches_high_precision_series(z):
    getcontext().prec = 60
    zz = Decimal(repr(z))
    ref = float(zz * (1 + _erf_series(zz / Decimal(2).sqrt())) / 2)
    got = float(oracle.gelu(z))
    # 1 + erf(z/sqrt2) cancels for z < 0, so the fp64 erf form is accurate to
    # about |z| * 2^-53 in absolute terms rather than relative to GELU(z).
    assert abs(got - ref) <= 4e-16 * max(abs(z), 1e-3), (z, got, ref)


def test_gelu_is_z_times_normal_cdf():
    # scipy's ndtr evaluates the normal CDF by its own route (Cephes erfc/erf);
    # GELU(z) = z * Phi(z) exactly.
    z = np.linspace(-12.0, 12.0, 2001)
    got = oracle.gelu(z)
    ref = z * scipy.special.ndtr(z)
    # relative for z > 0; absolute (|z| * 2^-53 scale) where 1 + erf cancels
    pos = z > 0
    assert np.max(np.abs(got - ref)[pos] / np.abs(ref[pos])) < 1e-15
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(z), 1e-3)) < 1e-15


def test_gelu_asymptotes():
    assert oracle.gelu(40.0) == 40.0
    assert abs(oracle.gelu(-40.0)) < 1e-300
    # odd part: GELU(z) - GELU(-z) = z (since Phi(z) + Phi(-z) = 1)
    z = np.linspace(-6, 6, 97)
    assert np.max(np.abs(oracle.gelu(z) - oracle.gelu(-z) - z)) < 1e-14


def test_softplus_against_logaddexp_and_identities():
    z = np.linspace(-60.0, 60.0, 4801)
    sp = oracle.softplus(z)
    ref = np.logaddexp(0.0, z)
    assert np.max(np.abs(sp - ref) / np.maximum(ref, 1e-300)) < 1e-14
    # softplus(z) - softplus(-z) = z
    assert np.max(np.abs(sp - oracle.softplus(-z) - z)) < 1e-13
    # strictly above max(z, 0) (where the gap e^-|z| is representable next to z)
    mid = np.abs(z) <= 30.0
    assert np.all(sp[mid] > np.maximum(z[mid], 0.0))
    assert np.all(sp >= np.maximum(z, 0.0))


def test_softplus_tails_keep_relative_accuracy():
    # ln(1 + e^z) ~ e^z for very negative z: a naive log(1 + exp(z)) gives 0 here.
    for z in (-50.0, -100.0, -700.0):
        assert abs(oracle.softplus(z) / math.exp(z) - 1.0) < 1e-15
    # no overflow for large z: softplus(z) = z + ln(1 + e^-z)
    assert oracle.softplus(1000.0) == 1000.0
    assert oracle.softplus(30.0) == 30.0 + math.exp(-30.0)


# ---------------------------------------------------------------------------
# GEMM + bias + act
# ---------------------------------------------------------------------------

SHAPES = [(1, 1, 1), (2, 3, 5), (7, 5, 3), (8, 16, 4), (17, 9, 33), (31, 65, 7), (3, 129, 64)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_integer_inputs_exact(M, N, K):
    A = datagen.to_f64(datagen.integer_matrix((M, K), 7, 3, 13, 6))
    B = datagen.to_f64(datagen.integer_matrix((K, N), 5, 11, 11, 5))
    bias = np.arange(N, dtype=np.float64) - 3.0
    exact = (A.astype(np.int64) @ B.astype(np.int64)) + bias.astype(np.int64)[None, :]
    got = oracle.gemm_bias_act(A, B, bias, act="none")
    assert np.array_equal(got, exact.astype(np.float64))


def test_gemm_accumulates_in_double():
    # Sums beyond 2^24 (not representable in float32) must still be exact.
    rng = np.random.default_rng(7)
    A = rng.integers(-4096, 4097, size=(9, 64)).astype(np.float64)
    B = rng.integers(-4096, 4097, size=(64, 11)).astype(np.float64)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.abs(exact).max() > 2 ** 25
    got = oracle.gemm_bias_act(A, B, None, act="none")
    assert np.array_equal(got, exact.astype(np.float64))


def test_gemm_pages_fill_patterns_exact_rational():
    # The README's index-exposing fills, checked against exact rational sums of
    # the very float64 values the oracle receives.
    M, K, N = 5, 7, 3
    A = datagen.to_f64(datagen.pattern_mod((M, K), 7, 13, 0.1, "f32"))
    B = datagen.to_f64(datagen.pattern_mod((K, N), 3, 11, 0.1, "f32"))
    got = oracle.gemm_bias_act(A, B, None, act="none")
    for i in range(M):
        for j in range(N):
            s = sum(Fraction(A[i, k]) * Fraction(B[k, j]) for k in range(K))
            assert abs(got[i, j] - float(s)) <= 1e-15 * max(abs(float(s)), 1.0)
    # square case: the fill tells A.B from the transposed-index mistake A^T.B,
    # which an all-ones fill cannot
    A4 = datagen.to_f64(datagen.pattern_mod((4, 4), 7, 13, 0.1, "f32"))
    B4 = datagen.to_f64(datagen.pattern_mod((4, 4), 3, 11, 0.1, "f32"))
    y4 = oracle.gemm_bias_act(A4, B4, None, act="none")
    assert np.max(np.abs(y4 - A4.T @ B4)) > 0.1
    ones = np.ones((4, 4))
    assert np.array_equal(oracle.gemm_bias_act(ones, ones, None, act="none"), ones.T @ ones)


@pytest.mark.parametrize("act,f", [("gelu", lambda b: b * scipy.special.ndtr(b)),
                                   ("softplus", lambda b: np.logaddexp(0.0, b)),
                                   ("relu", lambda b: np.where(b > 0, b, 0.0)),
                                   ("none", lambda b: b)])
def test_gemm_k0_is_act_of_bias_per_column(act, f):
    M, N = 4, 6
    bias = np.linspace(-3, 3, N)
    got = oracle.gemm_bias_act(np.zeros((M, 0)), np.zeros((0, N)), bias, act=act)
    ref = np.broadcast_to(f(bias)[None, :], (M, N))
    assert np.max(np.abs(got - ref)) < 1e-14
    # B = 0 gives the same, for any A
    got2 = oracle.gemm_bias_act(np.ones((M, 5)), np.zeros((5, N)), bias, act=act)
    assert np.max(np.abs(got2 - ref)) < 1e-14


def test_gemm_unit_accumulator_trick():
    # "Coalesce" README notes: B = 1/N puts the accumulator at 1.0, where GELU bends.
    M, K, N = 3, 256, 5
    A = np.ones((M, K))
    B = np.full((K, N), 1.0 / K)
    got = oracle.gemm_bias_act(A, B, None, act="gelu")
    assert np.all(np.abs(got - 0.8413447460685429) < 1e-15)
    bias = np.array([-2.0, -1.0, 0.0, 1.0, 2.0])
    got = oracle.gemm_bias_act(A, B, bias, act="gelu")
    ref = (1.0 + bias) * scipy.special.ndtr(1.0 + bias)
    assert np.max(np.abs(got - ref[None, :])) < 1e-14


def test_gemm_rows_and_samples_agree_with_full():
    w = datagen.FP32_512
    A, B, bias = datagen.gemm_inputs(w, M=37, N=45, K=29)
    A, B, bias = map(datagen.to_f64, (A, B, bias))
    full = oracle.gemm_bias_act(A, B, bias, act="gelu")
    rows = [36, 0, 5, 5]
    assert np.array_equal(oracle.gemm_bias_act(A, B, bias, act="gelu", rows=rows), full[rows])
    r = np.array([0, 36, 7, 12]); c = np.array([44, 0, 3, 9])
    assert np.array_equal(oracle.gemm_bias_act_at(A, B, bias, "gelu", r, c), full[r, c])
    # thread count does not change any bit (each k-sum is sequential)
    assert np.array_equal(oracle.gemm_bias_act(A, B, bias, act="gelu", nthreads=1), full)


# ---------------------------------------------------------------------------
# MLP chain
# ---------------------------------------------------------------------------

def _sp(z):
    return np.logaddexp(0.0, z)


@pytest.mark.parametrize("L", [2, 3, 5])
def test_mlp_identity_weights_closed_form(L):
    # W_l = I for every layer: out = softplus applied L-1 times, elementwise
    # (no activation after the last layer).
    D = 8
    x = np.linspace(-30.0, 30.0, 5 * D).reshape(5, D)
    out = oracle.mlp_forward(x, [np.eye(D)] * L)
    ref = x.copy()
    for _ in range(L - 1):
        ref = _sp(ref)
    assert np.max(np.abs(out - ref) / np.maximum(np.abs(ref), 1e-300)) < 1e-14


def test_mlp_layer_order_scaled_identities():
    # W_l = c_l I: out = c_3 sp(c_2 sp(c_1 x)).  Reversing the layers changes it.
    D = 4
    c = [0.5, -3.0, 2.0]
    x = np.linspace(-5, 5, 3 * D).reshape(3, D)
    out = oracle.mlp_forward(x, [ci * np.eye(D) for ci in c])
    ref = c[2] * _sp(c[1] * _sp(c[0] * x))
    assert np.max(np.abs(out - ref)) < 1e-13
    rev = c[0] * _sp(c[1] * _sp(c[2] * x))
    assert np.max(np.abs(out - rev)) > 1e-3


def test_mlp_zero_first_layer_and_zero_last_layer():
    rng = np.random.default_rng(3)
    D = 16
    x = rng.standard_normal((6, D))
    W2 = rng.standard_normal((D, D))
    W3 = rng.standard_normal((D, D))
    out = oracle.mlp_forward(x, [np.zeros((D, D)), W2, W3])
    # h1 = ln 2 everywhere, so every row is sp(ln2 * colsum(W2)) @ W3
    h2 = _sp(math.log(2.0) * W2.sum(axis=0))
    ref = np.broadcast_to(h2 @ W3, out.shape)
    assert np.max(np.abs(out - ref)) < 1e-12
    out0 = oracle.mlp_forward(x, [W2, W3, np.zeros((D, D))])
    assert np.array_equal(out0, np.zeros_like(out0))


def test_mlp_linear_chain_integer_exact_nonsquare():
    # hidden_act = none turns the chain into x W1 W2 W3 (exact integers), with
    # non-square widths so any transposed or mis-chained weight fails.
    x = datagen.to_f64(datagen.integer_matrix((5, 3), 3, 1, 7, 3))
    W1 = datagen.to_f64(datagen.integer_matrix((3, 6), 2, 5, 5, 2))
    W2 = datagen.to_f64(datagen.integer_matrix((6, 4), 1, 3, 3, 1))
    W3 = datagen.to_f64(datagen.integer_matrix((4, 2), 4, 1, 5, 2))
    out = oracle.mlp_forward(x, [W1, W2, W3], hidden_act="none")
    exact = x.astype(np.int64) @ W1.astype(np.int64) @ W2.astype(np.int64) @ W3.astype(np.int64)
    assert np.array_equal(out, exact.astype(np.float64))


def test_mlp_single_layer_is_plain_product():
    rng = np.random.default_rng(11)
    x = rng.integers(-9, 10, size=(7, 5)).astype(np.float64)
    W = rng.integers(-9, 10, size=(5, 3)).astype(np.float64)
    assert np.array_equal(oracle.mlp_forward(x, [W]), x @ W)


def test_mlp_rows_permute_and_subset():
    w = datagen.MLP3
    x, Ws = datagen.mlp_inputs(w, M=50, dims=(16, 8, 12, 4))
    x = datagen.to_f64(x); Ws = [datagen.to_f64(t) for t in Ws]
    full = oracle.mlp_forward(x, Ws)
    perm = np.random.default_rng(0).permutation(50)
    assert np.array_equal(oracle.mlp_forward(x[perm], Ws), full[perm])
    assert np.array_equal(oracle.mlp_forward(x, Ws, rows=perm[:9]), full[perm[:9]])


def test_relu_chain_by_hand_and_identity_closed_form():
    # 1 row, widths 2 -> 2 -> 1, relu between layers, evaluated by hand:
    # z1 = [1*1 + 2*0.25, 1*(-1) + 2*(-0.5)] = [1.5, -2], h1 = [1.5, 0],
    # out = 1.5*3 + 0*(-1) = 4.5
    x = np.array([[1.0, 2.0]])
    W1 = np.array([[1.0, -1.0], [0.25, -0.5]])
    W2 = np.array([[3.0], [-1.0]])
    assert oracle.mlp_forward(x, [W1, W2], hidden_act="relu")[0, 0] == 4.5
    # relu is idempotent: identity weights give out = relu(x) for any L >= 2
    xs = np.linspace(-3, 3, 24).reshape(3, 8)
    I = np.eye(8)
    for L in (2, 3, 5):
        got = oracle.mlp_forward(xs, [I] * L, hidden_act="relu")
        assert np.array_equal(got, np.where(xs > 0, xs, 0.0))
    # GEMM epilogue: relu(z) - relu(-z) = z, and relu(z) >= 0
    A = np.linspace(-2, 2, 15).reshape(5, 3)
    B = np.array([[1.0, -0.5], [2.0, 0.0], [-1.0, 3.0]])
    pos = oracle.gemm_bias_act(A, B, None, act="relu")
    neg = oracle.gemm_bias_act(-A, B, None, act="relu")
    assert np.all(pos >= 0) and np.allclose(pos - neg, oracle.gemm_bias_act(A, B, None, act="none"), atol=1e-15)


def test_mlp_small_chain_by_hand():
    # 1 row, widths 2 -> 2 -> 1, hand-evaluated.
    x = np.array([[1.0, -2.0]])
    W1 = np.array([[0.5, -1.0], [0.25, 2.0]])
    W2 = np.array([[3.0], [-1.0]])
    z1 = np.array([1.0 * 0.5 + -2.0 * 0.25, 1.0 * -1.0 + -2.0 * 2.0])  # [0, -5]
    h1 = np.array([math.log(2.0), math.log1p(math.exp(-5.0))])
    ref = 3.0 * h1[0] - h1[1]
    assert abs(oracle.mlp_forward(x, [W1, W2])[0, 0] - ref) < 1e-15
    assert z1[0] == 0.0
