"""Plain fp64 CPU oracle for the fused GEMM epilogue and the softplus MLP chain
(forward, and the training pair: forward with stored activations, backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP library
never calls it and shares no code with it; the two meet only through the
seeded inputs of ``datagen`` (which holds none of the method's arithmetic).

The arithmetic lives in ``coalesce_oracle.c`` (naive loops, double precision,
OpenMP over rows), built with gcc by :func:`build`.  This module only
marshals numpy arrays.  What each function computes, with the passages it
follows, is stated in that C file and in the docstrings below.

Every input must already hold the exact values the GPU consumed, widened to
float64 (bf16, fp16 and fp32 all widen to float64 exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coalesce_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT_NONE, ACT_GELU_ERF, ACT_SOFTPLUS, ACT_RELU = 0, 1, 2, 3
_ACTS = {"none": ACT_NONE, "gelu": ACT_GELU_ERF, "gelu_erf": ACT_GELU_ERF, "softplus": ACT_SOFTPLUS, "relu": ACT_RELU}

_lib = None


def build(force: bool = True) -> str:
    """Compile coalesce_oracle.c into liboracle.so with gcc (host only)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    d, i64, i32 = ctypes.c_double, ctypes.c_int64, ctypes.c_int
    p = ctypes.c_void_p
    lib.oracle_gelu.restype = d
    lib.oracle_gelu.argtypes = [d]
    lib.oracle_softplus.restype = d
    lib.oracle_softplus.argtypes = [d]
    lib.oracle_max_threads.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_gemm_bias_act.restype = i32
    lib.oracle_gemm_bias_act.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, i32]
    lib.oracle_gemm_bias_act_at.restype = i32
    lib.oracle_gemm_bias_act_at.argtypes = [p, p, p, p, p, i64, p, i64, i64, i64, i32, i32]
    lib.oracle_mlp_forward.restype = i32
    lib.oracle_mlp_forward.argtypes = [p, p, p, i32, p, p, i64, i64, i32, i32]
    lib.oracle_act_deriv.restype = d
    lib.oracle_act_deriv.argtypes = [d, i32]
    lib.oracle_mlp_forward_train.restype = i32
    lib.oracle_mlp_forward_train.argtypes = [p, p, p, i32, p, p, i64, i32, i32]
    lib.oracle_weight_norm.restype = i32
    lib.oracle_weight_norm.argtypes = [p, p, p, i64, i64]
    lib.oracle_weight_norm_backward.restype = i32
    lib.oracle_weight_norm_backward.argtypes = [p, p, p, p, p, i64, i64]
    lib.oracle_mlp_backward.restype = i32
    lib.oracle_mlp_backward.argtypes = [p, p, p, i32, p, p, p, i64, i32, i32]
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _act(act) -> int:
    if isinstance(act, str):
        return _ACTS[act]
    return int(act)


def max_threads() -> int:
    """Threads the oracle's OpenMP loops use by default."""
    return int(_load().oracle_max_threads())


def gelu(z) -> np.ndarray:
    """GELU, erf form: 0.5 z (1 + erf(z / sqrt 2)) ("Coalesce" README, notes)."""
    lib = _load()
    z = np.asarray(z, dtype=np.float64)
    return np.vectorize(lib.oracle_gelu, otypes=[np.float64])(z)


def softplus(z) -> np.ndarray:
    """softplus(z) = ln(1 + e^z), exact in fp64 ("MLP Megakernel" README)."""
    lib = _load()
    z = np.asarray(z, dtype=np.float64)
    return np.vectorize(lib.oracle_softplus, otypes=[np.float64])(z)


def gemm_bias_act(A, B, bias=None, act="gelu", rows: Optional[Sequence[int]] = None,
                  nthreads: int = 0) -> np.ndarray:
    """Y = act(A @ B + bias), fp64 naive triple loop.

    A: M x K, B: K x N, bias: length N or None.  ``rows`` selects a subset of
    the M rows (the result then has len(rows) rows).
    Pages: "Coalesce" README, "Fusion study" (the fused GEMM + bias + GELU).
    """
    lib = _load()
    A = _f64(A)
    B = _f64(B)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    b = None if bias is None else _f64(bias).reshape(-1)
    if b is not None and b.shape[0] != N:
        raise ValueError("bias must have N elements")
    if rows is None:
        r = None
        nrows = M
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = r.shape[0]
    Y = np.empty((nrows, N), dtype=np.float64)
    rc = lib.oracle_gemm_bias_act(_ptr(A), _ptr(B), _ptr(b), _ptr(Y), _ptr(r), nrows, M, N, K, _act(act),
                                  nthreads)
    if rc != 0:
        raise ValueError("oracle_gemm_bias_act rejected its arguments")
    return Y


def gemm_bias_act_at(A, B, bias, act, rows, cols, nthreads: int = 0) -> np.ndarray:
    """act(sum_k A[i,k] B[k,j] + bias[j]) for each sampled (i, j) pair."""
    lib = _load()
    A = _f64(A)
    B = _f64(B)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    b = None if bias is None else _f64(bias).reshape(-1)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    if r.shape != c.shape:
        raise ValueError("rows and cols must pair up")
    out = np.empty(r.shape[0], dtype=np.float64)
    rc = lib.oracle_gemm_bias_act_at(_ptr(A), _ptr(B), _ptr(b), _ptr(r), _ptr(c), r.shape[0], _ptr(out), M, N,
                                     K, _act(act), nthreads)
    if rc != 0:
        raise ValueError("oracle_gemm_bias_act_at rejected its arguments")
    return out


def mlp_forward(x, weights: Sequence, rows: Optional[Sequence[int]] = None, hidden_act="softplus",
                nthreads: int = 0) -> np.ndarray:
    """out = W_L(... softplus(softplus(x W_1) W_2) ...), no biases, last layer linear.

    x: M x d_0; weights[l]: d_l x d_{l+1} (the x @ W orientation).
    Pages: "MLP Megakernel" README, "Architecture".
    """
    lib = _load()
    x = _f64(x)
    Ws = [_f64(w) for w in weights]
    L = len(Ws)
    if L < 1:
        raise ValueError("need at least one layer")
    M, d0 = x.shape
    dims = [d0]
    for w in Ws:
        if w.shape[0] != dims[-1]:
            raise ValueError("layer widths do not chain")
        dims.append(w.shape[1])
    dims_arr = np.asarray(dims, dtype=np.int64)
    wptrs = (ctypes.c_void_p * L)(*[w.ctypes.data for w in Ws])
    if rows is None:
        r = None
        nrows = M
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = r.shape[0]
    out = np.empty((nrows, dims[-1]), dtype=np.float64)
    rc = lib.oracle_mlp_forward(_ptr(x), ctypes.cast(wptrs, ctypes.c_void_p), _ptr(dims_arr), L, _ptr(out), _ptr(r),
                                nrows, M, _act(hidden_act), nthreads)
    if rc != 0:
        raise ValueError("oracle_mlp_forward rejected its arguments")
    return out


def _chain(x, weights):
    x = _f64(x)
    Ws = [_f64(w) for w in weights]
    if len(Ws) < 1:
        raise ValueError("need at least one layer")
    if len(Ws) > 16:
        raise ValueError("at most 16 layers")
    M, d0 = x.shape
    dims = [d0]
    for w in Ws:
        if w.shape[0] != dims[-1]:
            raise ValueError("layer widths do not chain")
        dims.append(w.shape[1])
    return x, Ws, M, dims


def act_deriv(z, act="softplus") -> np.ndarray:
    """d act / dz: the logistic sigmoid for softplus, the step for relu, 1 for none."""
    lib = _load()
    z = np.asarray(z, dtype=np.float64)
    a = _act(act)
    return np.vectorize(lambda v: lib.oracle_act_deriv(v, a), otypes=[np.float64])(z)


def mlp_forward_train(x, weights: Sequence, hidden_act="softplus", nthreads: int = 0):
    """(out, [h_1 .. h_{L-1}]): the forward chain and the hidden activations
    h_l = act(z_l) that the training forward stores for the backward
    ("MLP Megakernel" README, "Key ideas")."""
    lib = _load()
    x, Ws, M, dims = _chain(x, weights)
    L = len(Ws)
    out = np.empty((M, dims[-1]), dtype=np.float64)
    acts = [np.empty((M, dims[l]), dtype=np.float64) for l in range(1, L)]
    wptrs = (ctypes.c_void_p * L)(*[w.ctypes.data for w in Ws])
    aptrs = (ctypes.c_void_p * max(1, L - 1))(*[a.ctypes.data for a in acts])
    dims_arr = np.asarray(dims, dtype=np.int64)
    rc = lib.oracle_mlp_forward_train(_ptr(x), ctypes.cast(wptrs, ctypes.c_void_p), _ptr(dims_arr), L, _ptr(out),
                                      ctypes.cast(aptrs, ctypes.c_void_p) if L > 1 else None, M,
                                      _act(hidden_act), nthreads)
    if rc != 0:
        raise ValueError("oracle_mlp_forward_train rejected its arguments")
    return out, acts


def mlp_backward(x, weights: Sequence, dout, hidden_act="softplus", want_dx: bool = True, nthreads: int = 0):
    """([dW_1 .. dW_L], dx or None): gradients of sum(dout * out) with respect
    to every weight and to x, by the chain rule in fp64, the forward
    recomputed from x and W ("MLP Megakernel" README, "Key ideas"; the
    backward multiplies by softplus' derivative, the logistic sigmoid)."""
    lib = _load()
    x, Ws, M, dims = _chain(x, weights)
    L = len(Ws)
    g = _f64(dout)
    if g.shape != (M, dims[-1]):
        raise ValueError("dout must be M x dims[L]")
    dWs = [np.empty((dims[l], dims[l + 1]), dtype=np.float64) for l in range(L)]
    dx = np.empty((M, dims[0]), dtype=np.float64) if want_dx else None
    wptrs = (ctypes.c_void_p * L)(*[w.ctypes.data for w in Ws])
    gptrs = (ctypes.c_void_p * L)(*[w.ctypes.data for w in dWs])
    dims_arr = np.asarray(dims, dtype=np.int64)
    rc = lib.oracle_mlp_backward(_ptr(x), ctypes.cast(wptrs, ctypes.c_void_p), _ptr(dims_arr), L, _ptr(g),
                                 ctypes.cast(gptrs, ctypes.c_void_p), _ptr(dx), M, _act(hidden_act), nthreads)
    if rc != 0:
        raise ValueError("oracle_mlp_backward rejected its arguments")
    return dWs, dx


def weight_norm(v, g) -> np.ndarray:
    """W = g * v / ||v|| per output unit (column of the x @ W matrix)
    ("MLP Megakernel" README, "Key ideas": fused weight normalisation)."""
    lib = _load()
    v = _f64(v)
    g = _f64(g).reshape(-1)
    din, dout = v.shape
    if g.shape[0] != dout:
        raise ValueError("g must have one gain per output unit")
    W = np.empty_like(v)
    if lib.oracle_weight_norm(_ptr(v), _ptr(g), _ptr(W), din, dout) != 0:
        raise ValueError("oracle_weight_norm rejected its arguments")
    return W


def weight_norm_backward(v, g, dW):
    """(dv, dg): gradients of sum(dW * weight_norm(v, g)) with respect to v and g."""
    lib = _load()
    v = _f64(v)
    g = _f64(g).reshape(-1)
    dW = _f64(dW)
    din, dout = v.shape
    if g.shape[0] != dout or dW.shape != v.shape:
        raise ValueError("shapes of v, g and dW do not match")
    dv = np.empty_like(v)
    dg = np.empty(dout, dtype=np.float64)
    if lib.oracle_weight_norm_backward(_ptr(v), _ptr(g), _ptr(dW), _ptr(dv), _ptr(dg), din, dout) != 0:
        raise ValueError("oracle_weight_norm_backward rejected its arguments")
    return dv, dg
