"""Host-side checks of the C ABI that need no GPU.

The library must load and export every entry point declared in
include/coalesce.h, and every invalid or unsupported request must be
rejected on the host, before any device call, with the documented status
(so these run with fake pointer values and no GPU present).
"""
import ctypes
import os
import re

import pytest

import mlp_megakernel_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coalesce.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(coalesce_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(mk.SIGNATURES), "binding signatures must cover exactly the header's entry points"


def test_library_exports_every_symbol():
    lib = mk.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.coalesce_version() == 100
    assert lib.coalesce_status_string(2) == b"COALESCE_ERR_UNSUPPORTED"


P = 0x10000  # a 16-byte aligned fake device address; never dereferenced
INV, UNS = mk.ERR_INVALID_ARGUMENT, mk.ERR_UNSUPPORTED


def gemm(**kw):
    a = dict(A=P, lda=64, B=P * 2, ldb=64, bias=None, Y=P * 4, ldy=64, M=8, N=64, K=64, i=mk.F32, o=mk.F32,
             act=mk.ACT_GELU_ERF)
    a.update(kw)
    lib = mk.load_library()
    return lib.coalesce_gemm_bias_act(a["A"], a["lda"], a["B"], a["ldb"], a["bias"], a["Y"], a["ldy"], a["M"],
                                      a["N"], a["K"], a["i"], a["o"], a["act"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INV), (dict(N=-3), INV), (dict(K=-2), INV),
    (dict(i=7), INV), (dict(act=9), INV),
    (dict(Y=None), INV), (dict(A=None), INV), (dict(B=None), INV),
    (dict(lda=63), INV), (dict(ldb=10), INV), (dict(ldy=60), INV),
    (dict(i=mk.F32, o=mk.BF16), UNS), (dict(i=mk.BF16, o=mk.F16), UNS), (dict(i=mk.F16, o=mk.BF16), UNS),
    (dict(A=P + 4), UNS), (dict(Y=P + 8), UNS), (dict(bias=P * 8 + 2), UNS),
    (dict(lda=66), UNS), (dict(ldy=65), UNS),
    (dict(M=1 << 31), UNS),
    (dict(Y=P + 256), INV),  # Y overlaps A
])
def test_gemm_rejects_before_launch(kw, status):
    assert gemm(**kw) == status
    assert len(mk.load_library().coalesce_last_error()) > 0


def test_gemm_empty_is_ok_without_device():
    assert gemm(M=0) == mk.OK
    assert gemm(N=0, Y=None) == mk.OK


def mlp(D=128, L=3, dims=None, **kw):
    lib = mk.load_library()
    dims = dims if dims is not None else [D] * (L + 1)
    W = (ctypes.c_void_p * max(L, 1))(*[P * (16 + l) for l in range(L)])
    d = (ctypes.c_int64 * len(dims))(*dims)
    a = dict(x=P, ldx=D, out=P * 64, ldo=D, M=100, dt=mk.F16, act=mk.ACT_SOFTPLUS, g=0)
    a.update(kw)
    return lib.coalesce_mlp_forward_grid(a["x"], a["ldx"], ctypes.cast(W, ctypes.c_void_p),
                                         ctypes.cast(d, ctypes.c_void_p), L, a["out"], a["ldo"], a["M"], a["dt"],
                                         a["act"], a["g"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), INV), (dict(M=-1), INV), (dict(g=-1), INV), (dict(dt=5), INV), (dict(act=4), INV),
    (dict(x=None), INV), (dict(out=None), INV), (dict(ldx=100), INV), (dict(ldo=127), INV),
    (dict(dt=mk.BF16), UNS), (dict(act=mk.ACT_GELU_ERF), UNS),
    (dict(D=100), UNS), (dict(D=264, ldx=264, ldo=264), UNS), (dict(D=64, L=17), UNS),
    (dict(dims=[128, 60, 128, 128]), UNS), (dict(L=3, dims=[256, 264, 64, 64]), UNS),
    (dict(x=P + 2), UNS), (dict(ldx=132), UNS),
])
def test_mlp_rejects_before_launch(kw, status):
    assert mlp(**kw) == status


@pytest.mark.parametrize("kw", [dict(D=136, ldx=136, ldo=136), dict(D=256, ldx=256, ldo=256), dict(D=128, L=5),
                                dict(D=64, L=9), dict(D=64, L=16), dict(L=5, dims=[64, 128, 64, 64, 64, 64])])
def test_mlp_accepts_chains_beyond_lds(kw):
    # deeper or wider than the resident kernel holds: the layer-streaming
    # kernel takes them, so validation passes and the call reaches the device
    # query (which fails here, without a GPU)
    assert mlp(**kw) == mk.ERR_DEVICE


def test_mlp_empty_batch_is_ok():
    assert mlp(M=0, x=None, out=None) == mk.OK


def test_elementwise_and_flush_reject():
    lib = mk.load_library()
    assert lib.coalesce_bias_add(P, 64, P * 2, P * 4, 64, 4, 64, mk.F32, mk.F16, mk.F32, None) == UNS
    assert lib.coalesce_bias_add(P, 64, None, P * 4, 64, 4, 64, mk.F32, mk.F32, mk.F32, None) == INV
    assert lib.coalesce_activation(P, 32, P * 4, 64, 4, 64, mk.F32, mk.ACT_GELU_ERF, None) == INV
    assert lib.coalesce_activation(P, 64, P + 64, 64, 4, 64, mk.F32, mk.ACT_GELU_ERF, None) == INV
    assert lib.coalesce_flush_caches(P + 4, 1024, P, None) == UNS
    assert lib.coalesce_flush_caches(None, 1024, P, None) == INV
    assert lib.coalesce_flush_caches(None, 0, None, None) == mk.OK


def mlp_train(D=128, L=3, **kw):
    lib = mk.load_library()
    dims = [D] * (L + 1)
    W = (ctypes.c_void_p * L)(*[P * (16 + l) for l in range(L)])
    d = (ctypes.c_int64 * len(dims))(*dims)
    acts = kw.pop("acts", [P * (256 + 64 * l) for l in range(max(L - 1, 1))])
    A = None if acts is None else ctypes.cast((ctypes.c_void_p * len(acts))(*acts), ctypes.c_void_p)
    a = dict(x=P, ldx=D, out=P * 64, ldo=D, lda=D, M=100, dt=mk.F16, act=mk.ACT_SOFTPLUS)
    a.update(kw)
    return lib.coalesce_mlp_forward_train(a["x"], a["ldx"], ctypes.cast(W, ctypes.c_void_p),
                                          ctypes.cast(d, ctypes.c_void_p), L, a["out"], a["ldo"], A, a["lda"],
                                          a["M"], a["dt"], a["act"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(acts=None), INV), (dict(acts=[P * 256, None]), INV), (dict(lda=100), INV),
    (dict(acts=[P * 256 + 4, P * 320]), UNS), (dict(lda=130), UNS), (dict(lda=(1 << 24) + 4), UNS),
    (dict(acts=[P * 64, P * 320]), INV),        # acts[0] overlaps out
    (dict(acts=[P * 256, P * 256 + 512]), INV),  # acts overlap each other
    (dict(act=mk.ACT_GELU_ERF), UNS), (dict(D=64, L=17), UNS), (dict(x=None), INV),
])
def test_mlp_forward_train_rejects_before_launch(kw, status):
    assert mlp_train(**kw) == status


def test_mlp_forward_train_empty_and_single_layer_need_no_acts():
    assert mlp_train(M=0, x=None, out=None, acts=None) == mk.OK


def mlp_bwd(D=128, L=3, **kw):
    lib = mk.load_library()
    dims = [D] * (L + 1)
    W = (ctypes.c_void_p * L)(*[P * (16 + l) for l in range(L)])
    d = (ctypes.c_int64 * len(dims))(*dims)
    acts = kw.pop("acts", [P * (256 + 64 * l) for l in range(max(L - 1, 1))])
    dW = kw.pop("dW", [P * (1024 + 4 * l) for l in range(L)])
    A = None if acts is None else ctypes.cast((ctypes.c_void_p * len(acts))(*acts), ctypes.c_void_p)
    G = None if dW is None else ctypes.cast((ctypes.c_void_p * len(dW))(*dW), ctypes.c_void_p)
    a = dict(x=P, ldx=D, lda=D, dout=P * 128, ldd=D, dx=P * 192, ldq=D, M=100, dt=mk.F16, act=mk.ACT_SOFTPLUS,
             ws=P * 4096, wsb=1 << 30)
    a.update(kw)
    return lib.coalesce_mlp_backward(a["x"], a["ldx"], ctypes.cast(W, ctypes.c_void_p),
                                     ctypes.cast(d, ctypes.c_void_p), L, A, a["lda"], a["dout"], a["ldd"], G,
                                     a["dx"], a["ldq"], a["M"], a["dt"], a["act"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dW=None), INV), (dict(dW=[P * 1024, None, P * 1032]), INV), (dict(dW=[P * 1024 + 2, P * 1028, P * 1032]), UNS),
    (dict(x=None), INV), (dict(dout=None), INV), (dict(acts=None), INV), (dict(ldd=100), INV), (dict(ldq=64), INV),
    (dict(dout=P * 128 + 8), UNS), (dict(lda=129), UNS), (dict(dx=P + 64), INV),  # dx overlaps x
    (dict(act=mk.ACT_GELU_ERF), UNS), (dict(dt=mk.F32), UNS), (dict(D=64, L=17), UNS), (dict(D=264), UNS),
    (dict(D=100), UNS),
    (dict(L=0), INV), (dict(M=-5), INV), (dict(act=11), INV),
])
def test_mlp_backward_rejects_before_launch(kw, status):
    assert mlp_bwd(**kw) == status
    assert len(mk.load_library().coalesce_last_error()) > 0


@pytest.mark.parametrize("kw", [dict(D=136), dict(D=256), dict(D=128, L=5), dict(D=64, L=9), dict(D=64, L=16)])
def test_mlp_backward_accepts_chains_beyond_lds(kw):
    # run layer by layer: validation passes and the call reaches the device
    # query (which fails here, without a GPU)
    D = kw["D"]
    assert mlp_bwd(ldx=D, lda=D, ldd=D, ldq=D, **kw) == mk.ERR_DEVICE


def test_mlp_backward_workspace_size_of_unsupported_chain_is_zero():
    lib = mk.load_library()
    for dims, M in (([96, 264], 10), ([64] * 18, 10), ([100, 64], 10), ([64, 64], -1), ([256] * 4, 2 ** 31)):
        d = (ctypes.c_int64 * len(dims))(*dims)
        assert lib.coalesce_mlp_backward_workspace_size(ctypes.cast(d, ctypes.c_void_p), len(dims) - 1, M) == 0
    assert lib.coalesce_mlp_backward_workspace_size(None, 3, 10) == 0


def wn(L=3, dims=None, back=False, **kw):
    lib = mk.load_library()
    dims = dims if dims is not None else [128] * (L + 1)
    arr = lambda xs: None if xs is None else ctypes.cast((ctypes.c_void_p * len(xs))(*xs), ctypes.c_void_p)
    v = kw.pop("v", [P * (16 + 4 * l) for l in range(L)])
    g = kw.pop("g", [P * (64 + l) for l in range(L)])
    d = (ctypes.c_int64 * len(dims))(*dims)
    dt = kw.pop("dt", mk.F16)
    if not back:
        W = kw.pop("W", [P * (128 + 4 * l) for l in range(L)])
        return lib.coalesce_weight_norm(arr(v), arr(g), arr(W), ctypes.cast(d, ctypes.c_void_p), L, dt, None)
    dW = kw.pop("dW", [P * (256 + 4 * l) for l in range(L)])
    dv = kw.pop("dv", [P * (512 + 4 * l) for l in range(L)])
    dg = kw.pop("dg", [P * (768 + l) for l in range(L)])
    return lib.coalesce_weight_norm_backward(arr(v), arr(g), arr(dW), arr(dv), arr(dg), ctypes.cast(d, ctypes.c_void_p),
                                             L, dt, None)


@pytest.mark.parametrize("back", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(L=0), INV), (dict(L=17, dims=[8] * 18), UNS), (dict(dims=[128, 0, 128, 128]), INV), (dict(dt=mk.F32), UNS),
    (dict(dt=9), INV), (dict(v=None), INV), (dict(g=[P * 64, None, P * 66]), INV), (dict(v=[P * 16 + 1, P * 20, P * 24]), UNS),
])
def test_weight_norm_rejects_before_launch(back, kw, status):
    assert wn(back=back, **kw) == status
    assert len(mk.load_library().coalesce_last_error()) > 0


def test_weight_norm_output_checks():
    assert wn(W=None) == INV
    assert wn(W=[P * 128, P * 16, P * 136]) == INV        # W[1] overlaps v[0]
    assert wn(W=[P * 128 + 1, P * 132, P * 136]) == UNS   # odd address
    assert wn(back=True, dg=[P * 768, P * 768, P * 770]) == INV  # dg[0] and dg[1] coincide
    assert wn(back=True, dv=[P * 256, P * 516, P * 520]) == INV  # dv[0] overlaps dW[0]
    assert wn(back=True, dW=[P * 256 + 2, P * 260, P * 264]) == UNS


def tune_gemm(ws=P * 64, wsb=1 << 20, iters=5, **kw):
    a = dict(A=P, lda=64, B=P * 2, ldb=64, bias=None, Y=P * 4, ldy=64, M=8, N=64, K=64, i=mk.F16, o=mk.F16,
             act=mk.ACT_GELU_ERF)
    a.update(kw)
    return mk.load_library().coalesce_autotune_gemm_bias_act(
        a["A"], a["lda"], a["B"], a["ldb"], a["bias"], a["Y"], a["ldy"], a["M"], a["N"], a["K"], a["i"], a["o"],
        a["act"], iters, ws, wsb, None, None)


def tune_mlp(D=128, L=3, ws=P * 256, wsb=1 << 20, iters=5, **kw):
    W = (ctypes.c_void_p * L)(*[P * (16 + l) for l in range(L)])
    d = (ctypes.c_int64 * (L + 1))(*([D] * (L + 1)))
    a = dict(x=P, ldx=D, out=P * 64, ldo=D, M=100, act=mk.ACT_SOFTPLUS)
    a.update(kw)
    return mk.load_library().coalesce_autotune_mlp_forward(
        a["x"], a["ldx"], ctypes.cast(W, ctypes.c_void_p), ctypes.cast(d, ctypes.c_void_p), L, a["out"], a["ldo"],
        a["M"], mk.F16, a["act"], iters, ws, wsb, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(iters=0), INV), (dict(iters=10001), INV), (dict(ws=None), INV), (dict(ws=P * 64 + 8), UNS),
    (dict(wsb=8 * 64 * 2 + 255), INV),  # the reference copy (1 KiB, rounded to 256) plus 256 bytes
    (dict(ws=P * 4), INV),  # the workspace is Y
    (dict(ws=P + 64), INV),  # the workspace overlaps A
    (dict(M=-1), INV), (dict(i=7), INV), (dict(ldy=60), INV), (dict(i=mk.F16, o=mk.BF16), UNS),
])
def test_autotune_gemm_rejects_before_launch(kw, status):
    assert tune_gemm(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(iters=0), INV), (dict(ws=None), INV), (dict(wsb=100 * 256 + 255), INV), (dict(ws=P * 64), INV),
    (dict(ws=P * 17), INV), (dict(L=0), INV), (dict(D=100), UNS), (dict(act=mk.ACT_GELU_ERF), UNS),
    (dict(ldo=127), INV),
])
def test_autotune_mlp_rejects_before_launch(kw, status):
    assert tune_mlp(**kw) == status


def test_autotune_empty_and_clear_need_no_device():
    assert tune_gemm(M=0) == mk.OK
    assert tune_mlp(M=0) == mk.OK
    assert mk.load_library().coalesce_autotune_clear() == mk.OK
