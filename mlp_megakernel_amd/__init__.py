"""Python binding of libcoalesce (argument marshalling only).

Every function here takes torch tensors that live on a ROCm device, checks
that their layout matches what the C ABI expects, and passes raw pointers,
leading dimensions and the current HIP stream to the ``coalesce_*`` entry
point of the same name.  All arithmetic happens in the gfx950 kernels of
``libcoalesce.so``; there is no fallback.  If the library is missing, every
call raises.  PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoalesce.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_DEVICE = 0, 1, 2, 3
F32, F16, BF16 = 0, 1, 2
ACT_NONE, ACT_GELU_ERF, ACT_SOFTPLUS, ACT_RELU = 0, 1, 2, 3

_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_ACTS = {"none": ACT_NONE, None: ACT_NONE, "gelu": ACT_GELU_ERF, "gelu_erf": ACT_GELU_ERF,
         "softplus": ACT_SOFTPLUS, "relu": ACT_RELU}

# Every exported entry point of include/coalesce.h with its ctypes signature.
_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "coalesce_gemm_bias_act": (_i32, [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "coalesce_mlp_forward": (_i32, [_p, _i64, _p, _p, _i32, _p, _i64, _i64, _i32, _i32, _p]),
    "coalesce_mlp_forward_grid": (_i32, [_p, _i64, _p, _p, _i32, _p, _i64, _i64, _i32, _i32, _i64, _p]),
    "coalesce_mlp_forward_train": (_i32, [_p, _i64, _p, _p, _i32, _p, _i64, _p, _i64, _i64, _i32, _i32, _p]),
    "coalesce_mlp_backward_workspace_size": (_sz, [_p, _i32, _i64]),
    "coalesce_mlp_backward": (_i32, [_p, _i64, _p, _p, _i32, _p, _i64, _p, _i64, _p, _p, _i64, _i64, _i32, _i32,
                                     _p, _sz, _p]),
    "coalesce_mlp_backward_noalloc": (_i32, [_p, _i64, _p, _p, _i32, _p, _i64, _p, _i64, _p, _p, _i64, _i64, _i32,
                                             _i32, _p]),
    "coalesce_weight_norm": (_i32, [_p, _p, _p, _p, _i32, _i32, _p]),
    "coalesce_weight_norm_backward": (_i32, [_p, _p, _p, _p, _p, _p, _i32, _i32, _p]),
    "coalesce_autotune_gemm_bias_act": (_i32, [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                               _i32, _p, _sz, _p, _p]),
    "coalesce_autotune_mlp_forward": (_i32, [_p, _i64, _p, _p, _i32, _p, _i64, _i64, _i32, _i32, _i32, _p, _sz, _p,
                                             _p]),
    "coalesce_autotune_clear": (_i32, []),
    "coalesce_bias_add": (_i32, [_p, _i64, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "coalesce_activation": (_i32, [_p, _i64, _p, _i64, _i64, _i64, _i32, _i32, _p]),
    "coalesce_flush_caches": (_i32, [_p, _sz, _p, _p]),
    "coalesce_matrix_rate": (_i32, [_p, _i32, _i32, _p, _p, _i64, _p, _p, _p]),
    "coalesce_device_cu_count": (_i32, []),
    "coalesce_status_string": (ctypes.c_char_p, [_i32]),
    "coalesce_last_error": (ctypes.c_char_p, []),
    "coalesce_version": (_i32, []),
}

_lib = None


class CoalesceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libcoalesce.so (once) and attach the ctypes signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libcoalesce.so is not built (%s); run __graft_entry__.build() or "
                          "python -m mlp_megakernel_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        lib = load_library()
        raise CoalesceError(status, "%s: %s" % (lib.coalesce_status_string(status).decode(),
                                                lib.coalesce_last_error().decode()))


# The current stream's raw handle without building a torch.cuda.Stream object
# (that costs about 2.7 us a call, a third of the binding's host time on a
# small launch); torch.cuda.current_stream() where this torch lacks the hook.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> Optional[int]:
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _matrix(t: torch.Tensor, name: str):
    """(rows, cols, ld) of a 2-D device tensor with unit inner stride."""
    shape = t.shape
    if len(shape) != 2:
        raise ValueError("%s must be 2-D" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    rows, cols = shape
    st = t.stride()
    if cols > 1 and st[1] != 1:
        raise ValueError("%s must have unit inner stride (row-major)" % name)
    ld = st[0] if rows > 1 else max(st[0], cols)
    return rows, cols, ld


def aligned_empty(rows: int, cols: int, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """rows x cols tensor whose leading dimension is padded to a multiple of 16 bytes."""
    es = torch.tensor([], dtype=dtype).element_size()
    per = 16 // es
    ld = max(per, (cols + per - 1) // per * per)
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def aligned_copy(t: torch.Tensor, device="cuda") -> torch.Tensor:
    out = aligned_empty(t.shape[0], t.shape[1], t.dtype, device)
    out.copy_(t)
    return out


def gemm_bias_act(A: torch.Tensor, B: torch.Tensor, bias: Optional[torch.Tensor] = None, act="gelu",
                  out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None, stream=None):
    """Y = act(A @ B + bias) in one fused kernel (coalesce_gemm_bias_act)."""
    lib = load_library()
    M, N, K, lda, ldb, ldy, out, odt = _gemm_args(A, B, bias, out_dtype, out)
    _check(lib.coalesce_gemm_bias_act(_ptr(A), lda, _ptr(B), ldb, _ptr(bias), _ptr(out), ldy, M, N, K,
                                      _DTYPES[A.dtype], _DTYPES[odt], _ACTS[act], _stream(stream)))
    return out


def _gemm_args(A, B, bias, out_dtype, out):
    M, K, lda = _matrix(A, "A")
    K2, N, ldb = _matrix(B, "B")
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if A.dtype != B.dtype:
        raise ValueError("A and B must share a dtype")
    if bias is not None:
        if bias.dim() != 1 or bias.shape[0] != N or bias.dtype != A.dtype or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous length-N vector of the input dtype")
    odt = out_dtype or (out.dtype if out is not None else A.dtype)
    if out is None:
        out = aligned_empty(M, N, odt, A.device)
    Mo, No, ldy = _matrix(out, "out")
    if (Mo, No) != (M, N) or out.dtype != odt:
        raise ValueError("out must be M x N of out_dtype")
    return M, N, K, lda, ldb, ldy, out, odt


def _chain_dims(x: torch.Tensor, weights: Sequence[torch.Tensor]):
    M, D0, ldx = _matrix(x, "x")
    dims = [D0]
    xdt = x.dtype
    for i, w in enumerate(weights):
        shape = w.shape
        if len(shape) != 2 or w.dtype != xdt or not w.is_cuda or not w.is_contiguous():
            raise ValueError("weight %d must be a contiguous 2-D device tensor of x's dtype" % i)
        if shape[0] != dims[-1]:
            raise ValueError("layer widths do not chain")
        dims.append(shape[1])
    return M, ldx, dims


# Host arrays of pointers and widths, cached by their values: building a
# ctypes array costs about a microsecond, which matters when a small launch
# is bound by the host.  The arrays hold only the values they are keyed by.
_array_cache = {}


def _c_array(ctype, values: tuple):
    key = (ctype, values)
    arr = _array_cache.get(key)
    if arr is None:
        if len(_array_cache) >= 512:
            _array_cache.clear()
        # the cast keeps a reference to the array it points into
        arr = ctypes.cast((ctype * max(len(values), 1))(*values), ctypes.c_void_p)
        _array_cache[key] = arr
    return arr


def _ptr_array(ts):
    return _c_array(ctypes.c_void_p, tuple([t.data_ptr() for t in ts]))


def _dims_array(dims):
    return _c_array(ctypes.c_int64, tuple(dims))


def mlp_forward(x: torch.Tensor, weights: Sequence[torch.Tensor], hidden_act="softplus",
                out: Optional[torch.Tensor] = None, num_workgroups: int = 0, stream=None):
    """out = W_L(... softplus(softplus(x W_1) W_2) ...) in one persistent launch."""
    lib = load_library()
    M, ldx, dims = _chain_dims(x, weights)
    L = len(weights)
    if out is None:
        out = aligned_empty(M, dims[-1], x.dtype, x.device)
    Mo, Do, ldo = _matrix(out, "out")
    if (Mo, Do) != (M, dims[-1]):
        raise ValueError("out must be M x dims[L]")
    _check(lib.coalesce_mlp_forward_grid(_ptr(x), ldx, _ptr_array(weights), _dims_array(dims), L, _ptr(out), ldo, M,
                                         _DTYPES[x.dtype], _ACTS[hidden_act], int(num_workgroups), _stream(stream)))
    return out


def _acts_pitch(acts: Sequence[torch.Tensor], M: int, dims):
    lda = None
    for i, a in enumerate(acts):
        r, c, ld = _matrix(a, "acts[%d]" % i)
        if (r, c) != (M, dims[i + 1]) or a.dtype != torch.float32:
            raise ValueError("acts[%d] must be M x dims[%d] float32" % (i, i + 1))
        if lda is not None and ld != lda:
            raise ValueError("every acts[l] must share one leading dimension")
        lda = ld
    return lda or dims[0]


def mlp_forward_train(x: torch.Tensor, weights: Sequence[torch.Tensor], hidden_act="softplus",
                      out: Optional[torch.Tensor] = None, acts: Optional[Sequence[torch.Tensor]] = None,
                      stream=None):
    """(out, acts): the forward of mlp_forward (same bits) plus the fp32
    hidden activations h_1 .. h_{L-1} the backward needs
    (coalesce_mlp_forward_train)."""
    lib = load_library()
    M, ldx, dims = _chain_dims(x, weights)
    L = len(weights)
    if out is None:
        out = aligned_empty(M, dims[-1], x.dtype, x.device)
    Mo, Do, ldo = _matrix(out, "out")
    if (Mo, Do) != (M, dims[-1]):
        raise ValueError("out must be M x dims[L]")
    if acts is None:
        pitch = max(4, (max(dims[1:-1], default=4) + 3) // 4 * 4)
        acts = [torch.empty((M, pitch), dtype=torch.float32, device=x.device)[:, :dims[l]] for l in range(1, L)]
    if len(acts) != L - 1:
        raise ValueError("need L - 1 activation buffers")
    lda = _acts_pitch(acts, M, dims)
    _check(lib.coalesce_mlp_forward_train(_ptr(x), ldx, _ptr_array(weights), _dims_array(dims), L,
                                          _ptr(out), ldo, _ptr_array(acts) if L > 1 else None, lda, M,
                                          _DTYPES[x.dtype], _ACTS[hidden_act], _stream(stream)))
    return out, list(acts)


def mlp_backward_workspace_size(dims: Sequence[int], M: int = 0) -> int:
    """Bytes of workspace coalesce_mlp_backward needs for this chain and M
    rows here (chains whose weights fit in LDS need the same for every M)."""
    L = len(dims) - 1
    n = int(load_library().coalesce_mlp_backward_workspace_size(_dims_array(dims), L, int(M)))
    if n == 0:
        raise CoalesceError(ERR_UNSUPPORTED, "no backward for dims %s on this device" % (list(dims),))
    return n


def mlp_backward(x: torch.Tensor, weights: Sequence[torch.Tensor], acts: Sequence[torch.Tensor],
                 dout: torch.Tensor, hidden_act="softplus", want_dx: bool = True,
                 dW: Optional[Sequence[torch.Tensor]] = None, dx: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """(dW list (fp32), dx or None): the backward of the chain from the
    stored activations (coalesce_mlp_backward): one fused kernel plus a
    fixed-order reduction, or for chains whose weights do not fit in LDS one
    fused kernel and one reduction launch per layer (per pair of layers at
    widths up to 128)."""
    lib = load_library()
    M, ldx, dims = _chain_dims(x, weights)
    L = len(weights)
    Md, Dd, ldd = _matrix(dout, "dout")
    if (Md, Dd) != (M, dims[-1]) or dout.dtype != x.dtype:
        raise ValueError("dout must be M x dims[L] of x's dtype")
    if len(acts) != L - 1:
        raise ValueError("need the L - 1 stored activations")
    lda = _acts_pitch(acts, M, dims)
    if dW is None:
        dW = [torch.empty((dims[l], dims[l + 1]), dtype=torch.float32, device=x.device) for l in range(L)]
    for l, g in enumerate(dW):
        if g.shape != (dims[l], dims[l + 1]) or g.dtype != torch.float32 or not g.is_contiguous():
            raise ValueError("dW[%d] must be a contiguous dims[l] x dims[l+1] float32 tensor" % l)
    ldq = 0
    if want_dx:
        if dx is None:
            dx = aligned_empty(M, dims[0], x.dtype, x.device)
        Mq, Dq, ldq = _matrix(dx, "dx")
        if (Mq, Dq) != (M, dims[0]) or dx.dtype != x.dtype:
            raise ValueError("dx must be M x dims[0] of x's dtype")
    else:
        dx = None
    need = mlp_backward_workspace_size(dims, M)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib.coalesce_mlp_backward(_ptr(x), ldx, _ptr_array(weights), _dims_array(dims), L,
                                     _ptr_array(acts) if L > 1 else None, lda, _ptr(dout), ldd, _ptr_array(dW),
                                     _ptr(dx), ldq, M, _DTYPES[x.dtype], _ACTS[hidden_act], _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return list(dW), dx


def mlp_backward_noalloc(x: torch.Tensor, weights: Sequence[torch.Tensor], acts: Sequence[torch.Tensor],
                         dout: torch.Tensor, dW: Sequence[torch.Tensor], dx: Optional[torch.Tensor] = None,
                         hidden_act="softplus", stream=None):
    """The backward into caller-provided dW (and dx, or None to skip it)
    through coalesce_mlp_backward_noalloc, whose partial sums live in the
    library's own device scratch: the call allocates nothing."""
    lib = load_library()
    M, ldx, dims = _chain_dims(x, weights)
    L = len(weights)
    Md, Dd, ldd = _matrix(dout, "dout")
    if (Md, Dd) != (M, dims[-1]) or dout.dtype != x.dtype:
        raise ValueError("dout must be M x dims[L] of x's dtype")
    if len(acts) != L - 1 or len(dW) != L:
        raise ValueError("need the L - 1 stored activations and L weight-gradient tensors")
    lda = _acts_pitch(acts, M, dims)
    for l, g in enumerate(dW):
        if g.shape != (dims[l], dims[l + 1]) or g.dtype != torch.float32 or not g.is_contiguous():
            raise ValueError("dW[%d] must be a contiguous dims[l] x dims[l+1] float32 tensor" % l)
    ldq = 0
    if dx is not None:
        Mq, Dq, ldq = _matrix(dx, "dx")
        if (Mq, Dq) != (M, dims[0]) or dx.dtype != x.dtype:
            raise ValueError("dx must be M x dims[0] of x's dtype")
    _check(lib.coalesce_mlp_backward_noalloc(_ptr(x), ldx, _ptr_array(weights), _dims_array(dims), L,
                                             _ptr_array(acts) if L > 1 else None, lda, _ptr(dout), ldd,
                                             _ptr_array(dW), _ptr(dx), ldq, M, _DTYPES[x.dtype], _ACTS[hidden_act],
                                             _stream(stream)))
    return list(dW), dx


def _wn_dims(vs, gs):
    if len(vs) != len(gs) or not vs:
        raise ValueError("need one gain vector per weight matrix")
    dims = [vs[0].shape[0]]
    for i, (v, g) in enumerate(zip(vs, gs)):
        if v.dim() != 2 or not v.is_contiguous() or not v.is_cuda or v.dtype != torch.float16:
            raise ValueError("v[%d] must be a contiguous 2-D fp16 device tensor" % i)
        if v.shape[0] != dims[-1]:
            raise ValueError("layer widths do not chain")
        if g.shape != (v.shape[1],) or not g.is_contiguous() or g.dtype != torch.float16 or not g.is_cuda:
            raise ValueError("g[%d] must be a contiguous fp16 device vector of v's column count" % i)
        dims.append(v.shape[1])
    return dims


def weight_norm(vs: Sequence[torch.Tensor], gs: Sequence[torch.Tensor], Ws: Optional[Sequence[torch.Tensor]] = None,
                stream=None):
    """[W_l = g_l * v_l / ||v_l||] (norm per column) for all layers in one
    launch (coalesce_weight_norm)."""
    lib = load_library()
    dims = _wn_dims(vs, gs)
    if Ws is None:
        Ws = [torch.empty_like(v) for v in vs]
    for W, v in zip(Ws, vs):
        if W.shape != v.shape or W.dtype != v.dtype or not W.is_contiguous():
            raise ValueError("every W must be a contiguous tensor shaped like its v")
    _check(lib.coalesce_weight_norm(_ptr_array(vs), _ptr_array(gs), _ptr_array(Ws), _dims_array(dims),
                                    len(vs), F16, _stream(stream)))
    return list(Ws)


def weight_norm_backward(vs: Sequence[torch.Tensor], gs: Sequence[torch.Tensor], dWs: Sequence[torch.Tensor],
                         stream=None):
    """(dv list, dg list), fp32, for all layers in one launch
    (coalesce_weight_norm_backward)."""
    lib = load_library()
    dims = _wn_dims(vs, gs)
    for i, (dW, v) in enumerate(zip(dWs, vs)):
        if dW.shape != v.shape or dW.dtype != torch.float32 or not dW.is_contiguous():
            raise ValueError("dW[%d] must be a contiguous float32 tensor shaped like v[%d]" % (i, i))
    dvs = [torch.empty(v.shape, dtype=torch.float32, device=v.device) for v in vs]
    dgs = [torch.empty(g.shape, dtype=torch.float32, device=g.device) for g in gs]
    _check(lib.coalesce_weight_norm_backward(_ptr_array(vs), _ptr_array(gs), _ptr_array(dWs), _ptr_array(dvs),
                                             _ptr_array(dgs), _dims_array(dims), len(vs), F16,
                                             _stream(stream)))
    return dvs, dgs


class TuneReport(ctypes.Structure):
    """coalesce_tune_report."""
    _fields_ = [("candidates", ctypes.c_int32), ("valid", ctypes.c_int32), ("default_us", ctypes.c_float),
                ("best_us", ctypes.c_float), ("grid", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("variant", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def _tune_workspace(rows, row_bytes, device):
    n = ((rows * row_bytes + 255) // 256) * 256 + 256
    return torch.empty(n, dtype=torch.uint8, device=device)


def autotune_gemm_bias_act(A: torch.Tensor, B: torch.Tensor, bias: Optional[torch.Tensor] = None, act="gelu",
                           out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                           iters: int = 10, stream=None):
    """(Y, report dict): tune the fused GEMM's launch configuration for this
    shape (coalesce_autotune_gemm_bias_act); later gemm_bias_act calls with
    the same shape use the winner."""
    lib = load_library()
    M, N, K, lda, ldb, ldy, out, odt = _gemm_args(A, B, bias, out_dtype, out)
    ws = _tune_workspace(M, N * out.element_size(), A.device)
    rep = TuneReport()
    _check(lib.coalesce_autotune_gemm_bias_act(_ptr(A), lda, _ptr(B), ldb, _ptr(bias), _ptr(out), ldy, M, N, K,
                                               _DTYPES[A.dtype], _DTYPES[odt], _ACTS[act], int(iters), _ptr(ws),
                                               ws.numel(), ctypes.byref(rep), _stream(stream)))
    return out, rep.as_dict()


def autotune_mlp_forward(x: torch.Tensor, weights: Sequence[torch.Tensor], hidden_act="softplus",
                         out: Optional[torch.Tensor] = None, iters: int = 10, stream=None):
    """(out, report dict): tune the megakernel's grid for this chain and
    batch (coalesce_autotune_mlp_forward); later mlp_forward calls with the
    same shape use the winner."""
    lib = load_library()
    M, ldx, dims = _chain_dims(x, weights)
    L = len(weights)
    if out is None:
        out = aligned_empty(M, dims[-1], x.dtype, x.device)
    Mo, Do, ldo = _matrix(out, "out")
    if (Mo, Do) != (M, dims[-1]):
        raise ValueError("out must be M x dims[L]")
    ws = _tune_workspace(M, dims[-1] * out.element_size(), x.device)
    rep = TuneReport()
    _check(lib.coalesce_autotune_mlp_forward(_ptr(x), ldx, _ptr_array(weights), _dims_array(dims), L,
                                             _ptr(out), ldo, M, _DTYPES[x.dtype], _ACTS[hidden_act], int(iters),
                                             _ptr(ws), ws.numel(), ctypes.byref(rep), _stream(stream)))
    return out, rep.as_dict()


def autotune_clear():
    """Forget all tuned configurations."""
    _check(load_library().coalesce_autotune_clear())


def bias_add(X: torch.Tensor, bias: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """Y = X + bias (unfused baseline step)."""
    lib = load_library()
    M, N, ldx = _matrix(X, "X")
    if out is None:
        out = aligned_empty(M, N, X.dtype, X.device)
    _, _, ldy = _matrix(out, "out")
    dt = _DTYPES[X.dtype]
    _check(lib.coalesce_bias_add(_ptr(X), ldx, _ptr(bias), _ptr(out), ldy, M, N, dt, _DTYPES[bias.dtype],
                                 _DTYPES[out.dtype], _stream(stream)))
    return out


def activation(X: torch.Tensor, act="gelu", out: Optional[torch.Tensor] = None, stream=None):
    """Y = act(X) elementwise (unfused baseline step)."""
    lib = load_library()
    M, N, ldx = _matrix(X, "X")
    if out is None:
        out = aligned_empty(M, N, X.dtype, X.device)
    _, _, ldy = _matrix(out, "out")
    _check(lib.coalesce_activation(_ptr(X), ldx, _ptr(out), ldy, M, N, _DTYPES[X.dtype], _ACTS[act],
                                   _stream(stream)))
    return out


def flush_caches(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream ``buf`` through L2 / MALL (timing harness helper)."""
    lib = load_library()
    _check(lib.coalesce_flush_caches(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def matrix_rate(ops: torch.Tensor, iters: int, sink: torch.Tensor, clocks: torch.Tensor, stream=None):
    """Run the matrix-core rate probe once (benchmark helper).  ``ops`` holds
    nsets x 24 x 64 x 8 bf16 operand fragments, ``sink`` float32 and ``clocks``
    int64 of at least 64 and 2 entries per wave.  Returns (waves,
    wallclock_khz); FLOP of the launch = waves x iters x 2^20."""
    lib = load_library()
    if ops.dtype != torch.bfloat16 or ops.numel() % (24 * 64 * 8):
        raise ValueError("ops must be bf16 with a multiple of 24 x 64 x 8 elements")
    if sink.dtype != torch.float32 or clocks.dtype != torch.int64:
        raise ValueError("sink must be float32 and clocks int64")
    cap = min(sink.numel() // 64, clocks.numel() // 2)
    waves, khz = ctypes.c_int32(0), ctypes.c_int64(0)
    _check(lib.coalesce_matrix_rate(_ptr(ops), ops.numel() // (24 * 64 * 8), int(iters), _ptr(sink), _ptr(clocks),
                                    cap, ctypes.byref(waves), ctypes.byref(khz), _stream(stream)))
    return waves.value, khz.value


def matrix_rate_waves() -> int:
    """Wave count of the matrix-core rate probe's launch on the current device."""
    lib = load_library()
    waves, khz = ctypes.c_int32(0), ctypes.c_int64(0)
    lib.coalesce_matrix_rate(None, 0, 0, None, None, 0, ctypes.byref(waves), ctypes.byref(khz), None)
    return waves.value


def device_cu_count() -> int:
    n = load_library().coalesce_device_cu_count()
    if n <= 0:
        raise CoalesceError(ERR_DEVICE, load_library().coalesce_last_error().decode())
    return n


def version() -> int:
    return int(load_library().coalesce_version())


class _FusedMLPFunction(torch.autograd.Function):
    """Training pair as one autograd node: forward = the training megakernel
    (which stores the fp32 hidden activations), backward = the fused backward.
    Weight gradients are computed in fp32 and returned in the weights' dtype."""

    @staticmethod
    def forward(ctx, x, hidden_act, *weights):
        out, acts = mlp_forward_train(x, list(weights), hidden_act=hidden_act)
        ctx.hidden_act = hidden_act
        ctx.save_for_backward(x, *weights, *acts)
        ctx.L = len(weights)
        return out

    @staticmethod
    def backward(ctx, dout):
        saved = ctx.saved_tensors
        L = ctx.L
        x, weights, acts = saved[0], list(saved[1:1 + L]), list(saved[1 + L:])
        if dout.dim() != 2 or dout.stride(-1) != 1 or (dout.data_ptr() % 16) or (dout.stride(0) * 2) % 16:
            dout = aligned_copy(dout.to(x.dtype), dout.device)
        dW, dx = mlp_backward(x, weights, acts, dout.to(x.dtype), hidden_act=ctx.hidden_act,
                              want_dx=ctx.needs_input_grad[0])
        return (dx, None) + tuple(g.to(w.dtype) for g, w in zip(dW, weights))


class FusedMLPSoftplus(torch.nn.Module):
    """Module with the page's constructor shape (D, H, out_features).

    Holds L weight matrices in the x @ W orientation (fp16).  Without
    gradients the forward is the inference megakernel; when a weight requires
    a gradient (or x does) it runs the training forward and its backward is
    the fused backward kernel.
    """

    def __init__(self, D: int = 128, H: int = 128, out_features: int = 128, layers: int = 3,
                 device="cuda", dtype=torch.float16, hidden_act="softplus", requires_grad: bool = True):
        super().__init__()
        dims = [D] + [H] * (layers - 1) + [out_features]
        self.hidden_act = hidden_act
        self.weights = torch.nn.ParameterList(
            [torch.nn.Parameter(torch.empty(dims[i], dims[i + 1], device=device, dtype=dtype),
                                requires_grad=requires_grad) for i in range(layers)])
        with torch.no_grad():
            for w in self.weights:
                torch.nn.init.normal_(w, std=w.shape[0] ** -0.5)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        ws = [w for w in self.weights]
        if torch.is_grad_enabled() and (x.requires_grad or any(w.requires_grad for w in ws)):
            return _FusedMLPFunction.apply(x, self.hidden_act, *ws)
        return mlp_forward(x, ws, hidden_act=self.hidden_act)


class _FusedMLPWNFunction(torch.autograd.Function):
    """Training step of the weight-normalised chain: one launch normalises
    every layer, the training megakernel runs the chain, and the backward is
    the fused backward followed by one weight-normalisation backward launch."""

    @staticmethod
    def forward(ctx, x, hidden_act, L, *vg):
        vs, gs = list(vg[:L]), list(vg[L:])
        Ws = weight_norm(vs, gs)
        out, acts = mlp_forward_train(x, Ws, hidden_act=hidden_act)
        ctx.hidden_act = hidden_act
        ctx.L = L
        ctx.save_for_backward(x, *vs, *gs, *Ws, *acts)
        return out

    @staticmethod
    def backward(ctx, dout):
        L = ctx.L
        saved = ctx.saved_tensors
        x, vs, gs, Ws, acts = saved[0], list(saved[1:1 + L]), list(saved[1 + L:1 + 2 * L]), \
            list(saved[1 + 2 * L:1 + 3 * L]), list(saved[1 + 3 * L:])
        if dout.dim() != 2 or dout.stride(-1) != 1 or (dout.data_ptr() % 16) or (dout.stride(0) * 2) % 16:
            dout = aligned_copy(dout.to(x.dtype), dout.device)
        dW, dx = mlp_backward(x, Ws, acts, dout.to(x.dtype), hidden_act=ctx.hidden_act,
                              want_dx=ctx.needs_input_grad[0])
        dvs, dgs = weight_norm_backward(vs, gs, dW)
        return (dx, None, None) + tuple(d.to(v.dtype) for d, v in zip(dvs, vs)) + \
            tuple(d.to(g.dtype) for d, g in zip(dgs, gs))


class FusedMLPSoftplusWN(torch.nn.Module):
    """The weight-normalised module of the page's quick start: parameters
    v_l (direction) and g_l (one gain per output unit), W_l = g_l v_l / ||v_l||
    computed for all layers in one launch before the megakernel."""

    def __init__(self, D: int = 128, H: int = 128, out_features: int = 128, layers: int = 3,
                 device="cuda", dtype=torch.float16, hidden_act="softplus"):
        super().__init__()
        dims = [D] + [H] * (layers - 1) + [out_features]
        self.hidden_act = hidden_act
        self.v = torch.nn.ParameterList(
            [torch.nn.Parameter(torch.empty(dims[i], dims[i + 1], device=device, dtype=dtype)) for i in range(layers)])
        self.g = torch.nn.ParameterList(
            [torch.nn.Parameter(torch.empty(dims[i + 1], device=device, dtype=dtype)) for i in range(layers)])
        with torch.no_grad():
            for v, g in zip(self.v, self.g):
                torch.nn.init.normal_(v, std=v.shape[0] ** -0.5)
                g.copy_(v.float().norm(dim=0).to(dtype))  # W starts equal to v

    def weights(self):
        return weight_norm([v for v in self.v], [g for g in self.g])

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        vs, gs = [v for v in self.v], [g for g in self.g]
        if torch.is_grad_enabled() and (x.requires_grad or any(p.requires_grad for p in vs + gs)):
            return _FusedMLPWNFunction.apply(x, self.hidden_act, len(vs), *vs, *gs)
        return mlp_forward(x, weight_norm(vs, gs), hidden_act=self.hidden_act)
