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
    "coalesce_bias_add": (_i32, [_p, _i64, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "coalesce_activation": (_i32, [_p, _i64, _p, _i64, _i64, _i64, _i32, _i32, _p]),
    "coalesce_flush_caches": (_i32, [_p, _sz, _p, _p]),
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


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _matrix(t: torch.Tensor, name: str):
    """(rows, cols, ld) of a 2-D device tensor with unit inner stride."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit inner stride (row-major)" % name)
    ld = t.stride(0) if rows > 1 else max(t.stride(0), cols)
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
    _check(lib.coalesce_gemm_bias_act(_ptr(A), lda, _ptr(B), ldb, _ptr(bias), _ptr(out), ldy, M, N, K,
                                      _DTYPES[A.dtype], _DTYPES[odt], _ACTS[act], _stream(stream)))
    return out


def mlp_forward(x: torch.Tensor, weights: Sequence[torch.Tensor], hidden_act="softplus",
                out: Optional[torch.Tensor] = None, num_workgroups: int = 0, stream=None):
    """out = W_L(... softplus(softplus(x W_1) W_2) ...) in one persistent launch."""
    lib = load_library()
    M, D0, ldx = _matrix(x, "x")
    L = len(weights)
    dims = [D0]
    for i, w in enumerate(weights):
        if w.dim() != 2 or not w.is_contiguous() or w.dtype != x.dtype or not w.is_cuda:
            raise ValueError("weight %d must be a contiguous 2-D device tensor of x's dtype" % i)
        if w.shape[0] != dims[-1]:
            raise ValueError("layer widths do not chain")
        dims.append(w.shape[1])
    if out is None:
        out = aligned_empty(M, dims[-1], x.dtype, x.device)
    Mo, Do, ldo = _matrix(out, "out")
    if (Mo, Do) != (M, dims[-1]):
        raise ValueError("out must be M x dims[L]")
    wp = (ctypes.c_void_p * max(L, 1))(*[w.data_ptr() for w in weights])
    dp = (ctypes.c_int64 * (L + 1))(*dims)
    _check(lib.coalesce_mlp_forward_grid(_ptr(x), ldx, ctypes.cast(wp, ctypes.c_void_p),
                                         ctypes.cast(dp, ctypes.c_void_p), L, _ptr(out), ldo, M,
                                         _DTYPES[x.dtype], _ACTS[hidden_act], int(num_workgroups), _stream(stream)))
    return out


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


def device_cu_count() -> int:
    n = load_library().coalesce_device_cu_count()
    if n <= 0:
        raise CoalesceError(ERR_DEVICE, load_library().coalesce_last_error().decode())
    return n


def version() -> int:
    return int(load_library().coalesce_version())


class FusedMLPSoftplus(torch.nn.Module):
    """Inference module with the page's constructor shape (D, H, out_features).

    Holds L weight matrices in the x @ W orientation (fp16) and runs the whole
    chain in one megakernel launch.  Forward only.
    """

    def __init__(self, D: int = 128, H: int = 128, out_features: int = 128, layers: int = 3,
                 device="cuda", dtype=torch.float16):
        super().__init__()
        dims = [D] + [H] * (layers - 1) + [out_features]
        self.weights = torch.nn.ParameterList(
            [torch.nn.Parameter(torch.empty(dims[i], dims[i + 1], device=device, dtype=dtype), requires_grad=False)
             for i in range(layers)])
        for w in self.weights:
            torch.nn.init.normal_(w, std=w.shape[0] ** -0.5)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return mlp_forward(x, [w for w in self.weights])
