"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds none of the method's arithmetic: it only draws numbers.
Both the HIP path and the oracle consume what it returns, so neither has to
import the other.

Recipe (the same everywhere):
  * generator: numpy ``default_rng([seed_id, tensor_id])`` (PCG64 seeded
    through a SeedSequence);
  * uniform tensors are ``2u - 1`` with u ~ U[0, 1), i.e. U[-1, 1);
  * normal tensors are standard normal draws times the standard deviation
    (``N(0, s)`` on the workload descriptions is read as s = standard
    deviation, so pre-activations come out at about unit scale);
  * values are drawn in float64, rounded to float32 (round to nearest even),
    then to bf16/fp16 (round to nearest even) when the input type is 16-bit;
  * tensor ids: A = 1, B = 2, bias = 3, x = 10, W_l = 10 + l (l = 1..L),
    the upstream gradient dout of the MLP backward = 30, weight-normalisation
    directions v_l = 40 + l and gains g_l = 60 + l.

Workloads (``WORKLOADS``) carry the shapes and value distributions of the
pages' problems: the FP32 square GEMM + bias + GELU shapes of the "Coalesce"
README's kernel sweep, a bf16 FFN up-projection, and the 3- and 5-layer
softplus MLPs of the "MLP Megakernel" README at large batch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

TENSOR_A, TENSOR_B, TENSOR_BIAS, TENSOR_X = 1, 2, 3, 10
TENSOR_DOUT = 30


def tensor_w(layer: int) -> int:
    """Tensor id of the weight of layer ``layer`` (1-based)."""
    return 10 + layer


_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _rng(seed_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(seed_id), int(tensor_id)])


def _quantize(a64: np.ndarray, dtype: str) -> torch.Tensor:
    a32 = torch.from_numpy(np.ascontiguousarray(a64.astype(np.float32)))
    if dtype == "f32":
        return a32
    return a32.to(_TORCH_DT[dtype])


def uniform(seed_id: int, tensor_id: int, shape: Sequence[int], dtype: str = "f32") -> torch.Tensor:
    """U[-1, 1) drawn as 2u - 1, rounded to ``dtype``; a CPU tensor."""
    u = _rng(seed_id, tensor_id).random(tuple(shape), dtype=np.float64)
    return _quantize(2.0 * u - 1.0, dtype)


def normal(seed_id: int, tensor_id: int, shape: Sequence[int], std: float, dtype: str = "f32") -> torch.Tensor:
    """N(0, std^2) (std is the standard deviation), rounded to ``dtype``; a CPU tensor."""
    g = _rng(seed_id, tensor_id).standard_normal(tuple(shape), dtype=np.float64)
    return _quantize(g * float(std), dtype)


# ---------------------------------------------------------------------------
# Structured test patterns (exact values; used to expose index mistakes).
# ---------------------------------------------------------------------------

def pattern_mod(shape: Sequence[int], mul: int, mod: int, scale: float, dtype: str = "f32") -> torch.Tensor:
    """Flat-index pattern ((i * mul) % mod) * scale.

    The "Coalesce" README's notes give ((i*7)%13)*0.1 and ((i*3)%11)*0.1 as
    the fills that expose transposed indices, where an all-ones fill hides
    them.
    """
    n = int(np.prod(shape))
    i = np.arange(n, dtype=np.int64)
    v = ((i * mul) % mod).astype(np.float64) * scale
    return _quantize(v.reshape(tuple(shape)), dtype)


def integer_matrix(shape: Sequence[int], a: int, b: int, mod: int, offset: int, dtype: str = "f32") -> torch.Tensor:
    """M[i, k] = ((a*i + b*k) mod ``mod``) - offset: small integers, exact in every input type."""
    r, c = shape
    i = np.arange(r, dtype=np.int64)[:, None]
    k = np.arange(c, dtype=np.int64)[None, :]
    v = ((a * i + b * k) % mod - offset).astype(np.float64)
    return _quantize(v, dtype)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class GemmWorkload:
    name: str
    seed_id: int
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    dist: str                # "uniform" (A, B, bias ~ U[-1,1)) or "ffn" (normal, see below)
    act: str = "gelu"
    description: str = ""

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def bytes(self) -> float:
        """Algorithmic bytes: A, B, bias read once and Y written once."""
        isz = 4 if self.in_dtype == "f32" else 2
        osz = 4 if self.out_dtype == "f32" else 2
        return float(isz * (self.M * self.K + self.K * self.N + self.N) + osz * self.M * self.N)


@dataclass(frozen=True)
class MlpWorkload:
    name: str
    seed_id: int
    M: int
    dims: Tuple[int, ...]
    dtype: str = "f16"
    description: str = ""

    @property
    def L(self) -> int:
        return len(self.dims) - 1

    def flops(self) -> float:
        return 2.0 * self.M * sum(self.dims[i] * self.dims[i + 1] for i in range(self.L))

    def bytes(self) -> float:
        """Algorithmic bytes: x read once, out written once (weights are a few KB)."""
        return 2.0 * self.M * (self.dims[0] + self.dims[-1])


WORKLOADS: Dict[str, object] = {}


def _reg(w):
    WORKLOADS[w.name] = w
    return w


FP32_512 = _reg(GemmWorkload("fp32_gemm_gelu_512", 1, 512, 512, 512, "f32", "f32", "uniform",
                             description="FP32 GEMM+bias+GELU(erf), M=N=K=512, U[-1,1) operands"))
FP32_1024 = _reg(GemmWorkload("fp32_gemm_gelu_1024", 2, 1024, 1024, 1024, "f32", "f32", "uniform",
                              description="FP32 GEMM+bias+GELU(erf), M=N=K=1024"))
FP32_2048 = _reg(GemmWorkload("fp32_gemm_gelu_2048", 2, 2048, 2048, 2048, "f32", "f32", "uniform",
                              description="FP32 GEMM+bias+GELU(erf), M=N=K=2048"))
FP32_4096 = _reg(GemmWorkload("fp32_gemm_gelu_4096", 2, 4096, 4096, 4096, "f32", "f32", "uniform",
                              description="FP32 GEMM+bias+GELU(erf), M=N=K=4096"))
BF16_FFN = _reg(GemmWorkload("bf16_ffn_up_gelu", 3, 8192, 16384, 4096, "bf16", "bf16", "ffn",
                             description="bf16 FFN up-projection + bias + GELU(erf): M=8192 tokens, K=4096, "
                                         "N=16384; A~N(0,1), B~N(0,1/64), bias~N(0,0.02)"))
MLP3 = _reg(MlpWorkload("fp16_mlp3_d128", 4, 1 << 20, (128, 128, 128, 128), "f16",
                        description="fp16 3-layer softplus MLP, D=H=out=128, 2^20 rows, x~N(0,1), "
                                    "W~N(0,1/sqrt(128))"))
MLP5 = _reg(MlpWorkload("fp16_mlp5_d64", 5, 1 << 22, (64, 64, 64, 64, 64, 64), "f16",
                        description="fp16 5-layer softplus MLP, D=H=out=64, 2^22 rows, x~N(0,1), "
                                    "W~N(0,1/8)"))
# Non-square chains of the quick start's FusedMLPSoftplus(D, H, out_features)
# kind (narrow input and output, wide hidden layers), same value recipe.
MLP_NS1 = _reg(MlpWorkload("fp16_mlp_32_128_128_16", 6, 1 << 20, (32, 128, 128, 16), "f16",
                           description="fp16 3-layer softplus MLP 32 -> 128 -> 128 -> 16, 2^20 rows"))
MLP_NS2 = _reg(MlpWorkload("fp16_mlp_64_128_96_128_32", 7, 1 << 20, (64, 128, 96, 128, 32), "f16",
                           description="fp16 4-layer softplus MLP 64 -> 128 -> 96 -> 128 -> 32, 2^20 rows"))
# Chains whose weights exceed the LDS (the N-layer generalisation: deeper and
# wider than the resident megakernel holds), same value recipe.
MLP6 = _reg(MlpWorkload("fp16_mlp6_d128", 8, 1 << 20, (128,) * 7, "f16",
                        description="fp16 6-layer softplus MLP, D=H=out=128 (192 KB of weights), 2^20 rows"))
MLP3W = _reg(MlpWorkload("fp16_mlp3_d256", 9, 1 << 20, (256,) * 4, "f16",
                         description="fp16 3-layer softplus MLP, D=H=out=256 (384 KB of weights), 2^20 rows"))


def gemm_inputs(w: GemmWorkload, M: Optional[int] = None, N: Optional[int] = None, K: Optional[int] = None):
    """(A, B, bias) CPU tensors for a GEMM workload (optionally resized, same recipe)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    if w.dist == "uniform":
        A = uniform(w.seed_id, TENSOR_A, (M, K), w.in_dtype)
        B = uniform(w.seed_id, TENSOR_B, (K, N), w.in_dtype)
        bias = uniform(w.seed_id, TENSOR_BIAS, (N,), w.in_dtype)
    elif w.dist == "ffn":
        A = normal(w.seed_id, TENSOR_A, (M, K), 1.0, w.in_dtype)
        B = normal(w.seed_id, TENSOR_B, (K, N), 1.0 / np.sqrt(K), w.in_dtype)
        bias = normal(w.seed_id, TENSOR_BIAS, (N,), 0.02, w.in_dtype)
    else:
        raise ValueError(w.dist)
    return A, B, bias


def mlp_inputs(w: MlpWorkload, M: Optional[int] = None, dims: Optional[Sequence[int]] = None):
    """(x, [W_1..W_L]) CPU tensors: x ~ N(0,1), W_l ~ N(0, 1/sqrt(d_{l-1}))."""
    M = w.M if M is None else M
    dims = tuple(w.dims if dims is None else dims)
    x = normal(w.seed_id, TENSOR_X, (M, dims[0]), 1.0, w.dtype)
    Ws = [normal(w.seed_id, tensor_w(l + 1), (dims[l], dims[l + 1]), 1.0 / np.sqrt(dims[l]), w.dtype)
          for l in range(len(dims) - 1)]
    return x, Ws


def mlp_grad_output(w: MlpWorkload, M: Optional[int] = None, dims: Optional[Sequence[int]] = None):
    """dout (M x d_L, the MLP's dtype) ~ N(0, 1): the upstream gradient fed to
    the backward (a unit-scale stand-in for dL/d(out) of a training loss)."""
    M = w.M if M is None else M
    dims = tuple(w.dims if dims is None else dims)
    return normal(w.seed_id, TENSOR_DOUT, (M, dims[-1]), 1.0, w.dtype)


def wn_inputs(w: MlpWorkload, dims: Optional[Sequence[int]] = None):
    """([v_1..v_L], [g_1..g_L]) CPU tensors of a weight-normalised chain:
    v_l ~ N(0, 1/sqrt(d_{l-1})) (d_{l-1} x d_l), g_l ~ N(1, 0.25) (d_l), in
    the workload's dtype."""
    dims = tuple(w.dims if dims is None else dims)
    vs = [normal(w.seed_id, 40 + l + 1, (dims[l], dims[l + 1]), 1.0 / np.sqrt(dims[l]), w.dtype)
          for l in range(len(dims) - 1)]
    gs = [_quantize(1.0 + 0.25 * _rng(w.seed_id, 60 + l + 1).standard_normal(dims[l + 1]), w.dtype)
          for l in range(len(dims) - 1)]
    return vs, gs


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (CPU or GPU) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
