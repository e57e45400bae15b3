"""Host-side checks that need no GPU: the seeded input recipe (datagen) and
bench.py's one-GPU contract.

datagen is shared by the tests, bench.py and smoke(); it holds no arithmetic
of the method, only seeded draws, so what is checked here is that the draws
are reproducible, have the stated distributions, and that a smaller input of
a workload is the leading rows of the full one (the full-size tests and the
CPU baseline rely on sampling rows of the same recipe).
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_draws_are_reproducible_and_seed_specific():
    a = datagen.normal(3, 1, (64, 32), 1.0, "f32")
    b = datagen.normal(3, 1, (64, 32), 1.0, "f32")
    c = datagen.normal(3, 2, (64, 32), 1.0, "f32")
    d = datagen.normal(4, 1, (64, 32), 1.0, "f32")
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, d)


def test_smaller_inputs_are_leading_rows_of_the_full_ones():
    w = datagen.MLP3
    x_small, W_small = datagen.mlp_inputs(w, M=1000)
    x_big, W_big = datagen.mlp_inputs(w, M=4096)
    assert torch.equal(x_small, x_big[:1000])
    assert all(torch.equal(p, q) for p, q in zip(W_small, W_big))
    A1, B1, b1 = datagen.gemm_inputs(datagen.BF16_FFN, M=64, N=128, K=96)
    A2, B2, b2 = datagen.gemm_inputs(datagen.BF16_FFN, M=128, N=128, K=96)
    assert torch.equal(A1, A2[:64]) and torch.equal(B1, B2) and torch.equal(b1, b2)


@pytest.mark.parametrize("name", ["fp32_gemm_gelu_512", "bf16_ffn_up_gelu"])
def test_gemm_input_distributions(name):
    w = datagen.WORKLOADS[name]
    A, B, bias = datagen.gemm_inputs(w, M=512, N=1024, K=w.K if w.K <= 4096 else 4096)
    A, B, bias = [datagen.to_f64(t) for t in (A, B, bias)]
    if w.dist == "uniform":  # U[-1, 1): mean 0, variance 1/3, bounded
        for t in (A, B):
            assert abs(t.mean()) < 0.02 and abs(t.var() - 1.0 / 3.0) < 0.02 and t.min() >= -1 and t.max() < 1
    else:  # A ~ N(0,1), B ~ N(0, 1/sqrt(K)), bias ~ N(0, 0.02)
        assert abs(A.mean()) < 0.01 and abs(A.std() - 1.0) < 0.01
        assert abs(B.std() - 1.0 / np.sqrt(w.K)) < 0.01 / np.sqrt(w.K) * 10
        assert abs(bias.std() - 0.02) < 0.003


def test_mlp_input_distributions():
    for w in (datagen.MLP3, datagen.MLP5, datagen.MLP_NS2):
        x, Ws = datagen.mlp_inputs(w, M=8192)
        x = datagen.to_f64(x)
        assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
        for l, W in enumerate(Ws):
            W = datagen.to_f64(W)
            assert W.shape == (w.dims[l], w.dims[l + 1])
            assert abs(W.std() * np.sqrt(w.dims[l]) - 1.0) < 0.1


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
