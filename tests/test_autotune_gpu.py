"""GPU checks of the per-shape autotuner (coalesce_autotune_gemm_bias_act,
coalesce_autotune_mlp_forward; "Coalesce" README, the plan's autotuning
phase; "MLP Megakernel" README, "Autotuning": exhaustive search per shape,
a cached fast path, correctness validated after tuning).

Every candidate configuration performs the same arithmetic per output
element, so the tuned launch must reproduce the default launch's output bit
for bit: checked on the call that tunes, on later calls of the ordinary
entry point (which now take the recorded configuration), after the record
is cleared, and against the fp64 oracle on the exact integer and random
cases.  The report must describe a search that happened: at least two
candidates, every one of them valid, the chosen one no slower than the
default.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import TOL, assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(autouse=True)
def _fresh_cache():
    mk.autotune_clear()
    yield
    mk.autotune_clear()


def _check_report(rep):
    # every candidate is built to give the default's bits, so every one of
    # them must be valid: a candidate that failed the bitwise check is a bug
    # in that configuration (the persistent multi-tile paths of the smaller
    # tile shapes run only through the reduced-grid candidates)
    assert rep["candidates"] >= 2, rep
    assert rep["valid"] == rep["candidates"], "a candidate configuration changed the output: %s" % rep
    assert 0 < rep["best_us"] <= rep["default_us"], rep


GEMM_CASES = [("bf16", "bf16", 8192, 16384, 4096, "gelu"),   # the FFN up-projection shape
              ("bf16", "f32", 2048, 4096, 1024, "gelu"),
              ("f16", "f16", 1000, 777, 300, "softplus"),
              ("f32", "f32", 1024, 1024, 1024, "gelu"),
              ("f32", "f32", 300, 520, 260, "relu")]


@pytest.mark.parametrize("i,o,M,N,K,act", GEMM_CASES, ids=lambda v: str(v))
def test_gemm_tuned_output_is_the_default_output(i, o, M, N, K, act):
    progress("autotune gemm %s->%s %dx%dx%d %s" % (i, o, M, N, K, act))
    gen = np.random.default_rng(M + N + K)
    A = torch.from_numpy(gen.standard_normal((M, K)).astype(np.float32)).to(DT[i])
    B = torch.from_numpy((gen.standard_normal((K, N)) / np.sqrt(K)).astype(np.float32)).to(DT[i])
    bias = torch.from_numpy(gen.standard_normal(N).astype(np.float32)).to(DT[i]).to("cuda")
    Ag, Bg = to_gpu(A), to_gpu(B)
    Y0 = mk.gemm_bias_act(Ag, Bg, bias, act=act, out_dtype=DT[o])
    Yt, rep = mk.autotune_gemm_bias_act(Ag, Bg, bias, act=act, out_dtype=DT[o], iters=3)
    Y1 = mk.gemm_bias_act(Ag, Bg, bias, act=act, out_dtype=DT[o])      # takes the recorded configuration
    torch.cuda.synchronize()
    progress("  report %s" % rep)
    _check_report(rep)
    assert torch.equal(Yt, Y0) and torch.equal(Y1, Y0)
    mk.autotune_clear()
    Y2 = mk.gemm_bias_act(Ag, Bg, bias, act=act, out_dtype=DT[o])
    assert torch.equal(Y2, Y0)
    if M * N * K <= 1 << 28:
        ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias.cpu()), act=act)
        assert_close(f64(Y1), ref, TOL[DT[o]] if DT[i] == torch.float32 else 2e-2, "tuned %s" % act)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_gemm_tuned_exact_integer_case(dt):
    M, N, K = 700, 530, 150
    A = datagen.integer_matrix((M, K), 7, 3, 13, 6, dt)
    B = datagen.integer_matrix((K, N), 5, 11, 11, 5, dt)
    bias = datagen.integer_matrix((1, N), 1, 3, 7, 3, dt).reshape(-1)
    _, rep = mk.autotune_gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act="none",
                                       out_dtype=torch.float32, iters=2)
    _check_report(rep)
    Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act="none", out_dtype=torch.float32)
    assert np.array_equal(f64(Y), oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="none"))


def test_gemm_record_is_per_shape():
    # tuning one shape leaves a neighbouring shape on the default path, and
    # both keep giving their default bits
    A, B = [to_gpu(datagen.uniform(9, t, s, "bf16")) for t, s in ((1, (1024, 512)), (2, (512, 2048)))]
    A2 = A[:1000]
    y_a = mk.gemm_bias_act(A, B)
    y_b = mk.gemm_bias_act(A2, B)
    mk.autotune_gemm_bias_act(A, B, iters=2)
    assert torch.equal(mk.gemm_bias_act(A, B), y_a)
    assert torch.equal(mk.gemm_bias_act(A2, B), y_b)


MLP_CASES = [("mlp3", (128,) * 4, 4096), ("mlp3", (128,) * 4, 100000), ("mlp3", (128,) * 4, 1 << 20),
             ("mlp5", (64,) * 6, 1 << 16), ("nonsquare", (120, 128, 24, 128, 40), 30000),
             ("streamed", (128,) * 7, 30000), ("streamed", (256, 136, 256), 20000)]


@pytest.mark.parametrize("name,dims,M", MLP_CASES, ids=lambda v: str(v))
def test_mlp_tuned_output_is_the_default_output(name, dims, M):
    progress("autotune mlp %s %s M=%d" % (name, dims, M))
    x, Ws = datagen.mlp_inputs(datagen.MLP3 if dims[0] == 128 else datagen.MLP5, M=M, dims=dims)
    xg = mk.aligned_copy(x)
    wg = [w.to("cuda") for w in Ws]
    y0 = mk.mlp_forward(xg, wg)
    yt, rep = mk.autotune_mlp_forward(xg, wg, iters=3)
    y1 = mk.mlp_forward(xg, wg)
    torch.cuda.synchronize()
    progress("  report %s" % rep)
    _check_report(rep)
    # chains whose weights fit in LDS try the resident kernel's launcher
    # choice and its three compiled launch configurations (32-row tiles with
    # fewer waves, 16-row tiles, 32-row tiles), each over six grids; the
    # others six grids
    assert rep["candidates"] == (24 if name != "streamed" else 6), rep
    assert torch.equal(yt, y0) and torch.equal(y1, y0)
    # an explicit grid still overrides the record
    assert torch.equal(mk.mlp_forward(xg, wg, num_workgroups=3), y0)
    if M <= 4096:
        assert_close(f64(y1), oracle.mlp_forward(f64(x), [f64(w) for w in Ws]), 2e-2, "tuned mlp")


def test_mlp_training_forward_ignores_the_record():
    dims = (128,) * 4
    x, Ws = datagen.mlp_inputs(datagen.MLP3, M=5000, dims=dims)
    xg = mk.aligned_copy(x)
    wg = [w.to("cuda") for w in Ws]
    out0, acts0 = mk.mlp_forward_train(xg, wg)
    mk.autotune_mlp_forward(xg, wg, iters=2)
    out1, acts1 = mk.mlp_forward_train(xg, wg)
    assert torch.equal(out0, out1) and all(torch.equal(a, b) for a, b in zip(acts0, acts1))
