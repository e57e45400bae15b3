"""GPU parity of coalesce_gemm_bias_act against the fp64 oracle.

Exact cases (integer-valued inputs, act = none) are compared bit for bit;
random cases use the gate metric max|y - o| / max(|o|, rms(o)) with the
tolerances 1e-4 (fp32) and 2e-2 (bf16 / fp16).  Shapes span several tiles
and ragged tails in M, N and K ("Fuse Elementwise Ops": test the last
partial tile and non-power-of-2 shapes).
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

# (M, N, K): single elements, sub-tile, tile-aligned, several tiles with
# ragged tails in every dimension, K below / at / above the K step.
EXACT_SHAPES = [(1, 1, 1), (7, 5, 3), (17, 33, 65), (64, 64, 64), (127, 129, 31), (255, 257, 129),
                (257, 255, 63), (129, 1, 33), (1, 300, 17), (300, 9, 5), (520, 530, 150), (513, 257, 200),
                (33, 600, 96), (600, 40, 257)]


def _integer_inputs(M, N, K, dt):
    A = datagen.integer_matrix((M, K), 7, 3, 13, 6, dt)
    B = datagen.integer_matrix((K, N), 5, 11, 11, 5, dt)
    bias = datagen.integer_matrix((1, N), 1, 3, 7, 3, dt).reshape(-1)
    return A, B, bias


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "f32"), ("bf16", "f32"), ("f16", "f32"), ("bf16", "bf16"),
                                          ("f16", "f16")])
def test_integer_inputs_bit_exact(in_dt, out_dt):
    for (M, N, K) in EXACT_SHAPES:
        progress("exact %s->%s M=%d N=%d K=%d" % (in_dt, out_dt, M, N, K))
        A, B, bias = _integer_inputs(M, N, K, in_dt)
        ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="none")
        # the exact integer, rounded once to the output type (round to nearest even)
        ref_t = torch.from_numpy(ref).to(torch.float32).to(DT[out_dt])
        Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act="none", out_dtype=DT[out_dt])
        torch.cuda.synchronize()
        got = Y.cpu()
        assert torch.equal(got.view(torch.int32 if out_dt == "f32" else torch.int16),
                           ref_t.view(torch.int32 if out_dt == "f32" else torch.int16)), (M, N, K)


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "f32"), ("bf16", "f32"), ("f16", "f32")])
def test_integer_inputs_relu_bit_exact(in_dt, out_dt):
    # relu of an exact integer sum is exact
    for (M, N, K) in [(1, 1, 1), (17, 33, 65), (257, 129, 127), (300, 520, 260)]:
        progress("exact relu %s->%s M=%d N=%d K=%d" % (in_dt, out_dt, M, N, K))
        A, B, bias = _integer_inputs(M, N, K, in_dt)
        ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="relu")
        Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act="relu", out_dtype=DT[out_dt])
        assert np.array_equal(f64(Y), ref), (M, N, K)


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("act", ["gelu", "softplus", "relu", "none"])
def test_random_parity(in_dt, out_dt, act):
    shapes = [(100, 70, 50), (300, 520, 260), (513, 300, 1000)]
    for (M, N, K) in shapes:
        progress("random %s->%s %s M=%d N=%d K=%d" % (in_dt, out_dt, act, M, N, K))
        w = datagen.FP32_512 if in_dt == "f32" else datagen.BF16_FFN
        w = datagen.GemmWorkload(w.name, w.seed_id, M, N, K, in_dt, out_dt, w.dist)
        A, B, bias = datagen.gemm_inputs(w)
        ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act=act)
        Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act=act, out_dtype=DT[out_dt])
        assert_close(f64(Y), ref, TOL[DT[in_dt]], "%s %s %s" % (in_dt, act, (M, N, K)))


@pytest.mark.parametrize("in_dt", ["f32", "bf16", "f16"])
def test_no_bias_and_k_zero(in_dt):
    M, N, K = 70, 90, 40
    A, B, bias = _integer_inputs(M, N, K, in_dt)
    ref = oracle.gemm_bias_act(f64(A), f64(B), None, act="gelu")
    Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), None, act="gelu", out_dtype=torch.float32)
    assert_close(f64(Y), ref, 1e-5, "no bias")
    # K = 0: Y = act(bias) for every row, A and B may be empty
    A0 = torch.empty((M, 0), dtype=DT[in_dt], device="cuda")
    B0 = torch.empty((0, N), dtype=DT[in_dt], device="cuda")
    bvals = torch.linspace(-4, 4, N).to(DT[in_dt])
    Y0 = mk.gemm_bias_act(A0, B0, bvals.to("cuda"), act="gelu", out_dtype=torch.float32)
    ref0 = np.broadcast_to(oracle.gelu(f64(bvals))[None, :], (M, N))
    assert_close(f64(Y0), ref0, 1e-6, "K=0")


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
def test_unit_accumulator_trick(in_dt):
    # "Coalesce" README notes: B = 1/K puts the accumulator at exactly 1.0,
    # where GELU bends; with a bias the output is GELU(1 + bias_j) per column.
    M, K, N = 300, 512, 260
    A = torch.ones((M, K), dtype=DT[in_dt])
    B = torch.full((K, N), 1.0 / K, dtype=DT[in_dt])
    bias = torch.linspace(-3, 3, N).to(DT[in_dt])
    Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act="gelu", out_dtype=torch.float32)
    ref = np.broadcast_to(oracle.gelu(1.0 + f64(bias))[None, :], (M, N))
    assert_close(f64(Y), ref, 1e-6, "unit accumulator")


def test_identity_sweep_gelu_and_softplus_fp32():
    # B = I, A = linspace(-30, 30): Y = act(A + bias) elementwise; crosses the
    # softplus guard at 20 and GELU's tails.
    M = K = N = 256
    A = torch.linspace(-30, 30, M * K, dtype=torch.float64).reshape(M, K).to(torch.float32)
    B = torch.eye(K, dtype=torch.float32)
    bias = torch.linspace(-0.5, 0.5, N, dtype=torch.float32)
    for act in ("gelu", "softplus"):
        Y = mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act=act)
        ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act=act)
        y = f64(Y)
        # relative error above |o| = 1, absolute below: in fp32 the erf form
        # 1 + erf(z / sqrt 2) cancels for z < 0, leaving an absolute error of
        # about |z| * 2^-24 there (inherent to the formula, not the kernel)
        err = np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)
        assert err.max() < 1e-6, (act, err.max())


def test_fused_equals_unfused_fp32_bitwise():
    # "Coalesce" README, Fusion study: fused and unfused are bit-identical in
    # FP32 -- same main loop, same fp32 bias add, same activation code.
    w = datagen.FP32_1024
    A, B, bias = datagen.gemm_inputs(w, M=520, N=777, K=300)
    A, B, bias = to_gpu(A), to_gpu(B), bias.to("cuda")
    Yf = mk.gemm_bias_act(A, B, bias, act="gelu")
    Z = mk.gemm_bias_act(A, B, None, act="none")
    Z2 = mk.bias_add(Z, bias)
    Yu = mk.activation(Z2, "gelu")
    torch.cuda.synchronize()
    assert torch.equal(Yf.cpu().view(torch.int32), Yu.cpu().view(torch.int32))


def test_fp32_large_problem_on_small_tiles():
    # Past one full round of 128 x 128 tiles the FP32 launcher may take 64 x 64
    # tiles (two K groups) when the last 128 x 128 round would be mostly
    # empty: 3000 x 3100 (600 tiles of 128 x 128 for 512 slots, 2303 of
    # 64 x 64) does, with ragged edges in M, N and K.  Sampled rows against
    # the oracle; fused and unfused bit for bit (the same tiles for both).
    w = datagen.FP32_1024
    M, N, K = 3000, 3100, 3000
    A, B, bias = datagen.gemm_inputs(w, M=M, N=N, K=K)
    progress("fp32 large on 64x64 tiles M=%d N=%d K=%d" % (M, N, K))
    Ag, Bg, bg = to_gpu(A), to_gpu(B), bias.to("cuda")
    Yf = mk.gemm_bias_act(Ag, Bg, bg, act="gelu")
    Yu = mk.activation(mk.bias_add(mk.gemm_bias_act(Ag, Bg, None, act="none"), bg), "gelu")
    torch.cuda.synchronize()
    assert torch.equal(Yf.cpu().view(torch.int32), Yu.cpu().view(torch.int32))
    rows = [0, 1, 63, 64, 1500, M - 1]
    ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="gelu", rows=rows)
    assert_close(f64(Yf)[rows], ref, 1e-4, "fp32 3000x3100x3000 rows")


def test_unfused_bf16_baseline_within_tolerance():
    w = datagen.BF16_FFN
    A, B, bias = datagen.gemm_inputs(w, M=300, N=520, K=256)
    ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="gelu")
    A, B, biasg = to_gpu(A), to_gpu(B), bias.to("cuda")
    Yu = mk.activation(mk.bias_add(mk.gemm_bias_act(A, B, None, act="none"), biasg), "gelu")
    assert_close(f64(Yu), ref, 2e-2, "unfused bf16")


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
def test_no_write_outside_output(in_dt):
    # Guard band: Y is a window of a larger NaN-filled buffer; nothing outside
    # the M x N window may change (last partial tile must be masked).
    M, N, K = 261, 135, 77
    A, B, bias = _integer_inputs(M, N, K, in_dt)
    big = torch.full((M + 3, 160), float("nan"), dtype=torch.float32, device="cuda")
    Y = big[1:M + 1, 8:8 + N]
    mk.gemm_bias_act(to_gpu(A), to_gpu(B), bias.to("cuda"), act="none", out_dtype=torch.float32, out=Y)
    torch.cuda.synchronize()
    b = big.cpu()
    mask = torch.ones_like(b, dtype=torch.bool)
    mask[1:M + 1, 8:8 + N] = False
    assert torch.isnan(b[mask]).all()
    assert not torch.isnan(b[~mask]).any()


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
def test_deterministic(in_dt):
    w = datagen.FP32_512 if in_dt == "f32" else datagen.BF16_FFN
    A, B, bias = datagen.gemm_inputs(w, M=600, N=700, K=400)
    A, B, bias = to_gpu(A), to_gpu(B), bias.to("cuda")
    ys = [mk.gemm_bias_act(A, B, bias, act="gelu").cpu() for _ in range(5)]
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16 if in_dt == "bf16" else torch.int32),
                           ys[0].view(torch.int16 if in_dt == "bf16" else torch.int32))


def _sampled_check(w, nsamp, rows_full):
    progress("full size %s" % w.name)
    A, B, bias = datagen.gemm_inputs(w)
    Y = mk.gemm_bias_act(to_gpu(A, padded=False), to_gpu(B, padded=False), bias.to("cuda"), act="gelu",
                         out_dtype=DT[w.out_dtype])
    torch.cuda.synchronize()
    y = Y.cpu()
    A64, B64, b64 = f64(A), f64(B), f64(bias)
    rng = np.random.default_rng(123)
    r = rng.integers(0, w.M, nsamp)
    c = rng.integers(0, w.N, nsamp)
    # include the corners of the problem
    r = np.concatenate([r, [0, 0, w.M - 1, w.M - 1]])
    c = np.concatenate([c, [0, w.N - 1, 0, w.N - 1]])
    ref = oracle.gemm_bias_act_at(A64, B64, b64, "gelu", r, c)
    got = y[r, c].to(torch.float64).numpy()
    # the floor is the rms of the sampled reference outputs
    e1 = assert_close(got, ref, TOL[DT[w.in_dtype]], w.name + " samples")
    rows = np.array(rows_full)
    ref_rows = oracle.gemm_bias_act(A64, B64, b64, act="gelu", rows=rows)
    e2 = assert_close(y[rows].to(torch.float64).numpy(), ref_rows, TOL[DT[w.in_dtype]], w.name + " rows")
    progress("%s: sampled E=%.3e rows E=%.3e" % (w.name, e1, e2))


@pytest.mark.parametrize("name", ["fp32_gemm_gelu_512", "fp32_gemm_gelu_1024", "fp32_gemm_gelu_2048",
                                  "fp32_gemm_gelu_4096"])
def test_fp32_full_size(name):
    w = datagen.WORKLOADS[name]
    if w.M <= 1024:
        A, B, bias = datagen.gemm_inputs(w)
        ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="gelu")
        Y = mk.gemm_bias_act(to_gpu(A, padded=False), to_gpu(B, padded=False), bias.to("cuda"), act="gelu")
        e = assert_close(f64(Y), ref, 1e-4, name)
        progress("%s: full E=%.3e" % (name, e))
    else:
        _sampled_check(w, 4000, [0, 1, w.M // 2, w.M - 1])


def test_bf16_ffn_full_size():
    _sampled_check(datagen.BF16_FFN, 4000, [0, 4095, 8191])


@pytest.mark.parametrize("in_dt,out_dt,act", [("bf16", "bf16", "gelu"), ("f16", "f32", "softplus"),
                                              ("bf16", "bf16", "none")])
def test_tile_shapes_agree_bitwise(in_dt, out_dt, act):
    # The 16-bit GEMM runs 64 x 64 tiles while 128 x 128 ones number fewer
    # than the CUs, 128 x 128 while all of them fit on the CUs at once (two
    # per CU) and 256 x 256 otherwise; all accumulate every output element in
    # the same k order, so they must give the same bits.  The full problem
    # (25 x 25 tiles of 128) takes 256 x 256 tiles with ragged edges in M, N
    # and K; its first 1536 rows (12 x 25 tiles of 128) take 128 x 128, its
    # first 300 rows (3 x 25) 64 x 64.
    w = datagen.BF16_FFN
    M, N, K = 3083, 3077, 200
    A, B, bias = datagen.gemm_inputs(w, M=M, N=N, K=K)
    if in_dt == "f16":
        A, B, bias = A.to(torch.float16), B.to(torch.float16), bias.to(torch.float16)
    progress("tile shapes %s->%s %s M=%d N=%d K=%d" % (in_dt, out_dt, act, M, N, K))
    Ag, Bg, bg = to_gpu(A), to_gpu(B), bias.to("cuda")
    big = mk.gemm_bias_act(Ag, Bg, bg, act=act, out_dtype=DT[out_dt])
    view = torch.int16 if out_dt != "f32" else torch.int32
    for rows in (1536, 300):
        part = mk.gemm_bias_act(Ag[:rows], Bg, bg, act=act, out_dtype=DT[out_dt])
        torch.cuda.synchronize()
        assert torch.equal(big[:rows].contiguous().view(view), part.contiguous().view(view)), rows
    rows = np.array([0, 1, 299, 300, 1500, 2047, 3071, 3072, M - 1])
    ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act=act, rows=rows)
    assert_close(f64(big[torch.from_numpy(rows).to("cuda")]), ref, TOL[DT[in_dt]], "tile shapes")
