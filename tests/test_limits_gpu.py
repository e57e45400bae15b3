"""GPU parity at the size limits the library accepts.

Two kinds of limit, both about addressing:
  * operands larger than 4 GiB, so that byte offsets of late rows do not fit
    in 32 bits (every tile's base is formed in 64-bit arithmetic and only the
    offsets inside a tile are 32-bit);
  * the largest leading dimensions the entry points accept (16-bit GEMM:
    lda = 2^23, ldb = 2^25; MLP: every pitch 2^24), where the offsets inside
    one tile come closest to 2^32.

Inputs follow the seeded recipe.  The large operands repeat a small seeded
block of P rows (built on the GPU), so every output row is a function of its
own input row only and rows P apart must agree bit for bit over the whole
output; sampled rows (the last ones included) are compared with the oracle.
The weight gradients of the periodic training input are q times the oracle's
gradient of one period plus that of the remaining rows.  The padded buffers
of the pitch tests are filled with NaN: a read of padding would reach the
outputs, and a write outside the outputs would overwrite the NaN.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import TOL, assert_close, f64, progress

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _periodic(t, M):
    """The first M rows of the P-row tensor t repeated (a contiguous copy on the GPU)."""
    P = t.shape[0]
    return t.to("cuda").repeat(-(-M // P), 1)[:M].contiguous()


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                       b.view(torch.int16 if b.element_size() == 2 else torch.int32))


def _sample_rows(M, n, last, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.integers(0, M, n), np.arange(M - last, M)]))


@pytest.mark.parametrize("name", ["bf16_ffn_up_gelu", "fp32_gemm_gelu_512"])
def test_gemm_operand_beyond_4gib(name):
    w = datagen.WORKLOADS[name]
    P, N, K = 1000, 320, 1152
    A, B, bias = datagen.gemm_inputs(w, M=P, N=N, K=K)
    es = A.element_size()
    M = (1 << 22) // es + 300  # A spans 4.8 GB; the last rows start past 2^32 bytes
    progress("gemm %s M=%d N=%d K=%d (A %.1f GB)" % (name, M, N, K, M * K * es / 1e9))
    Ag = _periodic(A, M)
    assert Ag.numel() * es > GIB4
    Y = mk.gemm_bias_act(Ag, B.to("cuda"), bias.to("cuda"), act="gelu")
    torch.cuda.synchronize()
    del Ag
    # rows P apart agree bit for bit (rows of the last, partial 256-row tile
    # take the masked epilogue and are checked against the oracle instead)
    full = M // 256 * 256
    assert _same_bits(Y[:full - P], Y[P:full])
    rows = _sample_rows(M, 512, 300, 11)
    ref = oracle.gemm_bias_act(f64(A)[rows % P], f64(B), f64(bias), act="gelu")
    got = f64(Y[torch.from_numpy(rows).to("cuda")])
    assert_close(got, ref, TOL[A.dtype], "rows of a 4.8 GB A (%s)" % name)


# N picks the tile shape the launcher takes for M = 300 (3 rows of 128 x 128
# tiles on 256 CUs): 200 -> 6 tiles of 128, fewer than the CUs: 64 x 64;
# 12000 -> 282, at most two per CU: 128 x 128; 22000 -> 516: 256 x 256, the
# shape whose 256-row A tile puts in-tile offsets closest to 2^32 bytes.
@pytest.mark.parametrize("N", [200, 12000, 22000])
def test_gemm_maximum_pitches(N):
    M, K = 300, 72  # ragged in every dimension
    lda, ldb, ldy = 1 << 23, 1 << 25, 1 << 23  # A 5.0 GB, B 4.8 GB, Y 5.0 GB
    A, B, bias = datagen.gemm_inputs(datagen.BF16_FFN, M=M, N=N, K=K)
    progress("gemm bf16 M=%d N=%d K=%d lda=2^23 ldb=2^25 ldy=2^23" % (M, N, K))
    nan = float("nan")
    Ab = torch.full((M, lda), nan, dtype=torch.bfloat16, device="cuda")
    Ab[:, :K] = A.to("cuda")
    Bb = torch.full((K, ldb), nan, dtype=torch.bfloat16, device="cuda")
    Bb[:, :N] = B.to("cuda")
    Yb = torch.full((M, ldy), nan, dtype=torch.bfloat16, device="cuda")
    mk.gemm_bias_act(Ab[:, :K], Bb[:, :N], bias.to("cuda"), act="gelu", out=Yb[:, :N])
    torch.cuda.synchronize()
    ref = oracle.gemm_bias_act(f64(A), f64(B), f64(bias), act="gelu")
    assert_close(f64(Yb[:, :N]), ref, TOL[torch.bfloat16], "maximum pitches")
    assert bool(torch.isnan(Yb[:, N:]).all()), "a write outside Y"


def test_mlp_forward_beyond_4gib():
    w = datagen.MLP3
    P = 4096
    M = (1 << 24) + 77  # x and out span 4.3 GB each; a ragged last tile
    x, Ws = datagen.mlp_inputs(w, M=P)
    progress("mlp forward %s M=%d" % (w.name, M))
    xg = _periodic(x, M)
    assert xg.numel() * 2 > GIB4
    out = mk.mlp_forward(xg, [t.to("cuda") for t in Ws])
    torch.cuda.synchronize()
    del xg
    assert out.numel() * 2 > GIB4
    assert _same_bits(out[:M - P], out[P:])
    rows = _sample_rows(M, 512, 77, 12)
    ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws], rows=rows % P)
    assert_close(f64(out[torch.from_numpy(rows).to("cuda")]), ref, 2e-2, "rows of a 4.3 GB x")


def test_training_pair_beyond_4gib():
    w = datagen.MLP3
    P = 4096
    M = (1 << 23) + 77  # each fp32 activation layer spans 4.3 GB
    L = w.L
    x, Ws = datagen.mlp_inputs(w, M=P)
    g = datagen.mlp_grad_output(w, M=P)
    progress("training pair %s M=%d" % (w.name, M))
    xg, gg = _periodic(x, M), _periodic(g, M)
    wg = [t.to("cuda") for t in Ws]
    out, acts = mk.mlp_forward_train(xg, wg)
    assert acts[0].shape[0] * acts[0].stride(0) * 4 > GIB4
    dW, dx = mk.mlp_backward(xg, wg, acts, gg)
    torch.cuda.synchronize()
    del xg, gg
    for name, t in [("out", out), ("dx", dx)] + [("acts[%d]" % l, a) for l, a in enumerate(acts)]:
        assert _same_bits(t[:M - P], t[P:]), name
    rows = _sample_rows(M, 256, 77, 13)
    rows_t = torch.from_numpy(rows).to("cuda")
    Wd = [f64(t) for t in Ws]
    _, o_acts = oracle.mlp_forward_train(f64(x), Wd)
    for l in range(L - 1):
        assert_close(f64(acts[l].index_select(0, rows_t)), o_acts[l][rows % P], 2e-2, "sampled acts[%d]" % l)
    o_dW, o_dx = oracle.mlp_backward(f64(x), Wd, f64(g))
    r = M % P
    o_dW_r, _ = oracle.mlp_backward(f64(x)[:r], Wd, f64(g)[:r], want_dx=False)
    for l in range(L):
        assert_close(f64(dW[l]), (M // P) * o_dW[l] + o_dW_r[l], 2e-2, "dW[%d]" % l)
    assert_close(f64(dx.index_select(0, rows_t)), o_dx[rows % P], 2e-2, "sampled dx")


def test_mlp_maximum_pitches():
    w = datagen.MLP3
    M, D, L = 70, 128, w.L  # two row tiles, the second ragged
    ld = 1 << 24  # every pitch at the limit: x, out, dout, dx 2.3 GB, each activation 4.7 GB
    x, Ws = datagen.mlp_inputs(w, M=M)
    g = datagen.mlp_grad_output(w, M=M)
    progress("mlp M=%d with every pitch 2^24" % M)
    nan = float("nan")

    def padded(rows, dtype, src=None):
        b = torch.full((rows, ld), nan, dtype=dtype, device="cuda")
        if src is not None:
            b[:, :D] = src.to("cuda")
        return b

    xb, gb = padded(M, torch.float16, x), padded(M, torch.float16, g)
    wg = [t.to("cuda") for t in Ws]
    ob = padded(M, torch.float16)
    mk.mlp_forward(xb[:, :D], wg, out=ob[:, :D])
    otb = padded(M, torch.float16)
    ab = [padded(M, torch.float32) for _ in range(L - 1)]
    mk.mlp_forward_train(xb[:, :D], wg, out=otb[:, :D], acts=[a[:, :D] for a in ab])
    dxb = padded(M, torch.float16)
    dW, _ = mk.mlp_backward(xb[:, :D], wg, [a[:, :D] for a in ab], gb[:, :D], dx=dxb[:, :D])
    torch.cuda.synchronize()
    Wd = [f64(t) for t in Ws]
    assert_close(f64(ob[:, :D]), oracle.mlp_forward(f64(x), Wd), 2e-2, "forward")
    assert _same_bits(otb[:, :D], ob[:, :D])
    _, o_acts = oracle.mlp_forward_train(f64(x), Wd)
    for l in range(L - 1):
        assert_close(f64(ab[l][:, :D]), o_acts[l], 2e-2, "acts[%d]" % l)
    o_dW, o_dx = oracle.mlp_backward(f64(x), Wd, f64(g))
    for l in range(L):
        assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d]" % l)
    assert_close(f64(dxb[:, :D]), o_dx, 2e-2, "dx")
    for name, b in [("out", ob), ("train out", otb), ("dx", dxb)] + [("acts[%d]" % l, a) for l, a in enumerate(ab)]:
        assert bool(torch.isnan(b[:, D:]).all()), "a write outside %s" % name
