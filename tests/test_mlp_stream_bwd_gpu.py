"""GPU parity of the layer-by-layer backward (mlp_bwd_stream.hip), which
coalesce_mlp_backward runs for the chains the layer-streaming forward takes:
more than 4 layers of width up to 128 or 8 of width up to 64, and any chain
with a layer wider than 128 (up to 256), up to 16 layers.

Exact cases: integer x and dout with signed partial-permutation weights make
a linear or relu chain exact in fp16 and fp32 (every dz and dx entry is one
signed term, every dW entry a sum of small integers), so dW and dx must equal
the oracle bit for bit; this pins the weight staging, both data-product
operands, the transposing reads of the weight gradient, the masking of
ragged widths and rows, the dz buffers between layers and the reduction.
Random softplus chains use the 2e-2 gate (max error over max(|ref|,
rms(ref))) of the other backward tests: the GPU rounds h_l and dz_l to fp16
as MFMA operands while the oracle stays in fp64.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

DEEP128 = (128,) * 7                      # 6 layers of 128
WIDE = (256, 256, 256, 256)               # 3 layers of 256
DEEP64 = (64,) * 13                       # 12 layers of 64
MIXED = (200, 256, 40, 136, 256, 8, 64)   # ragged widths, 256-wide layers
DEEP16 = (32, 96, 64, 128, 64, 96, 128, 32, 64, 128, 96, 64, 32, 128, 64, 96, 48)  # 16 layers
# an odd layer count at widths <= 128: two-layer launches, then the first
# layer on its own
ODD128 = (128,) * 6                       # 5 layers of 128
ODDRAG = (72, 128, 120, 8, 128, 104, 40, 128)  # 7 ragged layers
CHAINS = [DEEP128, WIDE, DEEP64, MIXED, DEEP16, ODD128, ODDRAG]
IDS = ["x".join(map(str, d)) for d in CHAINS]


def _signed_perm(rows, cols, seed):
    rng = np.random.default_rng(seed)
    P = np.zeros((rows, cols))
    n = min(rows, cols)
    P[rng.permutation(rows)[:n], rng.permutation(cols)[:n]] = rng.choice([-1.0, 1.0], n)
    return torch.from_numpy(P).to(torch.float16)


def _train(x, Ws, g, act="softplus", want_dx=True):
    xg = to_gpu(x)
    wg = [w.to("cuda") for w in Ws]
    out, acts = mk.mlp_forward_train(xg, wg, hidden_act=act)
    dW, dx = mk.mlp_backward(xg, wg, acts, to_gpu(g), hidden_act=act, want_dx=want_dx)
    torch.cuda.synchronize()
    return out, acts, dW, dx


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("dims", CHAINS, ids=IDS)
def test_exact_signed_permutation_chains(act, dims):
    L = len(dims) - 1
    for M in (33, 1000):
        progress("stream bwd exact %s %s M=%d" % (act, dims, M))
        x = datagen.integer_matrix((M, dims[0]), 3, 7, 17, 8, "f16")
        g = datagen.integer_matrix((M, dims[-1]), 5, 3, 13, 6, "f16")
        Ws = [_signed_perm(dims[l], dims[l + 1], 90 * L + l) for l in range(L)]
        _, _, dW, dx = _train(x, Ws, g, act=act)
        o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g), hidden_act=act)
        for l in range(L):
            assert np.array_equal(f64(dW[l]), o_dW[l]), "dW[%d] %s %s M=%d" % (l, act, dims, M)
        assert np.array_equal(f64(dx), o_dx), "dx %s %s M=%d" % (act, dims, M)


@pytest.mark.parametrize("dims", CHAINS, ids=IDS)
def test_random_softplus_parity_ragged_rows(dims):
    w = datagen.MLP3
    L = len(dims) - 1
    for M in (1, 65, 1000, 4097):
        progress("stream bwd random %s M=%d" % (dims, M))
        x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
        g = datagen.mlp_grad_output(w, M=M, dims=dims)
        _, _, dW, dx = _train(x, Ws, g)
        o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(t) for t in Ws], f64(g))
        for l in range(L):
            assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d] %s M=%d" % (l, dims, M))
        assert_close(f64(dx), o_dx, 2e-2, "dx %s M=%d" % (dims, M))


@pytest.mark.parametrize("dims", [DEEP128, WIDE], ids=["x".join(map(str, d)) for d in (DEEP128, WIDE)])
def test_larger_rows_linear_and_softplus(dims):
    # many tiles per workgroup (every workgroup sums dozens of tiles)
    w = datagen.MLP3
    L = len(dims) - 1
    M = 32768 + 19
    x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
    g = datagen.mlp_grad_output(w, M=M, dims=dims)
    for act in ("none", "softplus"):
        progress("stream bwd %s %s M=%d" % (act, dims, M))
        _, _, dW, dx = _train(x, Ws, g, act=act)
        o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(t) for t in Ws], f64(g), hidden_act=act)
        for l in range(L):
            assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d] %s %s" % (l, act, dims))
        assert_close(f64(dx), o_dx, 2e-2, "dx %s %s" % (act, dims))


@pytest.mark.parametrize("dims", [DEEP128, DEEP64], ids=["x".join(map(str, d)) for d in (DEEP128, DEEP64)])
def test_identity_weights_sigmoid_chain(dims):
    # W_l = I: dx = dout * prod_j sigmoid(z_j), z_1 = x, z_{j+1} = softplus(z_j)
    # (the same elementwise bound as for the fused backward: per layer one
    # fp16 rounding of dz and at most 2^-23 absolute in the derivative)
    D, L, M = dims[0], len(dims) - 1, 256
    x = torch.linspace(-30, 30, M * D, dtype=torch.float64).reshape(M, D).to(torch.float16)
    g = datagen.mlp_grad_output(datagen.MLP3, M=M, dims=dims)
    Ws = [torch.eye(D, dtype=torch.float16) for _ in range(L)]
    _, _, dW, dx = _train(x, Ws, g)
    _, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g))
    gg = np.abs(f64(g))
    bound = 4e-3 * L * np.abs(o_dx) + L * (2.0 ** -24 + gg * 2.0 ** -23)
    assert np.all(np.abs(f64(dx) - o_dx) <= bound), np.max(np.abs(f64(dx) - o_dx) / bound)


@pytest.mark.parametrize("dims", [WIDE, MIXED, DEEP128, ODDRAG],
                         ids=["x".join(map(str, d)) for d in (WIDE, MIXED, DEEP128, ODDRAG)])
def test_without_dx_deterministic_and_empty(dims):
    w = datagen.MLP3
    L = len(dims) - 1
    M = 5000
    x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
    g = datagen.mlp_grad_output(w, M=M, dims=dims)
    xg, gg = to_gpu(x), to_gpu(g)
    wg = [t.to("cuda") for t in Ws]
    _, acts = mk.mlp_forward_train(xg, wg)
    dW, dx = mk.mlp_backward(xg, wg, acts, gg)
    dW2, none = mk.mlp_backward(xg, wg, acts, gg, want_dx=False)
    dW3, dx3 = mk.mlp_backward(xg, wg, acts, gg)
    torch.cuda.synchronize()
    assert none is None
    for l in range(L):
        assert torch.equal(_bits(dW[l]), _bits(dW2[l])), "dW[%d] without dx" % l
        assert torch.equal(_bits(dW[l]), _bits(dW3[l])), "dW[%d] repeated call" % l
    assert torch.equal(_bits(dx), _bits(dx3))
    # M = 0: every dW is zero
    x0 = torch.empty((0, dims[0]), dtype=torch.float16, device="cuda")
    g0 = torch.empty((0, dims[-1]), dtype=torch.float16, device="cuda")
    _, acts0 = mk.mlp_forward_train(x0, wg)
    dW0 = [torch.full((dims[l], dims[l + 1]), float("nan"), device="cuda") for l in range(L)]
    mk.mlp_backward(x0, wg, acts0, g0, dW=dW0, want_dx=False)
    torch.cuda.synchronize()
    for l in range(L):
        assert torch.count_nonzero(dW0[l]).item() == 0, l
