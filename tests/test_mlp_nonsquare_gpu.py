"""GPU parity of the MLP megakernel on non-square chains: input width D,
hidden widths H_l and output width O in any mix (multiples of 8, at most
128), as the quick start's FusedMLPSoftplus(D, H, out_features) allows.

Such a chain runs at kernel width 64 or 128 with the weights zero-padded in
LDS and the x loads / out and activation stores limited to the true columns.
Tested: random parity against the oracle over ragged rows (the 2e-2 gate of
the forward), exact integer chains through selection weights (every output
unit copies one input unit with a sign), the training forward's activations,
and the masking itself: NaN in x beyond its width must not reach any result,
and nothing may be written beyond out's or an activation's width.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress

pytestmark = pytest.mark.gpu

CHAINS = [(32, 128, 16), (128, 64, 128, 128), (8, 64, 64, 64, 64, 8), (120, 128, 24, 128, 40), (64, 8, 64),
          (16, 24), (128, 96, 80, 56), (64, 64, 32, 64, 64, 64, 64, 64, 16)]


def _padded(t, extra, fill):
    """Device copy of a 2-D tensor inside a wider buffer whose pad columns hold `fill`."""
    M, N = t.shape
    buf = torch.full((M, N + extra), fill, dtype=t.dtype, device="cuda")
    buf[:, :N] = t.to("cuda")
    return buf[:, :N]


@pytest.mark.parametrize("dims", CHAINS, ids=lambda d: "x".join(map(str, d)))
def test_random_parity_ragged_rows(dims):
    for M in (1, 65, 1000, 4097):
        progress("nonsquare %s M=%d" % (dims, M))
        x, Ws = datagen.mlp_inputs(datagen.MLP3, M=M, dims=dims)
        out = mk.mlp_forward(mk.aligned_copy(x), [w.to("cuda") for w in Ws])
        ref = oracle.mlp_forward(f64(x), [f64(w) for w in Ws])
        assert_close(f64(out), ref, 2e-2, "%s M=%d" % (dims, M))


def _selection(K, N, seed):
    rng = np.random.default_rng(seed)
    W = np.zeros((K, N))
    W[rng.integers(0, K, N), np.arange(N)] = rng.choice([-1.0, 1.0], N)
    return torch.from_numpy(W).to(torch.float16)


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("dims", CHAINS, ids=lambda d: "x".join(map(str, d)))
def test_selection_chains_exact(act, dims):
    M = 333
    x = datagen.integer_matrix((M, dims[0]), 3, 7, 17, 8, "f16")
    Ws = [_selection(dims[l], dims[l + 1], 50 * l + len(dims)) for l in range(len(dims) - 1)]
    out = mk.mlp_forward(mk.aligned_copy(x), [w.to("cuda") for w in Ws], hidden_act=act)
    ref = oracle.mlp_forward(f64(x), [f64(w) for w in Ws], hidden_act=act)
    assert np.array_equal(f64(out), ref), (act, dims)


@pytest.mark.parametrize("dims", [(32, 128, 16), (120, 128, 24, 128, 40), (8, 64, 64, 64, 64, 8)],
                         ids=lambda d: "x".join(map(str, d)))
def test_training_forward_and_masking(dims):
    L = len(dims) - 1
    M = 1000
    x, Ws = datagen.mlp_inputs(datagen.MLP5, M=M, dims=dims)
    wg = [w.to("cuda") for w in Ws]
    xg = _padded(x, 24, float("nan"))          # NaN beyond x's width must never be read
    out = _padded(torch.zeros(M, dims[-1], dtype=torch.float16), 40, 7.0)
    H = max(dims[1:-1])
    acts = [torch.full((M, H + 12), -3.0, dtype=torch.float32, device="cuda")[:, :dims[l + 1]] for l in range(L - 1)]
    mk.mlp_forward_train(xg, wg, out=out, acts=acts)
    inf = mk.mlp_forward(xg, wg)
    torch.cuda.synchronize()
    assert torch.equal(out, inf), "training forward must match the inference forward bit for bit"
    o_out, o_acts = oracle.mlp_forward_train(f64(x), [f64(w) for w in Ws])
    assert_close(f64(out), o_out, 2e-2, "out")
    for l, a in enumerate(acts):
        assert_close(f64(a), o_acts[l], 1e-4 if l == 0 else 2e-2, "acts[%d]" % l)
        base = a.as_strided((M, a.stride(0)), (a.stride(0), 1))
        assert torch.all(base[:, dims[l + 1]:] == -3.0), "a store went past acts[%d]'s width" % l
    obase = out.as_strided((M, out.stride(0)), (out.stride(0), 1))
    assert torch.all(obase[:, dims[-1]:] == 7.0), "a store went past out's width"


def test_nonsquare_grid_invariance():
    dims = (120, 128, 24, 128, 40)
    x, Ws = datagen.mlp_inputs(datagen.MLP3, M=5000, dims=dims)
    xg = mk.aligned_copy(x)
    wg = [w.to("cuda") for w in Ws]
    a = mk.mlp_forward(xg, wg)
    b = mk.mlp_forward(xg, wg, num_workgroups=7)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dims", CHAINS, ids=lambda d: "x".join(map(str, d)))
def test_backward_random_parity(dims):
    L = len(dims) - 1
    for M in (65, 3001):
        progress("nonsquare backward %s M=%d" % (dims, M))
        x, Ws = datagen.mlp_inputs(datagen.MLP5, M=M, dims=dims)
        g = datagen.mlp_grad_output(datagen.MLP5, M=M, dims=dims)
        xg = _padded(x, 8, float("nan"))       # NaN beyond x's width must never be read
        gg = _padded(g, 16, float("nan"))      # nor beyond dout's
        wg = [w.to("cuda") for w in Ws]
        _, acts = mk.mlp_forward_train(xg, wg)
        dW = [torch.full((dims[l], dims[l + 1]), 5.0, device="cuda") for l in range(L)]
        dx = _padded(torch.zeros(M, dims[0], dtype=torch.float16), 24, 9.0)
        mk.mlp_backward(xg, wg, acts, gg, dW=dW, dx=dx)
        torch.cuda.synchronize()
        o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g))
        for l in range(L):
            assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d] %s M=%d" % (l, dims, M))
        assert_close(f64(dx), o_dx, 2e-2, "dx %s M=%d" % (dims, M))
        base = dx.as_strided((M, dx.stride(0)), (dx.stride(0), 1))
        assert torch.all(base[:, dims[0]:] == 9.0), "a store went past dx's width"


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("dims", CHAINS, ids=lambda d: "x".join(map(str, d)))
def test_backward_selection_chains_exact(act, dims):
    L = len(dims) - 1
    M = 333
    x = datagen.integer_matrix((M, dims[0]), 3, 7, 17, 8, "f16")
    g = datagen.integer_matrix((M, dims[-1]), 5, 3, 13, 6, "f16")
    Ws = [_selection(dims[l], dims[l + 1], 70 * l + len(dims)) for l in range(L)]
    xg, gg = mk.aligned_copy(x), mk.aligned_copy(g)
    wg = [w.to("cuda") for w in Ws]
    _, acts = mk.mlp_forward_train(xg, wg, hidden_act=act)
    dW, dx = mk.mlp_backward(xg, wg, acts, gg, hidden_act=act)
    torch.cuda.synchronize()
    o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g), hidden_act=act)
    for l in range(L):
        assert np.array_equal(f64(dW[l]), o_dW[l]), (act, dims, l)
    assert np.array_equal(f64(dx), o_dx), (act, dims)
