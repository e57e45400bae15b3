"""GPU parity of the MLP training pair (coalesce_mlp_forward_train and
coalesce_mlp_backward) against the fp64 oracle.

The backward consumes the activations the GPU's own training forward stored
(fp32), and rounds h_l and dz_l to fp16 as MFMA operands ("MLP Megakernel"
README, "Key ideas"); the oracle recomputes everything in fp64 from x, W
and dout.  Random cases use the same 2e-2 gate (max error over max(|ref|,
rms(ref))) as the forward.  Signed-permutation weights with small integer
inputs make the linear and relu chains exact in fp16/fp32, which pins every
layout step (staging swizzles, transposing reads, weight-gradient block
ownership, the unit order of the chained operands, the reduction) bit for
bit.  Random relu chains are left to those exact cases: where a rounded
pre-activation lands on the other side of 0 the derivative mask flips, an
O(1) change that no tolerance on the backward can absorb.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

CASES = [(128, 3), (64, 5), (128, 1), (128, 2), (128, 4), (64, 1), (64, 2), (64, 8)]


def _workload(D):
    return datagen.MLP3 if D == 128 else datagen.MLP5


def _inputs(D, L, M):
    w = _workload(D)
    dims = (D,) * (L + 1)
    x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
    g = datagen.mlp_grad_output(w, M=M, dims=dims)
    return x, Ws, g


def _gpu_train(x, Ws, g, act="softplus", want_dx=True):
    xg = to_gpu(x)
    wg = [w.to("cuda") for w in Ws]
    out, acts = mk.mlp_forward_train(xg, wg, hidden_act=act)
    dW, dx = mk.mlp_backward(xg, wg, acts, to_gpu(g), hidden_act=act, want_dx=want_dx)
    torch.cuda.synchronize()
    return out, acts, dW, dx


@pytest.mark.parametrize("D,L", CASES)
def test_forward_train_matches_forward_and_oracle(D, L):
    for M in (1, 65, 4097):
        progress("forward_train D=%d L=%d M=%d" % (D, L, M))
        x, Ws, _ = _inputs(D, L, M)
        xg = to_gpu(x)
        wg = [w.to("cuda") for w in Ws]
        out, acts = mk.mlp_forward_train(xg, wg)
        ref_out = mk.mlp_forward(xg, wg)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "training forward must give the inference forward's bits"
        o_out, o_acts = oracle.mlp_forward_train(f64(x), [f64(w) for w in Ws])
        assert_close(f64(out), o_out, 2e-2, "out D=%d L=%d M=%d" % (D, L, M))
        assert len(acts) == L - 1
        for l, a in enumerate(acts):
            # h_1 comes from exact fp16 products accumulated in fp32; deeper
            # layers carry the fp16 rounding of their inputs
            assert_close(f64(a), o_acts[l], 1e-4 if l == 0 else 2e-2, "acts[%d] D=%d L=%d M=%d" % (l, D, L, M))


@pytest.mark.parametrize("D,L", CASES)
def test_backward_random_parity_ragged_rows(D, L):
    for M in (1, 63, 64, 65, 1000, 4097):
        progress("backward D=%d L=%d M=%d" % (D, L, M))
        x, Ws, g = _inputs(D, L, M)
        _, _, dW, dx = _gpu_train(x, Ws, g)
        o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g))
        for l in range(L):
            assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d] D=%d L=%d M=%d" % (l, D, L, M))
        assert_close(f64(dx), o_dx, 2e-2, "dx D=%d L=%d M=%d" % (D, L, M))


@pytest.mark.parametrize("D,L", [(128, 3), (64, 5), (128, 4), (64, 8)])
def test_backward_linear_chain_random(D, L):
    M = 777
    x, Ws, g = _inputs(D, L, M)
    _, _, dW, dx = _gpu_train(x, Ws, g, act="none")
    o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g), hidden_act="none")
    for l in range(L):
        assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d]" % l)
    assert_close(f64(dx), o_dx, 2e-2, "dx")


def _signed_perm(D, seed):
    rng = np.random.default_rng(seed)
    P = np.zeros((D, D))
    P[np.arange(D), rng.permutation(D)] = rng.choice([-1.0, 1.0], D)
    return torch.from_numpy(P).to(torch.float16)


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("D,L", [(128, 1), (128, 2), (128, 3), (128, 4), (64, 1), (64, 3), (64, 5), (64, 8)])
def test_backward_signed_permutations_exact(act, D, L):
    # integer x and dout, signed-permutation weights: every product and sum is
    # an exact small integer in fp16 and fp32, so dW and dx equal the oracle
    for M in (200, 1000):
        x = datagen.integer_matrix((M, D), 3, 7, 17, 8, "f16")
        g = datagen.integer_matrix((M, D), 5, 3, 13, 6, "f16")
        Ws = [_signed_perm(D, 700 * L + 10 * D + l) for l in range(L)]
        out, acts, dW, dx = _gpu_train(x, Ws, g, act=act)
        o_out, o_acts = oracle.mlp_forward_train(f64(x), [f64(w) for w in Ws], hidden_act=act)
        assert np.array_equal(f64(out), o_out)
        for l, a in enumerate(acts):
            assert np.array_equal(f64(a), o_acts[l]), "acts[%d]" % l
        o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g), hidden_act=act)
        for l in range(L):
            assert np.array_equal(f64(dW[l]), o_dW[l]), "dW[%d] act=%s D=%d L=%d M=%d" % (l, act, D, L, M)
        assert np.array_equal(f64(dx), o_dx), "dx act=%s D=%d L=%d M=%d" % (act, D, L, M)


@pytest.mark.parametrize("D,L", [(128, 3), (64, 5)])
def test_identity_weights_sigmoid_chain(D, L):
    # W_l = I: dx = dout * prod_j sigmoid(z_j), z_1 = x, z_{j+1} = softplus(z_j).
    # x spans [-30, 30]: the forward's guard (z > 20) and tiny activations
    # (z down to -30, where 1 - e^{-h} cancels) are both crossed.
    M = 256
    x = torch.linspace(-30, 30, M * D, dtype=torch.float64).reshape(M, D).to(torch.float16)
    g = datagen.mlp_grad_output(_workload(D), M=M, dims=(D,) * (L + 1))
    Ws = [torch.eye(D, dtype=torch.float16) for _ in range(L)]
    _, _, dW, dx = _gpu_train(x, Ws, g)
    _, o_dx = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g))
    y = f64(dx)
    # elementwise, per layer: the derivative 1 - e^{-h} is off by at most
    # 2^-23 absolute (one fp32 ulp of e^{-h} < 1), i.e. |g| 2^-23 in dz since
    # every upstream factor is a sigmoid <= 1; and each of the L - 1 dz_l and
    # dx is rounded to fp16 once: at most 2^-11 relative, or 2^-25 absolute in
    # fp16's subnormal range (below 2^-14, where the spacing is 2^-24)
    gg = np.abs(f64(g))
    bound = 4e-3 * L * np.abs(o_dx) + L * (2.0 ** -24 + gg * 2.0 ** -23)
    assert np.all(np.abs(y - o_dx) <= bound), np.max(np.abs(y - o_dx) / bound)


def test_backward_is_deterministic_and_m0_gives_zero():
    D, L, M = 128, 3, 5000
    x, Ws, g = _inputs(D, L, M)
    xg, gg = to_gpu(x), to_gpu(g)
    wg = [w.to("cuda") for w in Ws]
    _, acts = mk.mlp_forward_train(xg, wg)
    a, dxa = mk.mlp_backward(xg, wg, acts, gg)
    b, dxb = mk.mlp_backward(xg, wg, acts, gg)
    torch.cuda.synchronize()
    for l in range(L):
        assert torch.equal(a[l], b[l])
    assert torch.equal(dxa, dxb)
    # M = 0: the weight gradients are an empty sum
    dW0 = [torch.full((D, D), 7.0, device="cuda") for _ in range(L)]
    x0 = mk.aligned_empty(0, D, torch.float16)
    a0 = [torch.empty((0, D), dtype=torch.float32, device="cuda") for _ in range(L - 1)]
    mk.mlp_backward(x0, wg, a0, mk.aligned_empty(0, D, torch.float16), dW=dW0)
    torch.cuda.synchronize()
    for t in dW0:
        assert torch.count_nonzero(t).item() == 0


def test_backward_without_dx_and_with_padded_pitches():
    D, L, M = 64, 5, 3001
    x, Ws, g = _inputs(D, L, M)
    xg = torch.zeros((M, D + 8), dtype=torch.float16, device="cuda")[:, :D]
    xg.copy_(x.to("cuda"))
    gg = torch.zeros((M, D + 16), dtype=torch.float16, device="cuda")[:, :D]
    gg.copy_(g.to("cuda"))
    wg = [w.to("cuda") for w in Ws]
    acts = [torch.zeros((M, D + 4), dtype=torch.float32, device="cuda")[:, :D] for _ in range(L - 1)]
    out, acts = mk.mlp_forward_train(xg, wg, acts=acts)
    dW, dx = mk.mlp_backward(xg, wg, acts, gg, want_dx=False)
    torch.cuda.synchronize()
    assert dx is None
    o_dW, _ = oracle.mlp_backward(f64(x), [f64(w) for w in Ws], f64(g), want_dx=False)
    for l in range(L):
        assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d]" % l)


def test_module_autograd_matches_oracle():
    # the page's quick start: loss = out.sum(); loss.backward()
    torch.manual_seed(0)
    model = mk.FusedMLPSoftplus(D=128, H=128, out_features=128, layers=3)
    x = datagen.mlp_inputs(datagen.MLP3, M=3000)[0]
    xg = to_gpu(x)
    out = model(xg)
    loss = out.float().sum()
    loss.backward()
    torch.cuda.synchronize()
    Ws = [f64(w.detach()) for w in model.weights]
    ones = np.ones((3000, 128))
    o_dW, _ = oracle.mlp_backward(f64(x), Ws, ones, want_dx=False)
    for l, w in enumerate(model.weights):
        assert w.grad is not None and w.grad.dtype == torch.float16
        assert_close(f64(w.grad), o_dW[l], 2e-2, "grad of W%d" % (l + 1))
    with torch.no_grad():
        assert torch.equal(model(xg), mk.mlp_forward(xg, [w for w in model.weights]))


@pytest.mark.parametrize("w", [datagen.MLP3, datagen.MLP5, datagen.MLP_NS1, datagen.MLP_NS2], ids=lambda w: w.name)
def test_full_size_periodic_rows_and_sampled_dx(w):
    # Full-size rows in the benchmark's launch configuration.  The rows repeat
    # with period P, so every weight gradient is (M / P) times the oracle's
    # gradient of one period (a property of the sum over rows, exact in
    # exact arithmetic); dx and the stored activations are checked on sampled
    # rows, each of which depends on its own row only.
    P = 4096
    M = w.M
    dims = w.dims
    L = len(dims) - 1
    x, Ws = datagen.mlp_inputs(w, M=P)
    g = datagen.mlp_grad_output(w, M=P)
    progress("full-size training pair %s M=%d" % (w.name, M))
    xg = to_gpu(x).repeat(M // P, 1)
    gg = to_gpu(g).repeat(M // P, 1)
    wg = [t.to("cuda") for t in Ws]
    out, acts = mk.mlp_forward_train(xg, wg)
    dW, dx = mk.mlp_backward(xg, wg, acts, gg)
    torch.cuda.synchronize()
    o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(t) for t in Ws], f64(g))
    for l in range(L):
        assert_close(f64(dW[l]), (M // P) * o_dW[l], 2e-2, "dW[%d] %s" % (l, w.name))
    rng = np.random.default_rng(99)
    rows = np.sort(rng.choice(M, 512, replace=False))
    rows_t = torch.from_numpy(rows).to("cuda")
    assert_close(f64(dx.index_select(0, rows_t)), o_dx[rows % P], 2e-2, "sampled dx %s" % w.name)
    _, o_acts = oracle.mlp_forward_train(f64(x), [f64(t) for t in Ws])
    for l in range(L - 1):
        assert_close(f64(acts[l].index_select(0, rows_t)), o_acts[l][rows % P], 2e-2, "sampled acts[%d]" % l)
