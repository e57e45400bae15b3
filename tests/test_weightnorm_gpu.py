"""GPU parity of the fused weight normalisation (coalesce_weight_norm and its
backward) against the fp64 oracle, and of the weight-normalised training
step ("MLP Megakernel" README, "Key ideas": W = g * v / ||v|| for every
layer in one launch; the quick start's FusedMLPSoftplusWN).

W is computed in fp32 and rounded once to fp16, so it must equal the oracle's
fp64 W rounded to fp16 to within one fp16 unit in the last place (the fp32
sum of squares is off by at most d_in 2^-24 relative, far below half an fp16
ulp, so almost every element matches exactly).  The backward is fp32
throughout: the 1e-4 gate of the FP32 GEMM.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

CHAINS = [("fp16_mlp3_d128", (128, 128, 128, 128)), ("fp16_mlp5_d64", (64,) * 6),
          ("nonsquare", (64, 96, 128, 32, 200)), ("tiny", (3, 1, 5)), ("eight", (64,) * 9)]


def _fp16_ulp(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _gpu(ts):
    return [t.to("cuda").contiguous() for t in ts]


@pytest.mark.parametrize("name,dims", CHAINS, ids=[c[0] for c in CHAINS])
def test_weight_norm_matches_oracle(name, dims):
    progress("weight_norm %s %s" % (name, dims))
    vs, gs = datagen.wn_inputs(datagen.MLP3, dims=dims)
    Ws = mk.weight_norm(_gpu(vs), _gpu(gs))
    torch.cuda.synchronize()
    exact = total = 0
    for l, (v, g, W) in enumerate(zip(vs, gs, Ws)):
        ref = oracle.weight_norm(f64(v), f64(g))
        ref16 = torch.from_numpy(ref).to(torch.float16).double().numpy()  # the oracle rounded to fp16 (RNE)
        y = f64(W)
        assert np.all(np.abs(y - ref16) <= _fp16_ulp(ref)), (name, l)
        exact += int(np.sum(y == ref16))
        total += y.size
    assert exact >= 0.99 * total, (exact, total)


def test_weight_norm_repeatable_and_zero_column():
    vs, gs = datagen.wn_inputs(datagen.MLP5)
    v, g = _gpu(vs), _gpu(gs)
    a = mk.weight_norm(v, g)
    b = mk.weight_norm(v, g)
    v[1][:, 7] = 0
    c = mk.weight_norm(v, g)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert torch.isnan(c[1][:, 7]).all()
    assert torch.equal(c[0], a[0]) and torch.equal(c[1][:, :7], a[1][:, :7])


@pytest.mark.parametrize("name,dims", CHAINS, ids=[c[0] for c in CHAINS])
def test_weight_norm_backward_matches_oracle(name, dims):
    vs, gs = datagen.wn_inputs(datagen.MLP5, dims=dims)
    rng = np.random.default_rng(len(dims))
    dWs = [torch.from_numpy(rng.standard_normal(v.shape).astype(np.float32)) for v in vs]
    dv, dg = mk.weight_norm_backward(_gpu(vs), _gpu(gs), _gpu(dWs))
    torch.cuda.synchronize()
    for l in range(len(vs)):
        o_dv, o_dg = oracle.weight_norm_backward(f64(vs[l]), f64(gs[l]), f64(dWs[l]))
        assert_close(f64(dv[l]), o_dv, 1e-4, "dv[%d] %s" % (l, name))
        assert_close(f64(dg[l]), o_dg, 1e-4, "dg[%d] %s" % (l, name))


@pytest.mark.parametrize("D,L", [(128, 3), (64, 5)])
def test_weight_normalised_training_step(D, L):
    # the page's quick start with weight normalisation: loss = out.sum()
    torch.manual_seed(1)
    model = mk.FusedMLPSoftplusWN(D=D, H=D, out_features=D, layers=L)
    with torch.no_grad():
        vs, gs = datagen.wn_inputs(datagen.MLP3 if D == 128 else datagen.MLP5, dims=(D,) * (L + 1))
        for p, t in zip(model.v, vs):
            p.copy_(t)
        for p, t in zip(model.g, gs):
            p.copy_(t)
    M = 2000
    x = datagen.mlp_inputs(datagen.MLP3 if D == 128 else datagen.MLP5, M=M, dims=(D,) * (L + 1))[0]
    out = model(to_gpu(x))
    out.float().sum().backward()
    torch.cuda.synchronize()
    Wo = [oracle.weight_norm(f64(v), f64(g)) for v, g in zip(vs, gs)]
    o_out = oracle.mlp_forward(f64(x), Wo)
    assert_close(f64(out.detach()), o_out, 2e-2, "out")
    o_dW, _ = oracle.mlp_backward(f64(x), Wo, np.ones((M, D)), want_dx=False)
    for l in range(L):
        o_dv, o_dg = oracle.weight_norm_backward(f64(vs[l]), f64(gs[l]), o_dW[l])
        assert model.v[l].grad.dtype == torch.float16
        assert_close(f64(model.v[l].grad), o_dv, 2e-2, "dv[%d]" % l)
        assert_close(f64(model.g[l].grad), o_dg, 2e-2, "dg[%d]" % l)
