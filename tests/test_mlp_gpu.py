"""GPU parity of the persistent MLP megakernel (coalesce_mlp_forward).

The GPU rounds every hidden activation to fp16 (the next layer's MFMA
operand, "MLP Megakernel" README: fp16 only at tile boundaries) while the
oracle keeps fp64 throughout, so random cases use the 2e-2 gate.  Signed
permutation weights make the linear chain exact, which pins the
register-to-register layer chaining bit for bit.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

CASES = [(64, 1), (64, 2), (64, 3), (64, 5), (64, 8), (128, 1), (128, 2), (128, 3), (128, 4)]


def _signed_perm(D, seed):
    rng = np.random.default_rng(seed)
    P = np.zeros((D, D))
    P[np.arange(D), rng.permutation(D)] = rng.choice([-1.0, 1.0], D)
    return torch.from_numpy(P).to(torch.float16)


@pytest.mark.parametrize("D,L", CASES)
def test_linear_chain_signed_permutations_exact(D, L):
    M = 200
    x = datagen.integer_matrix((M, D), 3, 7, 17, 8, "f16")
    Ws = [_signed_perm(D, 100 * L + l) for l in range(L)]
    out = mk.mlp_forward(to_gpu(x), [w.to("cuda") for w in Ws], hidden_act="none")
    ref = oracle.mlp_forward(f64(x), [f64(w) for w in Ws], hidden_act="none")
    assert np.array_equal(f64(out), ref), (D, L)


@pytest.mark.parametrize("D,L", [(64, 3), (64, 5), (128, 2), (128, 3)])
def test_relu_chains(D, L):
    # signed-permutation weights and integer x: every layer is exact in fp16
    M = 200
    x = datagen.integer_matrix((M, D), 3, 7, 17, 8, "f16")
    Ws = [_signed_perm(D, 300 * L + l) for l in range(L)]
    out = mk.mlp_forward(to_gpu(x), [w.to("cuda") for w in Ws], hidden_act="relu")
    ref = oracle.mlp_forward(f64(x), [f64(w) for w in Ws], hidden_act="relu")
    assert np.array_equal(f64(out), ref), (D, L)
    # random inputs, ragged rows, the 2e-2 gate
    w = datagen.MLP3 if D == 128 else datagen.MLP5
    x, Ws = datagen.mlp_inputs(w, M=1000, dims=(D,) * (L + 1))
    out = mk.mlp_forward(to_gpu(x), [t.to("cuda") for t in Ws], hidden_act="relu")
    ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws], hidden_act="relu")
    assert_close(f64(out), ref, 2e-2, "relu D=%d L=%d" % (D, L))


@pytest.mark.parametrize("D,L", CASES)
def test_random_parity_ragged_rows(D, L):
    w = datagen.MLP3 if D == 128 else datagen.MLP5
    for M in (1, 63, 65, 1000, 4097):
        progress("mlp D=%d L=%d M=%d" % (D, L, M))
        x, Ws = datagen.mlp_inputs(w, M=M, dims=(D,) * (L + 1))
        out = mk.mlp_forward(to_gpu(x), [t.to("cuda") for t in Ws])
        ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws])
        assert_close(f64(out), ref, 2e-2, "D=%d L=%d M=%d" % (D, L, M))


@pytest.mark.parametrize("D,L", [(64, 5), (128, 3)])
def test_identity_weights_softplus_sweep(D, L):
    # W_l = I: out = softplus applied L-1 times elementwise; x crosses the
    # guard at 20 and the underflow region.
    M = 256
    x = torch.linspace(-30, 30, M * D, dtype=torch.float64).reshape(M, D).to(torch.float16)
    Ws = [torch.eye(D, dtype=torch.float16) for _ in range(L)]
    out = mk.mlp_forward(to_gpu(x), [t.to("cuda") for t in Ws])
    ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws])
    y = f64(out)
    # elementwise: every hidden value is rounded to fp16 (2^-11 relative)
    err = np.abs(y - ref) / np.maximum(np.abs(ref), 1e-4)
    assert err.max() < 4e-3, err.max()


def test_zero_first_and_last_layer():
    D, L, M = 128, 3, 777
    x, Ws = datagen.mlp_inputs(datagen.MLP3, M=M)
    Ws0 = [torch.zeros_like(Ws[0])] + Ws[1:]
    out = f64(mk.mlp_forward(to_gpu(x), [t.to("cuda") for t in Ws0]))
    assert np.all(out == out[0:1, :]), "rows must be identical when W1 = 0"
    ref = oracle.mlp_forward(f64(x[:1]), [f64(t) for t in Ws0])
    assert_close(out[:1], ref, 2e-2, "W1 = 0")
    WsL = Ws[:-1] + [torch.zeros_like(Ws[-1])]
    outL = f64(mk.mlp_forward(to_gpu(x), [t.to("cuda") for t in WsL]))
    assert np.array_equal(outL, np.zeros_like(outL))


@pytest.mark.parametrize("D,L", [(64, 5), (128, 3)])
def test_grid_size_and_row_order_invariance(D, L):
    w = datagen.MLP3 if D == 128 else datagen.MLP5
    M = 64 * 300 + 17
    x, Ws = datagen.mlp_inputs(w, M=M, dims=(D,) * (L + 1))
    xg, Wg = to_gpu(x), [t.to("cuda") for t in Ws]
    tiles = (M + 63) // 64
    outs = [mk.mlp_forward(xg, Wg, num_workgroups=g).cpu() for g in (0, 1, 7, mk.device_cu_count(), tiles)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    perm = torch.from_numpy(np.random.default_rng(5).permutation(M))
    outp = mk.mlp_forward(to_gpu(x[perm]), Wg).cpu()
    assert torch.equal(outp.view(torch.int16), outs[0][perm].view(torch.int16))


@pytest.mark.parametrize("D,L", [(64, 5), (128, 3), (128, 2)])
def test_guard_recompute_mixed_rows(D, L):
    # A few rows with large inputs push softplus arguments past the guard at
    # z = 20 and past the fp32 range of exp (z > 88.7); the workgroups that
    # own them recompute their tiles with the guarded form.  Results must
    # match the oracle, and be bit-identical whichever wave and grid gets the
    # rows.
    w = datagen.MLP3 if D == 128 else datagen.MLP5
    M = 64 * 150 + 5
    x, Ws = datagen.mlp_inputs(w, M=M, dims=(D,) * (L + 1))
    big = [3, 700, 4001, M - 1]
    x[big] = (40.0 * torch.sign(x[big].float())).to(torch.float16)
    xg, Wg = to_gpu(x), [t.to("cuda") for t in Ws]
    out = mk.mlp_forward(xg, Wg).cpu()
    ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws])
    assert_close(f64(out), ref, 2e-2, "mixed large rows D=%d L=%d" % (D, L))
    for g in (1, 5, mk.device_cu_count()):
        o = mk.mlp_forward(xg, Wg, num_workgroups=g).cpu()
        assert torch.equal(o.view(torch.int16), out.view(torch.int16)), g
    perm = torch.from_numpy(np.random.default_rng(11).permutation(M))
    outp = mk.mlp_forward(to_gpu(x[perm]), Wg).cpu()
    assert torch.equal(outp.view(torch.int16), out[perm].view(torch.int16))


@pytest.mark.parametrize("D,L", [(64, 5), (128, 3)])
def test_nan_rows_stay_in_their_rows(D, L):
    # A NaN input row gives NaN outputs in that row only.  NaN also trips the
    # softplus guard's check (the maximum propagates NaN), so its workgroup
    # recomputes its tiles with the guarded form: every other row must keep
    # the bits of the run without NaN.
    w = datagen.MLP3 if D == 128 else datagen.MLP5
    M = 64 * 150 + 5
    x, Ws = datagen.mlp_inputs(w, M=M, dims=(D,) * (L + 1))
    Wg = [t.to("cuda") for t in Ws]
    clean = mk.mlp_forward(to_gpu(x), Wg).cpu()
    nan_rows = [2, 901, M - 1]
    xn = x.clone()
    xn[nan_rows] = float("nan")
    out = mk.mlp_forward(to_gpu(xn), Wg).cpu()
    keep = torch.ones(M, dtype=torch.bool)
    keep[nan_rows] = False
    assert torch.isnan(out[nan_rows]).all()
    assert torch.equal(out[keep].view(torch.int16), clean[keep].view(torch.int16))


def test_unfused_baseline_matches_oracle():
    # per-layer GEMM (fp16 out) + separate softplus kernel: the unfused chain
    D, L, M = 128, 3, 3000
    x, Ws = datagen.mlp_inputs(datagen.MLP3, M=M)
    h = to_gpu(x)
    for l, Wl in enumerate(Ws):
        h = mk.gemm_bias_act(h, Wl.to("cuda"), None, act="none")
        if l < L - 1:
            h = mk.activation(h, "softplus")
    ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws])
    assert_close(f64(h), ref, 2e-2, "unfused MLP")


@pytest.mark.parametrize("name", ["fp16_mlp3_d128", "fp16_mlp5_d64", "fp16_mlp_32_128_128_16",
                                  "fp16_mlp_64_128_96_128_32"])
def test_full_size_sampled_rows(name):
    w = datagen.WORKLOADS[name]
    progress("full size %s" % name)
    x, Ws = datagen.mlp_inputs(w)
    out = mk.mlp_forward(x.to("cuda"), [t.to("cuda") for t in Ws])
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.concatenate([rng.integers(0, w.M, 8192), [0, 1, w.M - 2, w.M - 1]])
    ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws], rows=rows)
    got = f64(out[torch.from_numpy(rows).to("cuda")])
    e = assert_close(got, ref, 2e-2, name)
    progress("%s: sampled E=%.3e" % (name, e))
    # deterministic across calls
    out2 = mk.mlp_forward(x.to("cuda"), [t.to("cuda") for t in Ws])
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
