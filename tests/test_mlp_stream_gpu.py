"""GPU parity of the layer-streaming MLP megakernel (mlp_stream.hip), which
runs the chains whose weights do not all fit in LDS at once: more than 4
layers of width up to 128 or 8 of width up to 64, and any chain with a
layer wider than 128 (up to 256), up to 16 layers ("MLP Megakernel" README:
the megakernel generalised to N layers and to D != H != out).

Exact cases: integer x, signed-permutation weights and a linear or relu
chain are exact in fp16 and fp32, so the output must equal the oracle bit
for bit; this pins the chunked weight staging, the transposing weight reads
in both k orders, the chaining of the result layout and the masked edges.
Random softplus chains use the 2e-2 gate of the other MLP tests.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

# (dims): beyond the resident kernel's LDS: deep at 128 and 64, wide, mixed
DEEP128 = (128,) * 7                      # 6 layers of 128
WIDE = (256, 256, 256, 256)               # 3 layers of 256
DEEP64 = (64,) * 13                       # 12 layers of 64
MIXED = (200, 256, 40, 136, 256, 8, 64)   # ragged widths, a 256 layer
DEEP16 = (32, 96, 64, 128, 64, 96, 128, 32, 64, 128, 96, 64, 32, 128, 64, 96, 48)  # 16 layers


def _signed_perm(rows, cols, seed):
    # a signed partial permutation (rows x cols): at most one +-1 per row and column
    rng = np.random.default_rng(seed)
    P = np.zeros((rows, cols))
    n = min(rows, cols)
    P[rng.permutation(rows)[:n], rng.permutation(cols)[:n]] = rng.choice([-1.0, 1.0], n)
    return torch.from_numpy(P).to(torch.float16)


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("dims", [DEEP128, WIDE, DEEP64, MIXED, DEEP16], ids=lambda d: "x".join(map(str, d)))
def test_exact_signed_permutation_chains(act, dims):
    L = len(dims) - 1
    for M in (33, 1000):
        progress("stream exact %s %s M=%d" % (act, dims, M))
        x = datagen.integer_matrix((M, dims[0]), 3, 7, 17, 8, "f16")
        Ws = [_signed_perm(dims[l], dims[l + 1], 50 * L + l) for l in range(L)]
        out = mk.mlp_forward(to_gpu(x), [w.to("cuda") for w in Ws], hidden_act=act)
        ref = oracle.mlp_forward(f64(x), [f64(w) for w in Ws], hidden_act=act)
        assert np.array_equal(f64(out), ref), (dims, act, M)


@pytest.mark.parametrize("dims", [DEEP128, WIDE, DEEP64, MIXED, DEEP16], ids=lambda d: "x".join(map(str, d)))
def test_random_softplus_parity_ragged_rows(dims):
    w = datagen.MLP3
    for M in (1, 65, 1000, 4097):
        progress("stream random %s M=%d" % (dims, M))
        x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
        out = mk.mlp_forward(to_gpu(x), [t.to("cuda") for t in Ws])
        ref = oracle.mlp_forward(f64(x), [f64(t) for t in Ws])
        assert_close(f64(out), ref, 2e-2, "%s M=%d" % (dims, M))


@pytest.mark.parametrize("dims", [DEEP128, WIDE, MIXED], ids=lambda d: "x".join(map(str, d)))
def test_training_forward(dims):
    w = datagen.MLP3
    L = len(dims) - 1
    M = 3001
    x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
    xg, wg = to_gpu(x), [t.to("cuda") for t in Ws]
    out, acts = mk.mlp_forward_train(xg, wg)
    ref_out = mk.mlp_forward(xg, wg)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "training forward must give the inference forward's bits"
    o_out, o_acts = oracle.mlp_forward_train(f64(x), [f64(t) for t in Ws])
    assert_close(f64(out), o_out, 2e-2, "out %s" % (dims,))
    assert len(acts) == L - 1
    for l, a in enumerate(acts):
        assert_close(f64(a), o_acts[l], 1e-4 if l == 0 else 2e-2, "acts[%d] %s" % (l, dims))


def test_grid_invariance_and_nan_free_padding():
    # results do not depend on the grid; padded units never leak into outputs
    dims = MIXED
    M = 8 * 32 * 37 + 5
    x, Ws = datagen.mlp_inputs(datagen.MLP3, M=M, dims=dims)
    xg, wg = to_gpu(x), [t.to("cuda") for t in Ws]
    outs = [mk.mlp_forward(xg, wg, num_workgroups=g).cpu() for g in (0, 1, 3, mk.device_cu_count())]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    # NaN-filled pitch padding of x must stay unread, of out unwritten
    D, O = dims[0], dims[-1]
    xb = torch.full((M, D + 24), float("nan"), dtype=torch.float16, device="cuda")
    xb[:, :D] = xg
    ob = torch.full((M, O + 8), float("nan"), dtype=torch.float16, device="cuda")
    mk.mlp_forward(xb[:, :D], wg, out=ob[:, :O])
    torch.cuda.synchronize()
    assert torch.equal(ob[:, :O].cpu().view(torch.int16), outs[0].view(torch.int16))
    assert bool(torch.isnan(ob[:, O:]).all())


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("dims", [DEEP128, WIDE], ids=lambda d: "x".join(map(str, d)))
def test_small_batches_equal_rows_of_a_large_batch(dims):
    # A round hands wave w of workgroup b the tile r G W + b + w G; small
    # batches leave most waves of a round without a tile (they copy the
    # chunks and pass the barriers, nothing else).  Each row's arithmetic does
    # not depend on which wave runs it, so a small batch must equal the same
    # rows of a large one bit for bit, forward and training forward (out and
    # the stored activations), on the default grid and on a few others.
    w = datagen.MLP3
    big = 70_000
    x, Ws = datagen.mlp_inputs(w, M=big, dims=dims)
    xg, wg = to_gpu(x), [t.to("cuda") for t in Ws]
    progress("stream small batches %s M=%d" % ("x".join(map(str, dims)), big))
    full = mk.mlp_forward(xg, wg)
    tout, tacts = mk.mlp_forward_train(xg, wg)
    torch.cuda.synchronize()
    assert torch.equal(_bits(tout), _bits(full))
    for m in (1, 33, 1000, 9000):
        for g in (0, 1, 7):
            part = mk.mlp_forward(xg[:m], wg, num_workgroups=g)
            assert torch.equal(_bits(part), _bits(full[:m])), (m, g)
        o, a = mk.mlp_forward_train(xg[:m], wg)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(full[:m])), m
        for l, (s, t) in enumerate(zip(a, tacts)):
            assert torch.equal(_bits(s), _bits(t[:m])), (m, l)
    ref = oracle.mlp_forward(f64(x[:1000]), [f64(t) for t in Ws])
    assert_close(f64(full[:1000]), ref, 2e-2, "small batch %s" % ("x".join(map(str, dims)),))
