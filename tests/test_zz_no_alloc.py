"""coalesce_mlp_backward_noalloc against coalesce_mlp_backward.

The no-allocation entry point runs the same kernels with the same grid as the
workspace entry point, only with the per-workgroup partial sums in the
library's own device scratch, so its weight gradients and dx must equal the
workspace entry point's bit for bit.  Two calls in a row share the scratch;
the second, on fewer rows (fewer workgroups, fewer partial sums), must not
see anything the first left behind.  Both calls are also held to the oracle
at the 2e-2 gate.  Chains run layer by layer keep their hidden gradients in
the scratch too, so they fit only up to a row count; beyond it the call is
rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu


def _case(D, L, M):
    w = datagen.MLP3 if D == 128 else datagen.MLP5
    dims = (D,) * (L + 1)
    x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
    g = datagen.mlp_grad_output(w, M=M, dims=dims)
    return x, Ws, g


def _same(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


@pytest.mark.parametrize("D,L,rows", [(128, 3, (20000, 3001)), (64, 5, (50000, 777)), (128, 4, (9000, 65)),
                                      (64, 8, (4097, 1))])
def test_noalloc_backward_equals_workspace_backward(D, L, rows):
    for M in rows:  # two calls in a row, the second on fewer rows
        progress("noalloc backward D=%d L=%d M=%d" % (D, L, M))
        x, Ws, g = _case(D, L, M)
        xg, gg = to_gpu(x), to_gpu(g)
        wg = [t.to("cuda") for t in Ws]
        _, acts = mk.mlp_forward_train(xg, wg)
        dW_ref, dx_ref = mk.mlp_backward(xg, wg, acts, gg)
        dW = [torch.full_like(t, float("nan")) for t in dW_ref]
        dx = torch.full_like(dx_ref, float("nan"))
        mk.mlp_backward_noalloc(xg, wg, acts, gg, dW=dW, dx=dx)
        torch.cuda.synchronize()
        for l in range(L):
            assert _same(dW[l], dW_ref[l]), "dW[%d] D=%d L=%d M=%d" % (l, D, L, M)
        assert _same(dx, dx_ref), "dx D=%d L=%d M=%d" % (D, L, M)
        if M <= 5000:
            o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(t) for t in Ws], f64(g))
            for l in range(L):
                assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d]" % l)
            assert_close(f64(dx), o_dx, 2e-2, "dx")


def test_noalloc_backward_without_dx_and_nonsquare():
    # a non-square chain (run padded) and dx skipped, again twice in a row
    w = datagen.MLP_NS2
    for M in (30000, 999):
        progress("noalloc backward %s M=%d" % (w.name, M))
        x, Ws = datagen.mlp_inputs(w, M=M)
        g = datagen.mlp_grad_output(w, M=M)
        xg, gg = to_gpu(x), to_gpu(g)
        wg = [t.to("cuda") for t in Ws]
        _, acts = mk.mlp_forward_train(xg, wg)
        dW_ref, _ = mk.mlp_backward(xg, wg, acts, gg, want_dx=False)
        dW = [torch.full_like(t, float("nan")) for t in dW_ref]
        _, dx = mk.mlp_backward_noalloc(xg, wg, acts, gg, dW=dW, dx=None)
        torch.cuda.synchronize()
        assert dx is None
        for l in range(len(Ws)):
            assert _same(dW[l], dW_ref[l]), "dW[%d] M=%d" % (l, M)


@pytest.mark.parametrize("dims,rows", [((128,) * 7, (20000, 777)), ((256, 128, 40, 136), (9000, 33))],
                         ids=["6x128", "256_128_40_136"])
def test_noalloc_backward_layer_by_layer_chains(dims, rows):
    # chains whose weights exceed the LDS: the scratch holds one layer's
    # partial sums and the fp16 hidden gradients of all M rows; two calls in
    # a row, the second on fewer rows
    w = datagen.MLP3
    L = len(dims) - 1
    for M in rows:
        progress("noalloc layer-by-layer backward %s M=%d" % (dims, M))
        x, Ws = datagen.mlp_inputs(w, M=M, dims=dims)
        g = datagen.mlp_grad_output(w, M=M, dims=dims)
        xg, gg = to_gpu(x), to_gpu(g)
        wg = [t.to("cuda") for t in Ws]
        _, acts = mk.mlp_forward_train(xg, wg)
        dW_ref, dx_ref = mk.mlp_backward(xg, wg, acts, gg)
        dW = [torch.full_like(t, float("nan")) for t in dW_ref]
        dx = torch.full_like(dx_ref, float("nan"))
        mk.mlp_backward_noalloc(xg, wg, acts, gg, dW=dW, dx=dx)
        torch.cuda.synchronize()
        for l in range(L):
            assert _same(dW[l], dW_ref[l]), "dW[%d] %s M=%d" % (l, dims, M)
        assert _same(dx, dx_ref), "dx %s M=%d" % (dims, M)
        if M <= 5000:
            o_dW, o_dx = oracle.mlp_backward(f64(x), [f64(t) for t in Ws], f64(g))
            for l in range(L):
                assert_close(f64(dW[l]), o_dW[l], 2e-2, "dW[%d]" % l)
            assert_close(f64(dx), o_dx, 2e-2, "dx")


def test_noalloc_backward_rejects_a_workspace_beyond_its_scratch():
    # 6 x 128 on 2^20 rows needs 2 x 256 MiB of hidden gradients: rejected
    # before anything is launched, the outputs untouched
    dims = (128,) * 7
    M = 1 << 20
    assert mk.mlp_backward_workspace_size(dims, M) > (64 << 20)
    x = torch.zeros((M, 128), dtype=torch.float16, device="cuda")
    Ws = [torch.zeros((128, 128), dtype=torch.float16, device="cuda") for _ in range(6)]
    acts = [torch.zeros((M, 128), dtype=torch.float32, device="cuda") for _ in range(5)]
    dW = [torch.full((128, 128), 7.0, device="cuda") for _ in range(6)]
    with pytest.raises(mk.CoalesceError) as e:
        mk.mlp_backward_noalloc(x, Ws, acts, x, dW=dW, dx=None)
    assert e.value.status == mk.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in dW)
