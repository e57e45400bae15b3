"""coalesce_mlp_backward_noalloc against coalesce_mlp_backward.

The no-allocation entry point runs the same kernels with the same grid as the
workspace entry point, only with the per-workgroup partial sums in the
library's own device scratch, so its weight gradients and dx must equal the
workspace entry point's bit for bit.  Two calls in a row share the scratch;
the second, on fewer rows (fewer workgroups, fewer partial sums), must not
see anything the first left behind.  Both calls are also held to the oracle
at the 2e-2 gate.
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
