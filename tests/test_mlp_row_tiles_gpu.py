"""The resident MLP megakernel's two wave-tile heights give the same bits.

Batches that give each wave of the grid few rows run 16-row wave tiles (the
latency of one tile's layer chain is then the kernel's); large inference
batches run 32-row tiles; the width-128 training forward runs 16-row tiles
at any size, the width-64 one 32-row tiles for large batches.  Every row goes
through the same MFMA accumulation order and the same activation
instructions either way, so the first rows of a large batch (32-row tiles)
must equal a small batch of the same rows (16-row tiles) bit for bit --
square and narrower chains, rows past the softplus guard, and the training
forward's stored activations.  The small batches are also checked against
the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk
import oracle
from helpers import assert_close, f64, progress, to_gpu

pytestmark = pytest.mark.gpu

# (workload, dims, large batch past the 16-row threshold of 96 rows per wave)
CASES = [(datagen.MLP3, (128, 128, 128, 128), 600_000), (datagen.MLP5, (64,) * 6, 700_000),
         (datagen.MLP3, (32, 128, 128, 16), 600_000), (datagen.MLP5, (48, 64, 40, 64, 24), 700_000)]


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("w,dims,big", CASES, ids=lambda v: str(v) if isinstance(v, tuple) else None)
def test_small_batch_tiles_equal_large_batch_tiles(w, dims, big):
    x, Ws = datagen.mlp_inputs(w, M=big, dims=dims)
    # a few rows far past the guard (z > 20) and past the fp32 range of exp
    x[[5, 3000, big - 1]] = (40.0 * torch.sign(x[[5, 3000, big - 1]].float())).to(torch.float16)
    xg, wg = to_gpu(x), [t.to("cuda") for t in Ws]
    progress("row tiles %s M=%d" % (dims, big))
    full = mk.mlp_forward(xg, wg)
    for m in (1, 4097, 60_000):
        part = mk.mlp_forward(xg[:m], wg)
        torch.cuda.synchronize()
        assert torch.equal(_bits(full[:m]), _bits(part)), (dims, m)
    ref = oracle.mlp_forward(f64(x[:4097]), [f64(t) for t in Ws])
    assert_close(f64(full[:4097]), ref, 2e-2, "small batch %s" % (dims,))


@pytest.mark.parametrize("w,dims,big", CASES[:2], ids=lambda v: str(v) if isinstance(v, tuple) else None)
def test_training_forward_tiles_agree(w, dims, big):
    # the width-64 training forward switches tile height with the batch size;
    # the width-128 one keeps 16-row tiles, and its output must still equal
    # the inference forward's (32-row tiles at this size)
    x, Ws = datagen.mlp_inputs(w, M=big, dims=dims)
    xg, wg = to_gpu(x), [t.to("cuda") for t in Ws]
    progress("training row tiles %s M=%d" % (dims, big))
    out, acts = mk.mlp_forward_train(xg, wg)
    inf = mk.mlp_forward(xg, wg)
    m = 5001
    out_s, acts_s = mk.mlp_forward_train(xg[:m], wg)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(inf))
    assert torch.equal(_bits(out[:m]), _bits(out_s))
    for a, b in zip(acts, acts_s):
        assert torch.equal(_bits(a[:m]), _bits(b))
    o_out, o_acts = oracle.mlp_forward_train(f64(x[:m]), [f64(t) for t in Ws])
    assert_close(f64(out_s), o_out, 2e-2, "training out")
    for l, a in enumerate(acts_s):
        # h_1 comes from exact fp16 products accumulated in fp32; deeper
        # layers carry the fp16 rounding of their inputs
        assert_close(f64(a), o_acts[l], 1e-4 if l == 0 else 2e-2, "training acts[%d]" % l)
