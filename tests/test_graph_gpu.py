"""The entry points under HIP graph capture: each one only enqueues kernels on
the caller's stream (no allocation, no memset, no synchronisation), so a
captured call replays the same work.  A graph holding the fused GEMM, the MLP
forward and the training pair is captured once and replayed several times,
with the inputs rewritten in place and eager work between the replays; every
replay must reproduce, bit for bit, what the eager calls give on the same
inputs (the small-batch setting where the pages time graphed launches).
"""
import pytest
import torch

import datagen
import mlp_megakernel_amd as mk

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    g = datagen.BF16_FFN
    A0, B, bias = datagen.gemm_inputs(g, M=512, N=1024, K=512)
    A = A0.to("cuda")
    B, bias = B.to("cuda"), bias.to("cuda")
    Y = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")

    w = datagen.MLP3
    M = 4096
    x0, Ws = datagen.mlp_inputs(w, M=M)
    x = x0.to("cuda")
    Ws = [t.to("cuda") for t in Ws]
    out = torch.empty((M, 128), dtype=torch.float16, device="cuda")
    out_t = torch.empty_like(out)
    acts = [torch.empty((M, 128), dtype=torch.float32, device="cuda") for _ in range(w.L - 1)]
    dout = datagen.mlp_grad_output(w, M=M).to("cuda")
    dW = [torch.empty((128, 128), dtype=torch.float32, device="cuda") for _ in range(w.L)]
    dx = torch.empty_like(x)
    ws = torch.empty(mk.mlp_backward_workspace_size(w.dims, w.M), dtype=torch.uint8, device="cuda")

    def work():
        mk.gemm_bias_act(A, B, bias, act="gelu", out=Y)
        mk.mlp_forward(x, Ws, out=out)
        mk.mlp_forward_train(x, Ws, out=out_t, acts=acts)
        mk.mlp_backward(x, Ws, acts, dout, dW=dW, dx=dx, workspace=ws)

    def snapshot():
        return [t.clone() for t in (Y, out, out_t, dx, *acts, *dW)]

    # eager warm-up: the library's per-device queries happen outside capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(4):
        # new inputs, written in place (the graph reads the same buffers)
        A.copy_(torch.randn(A.shape, generator=gen).to(A.dtype))
        x.copy_(torch.randn(x.shape, generator=gen).to(x.dtype))
        dout.copy_(torch.randn(dout.shape, generator=gen).to(dout.dtype))
        work()                       # eager reference on these inputs
        torch.cuda.synchronize()
        ref = snapshot()
        for t in (Y, out, out_t, dx, *acts, *dW):
            t.fill_(float("nan"))    # eager work between, and proof the replay writes everything
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (r, o) in enumerate(zip(ref, got)):
            assert torch.equal(r, o), "replay %d, output %d differs from the eager call" % (rep, i)
