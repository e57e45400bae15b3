"""The matrix-core rate probe behind the bench line's measured ceiling: its
launch covers every CU with 8 waves, its work is what it claims (exact sums
on all-ones operands: each round adds 2 x 32 to each of a lane's 128
accumulators), the per-wave counters are sane, and a call with buffers too
small for the launch is refused before any launch."""
import pytest
import torch

import mlp_megakernel_amd as mk

pytestmark = pytest.mark.gpu


def _buffers(waves):
    sink = torch.full((waves * 64,), float("nan"), dtype=torch.float32, device="cuda")
    clocks = torch.zeros(waves * 2, dtype=torch.int64, device="cuda")
    return sink, clocks


def test_launch_shape():
    assert mk.matrix_rate_waves() == 8 * mk.device_cu_count()


@pytest.mark.parametrize("iters", [1, 3, 64])
def test_all_ones_sums_are_exact(iters):
    waves = mk.matrix_rate_waves()
    ops = torch.ones((4, 24, 64, 8), dtype=torch.bfloat16, device="cuda")
    sink, clocks = _buffers(waves)
    got_waves, khz = mk.matrix_rate(ops, iters, sink, clocks)
    torch.cuda.synchronize()
    assert got_waves == waves and khz > 0
    assert torch.all(sink == 8192.0 * iters), sink.unique()[:8]


def test_zero_operands_and_counters():
    waves = mk.matrix_rate_waves()
    ops = torch.zeros((64, 24, 64, 8), dtype=torch.bfloat16, device="cuda")
    sink, clocks = _buffers(waves)
    iters = 256
    _, khz = mk.matrix_rate(ops, iters, sink, clocks)
    torch.cuda.synchronize()
    assert torch.all(sink == 0.0)
    c = clocks.view(-1, 2).cpu()
    assert torch.all(c > 0)
    # the engine clock of each wave's loop, from its two counters
    ghz = c[:, 0].double() / c[:, 1].double() * khz / 1e6
    assert float(ghz.min()) > 0.3 and float(ghz.max()) < 3.5, (float(ghz.min()), float(ghz.max()))
    # 64 MFMAs of >= 8 cycles each per round: no wave can finish faster
    assert int(c[:, 0].min()) >= 64 * 8 * iters


def test_random_operands_scale_with_rounds():
    waves = mk.matrix_rate_waves()
    gen = torch.Generator().manual_seed(3)
    ops = torch.randn((16, 24, 64, 8), generator=gen).to(torch.bfloat16).cuda()
    s1, c1 = _buffers(waves)
    s2, c2 = _buffers(waves)
    mk.matrix_rate(ops, 1, s1, c1)
    mk.matrix_rate(ops, 2, s2, c2)
    torch.cuda.synchronize()
    assert torch.isfinite(s1).all() and torch.isfinite(s2).all()
    # waves with the same operand set (w mod 16) give the same sums
    v1 = s1.view(-1, 64)
    assert torch.equal(v1[0], v1[16]) and torch.equal(v1[5], v1[5 + 16 * 3])
    assert torch.allclose(s2, 2 * s1, rtol=1e-4, atol=1e-2 * float(s1.abs().mean()))


def test_too_small_buffers_are_refused():
    waves = mk.matrix_rate_waves()
    ops = torch.ones((1, 24, 64, 8), dtype=torch.bfloat16, device="cuda")
    sink, clocks = _buffers(waves - 1)
    with pytest.raises(mk.CoalesceError):
        mk.matrix_rate(ops, 1, sink, clocks)
    torch.cuda.synchronize()
    assert torch.isnan(sink).all()
