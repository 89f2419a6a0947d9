"""The library keeps no state between calls: calls queued on two streams at
once give the same bits as the same calls run one after another."""
import pytest
import torch

import dsc_inputs as di
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_two_streams_match_serial():
    import dynamic_short_causal_amd as dsc
    dev = gu.dev()
    x = di.randn((2, 300, 1024), 1.0, 9800, "bf16").to(dev)
    w = di.randn((2, 300, 64, 4), 0.5, 9801, "bf16").to(dev)
    z = di.randn((2, 300, 16), 1.0, 9802, "bf16").to(dev)
    U = di.randn((16, 1024 * 4), 0.125, 9803, "bf16").to(dev)
    dy = di.randn((2, 300, 1024), 1.0, 9804, "bf16").to(dev)
    ref_h = dsc.headwise_bwd(x, w, dy, 16, True, True)
    ref_l = dsc.lowrank_bwd(x, z, U, dy, 4, 1, True, False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            h = dsc.headwise_bwd(x, w, dy, 16, True, True, stream=s1)
        with torch.cuda.stream(s2):
            l = dsc.lowrank_bwd(x, z, U, dy, 4, 1, True, False, stream=s2)
        outs.append((h, l))
    torch.cuda.synchronize()
    for h, l in outs:
        assert all(torch.equal(a, b) for a, b in zip(h, ref_h))
        assert all(torch.equal(a, b) for a, b in zip(l, ref_l))


def test_step_graph_replay_matches_eager():
    """The four ops of a training step (head-wise and low-rank, forward and
    backward, with a caller-owned workspace) captured in one HIP graph: every
    replay gives the eager bits, with eager work and synchronisations in
    between (the ops queue no memset and keep no state)."""
    import dynamic_short_causal_amd as dsc
    dev = gu.dev()
    B, T, D, W = 2, 300, 1024, 4
    x = di.randn((B, T, D), 1.0, 9810, "bf16").to(dev)
    w = di.randn((B, T, D // 16, W), 0.5, 9811, "bf16").to(dev)
    z = di.randn((B, T, 16), 1.0, 9812, "bf16").to(dev)
    U = di.randn((16, D * W), 0.125, 9813, "bf16").to(dev)
    dy = di.randn((B, T, D), 1.0, 9814, "bf16").to(dev)
    outs = [torch.empty_like(x), torch.empty_like(x), torch.empty_like(w), torch.empty_like(x),
            torch.empty_like(x), torch.empty_like(z), torch.empty_like(U)]
    y_h, dx_h, dw_h, y_l, dx_l, dz, dU = outs
    ws = dsc.lowrank_workspace(x, z, W, 1)

    def step(s):
        dsc.dsc_headwise_fwd(x, w, y_h, 16, True, False, s)
        dsc.dsc_headwise_bwd(x, w, dy, dx_h, dw_h, 16, True, False, s)
        dsc.dsc_lowrank_fwd(x, z, U, y_l, W, 1, True, False, s)
        dsc.dsc_lowrank_bwd(x, z, U, dy, dx_l, dz, dU, ws, W, 1, True, False, s)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()   # default priority
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y_h", "dx_h", "dw_h", "y_l", "dx_l", "dz", "dU"), outs, ref):
            assert torch.equal(a, b), f"replay {rep}: {name}"
        step(torch.cuda.current_stream())   # eager work between replays
        torch.cuda.synchronize()
