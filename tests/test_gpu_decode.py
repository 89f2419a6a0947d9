"""GPU parity of the one-token (decode) steps against the fp64 oracle.

A sequence is decoded token by token from the state left by a prompt (empty,
shorter than W-1, or long); every step's y must match the oracle's full
forward at that token, and every state must equal, bit for bit, the last W-1
inputs (zero before the sequence start) that the oracle's state function gives.
"""
import numpy as np
import pytest
import torch

import dsc_inputs as di
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsc():
    import dynamic_short_causal_amd as d
    return d


def own(t):
    """A fresh allocation (16-byte aligned), as a serving loop hands over per token."""
    return t.clone(memory_format=torch.contiguous_format)


def roll(dsc, orc, lowrank, B, T, D, W, H, dtype, residual, act, seed, T0=0, R=16):
    gu.say(f"  decode {'lowrank' if lowrank else 'headwise'} B={B} T={T} prompt={T0} D={D} "
           f"W={W} H={H} R={R} {dtype} res={residual} act={act}")
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    G = D // H
    x = di.randn((B, T, D), 1.0, seed, dt)
    if lowrank:
        z = di.randn((B, T, R), 1.0, seed + 2, dt)
        U = di.randn((R, G * W), (1.0 / (R * W)) ** 0.5, seed + 3, dt)
        full = orc.lowrank_fwd(gu.f64(x), gu.f64(z), gu.f64(U), W, H, residual, act)
        zd, Ud = z.to(gu.dev()), U.to(gu.dev())
    else:
        w = di.randn((B, T, G, W), 0.5, seed + 1, dt)
        full = orc.headwise_fwd(gu.f64(x), gu.f64(w), H, residual, act)
        wd = w.to(gu.dev())
    xd = x.to(gu.dev())
    state = dsc.decode_state(xd[:, :T0].contiguous(), W)
    torch.cuda.synchronize()
    assert np.array_equal(gu.f64(state), orc.decode_state(gu.f64(x[:, :T0]), W)), "prompt state"
    for t in range(T0, T):
        before = gu.f64(state)
        xt = own(xd[:, t])
        if lowrank:
            y = dsc.lowrank_decode(xt, own(zd[:, t]), Ud, state, W, H, residual, act)
            yo, so = orc.lowrank_decode(gu.f64(x[:, t]), gu.f64(z[:, t]), gu.f64(U), before, W, H,
                                        residual, act)
        else:
            y = dsc.headwise_decode(xt, own(wd[:, t]), state, H, residual, act)
            yo, so = orc.headwise_decode(gu.f64(x[:, t]), gu.f64(w[:, t]), before, H, residual,
                                         act)
        torch.cuda.synchronize()
        gu.check(f"y[t={t}] vs forward", y, full[:, t], dtype, "y")
        gu.check(f"y[t={t}] vs decode", y, yo, dtype, "y")
        assert np.array_equal(gu.f64(state), so), f"state after t={t}"
        assert np.array_equal(gu.f64(state), orc.decode_state(gu.f64(x[:, :t + 1]), W))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 2, 4, 8, 16, 64])
def test_headwise_tying(dsc, orc, dtype, H):
    # 3 sequences of 576 channels: 216 (bf16) or 432 (fp32) vectors, so one
    # full and one ragged 256-thread block in fp32
    roll(dsc, orc, False, 3, 9, 576, 4, H, dtype, True, False, 6000 + H)


@pytest.mark.parametrize("H,dtype", [(24, torch.bfloat16), (72, torch.bfloat16),
                                     (12, torch.float32)])
def test_headwise_groups_of_non_power_of_two_vectors(dsc, orc, H, dtype):
    roll(dsc, orc, False, 3, 9, 576, 4, H, dtype, True, True, 6100 + H)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 2, 4, 8, 16, 64])
def test_lowrank_tying(dsc, orc, dtype, H):
    # H above the vector width (fp32: 8, 16, 64; bf16: 16, 64): one group spans
    # several vectors
    roll(dsc, orc, True, 3, 9, 576, 4, H, dtype, True, False, 6100 + H)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 6, 7, 8])
def test_widths(dsc, orc, W):
    roll(dsc, orc, False, 2, W + 3, 256, W, 16, torch.bfloat16, True, True, 6200 + W)
    roll(dsc, orc, True, 2, W + 3, 256, W, 2, torch.float32, False, True, 6300 + W, R=3)


@pytest.mark.parametrize("residual,act", [(False, False), (True, False), (False, True),
                                          (True, True)])
def test_epilogues(dsc, orc, residual, act):
    roll(dsc, orc, False, 2, 6, 512, 4, 8, torch.bfloat16, residual, act, 6400)
    roll(dsc, orc, True, 2, 6, 512, 4, 1, torch.bfloat16, residual, act, 6500, R=5)


@pytest.mark.parametrize("T0", [1, 2, 3, 50])
def test_after_prompt(dsc, orc, T0):
    """The state of a prompt shorter than, equal to and longer than W-1."""
    roll(dsc, orc, False, 2, T0 + 4, 128, 4, 1, torch.bfloat16, True, False, 6600 + T0, T0=T0)
    roll(dsc, orc, True, 2, T0 + 4, 128, 4, 1, torch.float32, True, True, 6700 + T0, T0=T0,
         R=16)


@pytest.mark.parametrize("R", [1, 7, 16, 17, 40, 64])
def test_ranks(dsc, orc, R):
    roll(dsc, orc, True, 2, 6, 64, 4, 1, torch.bfloat16, True, False, 6800 + R, R=R)
    roll(dsc, orc, True, 3, 5, 64, 4, 2, torch.float32, True, True, 6850 + R, R=R)


def test_single_vector_and_large_batch(dsc, orc):
    roll(dsc, orc, False, 1, 5, 8, 4, 8, torch.bfloat16, True, False, 6900)
    roll(dsc, orc, True, 1, 5, 4, 4, 4, torch.float32, True, False, 6901, R=2)
    roll(dsc, orc, False, 300, 5, 24, 3, 1, torch.bfloat16, True, True, 6902)


@pytest.mark.parametrize("lowrank,D,H", [(True, 6144, 1), (False, 8192, 64),
                                         (True, 4608, 8)])
def test_serving_batch(dsc, orc, lowrank, D, H):
    """One step at a serving batch of 64 sequences and the workloads' widths,
    from the state of a 100-token prompt."""
    roll(dsc, orc, lowrank, 64, 101, D, 4, H, torch.bfloat16, True, H == 8, 7000 + H, T0=100)


@pytest.mark.parametrize("lowrank", [False, True], ids=["headwise", "lowrank"])
def test_graph_replay(dsc, orc, lowrank):
    """Decode steps captured in one HIP graph give, on every replay, the bits
    of the same steps launched eagerly (the kernels queue no memset)."""
    B, T, D, W, H, R = 4, 6, 512, 4, 1 if lowrank else 8, 16
    G = D // H
    dev = gu.dev()
    xs = [di.randn((B, D), 1.0, 7100 + t, "bf16").to(dev) for t in range(T)]
    if lowrank:
        zs = [di.randn((B, R), 1.0, 7200 + t, "bf16").to(dev) for t in range(T)]
        U = di.randn((R, G * W), 0.125, 7300, "bf16").to(dev)
    else:
        ws = [di.randn((B, G, W), 0.5, 7200 + t, "bf16").to(dev) for t in range(T)]
    init = di.randn((B, W - 1, D), 1.0, 7400, "bf16").to(dev)
    state = init.clone()
    ys = [torch.empty_like(xs[0]) for _ in range(T)]

    def steps(s):
        for t in range(T):
            if lowrank:
                dsc.dsc_lowrank_decode(xs[t], zs[t], U, state, ys[t], W, H, True, True, s)
            else:
                dsc.dsc_headwise_decode(xs[t], ws[t], state, ys[t], H, True, True, s)

    steps(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_y = [y.clone() for y in ys]
    ref_state = state.clone()
    # the eager steps agree with the oracle from the same initial state
    st = gu.f64(init)
    for t in range(T):
        if lowrank:
            yo, st = orc.lowrank_decode(gu.f64(xs[t]), gu.f64(zs[t]), gu.f64(U), st, W, H, True,
                                        True)
        else:
            yo, st = orc.headwise_decode(gu.f64(xs[t]), gu.f64(ws[t]), st, H, True, True)
        gu.check(f"eager y[{t}]", ref_y[t], yo, torch.bfloat16, "y")
    assert np.array_equal(gu.f64(ref_state), st)

    state.copy_(init)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(init)
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(ys[t], ref_y[t]), f"replay {rep} y[{t}]"
        assert torch.equal(state, ref_state), f"replay {rep} state"


@pytest.mark.parametrize("B,D,W,dtype,R", [(343, 6144, 4, torch.bfloat16, 16),
                                           (259, 4096, 4, torch.float32, 7),
                                           (343, 6144, 8, torch.bfloat16, 3)])
def test_lowrank_sequence_blocks(dsc, orc, B, D, W, dtype, R):
    """Batches large enough that each low-rank thread serves a block of
    sequences (a ragged last block here), with R a multiple of, above and
    below the rows of U loaded together."""
    roll(dsc, orc, True, B, 5, D, W, 1, dtype, True, False, 7500 + R, T0=3, R=R)
