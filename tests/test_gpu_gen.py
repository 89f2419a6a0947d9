"""GPU parity of the fused filter generation (w = xh M on chip, then the
head-wise convolution) against the fp64 oracle."""
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


def inputs(B, T, D, Dh, W, H, seed):
    G = D // H
    x = di.randn((B, T, D), 1.0, seed, "bf16")
    xh = di.randn((B, T, Dh), 1.0, seed + 1, "bf16")
    M = di.randn((Dh, G * W), (0.25 / Dh) ** 0.5, seed + 2, "bf16")  # w ~ N(0, 0.25)
    return x, xh, M


def mt(M):
    """M (Dh, G*W) as the kernel takes it: transposed, (G*W, Dh), on the GPU."""
    return M.t().contiguous().to(gu.dev())


def run_case(dsc, orc, B, T, D, Dh, W, H, residual, act, seed):
    gu.say(f"  gen B={B} T={T} D={D} Dh={Dh} W={W} H={H} res={residual} act={act}")
    x, xh, M = inputs(B, T, D, Dh, W, H, seed)
    y = dsc.headwise_gen_fwd(x.to(gu.dev()), xh.to(gu.dev()), mt(M), W, H, residual, act)
    torch.cuda.synchronize()
    yo = orc.headwise_gen_fwd(gu.f64(x), gu.f64(xh), gu.f64(M), H, residual, act)
    gu.check("y", y, yo, torch.bfloat16, "y")


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_widths(dsc, orc, W):
    # 2 sequences of 100 tokens: the 128-token tile crosses the sequence boundary
    run_case(dsc, orc, 2, 100, 1024, 128, W, 16, True, False, 9900 + W)


@pytest.mark.parametrize("H", [8, 24, 64])
def test_tying(dsc, orc, H):
    run_case(dsc, orc, 1, 70, 1536, 64, 4, H, False, True, 9910 + H)


def test_channel_blocks_and_ragged(dsc, orc):
    """Twelve full 128-column blocks; then a last block holding one group."""
    run_case(dsc, orc, 1, 130, 6144, 192, 4, 16, True, True, 9920)
    run_case(dsc, orc, 2, 33, 1032, 64, 8, 8, True, False, 9921)


def test_narrowest_shapes(dsc, orc):
    """The fewest filter columns the kernel takes (G*W = 8, one partial
    column block): D = 16 in two groups at W=4, D = 64 in eight groups at W=1."""
    run_case(dsc, orc, 1, 50, 16, 64, 4, 8, True, True, 9935)
    run_case(dsc, orc, 3, 5, 64, 128, 1, 8, False, False, 9936)


def test_one_token_sequences_and_short_batches(dsc, orc):
    run_case(dsc, orc, 5, 1, 512, 64, 4, 8, True, True, 9930)
    run_case(dsc, orc, 1, 3, 256, 64, 8, 32, False, False, 9931)


# Long reductions (Dh up to 2048, 64 K-tiles) at all widths: full oracle checks.
@pytest.mark.parametrize("B,T,D,Dh,W,H,residual,act", [
    (2, 300, 512, 256, 8, 8, True, False),
    (1, 520, 1024, 1024, 4, 16, False, True),  # ragged last tile
    (1, 200, 512, 2048, 1, 8, True, True),
    (3, 77, 1024, 2048, 2, 16, True, False),   # sequences inside a tile
    (2, 256, 1024, 256, 4, 16, True, False),   # XCD-grouped order: 4 token tiles x 2 column blocks
    (4, 1024, 2048, 512, 8, 16, False, True),  # XCD-grouped order over 32 token tiles
])
def test_long_reduction(dsc, orc, B, T, D, Dh, W, H, residual, act):
    run_case(dsc, orc, B, T, D, Dh, W, H, residual, act, 9960 + W + H)


def test_many_tiles_sampled(dsc, orc):
    """B=13, T=2500, D=1024, Dh=1024, W=4, H=16: 508 tiles of 128 tokens x
    128 columns, more than the CUs; the sequence length is no multiple of the
    tile."""
    sampled_case(dsc, orc, 13, 2500, 1024, 1024, 4, 16, True, True, 9970)


def test_qkv_shape_sampled(dsc, orc):
    """B=8, T=2048, D=6144, Dh=2048, W=4, H=16 (the Q,K,V projection of a
    2048-wide model); sampled tokens checked through the oracle on their
    causal window (the output at t depends on tokens t-W+1 .. t only)."""
    sampled_case(dsc, orc, 8, 2048, 6144, 2048, 4, 16, True, False, 9940)


def test_wide_sampled(dsc, orc):
    """B=16, T=2048, D=2048, Dh=128, W=4, H=16: 512 filter columns over
    32768 tokens."""
    sampled_case(dsc, orc, 16, 2048, 2048, 128, 4, 16, False, True, 9950)


def sampled_case(dsc, orc, B, T, D, Dh, W, H, residual, act, seed):
    gu.say(f"  gen sampled B={B} T={T} D={D} Dh={Dh} W={W} H={H}")
    x, xh, M = inputs(B, T, D, Dh, W, H, seed)
    y = dsc.headwise_gen_fwd(x.to(gu.dev()), xh.to(gu.dev()), mt(M), W, H, residual, act)
    torch.cuda.synchronize()
    Mf = gu.f64(M)
    got, ref = [], []
    for b, t in gu.sample_rows(B, T, 16, seed + 1):
        s0 = max(0, t - W + 1)
        yo = orc.headwise_gen_fwd(gu.f64(x[b:b + 1, s0:t + 1]), gu.f64(xh[b:b + 1, s0:t + 1]), Mf,
                                  H, residual, act)
        ref.append(yo[0, -1])
        got.append(gu.f64(y[b, t]))
    gu.check("sampled y", np.stack(got), np.stack(ref), torch.bfloat16, "y")


def test_graph_replay_and_streams(dsc, orc):
    """The fused kernel queues no memset and keeps no state: a HIP graph of
    it gives the eager bits on every replay, and calls on two streams at
    once give the bits of serial calls."""
    B, T, D, Dh, W, H = 2, 300, 1024, 256, 4, 16
    x, xh, M = inputs(B, T, D, Dh, W, H, 9980)
    dev = gu.dev()
    x, xh, Mt = x.to(dev), xh.to(dev), mt(M)
    y = torch.empty_like(x)
    dsc.dsc_headwise_gen_fwd(x, xh, Mt, y, W, H, True, True, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = y.clone()
    gu.check("eager y", ref, orc.headwise_gen_fwd(gu.f64(x), gu.f64(xh), gu.f64(M),
                                                   H, True, True), torch.bfloat16, "y")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsc.dsc_headwise_gen_fwd(x, xh, Mt, y, W, H, True, True, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    with torch.cuda.stream(s1):
        dsc.dsc_headwise_gen_fwd(x, xh, Mt, y1, W, H, True, True, s1)
    with torch.cuda.stream(s2):
        dsc.dsc_headwise_gen_fwd(x, xh, Mt, y2, W, H, True, True, s2)
    torch.cuda.synchronize()
    assert torch.equal(y1, ref) and torch.equal(y2, ref)
