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


def run_case(dsc, orc, B, T, D, Dh, W, H, residual, act, seed):
    gu.say(f"  gen B={B} T={T} D={D} Dh={Dh} W={W} H={H} res={residual} act={act}")
    x, xh, M = inputs(B, T, D, Dh, W, H, seed)
    y = dsc.headwise_gen_fwd(x.to(gu.dev()), xh.to(gu.dev()), M.to(gu.dev()), W, H, residual, act)
    torch.cuda.synchronize()
    yo = orc.headwise_gen_fwd(gu.f64(x), gu.f64(xh), gu.f64(M), H, residual, act)
    gu.check("y", y, yo, torch.bfloat16, "y")


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_widths(dsc, orc, W):
    # 2 sequences of 100 tokens: token tiles of 64 cross the sequence boundary
    run_case(dsc, orc, 2, 100, 1024, 128, W, 16, True, False, 9900 + W)


@pytest.mark.parametrize("H", [8, 24, 64])
def test_tying(dsc, orc, H):
    run_case(dsc, orc, 1, 70, 1536, 64, 4, H, False, True, 9910 + H)


def test_channel_blocks_and_ragged(dsc, orc):
    """Six full 256-column blocks; then a last block holding one group."""
    run_case(dsc, orc, 1, 130, 6144, 192, 4, 16, True, True, 9920)
    run_case(dsc, orc, 2, 33, 1032, 64, 8, 8, True, False, 9921)


def test_one_token_sequences_and_short_batches(dsc, orc):
    run_case(dsc, orc, 5, 1, 512, 64, 4, 8, True, True, 9930)
    run_case(dsc, orc, 1, 3, 256, 64, 8, 32, False, False, 9931)


def test_qkv_shape_sampled(dsc, orc):
    """B=8, T=2048, D=6144, Dh=2048, W=4, H=16 (the Q,K,V projection of a
    2048-wide model); sampled tokens checked through the oracle on their
    causal window (the output at t depends on tokens t-W+1 .. t only)."""
    B, T, D, Dh, W, H = 8, 2048, 6144, 2048, 4, 16
    x, xh, M = inputs(B, T, D, Dh, W, H, 9940)
    y = dsc.headwise_gen_fwd(x.to(gu.dev()), xh.to(gu.dev()), M.to(gu.dev()), W, H, True, False)
    torch.cuda.synchronize()
    Mf = gu.f64(M)
    got, ref = [], []
    for b, t in gu.sample_rows(B, T, 16, 9941):
        s0 = max(0, t - W + 1)
        yo = orc.headwise_gen_fwd(gu.f64(x[b:b + 1, s0:t + 1]), gu.f64(xh[b:b + 1, s0:t + 1]), Mf,
                                  H, True, False)
        ref.append(yo[0, -1])
        got.append(gu.f64(y[b, t]))
    gu.check("sampled y", np.stack(got), np.stack(ref), torch.bfloat16, "y")
