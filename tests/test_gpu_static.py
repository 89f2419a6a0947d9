"""GPU parity of the static-filter kernels against the fp64 oracle (through the C ABI)."""
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


def run_case(dsc, orc, B, T, D, W, H, dtype, residual, act, seed, w_std=0.5):
    gu.say(f"  static B={B} T={T} D={D} W={W} H={H} {dtype} res={residual} act={act}")
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    x = di.randn((B, T, D), 1.0, seed, dt)
    w = di.randn((D // H, W), w_std, seed + 1, dt)
    dy = di.randn((B, T, D), 1.0, seed + 4, dt)
    xd, wd, dyd = x.to(gu.dev()), w.to(gu.dev()), dy.to(gu.dev())
    y = dsc.static_fwd(xd, wd, H, residual, act)
    dx, dw = dsc.static_bwd(xd, wd, dyd, H, residual, act)
    torch.cuda.synchronize()
    yo = orc.static_fwd(gu.f64(x), gu.f64(w), H, residual, act)
    dxo, dwo = orc.static_bwd(gu.f64(x), gu.f64(w), gu.f64(dy), H, residual, act)
    gu.check("y", y, yo, dtype, "y")
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dw", dw, dwo, dtype, "dw")
    return y, dx, dw


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 2, 4, 8, 16, 64])
def test_tying_factors(dsc, orc, dtype, H):
    # 2 sequences of 600 tokens (one full 512-token span and a ragged one),
    # 2112 channels (33 blocks of 64 vectors at fp32, ragged at bf16)
    run_case(dsc, orc, 2, 600, 2112, 4, H, dtype, True, False, 8000 + H)


@pytest.mark.parametrize("H,dtype,act,D", [
    (24, torch.bfloat16, False, 2160), (8 * 33, torch.bfloat16, True, 2376),
    (12, torch.float32, True, 1200), (4 * 63, torch.float32, False, 1008)])
def test_groups_of_non_power_of_two_lanes(dsc, orc, H, dtype, act, D):
    """L = H / V lanes per group, not a power of two: each workgroup takes
    64 // L whole groups of lanes; D leaves a ragged last workgroup."""
    run_case(dsc, orc, 2, 600, D, 4, H, dtype, True, act, 8500 + H)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 6, 7, 8])
def test_widths(dsc, orc, W):
    run_case(dsc, orc, 2, 131, 512, W, 16, torch.bfloat16, True, False, 8100 + W)
    run_case(dsc, orc, 1, 70, 256, W, 2, torch.float32, False, True, 8200 + W)


@pytest.mark.parametrize("residual,act", [(False, False), (True, False), (False, True),
                                          (True, True)])
def test_epilogues(dsc, orc, residual, act):
    run_case(dsc, orc, 3, 97, 1024, 4, 1, torch.bfloat16, residual, act, 8300)
    run_case(dsc, orc, 1, 97, 512, 4, 4, torch.float32, residual, act, 8400)


@pytest.mark.parametrize("B,T,D,W,H", [(1, 1, 64, 4, 16), (2, 2, 64, 4, 1), (2, 3, 16, 4, 8),
                                       (3, 4, 8, 4, 8), (1, 65, 8, 8, 1), (4, 5, 128, 3, 128),
                                       (1, 64, 512, 4, 512), (1, 1024, 64, 4, 1)])
def test_edges(dsc, orc, B, T, D, W, H):
    """T < W, T = W, T = 1, one vector of channels, a group spanning 64 lanes,
    two spans of four full chunks."""
    run_case(dsc, orc, B, T, D, W, H, torch.bfloat16, True, True, 8500 + T)
    if H <= 4 or (H % 4 == 0 and H // 4 <= 64):
        run_case(dsc, orc, B, T, D, W, H, torch.float32, True, False, 8600 + T)


def test_empty_writes_zero_filter_gradient(dsc):
    for B, T in ((0, 16), (2, 0)):
        x = torch.zeros(B, T, 64, dtype=torch.bfloat16, device=gu.dev())
        w = torch.ones(64, 4, dtype=torch.bfloat16, device=gu.dev())
        y = dsc.static_fwd(x, w, 1)
        dx, dw = dsc.static_bwd(x, w, torch.zeros_like(x), 1)
        torch.cuda.synchronize()
        assert y.numel() == 0 and dx.numel() == 0
        assert torch.count_nonzero(dw).item() == 0


def test_qkv_shape(dsc, orc):
    """The Q,K,V workload's shape (B=8, T=2048, D=6144, W=4) with per-channel
    static filters, as the bench times it; every output checked."""
    run_case(dsc, orc, 8, 2048, 6144, 4, 1, torch.bfloat16, True, False, 8700)


def test_deterministic(dsc):
    x = di.randn((2, 700, 768), 1.0, 8800, "bf16").to(gu.dev())
    w = di.randn((768, 4), 0.5, 8801, "bf16").to(gu.dev())
    dy = di.randn((2, 700, 768), 1.0, 8802, "bf16").to(gu.dev())
    a = dsc.static_bwd(x, w, dy, 1, True, True)
    b = dsc.static_bwd(x, w, dy, 1, True, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
