"""GPU parity of the packed-row (varlen) entry points against the fp64 oracle.

Rows pack several documents; pos[b, t] is each token's index inside its
document.  Every output is compared with the oracle's masked definition, and a
row holding one document must give the dense path's bits exactly.
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


def packing(B, T, seed, ndocs=5, min_len=1):
    """Document positions of rows cut at random places (documents of at least
    min_len tokens; a final short document when T does not divide)."""
    rng = np.random.default_rng(seed)
    pos = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        k = min(ndocs - 1, max(0, T // max(min_len, 1) - 1))
        cuts = np.sort(rng.choice(np.arange(1, T), size=k, replace=False)) if k > 0 else []
        edges = [0] + list(cuts) + [T]
        for s0, e0 in zip(edges[:-1], edges[1:]):
            pos[b, s0:e0] = np.arange(e0 - s0)
    return pos


def hw_case(dsc, orc, B, T, D, W, H, dtype, residual, act, seed, pos):
    gu.say(f"  head-wise varlen B={B} T={T} D={D} W={W} H={H} {dtype} res={residual} act={act}")
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    x = di.randn((B, T, D), 1.0, seed, dt)
    w = di.randn((B, T, D // H, W), 0.5, seed + 1, dt)
    dy = di.randn((B, T, D), 1.0, seed + 4, dt)
    xd, wd, dyd = x.to(gu.dev()), w.to(gu.dev()), dy.to(gu.dev())
    pd = torch.from_numpy(pos).to(gu.dev())
    y = dsc.headwise_fwd_varlen(xd, wd, pd, H, residual, act)
    dx, dw = dsc.headwise_bwd_varlen(xd, wd, pd, dyd, H, residual, act)
    torch.cuda.synchronize()
    X, Wt, DY = gu.f64(x), gu.f64(w), gu.f64(dy)
    gu.check("y", y, orc.headwise_fwd_vl(X, Wt, pos, H, residual, act), dtype, "y")
    dxo, dwo = orc.headwise_bwd_vl(X, Wt, pos, DY, H, residual, act)
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dw", dw, dwo, dtype, "dw")
    return (xd, wd, dyd, pd), (y, dx, dw)


def lr_case(dsc, orc, B, T, D, W, H, R, dtype, residual, act, seed, pos):
    gu.say(f"  low-rank varlen B={B} T={T} D={D} W={W} H={H} R={R} {dtype} "
           f"res={residual} act={act}")
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    x = di.randn((B, T, D), 1.0, seed, dt)
    z = di.randn((B, T, R), 1.0, seed + 2, dt)
    U = di.randn((R, (D // H) * W), (1.0 / (R * W)) ** 0.5 * 2, seed + 3, dt)
    dy = di.randn((B, T, D), 1.0, seed + 4, dt)
    xd, zd, Ud, dyd = (t.to(gu.dev()) for t in (x, z, U, dy))
    pd = torch.from_numpy(pos).to(gu.dev())
    y = dsc.lowrank_fwd_varlen(xd, zd, Ud, pd, W, H, residual, act)
    dx, dz, dU = dsc.lowrank_bwd_varlen(xd, zd, Ud, pd, dyd, W, H, residual, act)
    torch.cuda.synchronize()
    X, Z, UU, DY = gu.f64(x), gu.f64(z), gu.f64(U), gu.f64(dy)
    gu.check("y", y, orc.lowrank_fwd_vl(X, Z, UU, pos, W, H, residual, act), dtype, "y")
    dxo, dzo, dUo = orc.lowrank_bwd_vl(X, Z, UU, pos, DY, W, H, residual, act)
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dz", dz, dzo, dtype, "dz")
    gu.check("dU", dU, dUo, dtype, "dU")
    return (xd, zd, Ud, dyd, pd), (y, dx, dz, dU)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 4, 16, 64])
def test_headwise_tying(dsc, orc, dtype, H):
    hw_case(dsc, orc, 2, 300, 1024, 4, H, dtype, True, False, 9000 + H, packing(2, 300, 1, 6))


@pytest.mark.parametrize("H,dtype", [(24, torch.bfloat16), (8 * 33, torch.bfloat16),
                                     (12, torch.float32)])
def test_headwise_groups_of_non_power_of_two_lanes(dsc, orc, H, dtype):
    # 1056 channels: 132 bf16 vectors (44 groups of 3, or 4 of 33), 264 fp32 (88 of 3)
    hw_case(dsc, orc, 2, 300, 1056, 4, H, dtype, True, True, 9050 + H, packing(2, 300, 1, 6))


@pytest.mark.parametrize("W", [2, 3, 5, 8])
def test_headwise_widths_silu(dsc, orc, W):
    hw_case(dsc, orc, 2, 150, 512, W, 8, torch.bfloat16, True, True, 9100 + W,
            packing(2, 150, W, 8))


@pytest.mark.parametrize("H,dtype", [(1, torch.bfloat16), (2, torch.bfloat16),
                                     (8, torch.bfloat16), (16, torch.bfloat16),
                                     (1, torch.float32), (2, torch.float32),
                                     (8, torch.float32)],
                         ids=["bf16-H1", "bf16-H2", "bf16-H8", "bf16-H16", "f32-H1", "f32-H2",
                              "f32-H8"])
def test_lowrank_tying(dsc, orc, H, dtype):
    # 150 tokens: chunks and tiles end inside documents
    lr_case(dsc, orc, 2, 150, 512, 4, H, 16, dtype, True, False, 9200 + H,
            packing(2, 150, 7 + H, 6))


@pytest.mark.parametrize("R,W,H,dtype", [(32, 4, 1, torch.bfloat16), (64, 8, 1, torch.bfloat16),
                                         (40, 3, 8, torch.bfloat16), (64, 4, 1, torch.float32)],
                         ids=["bf16-R32", "bf16-R64-W8", "bf16-R40-H8", "f32-R64"])
def test_lowrank_many_ranks(dsc, orc, R, W, H, dtype):
    lr_case(dsc, orc, 2, 97, 256, W, H, R, dtype, True, dtype == torch.bfloat16, 9250 + R + W,
            packing(2, 97, 40 + R, 6))


@pytest.mark.parametrize("W", [1, 2, 3])
def test_lowrank_tied_eight_widths(dsc, orc, W):
    """H = 8 in bf16 with W <= 4: the vector-ALU forward drops masked taps."""
    lr_case(dsc, orc, 2, 97, 576, W, 8, 16, torch.bfloat16, True, True, 9350 + W,
            packing(2, 97, 50 + W, 6))


@pytest.mark.parametrize("W", [1, 2, 3, 5, 8])
def test_lowrank_widths_silu(dsc, orc, W):
    lr_case(dsc, orc, 2, 97, 256, W, 1, 16, torch.bfloat16, True, True, 9300 + W,
            packing(2, 97, 20 + W, 6))
    lr_case(dsc, orc, 1, 70, 128, W, 2, 5, torch.float32, False, True, 9400 + W,
            packing(1, 70, 30 + W, 4))


def test_one_token_documents(dsc, orc):
    """Every token its own document: only tap 0 remains."""
    pos = np.zeros((2, 40), dtype=np.int32)
    hw_case(dsc, orc, 2, 40, 256, 4, 2, torch.bfloat16, True, True, 9500, pos)
    lr_case(dsc, orc, 2, 40, 256, 4, 1, 16, torch.bfloat16, True, True, 9501, pos)


def test_one_document_is_dense_bitwise(dsc, orc):
    """pos = t reproduces the dense entry points bit for bit."""
    B, T, D, W = 2, 200, 512, 4
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    (xd, wd, dyd, pd), outs = hw_case(dsc, orc, B, T, D, W, 8, torch.bfloat16, True, True,
                                      9600, pos)
    dense = (dsc.headwise_fwd(xd, wd, 8, True, True),) + dsc.headwise_bwd(xd, wd, dyd, 8, True,
                                                                          True)
    (xd, zd, Ud, dyd, pd), louts = lr_case(dsc, orc, B, T, D, W, 1, 16, torch.bfloat16, True,
                                           False, 9601, pos)
    ldense = (dsc.lowrank_fwd(xd, zd, Ud, W, 1, True, False),) + dsc.lowrank_bwd(
        xd, zd, Ud, dyd, W, 1, True, False)
    torch.cuda.synchronize()
    for a, b in zip(outs + louts, dense + ldense):
        assert torch.equal(a, b)


def test_qkv_shape(dsc, orc):
    """Two sequences at the Q,K,V width and length, each packing documents of
    random lengths (some shorter than W), both variants; every output checked."""
    pos = packing(2, 2048, 77, ndocs=40)
    hw_case(dsc, orc, 2, 2048, 6144, 4, 16, torch.bfloat16, True, False, 9700, pos)
    lr_case(dsc, orc, 2, 2048, 6144, 4, 1, 16, torch.bfloat16, True, False, 9701, pos)
