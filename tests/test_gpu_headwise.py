"""GPU parity of the head-wise kernels against the fp64 oracle (through the C ABI)."""
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


def run_case(dsc, orc, B, T, D, W, H, dtype, residual, act, seed, w_std=0.5, const_w=False):
    gu.say(f"  case B={B} T={T} D={D} W={W} H={H} {dtype} res={residual} act={act}")
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    x = di.randn((B, T, D), 1.0, seed, dt)
    w = di.randn((B, T, D // H, W), w_std, seed + 1, dt)
    if const_w:
        w = w[:, :1].expand(B, T, D // H, W).contiguous()
    dy = di.randn((B, T, D), 1.0, seed + 4, dt)
    xd, wd, dyd = x.to(gu.dev()), w.to(gu.dev()), dy.to(gu.dev())
    y = dsc.headwise_fwd(xd, wd, H, residual, act)
    dx, dw = dsc.headwise_bwd(xd, wd, dyd, H, residual, act)
    torch.cuda.synchronize()
    yo = orc.headwise_fwd(gu.f64(x), gu.f64(w), H, residual, act)
    dxo, dwo = orc.headwise_bwd(gu.f64(x), gu.f64(w), gu.f64(dy), H, residual, act)
    gu.check("y", y, yo, dtype, "y")
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dw", dw, dwo, dtype, "dw")
    return y, dx, dw


def test_tiny_f32_per_channel(dsc, orc):
    """The tiny oracle-check workload: fp32, B=1, T=64, D=64, W=4, H=1."""
    wl = di.WORKLOADS["tiny_f32"]
    run_case(dsc, orc, wl.B, wl.T, wl.D, wl.W, wl.H, torch.float32, False, False, 1000,
             w_std=wl.w_var ** 0.5)


def test_tiny_f32_width_one_and_static(dsc, orc):
    run_case(dsc, orc, 1, 64, 64, 1, 1, torch.float32, False, False, 1010)
    run_case(dsc, orc, 1, 64, 64, 4, 1, torch.float32, False, False, 1020, const_w=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 2, 4, 8, 16, 64])
def test_tying_factors(dsc, orc, dtype, H):
    # 2 sequences, 150 tokens (ragged against the 4- and 8-token chunks and the
    # 32-token backward workgroups), 2112 channels (a ragged last column)
    run_case(dsc, orc, 2, 150, 2112, 4, H, dtype, True, False, 2000 + H)


@pytest.mark.parametrize("H,dtype,act,W,D", [
    (24, torch.bfloat16, False, 4, 2160), (48, torch.bfloat16, True, 3, 2160),
    (40, torch.bfloat16, False, 7, 2000), (8 * 33, torch.bfloat16, True, 4, 2376),
    (12, torch.float32, False, 4, 1200), (20, torch.float32, True, 5, 1000),
    (4 * 63, torch.float32, False, 2, 1008)])
def test_groups_of_non_power_of_two_lanes(dsc, orc, H, dtype, act, W, D):
    """A group spans L = H / V lanes with L not a power of two (3, 6, 5, 33, 3,
    5, 63): the backward gives each wave 64 // L whole groups; D leaves a
    ragged last workgroup."""
    run_case(dsc, orc, 2, 150, D, W, H, dtype, True, act, 2500 + H)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 6, 7, 8])
def test_widths(dsc, orc, W):
    run_case(dsc, orc, 2, 131, 512, W, 16, torch.bfloat16, True, False, 3000 + W)
    run_case(dsc, orc, 1, 70, 256, W, 2, torch.float32, False, True, 3100 + W)


@pytest.mark.parametrize("T", [8, 9, 10, 31, 33, 34, 41, 42])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_chunk_boundaries(dsc, orc, T, W):
    """Lengths around the kernels' token chunks (4 per forward wave, 8 per
    backward wave, 32 per backward workgroup): a last chunk of 1 or 2 tokens,
    shorter than the W-1 tokens the previous chunk's dx needs from it, and
    chunks that open a new workgroup."""
    run_case(dsc, orc, 2, T, 1024, W, 16, torch.bfloat16, True, W == 3, 7000 + 10 * T + W)
    run_case(dsc, orc, 1, T, 512, W, 4, torch.float32, False, W == 2, 7100 + 10 * T + W)


@pytest.mark.parametrize("residual,act", [(False, False), (True, False), (False, True),
                                          (True, True)])
def test_epilogues(dsc, orc, residual, act):
    run_case(dsc, orc, 3, 97, 1024, 4, 8, torch.bfloat16, residual, act, 4000)
    run_case(dsc, orc, 1, 97, 512, 4, 4, torch.float32, residual, act, 4100)


@pytest.mark.parametrize("B,T,D,W,H", [(1, 1, 64, 4, 16), (2, 2, 64, 4, 1), (2, 3, 16, 4, 8),
                                       (3, 4, 8, 4, 8), (1, 65, 8, 8, 1), (4, 5, 128, 3, 128),
                                       (1, 64, 512, 4, 512)])
def test_edges(dsc, orc, B, T, D, W, H):
    """T < W, T = W, T = 1, one vector of channels, one group spanning lanes."""
    run_case(dsc, orc, B, T, D, W, H, torch.bfloat16, True, True, 5000 + T)
    if H <= 4 or (H % 4 == 0 and H // 4 <= 64):
        run_case(dsc, orc, B, T, D, W, H, torch.float32, True, False, 5100 + T)


def test_deterministic(dsc, orc):
    x = di.randn((2, 300, 2048), 1.0, 6000, "bf16").to(gu.dev())
    w = di.randn((2, 300, 128, 4), 0.5, 6001, "bf16").to(gu.dev())
    dy = di.randn((2, 300, 2048), 1.0, 6004, "bf16").to(gu.dev())
    a = dsc.headwise_bwd(x, w, dy, 16, True, True)
    b = dsc.headwise_bwd(x, w, dy, 16, True, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(dsc.headwise_fwd(x, w, 16, True), dsc.headwise_fwd(x, w, 16, True))


def test_outputs_fully_overwritten(dsc, orc):
    """Outputs are overwritten, not accumulated into (pre-filled with NaN)."""
    x = di.randn((1, 70, 512), 1.0, 6100, "bf16").to(gu.dev())
    w = di.randn((1, 70, 32, 4), 0.5, 6101, "bf16").to(gu.dev())
    dy = di.randn((1, 70, 512), 1.0, 6104, "bf16").to(gu.dev())
    y = torch.full_like(x, float("nan"))
    dx, dw = torch.full_like(x, float("nan")), torch.full_like(w, float("nan"))
    dsc.dsc_headwise_fwd(x, w, y, 16, True)
    dsc.dsc_headwise_bwd(x, w, dy, dx, dw, 16, True)
    torch.cuda.synchronize()
    for t in (y, dx, dw):
        assert torch.isfinite(t).all()


def _full_size(dsc, orc, wl, nrows, seed_offset=0):
    gu.say(f"  full-size {wl.name} W={wl.W}: generating inputs")
    inp = di.make(wl, seed_offset=seed_offset)
    xd, wd, dyd = (inp[k].to(gu.dev()) for k in ("x", "w", "dy"))
    y = dsc.headwise_fwd(xd, wd, wl.H, wl.residual, wl.act)
    dx, dw = dsc.headwise_bwd(xd, wd, dyd, wl.H, wl.residual, wl.act)
    torch.cuda.synchronize()
    gu.say("  kernels done; oracle on sampled rows")
    rows = gu.sample_rows(wl.B, wl.T, nrows, seed=wl.case)
    yg, dxg, dwg, yo, dxo, dwo = [], [], [], [], [], []
    for (b, s, e, loc) in gu.windows(wl.T, wl.W, rows):
        t = s + loc
        xs, ws, dys = (gu.f64(inp[k][b:b + 1, s:e]) for k in ("x", "w", "dy"))
        yo.append(orc.headwise_fwd_rows(xs, ws, wl.H, [loc], wl.residual, wl.act)[0])
        a, c = orc.headwise_bwd_rows(xs, ws, dys, wl.H, [loc], wl.residual, wl.act)
        dxo.append(a[0])
        dwo.append(c[0])
        yg.append(gu.f64(y[b, t]))
        dxg.append(gu.f64(dx[b, t]))
        dwg.append(gu.f64(dw[b, t]))
    dtype = torch.bfloat16
    gu.check("y rows", np.array(yg), np.array(yo), dtype, "y")
    gu.check("dx rows", np.array(dxg), np.array(dxo), dtype, "dx")
    gu.check("dw rows", np.array(dwg), np.array(dwo), dtype, "dw")
    # adjoint identity over the whole tensor: <y - rho x, dy> = <x, dx - rho dy>
    rho = 1.0 if wl.residual else 0.0
    yf, xf, dyf, dxf = (t.double() for t in (y, xd, dyd, dx))
    lhs = float(((yf - rho * xf) * dyf).sum())
    rhs = float((xf * (dxf - rho * dyf)).sum())
    scale = float((yf - rho * xf).abs().mul(dyf.abs()).sum())
    gu.say(f"    adjoint: {lhs:.6e} vs {rhs:.6e} (scale {scale:.3e})")
    assert abs(lhs - rhs) <= 1e-2 * scale ** 0.5 + 1e-4 * abs(lhs)


def test_full_size_qkv(dsc, orc):
    """D=6144, T=2048, B=8, W=4, H=16, residual: every element of y, dx and dw
    against the whole-batch fp64 oracle."""
    wl = di.WORKLOADS["qkv_headwise"]
    gu.say(f"  full-size {wl.name}: generating inputs")
    inp = di.make(wl)
    xd, wd, dyd = (inp[k].to(gu.dev()) for k in ("x", "w", "dy"))
    y = dsc.headwise_fwd(xd, wd, wl.H, wl.residual, wl.act)
    dx, dw = dsc.headwise_bwd(xd, wd, dyd, wl.H, wl.residual, wl.act)
    torch.cuda.synchronize()
    del xd, wd, dyd
    gu.say("  kernels done; whole-batch oracle")
    X, Wt, DY = (gu.f64(inp[k]) for k in ("x", "w", "dy"))
    dtype = torch.bfloat16
    gu.check("y", y, orc.headwise_fwd(X, Wt, wl.H, wl.residual, wl.act), dtype, "y")
    dxo, dwo = orc.headwise_bwd(X, Wt, DY, wl.H, wl.residual, wl.act)
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dw", dw, dwo, dtype, "dw")


@pytest.mark.parametrize("W", [2, 3, 4, 8])
def test_full_size_mlp_width_sweep(dsc, orc, W):
    wl = di.WORKLOADS["mlp_headwise"].with_(W=W)
    _full_size(dsc, orc, wl, 24, seed_offset=10 * W)
