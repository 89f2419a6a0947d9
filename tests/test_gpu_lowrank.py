"""GPU parity of the low-rank kernels (on-chip zU) against the fp64 oracle."""
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


def run_case(dsc, orc, B, T, D, W, H, R, dtype, residual, act, seed, u_std=None):
    gu.say(f"  case B={B} T={T} D={D} W={W} H={H} R={R} {dtype} res={residual} act={act}")
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    u_std = u_std if u_std is not None else (1.0 / (R * W)) ** 0.5 * 2
    x = di.randn((B, T, D), 1.0, seed, dt)
    z = di.randn((B, T, R), 1.0, seed + 2, dt)
    U = di.randn((R, (D // H) * W), u_std, seed + 3, dt)
    dy = di.randn((B, T, D), 1.0, seed + 4, dt)
    xd, zd, Ud, dyd = (t.to(gu.dev()) for t in (x, z, U, dy))
    y = dsc.lowrank_fwd(xd, zd, Ud, W, H, residual, act)
    dx, dz, dU = dsc.lowrank_bwd(xd, zd, Ud, dyd, W, H, residual, act)
    torch.cuda.synchronize()
    X, Z, UU, DY = gu.f64(x), gu.f64(z), gu.f64(U), gu.f64(dy)
    yo = orc.lowrank_fwd(X, Z, UU, W, H, residual, act)
    dxo, dzo, dUo = orc.lowrank_bwd(X, Z, UU, DY, W, H, residual, act)
    gu.check("y", y, yo, dtype, "y")
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dz", dz, dzo, dtype, "dz")
    gu.check("dU", dU, dUo, dtype, "dU")
    return y, dx, dz, dU


@pytest.mark.parametrize("H", [1, 2, 4, 8])
def test_tying_bf16(dsc, orc, H):
    # 150 tokens: several 16-token tiles, a ragged tail, several backward chunks
    run_case(dsc, orc, 2, 150, 1024 + 8 * 16 * H, 4, H, 16, torch.bfloat16, True, False,
             7000 + H)


@pytest.mark.parametrize("H", [1, 2, 4])
def test_tying_f32(dsc, orc, H):
    run_case(dsc, orc, 2, 150, 512 + 64 * H, 4, H, 16, torch.float32, True, False, 7100 + H)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 6, 7, 8])
def test_widths(dsc, orc, W):
    run_case(dsc, orc, 2, 67, 256, W, 1, 16, torch.bfloat16, True, False, 7200 + W)
    run_case(dsc, orc, 1, 70, 128, W, 2, 16, torch.float32, False, True, 7300 + W)


@pytest.mark.parametrize("R", [1, 3, 8, 12, 16])
def test_ranks(dsc, orc, R):
    run_case(dsc, orc, 2, 45, 256, 4, 1, R, torch.bfloat16, True, False, 7400 + R)
    run_case(dsc, orc, 1, 45, 64, 4, 4, R, torch.float32, False, False, 7500 + R)


@pytest.mark.parametrize("residual,act", [(False, False), (True, False), (False, True),
                                          (True, True)])
def test_epilogues(dsc, orc, residual, act):
    run_case(dsc, orc, 2, 97, 1024, 4, 8, 16, torch.bfloat16, residual, act, 7600)
    # per-channel filters in bf16 take the one-channel-per-lane backward
    run_case(dsc, orc, 2, 97, 392, 4, 1, 16, torch.bfloat16, residual, act, 7650)
    run_case(dsc, orc, 2, 97, 256, 4, 1, 16, torch.float32, residual, act, 7700)


@pytest.mark.parametrize("B,T,D,W,H", [(1, 1, 8, 4, 1), (2, 2, 16, 4, 8), (1, 3, 136, 4, 1),
                                       (3, 16, 520, 4, 8), (2, 17, 64, 4, 2),
                                       (1, 33, 8, 8, 1), (2, 1000, 128, 4, 1)])
def test_edges(dsc, orc, B, T, D, W, H):
    """T = 1, T < W, one vector, ragged channel blocks, exact and ragged tiles."""
    run_case(dsc, orc, B, T, D, W, H, 16, torch.bfloat16, True, True, 7800 + T)
    if H <= 4 and D % 4 == 0:
        run_case(dsc, orc, B, T, D, W, H, 16, torch.float32, True, False, 7900 + T)


def test_empty_batch_zeroes_dU(dsc, orc):
    x = torch.empty((0, 5, 64), dtype=torch.bfloat16, device=gu.dev())
    z = torch.empty((0, 5, 16), dtype=torch.bfloat16, device=gu.dev())
    U = di.randn((16, 64 * 4), 0.1, 8000, "bf16").to(gu.dev())
    dU = torch.full_like(U, float("nan"))
    dz = torch.empty_like(z)
    dx = torch.empty_like(x)
    ws = dsc.lowrank_workspace(x, z, 4, 1)
    dsc.dsc_lowrank_bwd(x, z, U, x, dx, dz, dU, ws, 4, 1)
    torch.cuda.synchronize()
    assert torch.all(dU == 0)


def test_deterministic(dsc, orc):
    x = di.randn((2, 300, 1024), 1.0, 8100, "bf16").to(gu.dev())
    z = di.randn((2, 300, 16), 1.0, 8102, "bf16").to(gu.dev())
    U = di.randn((16, 1024 * 4), 0.125, 8103, "bf16").to(gu.dev())
    dy = di.randn((2, 300, 1024), 1.0, 8104, "bf16").to(gu.dev())
    a = dsc.lowrank_bwd(x, z, U, dy, 4, 1, True, False)
    b = dsc.lowrank_bwd(x, z, U, dy, 4, 1, True, False)
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    assert torch.equal(dsc.lowrank_fwd(x, z, U, 4, 1, True), dsc.lowrank_fwd(x, z, U, 4, 1, True))


def test_lowrank_equals_headwise_on_gpu(dsc, orc):
    """The fused low-rank forward equals the head-wise kernel fed w = zU.

    w is formed in fp32 on the host from the same bf16 z and U, then given to the
    fp32 head-wise kernel; both GPU paths must agree to fp32 rounding."""
    B, T, D, W, H, R = 2, 80, 256, 4, 2, 16
    x = di.randn((B, T, D), 1.0, 8200, "f32")
    z = di.randn((B, T, R), 1.0, 8202, "f32")
    U = di.randn((R, (D // H) * W), 0.125, 8203, "f32")
    w = (z.double() @ U.double()).reshape(B, T, D // H, W).float()
    y1 = dsc.lowrank_fwd(x.to(gu.dev()), z.to(gu.dev()), U.to(gu.dev()), W, H, True)
    y2 = dsc.headwise_fwd(x.to(gu.dev()), w.to(gu.dev()), H, True)
    torch.cuda.synchronize()
    assert float((y1 - y2).abs().max()) < 1e-5


def _full_size(dsc, orc, wl, nrows, ncols):
    gu.say(f"  full-size {wl.name}: generating inputs")
    inp = di.make(wl)
    xd, zd, Ud, dyd = (inp[k].to(gu.dev()) for k in ("x", "z", "U", "dy"))
    y = dsc.lowrank_fwd(xd, zd, Ud, wl.W, wl.H, wl.residual, wl.act)
    dx, dz, dU = dsc.lowrank_bwd(xd, zd, Ud, dyd, wl.W, wl.H, wl.residual, wl.act)
    torch.cuda.synchronize()
    gu.say("  kernels done; oracle on sampled rows")
    UU = gu.f64(inp["U"])
    rows = gu.sample_rows(wl.B, wl.T, nrows, seed=wl.case)
    yg, dxg, dzg, yo, dxo, dzo = [], [], [], [], [], []
    for (b, s, e, loc) in gu.windows(wl.T, wl.W, rows):
        t = s + loc
        xs, zs, dys = (gu.f64(inp[k][b:b + 1, s:e]) for k in ("x", "z", "dy"))
        yo.append(orc.lowrank_fwd_rows(xs, zs, UU, wl.W, wl.H, [loc], wl.residual, wl.act)[0])
        a, c = orc.lowrank_bwd_rows(xs, zs, UU, dys, wl.W, wl.H, [loc], wl.residual, wl.act)
        dxo.append(a[0])
        dzo.append(c[0])
        yg.append(gu.f64(y[b, t]))
        dxg.append(gu.f64(dx[b, t]))
        dzg.append(gu.f64(dz[b, t]))
    dtype = torch.bfloat16
    gu.check("y rows", np.array(yg), np.array(yo), dtype, "y")
    gu.check("dx rows", np.array(dxg), np.array(dxo), dtype, "dx")
    gu.check("dz rows", np.array(dzg), np.array(dzo), dtype, "dz")
    gu.say("  oracle on sampled dU columns (sums over every token)")
    rng = np.random.default_rng(wl.case)
    GW = wl.G * wl.W
    cols = sorted(set([0, 1, wl.W, GW - 1] + [int(c) for c in rng.integers(0, GW, ncols)]))
    X, Z, DY = (gu.f64(inp[k]) for k in ("x", "z", "dy"))
    dUo = orc.lowrank_dU_cols(X, Z, UU, DY, wl.W, wl.H, cols, wl.act)
    del X, Z, DY
    # relative to the whole dU's norm (as for the other outputs)
    a = float(np.max(np.abs(gu.f64(dU)[:, cols] - dUo)))
    m = float(gu.f64(dU).__abs__().max())
    gu.say(f"    dU cols: max abs err {a:.3e}, max|dU| {m:.3e}, rel {a / m:.3e}")
    assert a / m <= gu.TOL_BF16["dU"]


def test_full_size_qkv_lowrank(dsc, orc):
    """D=6144, T=2048, B=8, W=4, R=16, H=1, residual."""
    _full_size(dsc, orc, di.WORKLOADS["qkv_lowrank"], 40, 24)


def test_full_size_rnn_lowrank_silu(dsc, orc):
    """B=16, T=4096, D=4608, W=4, R=16, H=8, SiLU."""
    _full_size(dsc, orc, di.WORKLOADS["rnn_lowrank_silu"], 24, 12)


@pytest.mark.parametrize("W,H,dt", [(7, 8, "bf16"), (7, 4, "bf16"), (5, 8, "bf16"),
                                    (5, 4, "f32"), (7, 4, "f32"), (6, 2, "f32")])
def test_slot_counts_not_multiple_of_four(dsc, orc, W, H, dt):
    """Shapes whose per-lane filter-slot count leaves a partial dU MFMA block."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    run_case(dsc, orc, 2, 40, 512, W, H, 16, dtype, True, True, 8300 + 10 * W + H)
