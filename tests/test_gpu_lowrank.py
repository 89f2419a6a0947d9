"""GPU parity of the low-rank kernels (on-chip zU) against the fp64 oracle."""
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


# Filters tied over several channel vectors (H a multiple of the vector width:
# 16, 24 and 64 in bf16, 8 and 32 in fp32): the kernels tile one group per
# vector, read U's column of group c / H and fold the vector groups' dU
# partials in the reduction.  D leaves a partial last channel block.
@pytest.mark.parametrize("H,dt,act,R,D", [(16, "bf16", False, 16, 1072), (64, "bf16", True, 16, 1088),
                                          (24, "bf16", False, 16, 1080), (16, "bf16", True, 40, 1072),
                                          (8, "f32", False, 16, 552), (32, "f32", True, 7, 608)])
def test_tying_wider_than_a_vector(dsc, orc, H, dt, act, R, D):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    run_case(dsc, orc, 2, 150, D, 4, H, R, dtype, True, act, 7700 + H + R)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 6, 7, 8])
def test_widths(dsc, orc, W):
    run_case(dsc, orc, 2, 67, 256, W, 1, 16, torch.bfloat16, True, False, 7200 + W)
    run_case(dsc, orc, 1, 70, 128, W, 2, 16, torch.float32, False, True, 7300 + W)


@pytest.mark.parametrize("R", [1, 3, 8, 12, 16, 17, 24, 32, 33, 48, 64])
def test_ranks(dsc, orc, R):
    """Ranks within one 16-rank block and across two and four (the backward
    then runs one pass per block)."""
    run_case(dsc, orc, 2, 45, 256, 4, 1, R, torch.bfloat16, True, False, 7400 + R)
    run_case(dsc, orc, 1, 45, 64, 4, 4, R, torch.float32, False, False, 7500 + R)


@pytest.mark.parametrize("R", [20, 64])
@pytest.mark.parametrize("H,act", [(1, True), (8, False), (2, True)])
def test_many_ranks_tied_and_silu(dsc, orc, R, H, act):
    run_case(dsc, orc, 2, 150, 512 + 8 * 16 * H, 4, H, R, torch.bfloat16, True, act,
             7550 + R + 10 * H)


@pytest.mark.parametrize("W,H,dt", [(8, 1, "bf16"), (7, 1, "bf16"), (8, 2, "f32"), (1, 1, "f32")])
def test_many_ranks_widths(dsc, orc, W, H, dt):
    """The widest filters at 64 ranks (the largest resident fragment sets)."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    run_case(dsc, orc, 2, 70, 256, W, H, 64, dtype, True, dt == "bf16", 7580 + W + H)


@pytest.mark.parametrize("B,T", [(1, 1), (2, 3), (1, 17)])
def test_many_ranks_short_sequences(dsc, orc, B, T):
    run_case(dsc, orc, B, T, 128, 4, 1, 48, torch.bfloat16, True, True, 7590 + T)
    run_case(dsc, orc, B, T, 64, 4, 2, 33, torch.float32, True, False, 7595 + T)


@pytest.mark.parametrize("B,T,D,W,act", [(4, 1041, 1536, 4, False), (2, 1041, 1536, 8, True),
                                         (3, 129, 640, 2, True), (2, 527, 1000, 3, False)])
def test_per_channel_chunks(dsc, orc, B, T, D, W, act):
    """Per-channel bf16 filters (one channel per lane in both directions)
    over lengths whose token chunks and 16-token steps end ragged, every
    element checked."""
    run_case(dsc, orc, B, T, D, W, 1, 16, torch.bfloat16, True, act, 7950 + T + W)


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


@pytest.mark.parametrize("B,T", [(0, 5), (1, 0), (3, 0)])
def test_empty_batch_zeroes_dU(dsc, orc, B, T):
    """No sequences, or sequences of length 0: dU is still written, as zeros."""
    x = torch.empty((B, T, 64), dtype=torch.bfloat16, device=gu.dev())
    z = torch.empty((B, T, 16), dtype=torch.bfloat16, device=gu.dev())
    U = di.randn((16, 64 * 4), 0.1, 8000, "bf16").to(gu.dev())
    dU = torch.full_like(U, float("nan"))
    dz = torch.empty_like(z)
    dx = torch.empty_like(x)
    ws = dsc.lowrank_workspace(x, z, 4, 1)
    dsc.dsc_lowrank_bwd(x, z, U, x, dx, dz, dU, ws, 4, 1)
    torch.cuda.synchronize()
    assert torch.all(dU == 0)


@pytest.mark.parametrize("H,act", [(1, False), (8, True)])
def test_deterministic(dsc, orc, H, act):
    """Repeated calls give the same bits: per-channel filters (channel-per-lane
    backward) and filters tied over 8 channels with SiLU (vector-ALU forward,
    token-per-lane backward)."""
    x = di.randn((2, 300, 1024), 1.0, 8100, "bf16").to(gu.dev())
    z = di.randn((2, 300, 16), 1.0, 8102, "bf16").to(gu.dev())
    U = di.randn((16, (1024 // H) * 4), 0.125, 8103, "bf16").to(gu.dev())
    dy = di.randn((2, 300, 1024), 1.0, 8104, "bf16").to(gu.dev())
    a = dsc.lowrank_bwd(x, z, U, dy, 4, H, True, act)
    b = dsc.lowrank_bwd(x, z, U, dy, 4, H, True, act)
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    assert torch.equal(dsc.lowrank_fwd(x, z, U, 4, H, True, act),
                       dsc.lowrank_fwd(x, z, U, 4, H, True, act))


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


def _full_tensor(dsc, orc, wl):
    """Every element of y, dx, dz and dU against the whole-batch fp64 oracle
    (each tolerance relative to the oracle's max-norm)."""
    gu.say(f"  full-size {wl.name}: generating inputs")
    inp = di.make(wl)
    xd, zd, Ud, dyd = (inp[k].to(gu.dev()) for k in ("x", "z", "U", "dy"))
    y = dsc.lowrank_fwd(xd, zd, Ud, wl.W, wl.H, wl.residual, wl.act)
    dx, dz, dU = dsc.lowrank_bwd(xd, zd, Ud, dyd, wl.W, wl.H, wl.residual, wl.act)
    torch.cuda.synchronize()
    del xd, zd, Ud, dyd
    gu.say("  kernels done; whole-batch oracle")
    X, Z, UU, DY = (gu.f64(inp[k]) for k in ("x", "z", "U", "dy"))
    dtype = torch.bfloat16
    gu.check("y", y, orc.lowrank_fwd(X, Z, UU, wl.W, wl.H, wl.residual, wl.act), dtype, "y")
    del y
    dxo, dzo, dUo = orc.lowrank_bwd(X, Z, UU, DY, wl.W, wl.H, wl.residual, wl.act)
    del X, DY
    gu.check("dx", dx, dxo, dtype, "dx")
    gu.check("dz", dz, dzo, dtype, "dz")
    gu.check("dU", dU, dUo, dtype, "dU")


def test_full_size_qkv_lowrank(dsc, orc):
    """D=6144, T=2048, B=8, W=4, R=16, H=1, residual: every element."""
    _full_tensor(dsc, orc, di.WORKLOADS["qkv_lowrank"])


def test_full_size_rnn_lowrank_silu(dsc, orc):
    """B=16, T=4096, D=4608, W=4, R=16, H=8, SiLU: every element."""
    _full_tensor(dsc, orc, di.WORKLOADS["rnn_lowrank_silu"])


@pytest.mark.parametrize("W,H,dt", [(7, 8, "bf16"), (7, 4, "bf16"), (5, 8, "bf16"),
                                    (5, 4, "f32"), (7, 4, "f32"), (6, 2, "f32")])
def test_slot_counts_not_multiple_of_four(dsc, orc, W, H, dt):
    """Shapes whose per-lane filter-slot count leaves a partial dU MFMA block."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    run_case(dsc, orc, 2, 40, 512, W, H, 16, dtype, True, True, 8300 + 10 * W + H)


@pytest.mark.parametrize("W,R,T,residual,act", [
    (1, 16, 70, True, False), (2, 8, 70, False, True), (3, 12, 33, True, True),
    (4, 2, 70, True, True), (4, 16, 1, True, True), (3, 16, 2, False, False),
    (4, 5, 70, True, True), (2, 16, 129, True, False)])
def test_tied_eight_vector_alu_forward(dsc, orc, W, R, T, residual, act):
    """bf16 filters tied over 8 channels form their taps on the vector ALUs
    when W <= 4 and R is even (R = 5 takes the matrix-core kernel).  D = 576
    is 72 channel vectors: one wave and a part-filled second per row."""
    run_case(dsc, orc, 2, T, 576, W, 8, R, torch.bfloat16, residual, act,
             8400 + 10 * W + R + T)


@pytest.mark.parametrize("T,act,residual", [(300, True, False), (70, False, True), (1, True, True)])
def test_vector_alu_backward_yardstick(dsc, orc, T, act, residual):
    """The vector-ALU backward kept in libdsc_yard.so (measured against the
    library's matrix-core backward by the benchmark) matches the oracle at
    the bar of the library's own kernels: bf16, W=4, H=8, R=16, D=576 (one
    full and one part-filled wave per row)."""
    import ctypes
    import os
    lib = ctypes.CDLL(os.path.join(os.path.dirname(dsc.__file__), "libdsc_yard.so"))
    lib.dsc_yard_lowrank_bwd_valu_workspace.restype = ctypes.c_size_t
    lib.dsc_yard_lowrank_bwd_valu_workspace.argtypes = [ctypes.c_int64] * 3
    lib.dsc_yard_lowrank_bwd_valu.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int64] * 3
                                              + [ctypes.c_int] * 3 + [ctypes.c_void_p])
    B, D, W, H, R, seed = 2, 576, 4, 8, 16, 8500 + T
    gu.say(f"  case yardstick B={B} T={T} D={D} act={act} res={residual}")
    x = di.randn((B, T, D), 1.0, seed, "bf16")
    z = di.randn((B, T, R), 1.0, seed + 2, "bf16")
    U = di.randn((R, (D // H) * W), (1.0 / (R * W)) ** 0.5 * 2, seed + 3, "bf16")
    dy = di.randn((B, T, D), 1.0, seed + 4, "bf16")
    xd, zd, Ud, dyd = (t.to(gu.dev()) for t in (x, z, U, dy))
    dx, dz, dU = torch.empty_like(xd), torch.empty_like(zd), torch.empty_like(Ud)
    ws = torch.empty(lib.dsc_yard_lowrank_bwd_valu_workspace(B, T, D), dtype=torch.uint8,
                     device=gu.dev())
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s = torch.cuda.current_stream()
    assert lib.dsc_yard_lowrank_bwd_valu(P(xd), P(zd), P(Ud), P(dyd), P(dx), P(dz), P(dU), P(ws),
                                         B, T, D, R, int(residual), int(act),
                                         ctypes.c_void_p(s.cuda_stream)) == 0
    torch.cuda.synchronize()
    X, Z, UU, DY = gu.f64(x), gu.f64(z), gu.f64(U), gu.f64(dy)
    dxo, dzo, dUo = orc.lowrank_bwd(X, Z, UU, DY, W, H, residual, act)
    gu.check("dx", dx, dxo, torch.bfloat16, "dx")
    gu.check("dz", dz, dzo, torch.bfloat16, "dz")
    gu.check("dU", dU, dUo, torch.bfloat16, "dU")
