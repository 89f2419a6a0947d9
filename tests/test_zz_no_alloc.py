"""The allocation-free low-rank backward (dsc_lowrank_bwd_noalloc) against the
entry point with a caller-owned workspace (dsc_lowrank_bwd), through the C ABI.

Both run the same kernels, so their results must agree bit for bit; the
smaller case is also held to the oracle's tolerance.  Two calls in a row
share the library's buffer, the second with a smaller input, so a stale
partial sum left by the first would show in the second.
"""
import pytest
import torch

import dsc_inputs as di
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsc():
    import dynamic_short_causal_amd as d
    return d


def _inputs(wl, seed_offset=0):
    inp = di.make(wl, seed_offset=seed_offset)
    return {k: v.to(gu.dev()) for k, v in inp.items()}


def _both(dsc, d, wl):
    ref = dsc.lowrank_bwd(d["x"], d["z"], d["U"], d["dy"], wl.W, wl.H, wl.residual, wl.act)
    out = (torch.full_like(d["x"], float("nan")), torch.full_like(d["z"], float("nan")),
           torch.full_like(d["U"], float("nan")))
    dsc.dsc_lowrank_bwd_noalloc(d["x"], d["z"], d["U"], d["dy"], *out, wl.W, wl.H,
                                wl.residual, wl.act)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_entry_two_calls(dsc, orc):
    big = di.WORKLOADS["qkv_lowrank"]            # B=8 T=2048 D=6144 W=4 R=16 H=1
    small = big.with_(name="small", case=31, B=2, T=150, D=1024, H=2, act=True)
    for wl in (big, small):
        gu.say(f"  noalloc {wl.name}: B={wl.B} T={wl.T} D={wl.D} H={wl.H} act={wl.act}")
        d = _inputs(wl)
        ref, out = _both(dsc, d, wl)
        for name, a, b in zip(("dx", "dz", "dU"), ref, out):
            assert torch.equal(a, b), f"{wl.name} {name} differs from dsc_lowrank_bwd"
    X, Z, UU, DY = (gu.f64(d[k]) for k in ("x", "z", "U", "dy"))
    dxo, dzo, dUo = orc.lowrank_bwd(X, Z, UU, DY, small.W, small.H, small.residual, small.act)
    for name, g, r in zip(("dx", "dz", "dU"), out, (dxo, dzo, dUo)):
        gu.check(name, g, r, torch.bfloat16, name)


def test_noalloc_rejects_shapes_above_its_buffer(dsc):
    """A shape whose partial sums exceed the buffer fails on the host."""
    B, T, D, W, H, R = 16, 4096, 8192, 4, 1, 16
    need = dsc.LIB.dsc_lowrank_bwd_workspace_bytes(B, T, D, W, H, R, dsc.DSC_BF16)
    assert need > dsc.NOALLOC_SCRATCH_BYTES
    import ctypes
    p = ctypes.c_void_p
    A, BIG = 1 << 20, 1 << 40
    st = dsc.LIB.dsc_lowrank_bwd_noalloc(p(A), p(A + BIG), p(A + 2 * BIG), p(A + 3 * BIG),
                                         p(A + 4 * BIG), p(A + 5 * BIG), p(A + 6 * BIG), B, T, D,
                                         W, H, R, dsc.DSC_BF16, 0, None)
    assert st == dsc.DSC_ERR_WORKSPACE, st
