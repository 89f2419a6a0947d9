"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before anything is queued.

No call here reaches a kernel launch: every case fails a host-side check (or
is empty, which queues nothing), so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsc.h")


@pytest.fixture(scope="module")
def lib():
    import __graft_entry__ as ge
    if not os.path.exists(os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc.so")):
        ge._library_builder().build()
    import dynamic_short_causal_amd as d
    return d.LIB


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsc_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    import dynamic_short_causal_amd as d
    names = declared()
    assert names and set(names) == set(d.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_match_header(lib):
    """Every binding declares as many arguments as the header, with 64-bit
    types where the header has int64_t or size_t."""
    import ctypes as ct
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, params in re.findall(r"\b(dsc_[a-z_0-9]+)\s*\(([^)]*)\)\s*;", text):
        params = [q.strip() for q in params.split(",") if q.strip() and q.strip() != "void"]
        fn = getattr(lib, name)
        got = fn.argtypes or []
        assert len(got) == len(params), (name, len(got), len(params))
        for q, t in zip(params, got):
            if q.startswith("int64_t"):
                assert t is ct.c_int64, (name, q)
            elif q.startswith("size_t"):
                assert t is ct.c_size_t, (name, q)
            elif "*" in q:
                assert t is ct.c_void_p, (name, q)
        if re.search(r"size_t\s+" + name + r"\s*\(", text):
            assert fn.restype is ct.c_size_t, name


def test_status_strings(lib):
    assert lib.dsc_status_string(0) == b"DSC_OK"
    assert lib.dsc_status_string(3) == b"DSC_ERR_WORKSPACE"
    assert lib.dsc_version() >= 10000


A = 1 << 20          # fake, 16-byte aligned, never dereferenced
BIG = 1 << 40


def hw(lib, x=A, w=A + BIG, y=A + 2 * BIG, B=1, T=8, D=64, W=4, H=1, dt=1, fl=0):
    return lib.dsc_headwise_fwd(ctypes.c_void_p(x), ctypes.c_void_p(w), ctypes.c_void_p(y),
                                B, T, D, W, H, dt, fl, None)


def hwb(lib, x=A, w=A + BIG, dy=A + 2 * BIG, dx=A + 3 * BIG, dw=A + 4 * BIG, B=1, T=8, D=64,
        W=4, H=1, dt=1, fl=0):
    p = ctypes.c_void_p
    return lib.dsc_headwise_bwd(p(x), p(w), p(dy), p(dx), p(dw), B, T, D, W, H, dt, fl, None)


def lr(lib, x=A, z=A + BIG, U=A + 2 * BIG, y=A + 3 * BIG, B=1, T=8, D=64, W=4, H=1, R=16,
       dt=1, fl=0):
    p = ctypes.c_void_p
    return lib.dsc_lowrank_fwd(p(x), p(z), p(U), p(y), B, T, D, W, H, R, dt, fl, None)


def lrb(lib, ws=A + 7 * BIG, wsb=None, B=1, T=8, D=64, W=4, H=1, R=16, dt=1, fl=0, dx=None):
    p = ctypes.c_void_p
    if wsb is None:
        wsb = lib.dsc_lowrank_bwd_workspace_bytes(B, T, D, W, H, R, dt)
    return lib.dsc_lowrank_bwd(p(A), p(A + BIG), p(A + 2 * BIG), p(A + 3 * BIG),
                               p(dx if dx is not None else A + 4 * BIG), p(A + 5 * BIG),
                               p(A + 6 * BIG), p(ws), wsb, B, T, D, W, H, R, dt, fl, None)


INVALID, UNSUP, WS = 1, 2, 3


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), UNSUP), (dict(fl=4), UNSUP), (dict(B=-1), INVALID), (dict(T=-2), INVALID),
    (dict(D=0), INVALID), (dict(W=0), UNSUP), (dict(W=9), UNSUP), (dict(H=0), INVALID),
    (dict(D=60, H=7), INVALID), (dict(D=36, H=1), INVALID), (dict(D=36, H=1, dt=0), OK := 0),
    (dict(H=3, D=48), UNSUP), (dict(H=12, D=48), UNSUP), (dict(H=8 * 128, D=8192), UNSUP),
    (dict(H=8 * 65, D=8 * 65), UNSUP), (dict(H=6, D=48, dt=0), UNSUP),
    (dict(x=0), INVALID), (dict(y=0), INVALID), (dict(w=A + BIG + 2), INVALID),
    (dict(y=A + 8), INVALID), (dict(y=A + 64 * 8 * 2 - 16), INVALID),
    (dict(B=1 << 31), INVALID), (dict(B=1 << 20, T=1 << 10, D=512), INVALID),
])
def test_headwise_fwd_checks(lib, kw, code):
    if code == 0:
        pytest.skip("valid arguments would launch a kernel")
    assert hw(lib, **kw) == code, lib.dsc_last_error()
    assert lib.dsc_last_error() != b""


def test_headwise_bwd_overlaps(lib):
    assert hwb(lib, dx=A + 2 * BIG + 16) == INVALID          # dx overlaps dy
    assert hwb(lib, dw=A + 3 * BIG + 32) == INVALID          # dw overlaps dx
    assert hwb(lib, dw=A + 16) == INVALID                    # dw overlaps x
    assert b"overlaps" in lib.dsc_last_error()
    assert hwb(lib, dy=0) == INVALID
    assert hwb(lib, H=5, D=40) == UNSUP


def test_empty_is_ok_and_queues_nothing(lib):
    assert hw(lib, B=0, x=0, w=0, y=0) == 0
    assert hw(lib, T=0, x=0, w=0, y=0) == 0
    assert hwb(lib, B=0, x=0, w=0, dy=0, dx=0, dw=0) == 0
    assert lr(lib, T=0, x=0, z=0, y=0) == 0


def test_lowrank_checks(lib):
    assert lr(lib, H=12, D=48) == UNSUP                     # neither divides 8 nor a multiple of it
    assert lr(lib, R=0) == UNSUP
    assert lr(lib, R=65) == UNSUP
    assert lr(lib, U=0) == INVALID
    assert lr(lib, y=A + BIG + 8) == INVALID                 # y overlaps z
    assert lr(lib, H=3, D=48, dt=0) == UNSUP
    assert lr(lib, H=2, D=48, dt=0, x=A + 4) == INVALID


def test_workspace_checks(lib):
    n = lib.dsc_lowrank_bwd_workspace_bytes(8, 2048, 6144, 4, 1, 16, 1)
    assert n > 0
    assert lib.dsc_lowrank_bwd_workspace_bytes(8, 2048, 6144, 4, 12, 16, 1) == 0  # H=12
    # H=16 (two bf16 vectors per group): partials of one group per vector
    assert (lib.dsc_lowrank_bwd_workspace_bytes(8, 2048, 6144, 4, 16, 16, 1)
            == lib.dsc_lowrank_bwd_workspace_bytes(8, 2048, 6144, 4, 8, 16, 1))
    assert lib.dsc_lowrank_bwd_workspace_bytes(8, 2048, 6144, 9, 1, 16, 1) == 0
    assert lrb(lib, wsb=lib.dsc_lowrank_bwd_workspace_bytes(1, 8, 64, 4, 1, 16, 1) - 1) == WS
    assert lrb(lib, ws=0) == WS
    assert lrb(lib, ws=A + 4 * BIG + 16) == INVALID          # workspace overlaps dx
    assert lrb(lib, R=70) == UNSUP
    assert lrb(lib, dx=A + 8) == INVALID
    # 16 rows of x must fit the backward's 32-bit slab offsets
    assert lrb(lib, B=1, T=1, D=1 << 26) == UNSUP            # bf16: 16 * 2^26 * 2 = 2^31
    assert lrb(lib, B=1, T=1, D=(1 << 25), dt=0) == UNSUP    # fp32: 16 * 2^25 * 4 = 2^31
    assert lrb(lib, B=0, T=1, D=(1 << 26) - 8) != UNSUP


def test_empty_sequence_workspace_and_checks():
    """T = 0 (and B = 0) through the backward's tiling plan: the workspace query
    is 0 and a call that then fails a pointer check returns INVALID.  Run in a
    child process, since a division by zero in the plan would kill it."""
    import subprocess
    import sys
    code = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import dynamic_short_causal_amd as d\n"
        "lib = d.LIB\n"
        "for (B, T) in ((1, 0), (0, 5), (0, 0), (3, 0)):\n"
        "    for dt in (0, 1):\n"
        "        for H in (1, 2):\n"
        "            n = lib.dsc_lowrank_bwd_workspace_bytes(B, T, 64, 4, H, 16, dt)\n"
        "            assert n == 0, (B, T, dt, H, n)\n"
        "p = ctypes.c_void_p\n"
        "A, BIG = 1 << 20, 1 << 40\n"
        "# dU is non-empty (R x G*W) even for T = 0: NULL must be rejected\n"
        "st = lib.dsc_lowrank_bwd(p(A), p(A + BIG), p(A + 2 * BIG), p(A + 3 * BIG), p(A + 4 * BIG),\n"
        "                         p(A + 5 * BIG), p(0), p(0), 0, 1, 0, 64, 4, 1, 16, 1, 0, None)\n"
        "assert st == 1, st\n"
        "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stderr[-2000:])


def hdec(lib, x=A, w=A + BIG, st=A + 2 * BIG, y=A + 3 * BIG, B=2, D=64, W=4, H=1, dt=1, fl=0):
    p = ctypes.c_void_p
    return lib.dsc_headwise_decode(p(x), p(w), p(st), p(y), B, D, W, H, dt, fl, None)


def ldec(lib, x=A, z=A + BIG, U=A + 2 * BIG, st=A + 3 * BIG, y=A + 4 * BIG, B=2, D=64, W=4, H=1,
         R=16, dt=1, fl=0):
    p = ctypes.c_void_p
    return lib.dsc_lowrank_decode(p(x), p(z), p(U), p(st), p(y), B, D, W, H, R, dt, fl, None)


def dstate(lib, x=A, st=A + BIG, B=2, T=8, D=64, W=4, dt=1):
    p = ctypes.c_void_p
    return lib.dsc_decode_state(p(x), p(st), B, T, D, W, dt, None)


def test_decode_checks(lib):
    assert hdec(lib, W=9) == UNSUP
    assert hdec(lib, fl=8) == UNSUP
    assert hdec(lib, H=3, D=48) == UNSUP
    assert hdec(lib, D=36) == INVALID                        # not a multiple of 8 (bf16)
    assert hdec(lib, st=0) == INVALID
    assert hdec(lib, st=A + 8) == INVALID                    # misaligned
    assert hdec(lib, st=A + 3 * BIG - 16) == INVALID         # state runs into y
    assert b"overlaps" in lib.dsc_last_error()
    assert hdec(lib, y=A + 2 * BIG + 16) == INVALID          # y inside the state
    assert hdec(lib, B=-1) == INVALID
    assert ldec(lib, H=12, D=48) == UNSUP                    # low-rank: H | 8 or 8 | H
    assert ldec(lib, R=0) == UNSUP
    assert ldec(lib, U=0) == INVALID
    assert ldec(lib, st=A + BIG) == INVALID                  # state overlaps z
    assert dstate(lib, W=0) == UNSUP
    assert dstate(lib, T=-1) == INVALID
    assert dstate(lib, st=A + 16) == INVALID                 # state overlaps x
    assert dstate(lib, x=0) == INVALID


def test_decode_empty(lib):
    assert hdec(lib, B=0, x=0, w=0, st=0, y=0) == 0
    assert ldec(lib, B=0, x=0, z=0, st=0, y=0) == 0
    assert dstate(lib, B=0, x=0, st=0) == 0
    # W == 1 keeps no state: the pointer is not used, but x, w and y still are
    assert dstate(lib, W=1, st=0) == 0
    assert hdec(lib, W=1, st=0, y=0) == INVALID


def sfw(lib, x=A, w=A + BIG, y=A + 2 * BIG, B=1, T=8, D=64, W=4, H=1, dt=1, fl=0):
    p = ctypes.c_void_p
    return lib.dsc_static_fwd(p(x), p(w), p(y), B, T, D, W, H, dt, fl, None)


def sbw(lib, ws=A + 5 * BIG, wsb=None, B=1, T=8, D=64, W=4, H=1, dt=1, fl=0, dw=A + 4 * BIG):
    p = ctypes.c_void_p
    if wsb is None:
        wsb = lib.dsc_static_bwd_workspace_bytes(B, T, D, W, H, dt)
    return lib.dsc_static_bwd(p(A), p(A + BIG), p(A + 2 * BIG), p(A + 3 * BIG), p(dw), p(ws),
                              wsb, B, T, D, W, H, dt, fl, None)


def test_static_checks(lib):
    assert sfw(lib, W=9) == UNSUP
    assert sfw(lib, H=3, D=48) == UNSUP
    assert sfw(lib, D=36) == INVALID
    assert sfw(lib, w=0) == INVALID
    assert sfw(lib, y=A + BIG + 16) == INVALID               # y overlaps w
    n = lib.dsc_static_bwd_workspace_bytes(1, 8, 64, 4, 1, 1)
    assert n == 64 * 4 * 4                                   # one 512-token span: G*W fp32
    assert lib.dsc_static_bwd_workspace_bytes(8, 2048, 6144, 4, 1, 1) == 8 * 4 * 6144 * 4 * 4
    assert lib.dsc_static_bwd_workspace_bytes(1, 8, 64, 9, 1, 1) == 0
    assert lib.dsc_static_bwd_workspace_bytes(0, 8, 64, 4, 1, 1) == 0
    assert sbw(lib, wsb=n - 1) == WS
    assert sbw(lib, ws=0) == WS
    assert sbw(lib, ws=A + 3 * BIG + 16) == INVALID          # workspace overlaps dx
    assert sbw(lib, dw=A + BIG) == INVALID                   # dw overlaps w
    assert sbw(lib, fl=16) == UNSUP


def test_varlen_checks(lib):
    p = ctypes.c_void_p
    POS = A + 9 * BIG
    hv = lambda pos=POS, **kw: lib.dsc_headwise_fwd_varlen(
        p(A), p(A + BIG), p(pos), p(A + 2 * BIG), kw.get("B", 1), 8, 64, 4, kw.get("H", 1), 1, 0,
        None)
    assert hv(pos=0) == INVALID                              # pos is NULL
    assert hv(pos=POS + 4) == INVALID                        # not 16-byte aligned
    assert hv(pos=A + 2 * BIG + 16) == INVALID               # y overlaps pos
    assert hv(H=3) == INVALID                                # 64 % 3
    assert hv(B=0, pos=0) == 0                               # empty: pos unused
    lv = lambda pos=POS: lib.dsc_lowrank_bwd_varlen(
        p(A), p(A + BIG), p(A + 2 * BIG), p(pos), p(A + 3 * BIG), p(A + 4 * BIG), p(A + 5 * BIG),
        p(A + 6 * BIG), p(A + 7 * BIG), lib.dsc_lowrank_bwd_workspace_bytes(1, 8, 64, 4, 1, 16, 1),
        1, 8, 64, 4, 1, 16, 1, 0, None)
    assert lv(pos=0) == INVALID
    assert lv(pos=A + 4 * BIG + 64) == INVALID               # dx overlaps pos


def gfw(lib, x=A, xh=A + BIG, Mt=A + 2 * BIG, y=A + 3 * BIG, B=1, T=8, D=64, Dh=64, W=4, H=8,
        dt=1, fl=0):
    p = ctypes.c_void_p
    return lib.dsc_headwise_gen_fwd(p(x), p(xh), p(Mt), p(y), B, T, D, Dh, W, H, dt, fl, None)


def test_generated_filter_checks(lib):
    assert gfw(lib, dt=0) == UNSUP                           # bf16 only
    assert gfw(lib, W=3) == UNSUP                            # W in {1, 2, 4, 8}
    assert gfw(lib, H=4) == UNSUP                            # H a multiple of 8
    assert gfw(lib, Dh=96) == UNSUP                          # Dh a multiple of 64
    assert gfw(lib, Dh=0) == UNSUP
    assert gfw(lib, D=72, H=24, W=1) == UNSUP                # G*W = 3
    assert gfw(lib, D=8, H=8, W=4) == UNSUP                  # G*W = 4
    assert gfw(lib, Mt=0) == INVALID
    assert gfw(lib, y=A + 2 * BIG + 16) == INVALID           # y overlaps Mt
    assert gfw(lib, B=0, x=0, xh=0, y=0) == 0                # empty: nothing is read


def test_noalloc_checks(lib):
    """The allocation-free backward: argument errors as dsc_lowrank_bwd, and a
    shape needing more partial-sum space than the library buffer is refused
    on the host (no device is touched)."""
    import dynamic_short_causal_amd as d
    p = ctypes.c_void_p

    def call(B=1, T=8, D=64, W=4, H=1, R=16, dt=1, fl=0, x=A, dU=A + 6 * BIG):
        return lib.dsc_lowrank_bwd_noalloc(p(x), p(A + BIG), p(A + 2 * BIG), p(A + 3 * BIG),
                                           p(A + 4 * BIG), p(A + 5 * BIG), p(dU), B, T, D, W, H,
                                           R, dt, fl, None)
    assert call(R=0) == UNSUP
    assert call(W=9) == UNSUP
    assert call(x=0) == INVALID
    assert call(dU=A + 4 * BIG + 16) == INVALID               # dU overlaps dx
    B, T, D = 16, 4096, 8192
    assert lib.dsc_lowrank_bwd_workspace_bytes(B, T, D, 4, 1, 16, 1) > d.NOALLOC_SCRATCH_BYTES
    assert call(B=B, T=T, D=D) == WS
    assert b"library buffer" in lib.dsc_last_error()


def test_yardstick_library_checks():
    """libdsc_yard.so (the matrix-core forward the benchmark times beside the
    vector-ALU kernel for filters tied over 8 channels) loads, exports its one
    call, and refuses arguments outside its case before touching a device."""
    path = os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc_yard.so")
    if not os.path.exists(path):
        import __graft_entry__ as ge
        ge._library_builder().build()
    y = ctypes.CDLL(path)
    f = y.dsc_yard_lowrank_fwd_mfma
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_int] * 3 + [
        ctypes.c_void_p]
    p = ctypes.c_void_p
    ok = dict(x=A, z=A + BIG, U=A + 2 * BIG, y=A + 3 * BIG, B=1, T=8, D=64, R=16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(p(a["x"]), p(a["z"]), p(a["U"]), p(a["y"]), a["B"], a["T"], a["D"], a["R"], 1,
                 1, None)
    assert call(x=0) == -1
    assert call(R=17) == -1
    assert call(R=0) == -1
    assert call(D=60) == -1
    assert call(B=-1) == -1
    # the vector-ALU backward yardstick: workspace query and argument checks
    y.dsc_yard_lowrank_bwd_valu_workspace.restype = ctypes.c_size_t
    y.dsc_yard_lowrank_bwd_valu_workspace.argtypes = [ctypes.c_int64] * 3
    assert y.dsc_yard_lowrank_bwd_valu_workspace(2, 300, 1024) > 0
    assert y.dsc_yard_lowrank_bwd_valu_workspace(2, 300, 1020) == 0
    g = y.dsc_yard_lowrank_bwd_valu
    g.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int64] * 3 + [ctypes.c_int] * 3 + [
        ctypes.c_void_p]
    ptrs = [p(A + i * BIG) for i in range(8)]
    assert g(*([p(0)] + ptrs[1:]), 1, 8, 64, 16, 1, 1, None) == -1   # null x
    assert g(*ptrs, 1, 8, 64, 15, 1, 1, None) == -1                  # odd R
    assert g(*ptrs, 1, 8, 64, 18, 1, 1, None) == -1                  # R > 16
    assert g(*ptrs, 1, 8, 60, 16, 1, 1, None) == -1                  # D not a multiple of 8
