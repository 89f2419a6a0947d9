"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a fact fixed by the pages or by mathematics:
a hand-worked example, a closed form, a library routine, an invariant, or a
brute-force finite difference.  ``test_oracle_pins.py`` runs them against the
real oracle, ``test_oracle_mutants.py`` against copies of it with planted
mistakes (each of which must trip at least one pin).
"""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from tests import torch_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "handworked.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    tol = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.3e}"


# ---------------------------------------------------------------- worked example
def pin_handworked(orc):
    """Numbers worked by hand from the defining sum (tests/golden/handworked.json)."""
    g = json.load(open(GOLDEN))
    x, dy = np.array(g["x"], float), np.array(g["dy"], float)
    pc = g["per_channel"]
    w = np.array(pc["w"], float)
    _close(orc.headwise_fwd(x, w, 1), pc["y"], what="hand y")
    _close(orc.headwise_fwd(x, w, 1, residual=True), pc["y_residual"], what="hand y+x")
    dx, dw = orc.headwise_bwd(x, w, dy, 1)
    _close(dx, pc["dx"], what="hand dx")
    _close(dw, pc["dw"], what="hand dw")
    dx, _ = orc.headwise_bwd(x, w, dy, 1, residual=True)
    _close(dx, pc["dx_residual"], what="hand dx+dy")
    td = g["tied_H2"]
    w = np.array(td["w"], float)
    _close(orc.headwise_fwd(x, w, 2), td["y"], what="hand tied y")
    dx, dw = orc.headwise_bwd(x, w, dy, 2)
    _close(dx, td["dx"], what="hand tied dx")
    _close(dw, td["dw"], what="hand tied dw")
    lr = g["lowrank_H2_R1"]
    z, U = np.array(lr["z"], float), np.array(lr["U"], float)
    _close(orc.lowrank_w(z, U, 2), lr["w"], what="hand zU")
    _close(orc.lowrank_fwd(x, z, U, 2, 2), lr["y"], what="hand lowrank y")
    dx, dz, dU = orc.lowrank_bwd(x, z, U, dy, 2, 2)
    _close(dx, lr["dx"], what="hand lowrank dx")
    _close(dz, lr["dz"], what="hand lowrank dz")
    _close(dU, lr["dU"], what="hand lowrank dU")


# ---------------------------------------------------------------- closed forms
def pin_width_one_is_scale(orc):
    """W = 1: y = w[...,0] (.) x, the dynamic filter reduces to a per-token scale."""
    rng = _rng(1)
    for H in (1, 2, 3):
        x = _rand(rng, 2, 9, 6)
        w = _rand(rng, 2, 9, 6 // H, 1)
        wc = np.repeat(w[..., 0], H, axis=2)
        _close(orc.headwise_fwd(x, w, H), wc * x, what=f"W=1 H={H}")
        _close(orc.headwise_fwd(x, w, H, residual=True), wc * x + x, what="W=1 res")
        dy = _rand(rng, 2, 9, 6)
        dx, dw = orc.headwise_bwd(x, w, dy, H)
        _close(dx, wc * dy, what="W=1 dx")
        _close(dw[..., 0], (dy * x).reshape(2, 9, 6 // H, H).sum(-1), what="W=1 dw")


def pin_silu_values(orc):
    """With W = 1 and w = 1 the op is the activation itself: SiLU(s) = s/(1+e^-s)."""
    s = np.array([[[0.0, 1.0, -1.0, 2.5, -3.0, 20.0]]])
    w = np.ones((1, 1, 6, 1))
    y = orc.headwise_fwd(s, w, 1, act=True)
    expect = np.array([v / (1.0 + math.exp(-v)) for v in s[0, 0]])
    _close(y[0, 0], expect, rtol=1e-14, atol=1e-15, what="silu values")
    # sigmoid(1) = e / (e + 1); SiLU(-1) = -1 / (1 + e)
    assert abs(y[0, 0, 1] - math.e / (math.e + 1)) < 1e-15
    assert abs(y[0, 0, 2] + 1.0 / (1.0 + math.e)) < 1e-15
    # d/dx SiLU(w x) at w=1: sigmoid(s) (1 + s (1 - sigmoid(s))); at s=0 it is 1/2
    dx, _ = orc.headwise_bwd(s, w, np.ones_like(s), 1, act=True)
    sg = 1.0 / (1.0 + np.exp(-s[0, 0]))
    _close(dx[0, 0], sg * (1 + s[0, 0] * (1 - sg)), what="silu grad")
    assert abs(dx[0, 0, 0] - 0.5) < 1e-15


# ---------------------------------------------------------------- library routine
def pin_static_filter_is_conv1d(orc):
    """w constant in t reduces to a static depthwise causal conv (torch conv1d)."""
    rng = _rng(2)
    for (B, T, D, W, H) in [(2, 13, 8, 4, 1), (1, 7, 6, 3, 2), (2, 3, 4, 5, 4)]:
        x = _rand(rng, B, T, D)
        w0 = _rand(rng, B, D // H, W)
        w = np.broadcast_to(w0[:, None], (B, T, D // H, W)).copy()
        y = orc.headwise_fwd(x, w, H)
        for b in range(B):
            wt = torch.tensor(np.repeat(w0[b], H, axis=0)[:, ::-1].copy())  # (D, W) flipped
            ref = F.conv1d(torch.tensor(x[b].T[None]), wt[:, None, :], padding=W - 1,
                           groups=D)[0, :, :T].T.numpy()
            _close(y[b], ref, what=f"conv1d B={B} T={T} W={W} H={H}")


# ---------------------------------------------------------------- invariants
def pin_causality(orc):
    """Changing x at t' > t leaves y at t bitwise unchanged; no leakage across b."""
    rng = _rng(3)
    B, T, D, W = 3, 11, 4, 4
    x = _rand(rng, B, T, D)
    w = _rand(rng, B, T, D, W)
    y = orc.headwise_fwd(x, w, 1, residual=True, act=True)
    for tp in (0, 5, 10):
        x2 = x.copy()
        x2[1, tp] += 7.0
        y2 = orc.headwise_fwd(x2, w, 1, residual=True, act=True)
        assert np.array_equal(y2[:, :tp], y[:, :tp]), "future leaked into the past"
        assert np.array_equal(y2[0], y[0]) and np.array_equal(y2[2], y[2]), "batch leak"
        hit = np.any(y2[1, tp:min(T, tp + W)] != y[1, tp:min(T, tp + W)], axis=1)
        assert hit.all(), "x_t' did not reach y at t' .. t'+W-1"
        if tp + W < T:
            assert np.array_equal(y2[1, tp + W:], y[1, tp + W:]), "window longer than W"


def pin_linearity(orc):
    """Without activation, y is linear in x and, separately, in w."""
    rng = _rng(4)
    B, T, D, W, H = 2, 10, 6, 3, 2
    x1, x2 = _rand(rng, B, T, D), _rand(rng, B, T, D)
    w1, w2 = _rand(rng, B, T, D // H, W), _rand(rng, B, T, D // H, W)
    a, b = 0.75, -1.5
    _close(orc.headwise_fwd(a * x1 + b * x2, w1, H),
           a * orc.headwise_fwd(x1, w1, H) + b * orc.headwise_fwd(x2, w1, H),
           rtol=1e-13, atol=1e-13, what="linear in x")
    _close(orc.headwise_fwd(x1, a * w1 + b * w2, H),
           a * orc.headwise_fwd(x1, w1, H) + b * orc.headwise_fwd(x1, w2, H),
           rtol=1e-13, atol=1e-13, what="linear in w")


def pin_residual_is_tap0_shift(orc):
    """rho = 1 equals rho = 0 with w[..., 0] += 1 (for y, dx; dw is unchanged)."""
    rng = _rng(5)
    B, T, D, W, H = 2, 9, 8, 4, 4
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    w = _rand(rng, B, T, D // H, W)
    w1 = w.copy()
    w1[..., 0] += 1.0
    _close(orc.headwise_fwd(x, w, H, residual=True), orc.headwise_fwd(x, w1, H),
           rtol=1e-13, atol=1e-13, what="residual fwd")
    dxa, dwa = orc.headwise_bwd(x, w, dy, H, residual=True)
    dxb, dwb = orc.headwise_bwd(x, w1, dy, H)
    _close(dxa, dxb, rtol=1e-13, atol=1e-13, what="residual dx")
    _close(dwa, dwb, rtol=1e-13, atol=1e-13, what="residual dw")


def pin_tying_is_repeat(orc):
    """H-tied filters equal per-channel filters repeated H times along channels."""
    rng = _rng(6)
    B, T, D, W = 2, 8, 12, 3
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    for H in (2, 3, 4, 6, 12):
        w = _rand(rng, B, T, D // H, W)
        wr = np.repeat(w, H, axis=2)
        for act in (False, True):
            _close(orc.headwise_fwd(x, w, H, act=act), orc.headwise_fwd(x, wr, 1, act=act),
                   rtol=1e-13, atol=1e-13, what=f"tying fwd H={H}")
            dx, dw = orc.headwise_bwd(x, w, dy, H, act=act)
            dxr, dwr = orc.headwise_bwd(x, wr, dy, 1, act=act)
            _close(dx, dxr, rtol=1e-13, atol=1e-13, what=f"tying dx H={H}")
            _close(dw, dwr.reshape(B, T, D // H, H, W).sum(3), rtol=1e-12, atol=1e-12,
                   what=f"tying dw H={H}")


def pin_lowrank_is_headwise(orc):
    """Low-rank equals head-wise with w = (z @ U).reshape(B,T,G,W) materialised."""
    rng = _rng(7)
    B, T, D, W, R = 2, 9, 8, 4, 3
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    for H in (1, 2, 8):
        G = D // H
        z, U = _rand(rng, B, T, R), _rand(rng, R, G * W)
        w = (z @ U).reshape(B, T, G, W)
        _close(orc.lowrank_w(z, U, W), w, rtol=1e-13, atol=1e-13, what="zU")
        for res, act in ((True, False), (False, True)):
            _close(orc.lowrank_fwd(x, z, U, W, H, residual=res, act=act),
                   orc.headwise_fwd(x, w, H, residual=res, act=act),
                   rtol=1e-13, atol=1e-13, what=f"lowrank fwd H={H}")
            dx, dz, dU = orc.lowrank_bwd(x, z, U, dy, W, H, residual=res, act=act)
            dxh, dwh = orc.headwise_bwd(x, w, dy, H, residual=res, act=act)
            _close(dx, dxh, rtol=1e-13, atol=1e-13, what="lowrank dx")
            dw2 = dwh.reshape(B * T, G * W)
            _close(dz, (dw2 @ U.T).reshape(B, T, R), rtol=1e-12, atol=1e-12, what="dz")
            _close(dU, z.reshape(B * T, R).T @ dw2, rtol=1e-12, atol=1e-12, what="dU")


# ---------------------------------------------------------------- identities
def pin_adjoint(orc):
    """<conv_w(x), u> = <x, conv_w^T(u)>: dx is the adjoint applied to dy."""
    rng = _rng(8)
    for (B, T, D, W, H) in [(2, 17, 8, 4, 2), (1, 3, 4, 5, 1)]:
        x, u = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, B, T, D // H, W)
        y = orc.headwise_fwd(x, w, H)
        dx, _ = orc.headwise_bwd(x, w, u, H)
        lhs, rhs = np.sum(y * u), np.sum(x * dx)
        assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), (lhs, rhs)


def pin_euler(orc):
    """Bilinearity: sum dw*w = sum dz*z = sum dU*U = sum ds*s (ds = grad at s)."""
    rng = _rng(9)
    B, T, D, W, H, R = 2, 12, 8, 3, 2, 4
    G = D // H
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    z, U = _rand(rng, B, T, R), _rand(rng, R, G * W)
    w = (z @ U).reshape(B, T, G, W)
    for act in (False, True):
        s = orc.headwise_fwd(x, w, H)           # pre-activation
        sg = 1.0 / (1.0 + np.exp(-s))
        ds = dy * (sg * (1 + s * (1 - sg)) if act else 1.0)
        ref = np.sum(ds * s)
        _, dw = orc.headwise_bwd(x, w, dy, H, residual=True, act=act)
        _, dz, dU = orc.lowrank_bwd(x, z, U, dy, W, H, residual=True, act=act)
        for name, v in (("dw.w", np.sum(dw * w)), ("dz.z", np.sum(dz * z)),
                        ("dU.U", np.sum(dU * U))):
            assert abs(v - ref) <= 1e-10 * max(1.0, abs(ref)), (name, v, ref)


# ---------------------------------------------------------------- brute force
def _fd(f, a, eps=1e-6):
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        ap, am = a.copy(), a.copy()
        ap[i] += eps
        am[i] -= eps
        g[i] = (f(ap) - f(am)) / (2 * eps)
    return g


def pin_finite_differences(orc):
    """Central differences of L = <y, dy> in fp64 against every gradient."""
    rng = _rng(10)
    cases = [(2, 7, 12, 3, 1, 3), (2, 7, 12, 3, 3, 3), (1, 7, 12, 3, 4, 2),
             (1, 2, 4, 4, 2, 3)]                    # last one: T=2 < W=4
    for (B, T, D, W, H, R) in cases:
        G = D // H
        x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, B, T, G, W, std=0.5)
        z, U = _rand(rng, B, T, R), _rand(rng, R, G * W, std=0.5)
        for res, act in ((False, False), (True, False), (False, True), (True, True)):
            def Lh_x(xx): return np.sum(orc.headwise_fwd(xx, w, H, res, act) * dy)
            def Lh_w(ww): return np.sum(orc.headwise_fwd(x, ww, H, res, act) * dy)
            dx, dw = orc.headwise_bwd(x, w, dy, H, res, act)
            _close(dx, _fd(Lh_x, x), rtol=1e-7, atol=1e-7, what=f"fd dx {B,T,D,W,H}")
            _close(dw, _fd(Lh_w, w), rtol=1e-7, atol=1e-7, what=f"fd dw {B,T,D,W,H}")
            def Ll_z(zz): return np.sum(orc.lowrank_fwd(x, zz, U, W, H, res, act) * dy)
            def Ll_U(uu): return np.sum(orc.lowrank_fwd(x, z, uu, W, H, res, act) * dy)
            def Ll_x(xx): return np.sum(orc.lowrank_fwd(xx, z, U, W, H, res, act) * dy)
            dxl, dz, dU = orc.lowrank_bwd(x, z, U, dy, W, H, res, act)
            _close(dxl, _fd(Ll_x, x), rtol=1e-7, atol=1e-7, what="fd lowrank dx")
            _close(dz, _fd(Ll_z, z), rtol=1e-7, atol=1e-7, what="fd dz")
            _close(dU, _fd(Ll_U, U), rtol=1e-7, atol=1e-7, what="fd dU")


def pin_torch_autograd(orc):
    """An independent unfold + autograd formulation in fp64 agrees to rounding."""
    rng = _rng(11)
    for (B, T, D, W, H, R) in [(2, 33, 16, 4, 1, 5), (3, 20, 24, 3, 4, 16),
                               (1, 5, 8, 8, 8, 2)]:
        G = D // H
        x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, B, T, G, W, std=0.5)
        z, U = _rand(rng, B, T, R), _rand(rng, R, G * W, std=0.3)
        for res, act in ((False, False), (True, False), (False, True)):
            y, dx, dw = torch_ref.headwise_grads(x, w, dy, H, res, act)
            _close(orc.headwise_fwd(x, w, H, res, act), y, rtol=1e-12, atol=1e-12,
                   what="torch y")
            dxo, dwo = orc.headwise_bwd(x, w, dy, H, res, act)
            _close(dxo, dx, rtol=1e-12, atol=1e-12, what="torch dx")
            _close(dwo, dw, rtol=1e-12, atol=1e-12, what="torch dw")
            y, dx, dz, dU = torch_ref.lowrank_grads(x, z, U, dy, W, H, res, act)
            _close(orc.lowrank_fwd(x, z, U, W, H, res, act), y, rtol=1e-12, atol=1e-12,
                   what="torch lowrank y")
            dxo, dzo, dUo = orc.lowrank_bwd(x, z, U, dy, W, H, res, act)
            _close(dxo, dx, rtol=1e-12, atol=1e-12, what="torch lowrank dx")
            _close(dzo, dz, rtol=1e-12, atol=1e-12, what="torch dz")
            _close(dUo, dU, rtol=1e-12, atol=1e-12, what="torch dU")


# ---------------------------------------------------------------- sampled entry points
def pin_sampled_match_full(orc):
    """Row / column evaluators (used at full benchmark sizes) equal the full pass."""
    rng = _rng(12)
    B, T, D, W, H, R = 2, 19, 16, 4, 2, 5
    G = D // H
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    w = _rand(rng, B, T, G, W)
    z, U = _rand(rng, B, T, R), _rand(rng, R, G * W)
    rows = [0, 1, 2, 3, 18, 19, 20, 37]
    cols = [0, 1, 5, G * W - 1]
    for res, act in ((True, False), (False, True)):
        y = orc.headwise_fwd(x, w, H, res, act).reshape(B * T, D)
        _close(orc.headwise_fwd_rows(x, w, H, rows, res, act), y[rows],
               rtol=1e-14, atol=1e-14, what="fwd rows")
        dx, dw = orc.headwise_bwd(x, w, dy, H, res, act)
        dxr, dwr = orc.headwise_bwd_rows(x, w, dy, H, rows, res, act)
        _close(dxr, dx.reshape(B * T, D)[rows], rtol=1e-14, atol=1e-14, what="dx rows")
        _close(dwr, dw.reshape(B * T, G, W)[rows], rtol=1e-14, atol=1e-14, what="dw rows")
        yl = orc.lowrank_fwd(x, z, U, W, H, res, act).reshape(B * T, D)
        _close(orc.lowrank_fwd_rows(x, z, U, W, H, rows, res, act), yl[rows],
               rtol=1e-13, atol=1e-13, what="lowrank fwd rows")
        dxl, dz, dU = orc.lowrank_bwd(x, z, U, dy, W, H, res, act)
        dxr, dzr = orc.lowrank_bwd_rows(x, z, U, dy, W, H, rows, res, act)
        _close(dxr, dxl.reshape(B * T, D)[rows], rtol=1e-13, atol=1e-13, what="lr dx rows")
        _close(dzr, dz.reshape(B * T, R)[rows], rtol=1e-12, atol=1e-12, what="lr dz rows")
        _close(orc.lowrank_dU_cols(x, z, U, dy, W, H, cols, act), dU[:, cols],
               rtol=1e-12, atol=1e-12, what="dU cols")



# ---------------------------------------------------------------- streaming steps
def pin_decode_handworked(orc):
    """One step worked by hand (tests/golden/handworked.json, "decode")."""
    d = json.load(open(GOLDEN))["decode"]
    st, x = np.array(d["state"], float), np.array(d["x"], float)
    y, st2 = orc.headwise_decode(x, np.array(d["per_channel_w"], float), st, 1)
    _close(y, d["y"], what="decode y")
    _close(st2, d["state_after"], what="decode state")
    y, _ = orc.headwise_decode(x, np.array(d["per_channel_w"], float), st, 1, residual=True)
    _close(y, d["y_residual"], what="decode y+x")
    y, _ = orc.headwise_decode(x, np.array(d["tied_H2_w"], float), st, 2)
    _close(y, d["tied_H2_y"], what="decode tied y")
    y, _ = orc.lowrank_decode(x, np.array(d["lowrank_H2_R1_z"], float),
                              np.array(d["lowrank_H2_R1_U"], float), st, d["W"], 2)
    _close(y, d["tied_H2_y"], what="decode low-rank y")
    _close(orc.decode_state(np.array(d["prompt_short"], float), d["W"]), d["state_short"],
           what="state after a short prompt")
    _close(orc.decode_state(np.array(d["prompt_long"], float), d["W"]), d["state_long"],
           what="state after a long prompt")


def pin_decode_rolls_forward(orc):
    """Stepping token by token from an empty state reproduces the whole-sequence
    forward at every position, and the state is always the last W-1 inputs."""
    rng = _rng(31)
    for (B, T, D, W, H, res, act) in [(2, 9, 6, 3, 2, True, True), (1, 7, 4, 4, 1, False, False),
                                      (2, 5, 8, 1, 4, True, False)]:
        x = _rand(rng, B, T, D)
        w = _rand(rng, B, T, D // H, W, std=0.5)
        y = orc.headwise_fwd(x, w, H, residual=res, act=act)
        st = np.zeros((B, W - 1, D))
        for t in range(T):
            yt, st = orc.headwise_decode(x[:, t], w[:, t], st, H, residual=res, act=act)
            _close(yt, y[:, t], what=f"decode t={t}")
            _close(st, orc.decode_state(x[:, :t + 1], W), what=f"state t={t}")
        R = 3
        z = _rand(rng, B, T, R)
        U = _rand(rng, R, (D // H) * W, std=0.5)
        yl = orc.lowrank_fwd(x, z, U, W, H, residual=res, act=act)
        for T0 in sorted({0, 1, max(0, W - 2), T - 1}):
            st = orc.decode_state(x[:, :T0], W)
            yt, _ = orc.lowrank_decode(x[:, T0], z[:, T0], U, st, W, H, residual=res, act=act)
            _close(yt, yl[:, T0], what=f"low-rank decode after a {T0}-token prompt")

# ---------------------------------------------------------------- static filters
def _conv1d_static(x, w, H, residual, act, dy):
    """y and the gradients of <y, dy> through torch's depthwise conv1d (fp64):
    the (G, W) filter repeated over its H channels, taps flipped (conv1d's last
    weight meets the newest input), W-1 zeros of left padding."""
    B, T, D = x.shape
    W = w.shape[1]
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    kern = wt.repeat_interleave(H, dim=0).flip(-1)[:, None, :]       # (D, 1, W)
    s = F.conv1d(xt.transpose(1, 2), kern, padding=W - 1, groups=D)[:, :, :T].transpose(1, 2)
    y = F.silu(s) if act else s
    if residual:
        y = y + xt
    y.backward(torch.tensor(dy))
    return y.detach().numpy(), xt.grad.numpy(), wt.grad.numpy()


def pin_static_is_conv1d(orc):
    """The static forward and both gradients equal torch conv1d + autograd."""
    rng = _rng(40)
    for (B, T, D, W, H) in [(2, 13, 8, 4, 1), (3, 5, 12, 3, 4), (1, 3, 8, 6, 2),
                            (2, 9, 16, 1, 16)]:
        x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, D // H, W, std=0.5)
        for res, act in ((False, False), (True, False), (False, True), (True, True)):
            y, dx, dw = _conv1d_static(x, w, H, res, act, dy)
            _close(orc.static_fwd(x, w, H, res, act), y, what=f"static y {B,T,D,W,H}")
            dxo, dwo = orc.static_bwd(x, w, dy, H, res, act)
            _close(dxo, dx, what=f"static dx {B,T,D,W,H}")
            _close(dwo, dw, rtol=1e-11, atol=1e-11, what=f"static dw {B,T,D,W,H}")


def pin_static_is_broadcast_dynamic(orc):
    """A static filter is a dynamic one repeated over (b, t): same y and dx,
    and the static dw is the dynamic dw summed over every sequence and token."""
    rng = _rng(41)
    for (B, T, D, W, H) in [(2, 11, 8, 4, 2), (3, 4, 6, 5, 3)]:
        x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, D // H, W, std=0.5)
        wb = np.broadcast_to(w, (B, T) + w.shape).copy()
        for res, act in ((True, False), (False, True)):
            _close(orc.static_fwd(x, w, H, res, act), orc.headwise_fwd(x, wb, H, res, act),
                   what="static vs broadcast y")
            dxs, dws = orc.static_bwd(x, w, dy, H, res, act)
            dxh, dwh = orc.headwise_bwd(x, wb, dy, H, res, act)
            _close(dxs, dxh, what="static vs broadcast dx")
            _close(dws, dwh.sum(axis=(0, 1)), rtol=1e-11, atol=1e-11,
                   what="static dw vs summed dynamic dw")


def pin_static_finite_differences(orc):
    """Central differences of L = <y, dy> for dx and dw, T < W included."""
    rng = _rng(42)
    for (B, T, D, W, H) in [(2, 6, 6, 3, 3), (1, 2, 4, 4, 1)]:
        x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, D // H, W, std=0.5)
        for res, act in ((False, False), (True, True)):
            def Lx(xx): return np.sum(orc.static_fwd(xx, w, H, res, act) * dy)
            def Lw(ww): return np.sum(orc.static_fwd(x, ww, H, res, act) * dy)
            dx, dw = orc.static_bwd(x, w, dy, H, res, act)
            _close(dx, _fd(Lx, x), rtol=1e-7, atol=1e-7, what="fd static dx")
            _close(dw, _fd(Lw, w), rtol=1e-7, atol=1e-7, what="fd static dw")

# ---------------------------------------------------------------- packed documents
def _packing(rng, B, T, max_docs=4):
    """pos[b, t] for rows packed with documents of random lengths (>= 1)."""
    pos = np.zeros((B, T), dtype=np.int32)
    spans = []
    for b in range(B):
        cuts = sorted(rng.choice(np.arange(1, T), size=min(max_docs - 1, T - 1),
                                 replace=False)) if T > 1 else []
        edges = [0] + list(cuts) + [T]
        row = []
        for s0, e0 in zip(edges[:-1], edges[1:]):
            pos[b, s0:e0] = np.arange(e0 - s0)
            row.append((s0, e0))
        spans.append(row)
    return pos, spans


def pin_varlen_one_document_is_dense(orc):
    """pos[b, t] = t (one document per row) gives the dense results."""
    rng = _rng(50)
    B, T, D, W, H, R = 2, 9, 8, 4, 2, 3
    G = D // H
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    w = _rand(rng, B, T, G, W, std=0.5)
    z, U = _rand(rng, B, T, R), _rand(rng, R, G * W, std=0.5)
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    for res, act in ((True, False), (False, True)):
        _close(orc.headwise_fwd_vl(x, w, pos, H, res, act), orc.headwise_fwd(x, w, H, res, act),
               what="vl dense y")
        for a, b in zip(orc.headwise_bwd_vl(x, w, pos, dy, H, res, act),
                        orc.headwise_bwd(x, w, dy, H, res, act)):
            _close(a, b, what="vl dense head-wise grads")
        _close(orc.lowrank_fwd_vl(x, z, U, pos, W, H, res, act),
               orc.lowrank_fwd(x, z, U, W, H, res, act), what="vl dense low-rank y")
        for a, b in zip(orc.lowrank_bwd_vl(x, z, U, pos, dy, W, H, res, act),
                        orc.lowrank_bwd(x, z, U, dy, W, H, res, act)):
            _close(a, b, what="vl dense low-rank grads")


def pin_varlen_documents_are_independent(orc):
    """A packed row gives, document by document, what the dense operation gives
    on that document alone; dU is the sum of the documents' dU."""
    rng = _rng(51)
    for (B, T, D, W, H, R) in [(2, 17, 8, 4, 2, 3), (3, 12, 6, 3, 3, 2), (1, 9, 4, 5, 1, 4)]:
        G = D // H
        x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
        w = _rand(rng, B, T, G, W, std=0.5)
        z, U = _rand(rng, B, T, R), _rand(rng, R, G * W, std=0.5)
        pos, spans = _packing(rng, B, T)
        for res, act in ((True, False), (False, True), (True, True)):
            y = orc.headwise_fwd_vl(x, w, pos, H, res, act)
            dx, dw = orc.headwise_bwd_vl(x, w, pos, dy, H, res, act)
            yl = orc.lowrank_fwd_vl(x, z, U, pos, W, H, res, act)
            dxl, dz, dU = orc.lowrank_bwd_vl(x, z, U, pos, dy, W, H, res, act)
            dU_sum = np.zeros_like(U)
            for b in range(B):
                for s0, e0 in spans[b]:
                    sl = (slice(b, b + 1), slice(s0, e0))
                    xs, ws, dys, zs = x[sl], w[sl], dy[sl], z[sl]
                    _close(y[sl], orc.headwise_fwd(xs, ws, H, res, act), what="vl doc y")
                    ddx, ddw = orc.headwise_bwd(xs, ws, dys, H, res, act)
                    _close(dx[sl], ddx, what="vl doc dx")
                    _close(dw[sl], ddw, what="vl doc dw")
                    _close(yl[sl], orc.lowrank_fwd(xs, zs, U, W, H, res, act),
                           what="vl doc low-rank y")
                    ldx, ldz, ldU = orc.lowrank_bwd(xs, zs, U, dys, W, H, res, act)
                    _close(dxl[sl], ldx, what="vl doc low-rank dx")
                    _close(dz[sl], ldz, what="vl doc dz")
                    dU_sum += ldU
            _close(dU, dU_sum, rtol=1e-11, atol=1e-11, what="vl dU over documents")


def pin_varlen_finite_differences(orc):
    """Central differences of <y, dy> through packed rows."""
    rng = _rng(52)
    B, T, D, W, H, R = 2, 7, 4, 3, 2, 2
    G = D // H
    x, dy = _rand(rng, B, T, D), _rand(rng, B, T, D)
    w = _rand(rng, B, T, G, W, std=0.5)
    z, U = _rand(rng, B, T, R), _rand(rng, R, G * W, std=0.5)
    pos, _ = _packing(rng, B, T, max_docs=3)
    for res, act in ((False, False), (True, True)):
        dx, dw = orc.headwise_bwd_vl(x, w, pos, dy, H, res, act)
        _close(dx, _fd(lambda a: np.sum(orc.headwise_fwd_vl(a, w, pos, H, res, act) * dy), x),
               rtol=1e-7, atol=1e-7, what="fd vl dx")
        _close(dw, _fd(lambda a: np.sum(orc.headwise_fwd_vl(x, a, pos, H, res, act) * dy), w),
               rtol=1e-7, atol=1e-7, what="fd vl dw")
        _, dz, dU = orc.lowrank_bwd_vl(x, z, U, pos, dy, W, H, res, act)
        _close(dz, _fd(lambda a: np.sum(orc.lowrank_fwd_vl(x, a, U, pos, W, H, res, act) * dy),
                       z), rtol=1e-7, atol=1e-7, what="fd vl dz")
        _close(dU, _fd(lambda a: np.sum(orc.lowrank_fwd_vl(x, z, a, pos, W, H, res, act) * dy),
                       U), rtol=1e-7, atol=1e-7, what="fd vl dU")

# ---------------------------------------------------------------- generated filters
def pin_generated_filters(orc):
    """The fused generator equals the head-wise forward fed w = xh @ M (numpy
    matmul), with the filter columns laid out g*W + k."""
    rng = _rng(60)
    for (B, T, D, Dh, W, H) in [(2, 9, 16, 12, 4, 8), (1, 5, 8, 3, 2, 8), (2, 4, 12, 7, 3, 4)]:
        G = D // H
        x, xh = _rand(rng, B, T, D), _rand(rng, B, T, Dh)
        M = _rand(rng, Dh, G * W, std=0.3)
        w = (xh.reshape(-1, Dh) @ M).reshape(B, T, G, W)
        for res, act in ((False, False), (True, True)):
            _close(orc.headwise_gen_fwd(x, xh, M, H, res, act), orc.headwise_fwd(x, w, H, res, act),
                   what=f"generated filters {B,T,D,Dh,W,H}")
    # one token, one group: y = sum_k (xh M)[k] x_{t-k}, worked by hand
    x = np.array([[[1.0], [2.0]]])                 # B=1, T=2, D=1
    xh = np.array([[[1.0, 0.0], [0.5, 2.0]]])      # Dh=2
    M = np.array([[1.0, -1.0], [0.25, 3.0]])       # W=2: w_t = (xh_t0 + 0.25 xh_t1, -xh_t0 + 3 xh_t1)
    # t=0: w = (1, -1), y = 1*1 = 1;  t=1: w = (1, 5.5), y = 1*2 + 5.5*1 = 7.5
    _close(orc.headwise_gen_fwd(x, xh, M, 1), [[[1.0], [7.5]]], what="generated filters by hand")


ALL_PINS = [pin_handworked, pin_width_one_is_scale, pin_silu_values,
            pin_static_filter_is_conv1d, pin_causality, pin_linearity,
            pin_residual_is_tap0_shift, pin_tying_is_repeat, pin_lowrank_is_headwise,
            pin_adjoint, pin_euler, pin_finite_differences, pin_torch_autograd,
            pin_sampled_match_full, pin_decode_handworked, pin_decode_rolls_forward,
            pin_static_is_conv1d, pin_static_is_broadcast_dynamic,
            pin_static_finite_differences, pin_varlen_one_document_is_dense,
            pin_varlen_documents_are_independent, pin_varlen_finite_differences,
            pin_generated_filters]
