"""fp64 CPU oracle of the dynamic short causal convolution.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``dynamic_short_causal_amd``) never imports, links or calls it, and this
package imports nothing from there.

Every function takes float64 NumPy arrays in the layouts of ``dsc_oracle.c``
(x, y, dy, dx: (B,T,D); w, dw: (B,T,G,W); z, dz: (B,T,R); U, dU: (R,G*W)) and
returns float64 arrays.  The arithmetic lives in ``dsc_oracle.c``; this module
only marshals arguments.  See that file's header for the passages each
function follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_i64 = ctypes.c_int64
_int = ctypes.c_int
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)
_ip = ctypes.POINTER(ctypes.c_int32)


def _declare(lib):
    sigs = {
        "oracle_headwise_fwd": [_dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int, _int],
        "oracle_headwise_fwd_rows": [_dp, _dp, _i64, _i64, _i64, _int, _int, _int, _int,
                                     _i64, _lp, _dp],
        "oracle_headwise_bwd": [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _int, _int,
                                _int, _int],
        "oracle_headwise_bwd_rows": [_dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int,
                                     _int, _i64, _lp, _dp, _dp],
        "oracle_lowrank_w": [_dp, _dp, _dp, _i64, _i64, _i64, _int, _int],
        "oracle_lowrank_fwd": [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int,
                               _int, _int],
        "oracle_lowrank_bwd": [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _int,
                               _int, _int, _int, _int],
        "oracle_lowrank_fwd_rows": [_dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int,
                                    _int, _int, _i64, _lp, _dp],
        "oracle_lowrank_bwd_rows": [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _int, _int,
                                    _int, _int, _int, _i64, _lp, _dp, _dp],
        "oracle_lowrank_dU_cols": [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int,
                                   _int, _i64, _lp, _dp],
        "oracle_headwise_decode": [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _int, _int, _int,
                                   _int],
        "oracle_lowrank_decode": [_dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _int, _int,
                                  _int, _int, _int],
        "oracle_decode_state": [_dp, _dp, _i64, _i64, _i64, _int],
        "oracle_headwise_fwd_vl": [_dp, _dp, _ip, _dp, _i64, _i64, _i64, _int, _int, _int,
                                   _int],
        "oracle_headwise_bwd_vl": [_dp, _dp, _ip, _dp, _dp, _dp, _i64, _i64, _i64, _int, _int,
                                   _int, _int],
        "oracle_lowrank_fwd_vl": [_dp, _dp, _dp, _ip, _dp, _i64, _i64, _i64, _int, _int, _int,
                                  _int, _int],
        "oracle_lowrank_bwd_vl": [_dp, _dp, _dp, _ip, _dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                  _int, _int, _int, _int, _int],
        "oracle_headwise_gen_fwd": [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _int, _int,
                                    _int, _int],
        "oracle_static_fwd": [_dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int, _int],
        "oracle_static_bwd": [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _int, _int, _int,
                              _int],
        "oracle_num_threads": [],
        "oracle_set_num_threads": [_int],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _int if name == "oracle_num_threads" else None
    return lib


def load(path=None):
    """Load (building if absent) the oracle library; returns the ctypes handle."""
    global _LIB
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _declare(ctypes.CDLL(_build.LIB))
    return _LIB


def _c(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _p(a):
    return a.ctypes.data_as(_dp)


def _rows(rows):
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.ctypes.data_as(_lp)


class Oracle:
    """Thin marshalling wrapper around one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def num_threads(self):
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n):
        self.lib.oracle_set_num_threads(int(n))

    # ---- head-wise tying -------------------------------------------------
    def headwise_fwd(self, x, w, H, residual=False, act=False):
        x, w = _c(x), _c(w)
        B, T, D = x.shape
        W = w.shape[-1]
        assert w.shape == (B, T, D // H, W)
        y = np.empty_like(x)
        self.lib.oracle_headwise_fwd(_p(x), _p(w), _p(y), B, T, D, W, H,
                                     int(residual), int(act))
        return y

    def headwise_fwd_rows(self, x, w, H, rows, residual=False, act=False):
        x, w = _c(x), _c(w)
        B, T, D = x.shape
        W = w.shape[-1]
        r, rp = _rows(rows)
        out = np.empty((len(r), D))
        self.lib.oracle_headwise_fwd_rows(_p(x), _p(w), B, T, D, W, H, int(residual),
                                          int(act), len(r), rp, _p(out))
        return out

    def headwise_bwd(self, x, w, dy, H, residual=False, act=False):
        x, w, dy = _c(x), _c(w), _c(dy)
        B, T, D = x.shape
        W = w.shape[-1]
        dx = np.empty_like(x)
        dw = np.empty_like(w)
        self.lib.oracle_headwise_bwd(_p(x), _p(w), _p(dy), _p(dx), _p(dw), B, T, D, W,
                                     H, int(residual), int(act))
        return dx, dw

    def headwise_bwd_rows(self, x, w, dy, H, rows, residual=False, act=False):
        x, w, dy = _c(x), _c(w), _c(dy)
        B, T, D = x.shape
        W = w.shape[-1]
        r, rp = _rows(rows)
        dx = np.empty((len(r), D))
        dw = np.empty((len(r), D // H, W))
        self.lib.oracle_headwise_bwd_rows(_p(x), _p(w), _p(dy), B, T, D, W, H,
                                          int(residual), int(act), len(r), rp, _p(dx),
                                          _p(dw))
        return dx, dw

    # ---- low-rank --------------------------------------------------------
    def lowrank_w(self, z, U, W):
        z, U = _c(z), _c(U)
        B, T, R = z.shape
        GW = U.shape[1]
        assert U.shape[0] == R and GW % W == 0
        w = np.empty((B, T, GW // W, W))
        self.lib.oracle_lowrank_w(_p(z), _p(U), _p(w), B, T, GW // W, W, R)
        return w

    def lowrank_fwd(self, x, z, U, W, H, residual=False, act=False):
        x, z, U = _c(x), _c(z), _c(U)
        B, T, D = x.shape
        R = z.shape[-1]
        assert U.shape == (R, (D // H) * W)
        y = np.empty_like(x)
        self.lib.oracle_lowrank_fwd(_p(x), _p(z), _p(U), _p(y), B, T, D, W, H, R,
                                    int(residual), int(act))
        return y

    def lowrank_bwd(self, x, z, U, dy, W, H, residual=False, act=False):
        x, z, U, dy = _c(x), _c(z), _c(U), _c(dy)
        B, T, D = x.shape
        R = z.shape[-1]
        dx = np.empty_like(x)
        dz = np.empty_like(z)
        dU = np.empty_like(U)
        self.lib.oracle_lowrank_bwd(_p(x), _p(z), _p(U), _p(dy), _p(dx), _p(dz), _p(dU),
                                    B, T, D, W, H, R, int(residual), int(act))
        return dx, dz, dU

    def lowrank_fwd_rows(self, x, z, U, W, H, rows, residual=False, act=False):
        x, z, U = _c(x), _c(z), _c(U)
        B, T, D = x.shape
        R = z.shape[-1]
        r, rp = _rows(rows)
        out = np.empty((len(r), D))
        self.lib.oracle_lowrank_fwd_rows(_p(x), _p(z), _p(U), B, T, D, W, H, R,
                                         int(residual), int(act), len(r), rp, _p(out))
        return out

    def lowrank_bwd_rows(self, x, z, U, dy, W, H, rows, residual=False, act=False):
        x, z, U, dy = _c(x), _c(z), _c(U), _c(dy)
        B, T, D = x.shape
        R = z.shape[-1]
        r, rp = _rows(rows)
        dx = np.empty((len(r), D))
        dz = np.empty((len(r), R))
        self.lib.oracle_lowrank_bwd_rows(_p(x), _p(z), _p(U), _p(dy), B, T, D, W, H, R,
                                         int(residual), int(act), len(r), rp, _p(dx),
                                         _p(dz))
        return dx, dz

    def lowrank_dU_cols(self, x, z, U, dy, W, H, cols, act=False):
        x, z, U, dy = _c(x), _c(z), _c(U), _c(dy)
        B, T, D = x.shape
        R = z.shape[-1]
        c, cp = _rows(cols)
        out = np.empty((R, len(c)))
        self.lib.oracle_lowrank_dU_cols(_p(x), _p(z), _p(U), _p(dy), B, T, D, W, H, R,
                                        int(act), len(c), cp, _p(out))
        return out

    # ---- one-token steps (inference) -------------------------------------
    def headwise_decode(self, x, w, state, H, residual=False, act=False):
        """x (B,D), w (B,G,W), state (B,W-1,D) -> (y (B,D), new state)."""
        x, w, state = _c(x), _c(w), _c(state)
        B, D = x.shape
        W = w.shape[-1]
        assert w.shape == (B, D // H, W) and state.shape == (B, W - 1, D)
        y = np.empty_like(x)
        out = np.empty_like(state)
        self.lib.oracle_headwise_decode(_p(x), _p(w), _p(state), _p(out), _p(y), B, D, W,
                                        H, int(residual), int(act))
        return y, out

    def lowrank_decode(self, x, z, U, state, W, H, residual=False, act=False):
        """x (B,D), z (B,R), U (R,G*W), state (B,W-1,D) -> (y, new state)."""
        x, z, U, state = _c(x), _c(z), _c(U), _c(state)
        B, D = x.shape
        R = z.shape[-1]
        assert U.shape == (R, (D // H) * W) and state.shape == (B, W - 1, D)
        y = np.empty_like(x)
        out = np.empty_like(state)
        self.lib.oracle_lowrank_decode(_p(x), _p(z), _p(U), _p(state), _p(out), _p(y), B,
                                       D, W, H, R, int(residual), int(act))
        return y, out

    def decode_state(self, x, W):
        """State (B, W-1, D) after the prompt x (B, T, D)."""
        x = _c(x)
        B, T, D = x.shape
        st = np.empty((B, W - 1, D))
        self.lib.oracle_decode_state(_p(x), _p(st), B, T, D, W)
        return st

    # ---- static short convolution (one filter for all positions) ----------
    def static_fwd(self, x, w, H, residual=False, act=False):
        """x (B,T,D), w (G,W) -> y (B,T,D)."""
        x, w = _c(x), _c(w)
        B, T, D = x.shape
        assert w.shape[0] == D // H
        y = np.empty_like(x)
        self.lib.oracle_static_fwd(_p(x), _p(w), _p(y), B, T, D, w.shape[1], H,
                                   int(residual), int(act))
        return y

    def static_bwd(self, x, w, dy, H, residual=False, act=False):
        """-> (dx (B,T,D), dw (G,W))."""
        x, w, dy = _c(x), _c(w), _c(dy)
        B, T, D = x.shape
        assert w.shape[0] == D // H and dy.shape == x.shape
        dx = np.empty_like(x)
        dw = np.empty_like(w)
        self.lib.oracle_static_bwd(_p(x), _p(w), _p(dy), _p(dx), _p(dw), B, T, D, w.shape[1],
                                   H, int(residual), int(act))
        return dx, dw

    # ---- filter generation fused with the convolution --------------------
    def headwise_gen_fwd(self, x, xh, M, H, residual=False, act=False):
        """x (B,T,D), xh (B,T,Dh), M (Dh, G*W) -> y (B,T,D) with w = xh M."""
        x, xh, M = _c(x), _c(xh), _c(M)
        B, T, D = x.shape
        Dh = xh.shape[-1]
        G = D // H
        W = M.shape[1] // G
        assert xh.shape == (B, T, Dh) and M.shape == (Dh, G * W)
        y = np.empty_like(x)
        self.lib.oracle_headwise_gen_fwd(_p(x), _p(xh), _p(M), _p(y), B, T, D, Dh, W, H,
                                         int(residual), int(act))
        return y

    # ---- packed variable-length sequences ---------------------------------
    @staticmethod
    def _pos(pos, B, T):
        p = np.ascontiguousarray(pos, dtype=np.int32)
        assert p.shape == (B, T)
        return p, p.ctypes.data_as(_ip)

    def headwise_fwd_vl(self, x, w, pos, H, residual=False, act=False):
        """As headwise_fwd, tap k of token t only when k <= pos[b, t]."""
        x, w = _c(x), _c(w)
        B, T, D = x.shape
        p, pp = self._pos(pos, B, T)
        y = np.empty_like(x)
        self.lib.oracle_headwise_fwd_vl(_p(x), _p(w), pp, _p(y), B, T, D, w.shape[-1], H,
                                        int(residual), int(act))
        return y

    def headwise_bwd_vl(self, x, w, pos, dy, H, residual=False, act=False):
        x, w, dy = _c(x), _c(w), _c(dy)
        B, T, D = x.shape
        p, pp = self._pos(pos, B, T)
        dx, dw = np.empty_like(x), np.empty_like(w)
        self.lib.oracle_headwise_bwd_vl(_p(x), _p(w), pp, _p(dy), _p(dx), _p(dw), B, T, D,
                                        w.shape[-1], H, int(residual), int(act))
        return dx, dw

    def lowrank_fwd_vl(self, x, z, U, pos, W, H, residual=False, act=False):
        x, z, U = _c(x), _c(z), _c(U)
        B, T, D = x.shape
        p, pp = self._pos(pos, B, T)
        y = np.empty_like(x)
        self.lib.oracle_lowrank_fwd_vl(_p(x), _p(z), _p(U), pp, _p(y), B, T, D, W, H,
                                       z.shape[-1], int(residual), int(act))
        return y

    def lowrank_bwd_vl(self, x, z, U, pos, dy, W, H, residual=False, act=False):
        x, z, U, dy = _c(x), _c(z), _c(U), _c(dy)
        B, T, D = x.shape
        p, pp = self._pos(pos, B, T)
        dx, dz, dU = np.empty_like(x), np.empty_like(z), np.empty_like(U)
        self.lib.oracle_lowrank_bwd_vl(_p(x), _p(z), _p(U), pp, _p(dy), _p(dx), _p(dz),
                                       _p(dU), B, T, D, W, H, z.shape[-1], int(residual),
                                       int(act))
        return dx, dz, dU


_DEFAULT = None


def default():
    """The oracle built from ``dsc_oracle.c`` in this directory."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT

