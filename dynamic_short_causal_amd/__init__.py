"""Python binding of ``libdsc.so``, the gfx950 dynamic short causal convolution.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/dsc.h``.  PyTorch supplies device memory
and the current stream.  There is no CPU or PyTorch fallback: if the library
is missing, importing this package raises.

The functions named like the C entry points (``dsc_headwise_fwd`` ...) take
pre-allocated output tensors; ``headwise_fwd`` and friends allocate them with
``torch.empty`` and call the former.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsc.so")

DSC_OK, DSC_ERR_INVALID_ARG, DSC_ERR_UNSUPPORTED, DSC_ERR_WORKSPACE, DSC_ERR_HIP = range(5)
DSC_F32, DSC_BF16 = 0, 1
DSC_RESIDUAL, DSC_ACT_SILU = 1, 2

# every symbol declared in include/dsc.h
EXPORTS = ("dsc_version", "dsc_status_string", "dsc_last_error", "dsc_headwise_fwd",
           "dsc_headwise_bwd", "dsc_lowrank_fwd", "dsc_lowrank_bwd_workspace_bytes",
           "dsc_lowrank_bwd", "dsc_headwise_decode", "dsc_lowrank_decode",
           "dsc_decode_state", "dsc_static_fwd", "dsc_static_bwd_workspace_bytes",
           "dsc_static_bwd", "dsc_headwise_fwd_varlen", "dsc_headwise_bwd_varlen",
           "dsc_lowrank_fwd_varlen", "dsc_lowrank_bwd_varlen", "dsc_headwise_gen_fwd",
           "dsc_lowrank_bwd_noalloc")

# bytes of the library-owned buffer behind dsc_lowrank_bwd_noalloc (include/dsc.h)
NOALLOC_SCRATCH_BYTES = 128 << 20


class DscError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with dynamic_short_causal_amd/build.py "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    lib.dsc_version.restype = ci
    lib.dsc_status_string.restype = ctypes.c_char_p
    lib.dsc_status_string.argtypes = [ci]
    lib.dsc_last_error.restype = ctypes.c_char_p
    lib.dsc_headwise_fwd.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, cu, vp]
    lib.dsc_headwise_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, cu, vp]
    lib.dsc_lowrank_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, ci, cu, vp]
    lib.dsc_lowrank_bwd_workspace_bytes.argtypes = [i64, i64, i64, ci, ci, ci, ci]
    lib.dsc_lowrank_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.dsc_lowrank_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64,
                                    i64, ci, ci, ci, ci, cu, vp]
    lib.dsc_lowrank_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, ci, ci,
                                            ci, ci, cu, vp]
    lib.dsc_headwise_decode.argtypes = [vp, vp, vp, vp, i64, i64, ci, ci, ci, cu, vp]
    lib.dsc_lowrank_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, ci, ci, ci, ci, cu, vp]
    lib.dsc_decode_state.argtypes = [vp, vp, i64, i64, i64, ci, ci, vp]
    lib.dsc_static_fwd.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, cu, vp]
    lib.dsc_static_bwd_workspace_bytes.argtypes = [i64, i64, i64, ci, ci, ci]
    lib.dsc_static_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.dsc_static_bwd.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, ci,
                                   ci, ci, cu, vp]
    lib.dsc_headwise_gen_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, ci, cu, vp]
    lib.dsc_headwise_fwd_varlen.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, cu, vp]
    lib.dsc_headwise_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ci,
                                            cu, vp]
    lib.dsc_lowrank_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, ci,
                                           cu, vp]
    lib.dsc_lowrank_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                           i64, i64, i64, ci, ci, ci, ci, cu, vp]
    for name in ("dsc_headwise_fwd", "dsc_headwise_bwd", "dsc_lowrank_fwd",
                 "dsc_lowrank_bwd", "dsc_headwise_decode", "dsc_lowrank_decode",
                 "dsc_decode_state", "dsc_static_fwd", "dsc_static_bwd",
                 "dsc_headwise_fwd_varlen", "dsc_headwise_bwd_varlen",
                 "dsc_lowrank_fwd_varlen", "dsc_lowrank_bwd_varlen", "dsc_headwise_gen_fwd",
                 "dsc_lowrank_bwd_noalloc"):
        getattr(lib, name).restype = ci
    return lib


LIB = _load()


def _status_name(s):
    return LIB.dsc_status_string(int(s)).decode()


def version():
    return int(LIB.dsc_version())


def _check(status):
    if status != DSC_OK:
        raise DscError(status, LIB.dsc_last_error().decode())


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return DSC_BF16
    if t.dtype == torch.float32:
        return DSC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _flags(residual, act):
    return (DSC_RESIDUAL if residual else 0) | (DSC_ACT_SILU if act else 0)


def _need(t, name, shape, dtype):
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


# --------------------------------------------------------------- C-named calls
def dsc_headwise_fwd(x, w, y, H, residual=False, act=False, stream=None):
    B, T, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("w", w, (B, T, D // H, W)), ("y", y, (B, T, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_headwise_fwd(_ptr(x), _ptr(w), _ptr(y), B, T, D, W, H, _dtype(x),
                                _flags(residual, act), _stream(stream)))
    return y


def dsc_headwise_bwd(x, w, dy, dx, dw, H, residual=False, act=False, stream=None):
    B, T, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("w", w, (B, T, D // H, W)), ("dy", dy, (B, T, D)),
                    ("dx", dx, (B, T, D)), ("dw", dw, (B, T, D // H, W))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_headwise_bwd(_ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), B, T, D, W, H,
                                _dtype(x), _flags(residual, act), _stream(stream)))
    return dx, dw


def dsc_lowrank_fwd(x, z, U, y, W, H, residual=False, act=False, stream=None):
    B, T, D = x.shape
    R = z.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("z", z, (B, T, R)), ("U", U, (R, (D // H) * W)),
                    ("y", y, (B, T, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_lowrank_fwd(_ptr(x), _ptr(z), _ptr(U), _ptr(y), B, T, D, W, H, R,
                               _dtype(x), _flags(residual, act), _stream(stream)))
    return y


def dsc_lowrank_bwd_workspace_bytes(B, T, D, W, H, R, dtype):
    d = DSC_BF16 if dtype == torch.bfloat16 else DSC_F32
    return int(LIB.dsc_lowrank_bwd_workspace_bytes(B, T, D, W, H, R, d))


def dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, workspace, W, H, residual=False, act=False,
                    stream=None):
    B, T, D = x.shape
    R = z.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("z", z, (B, T, R)), ("U", U, (R, (D // H) * W)),
                    ("dy", dy, (B, T, D)), ("dx", dx, (B, T, D)), ("dz", dz, (B, T, R)),
                    ("dU", dU, (R, (D // H) * W))):
        _need(t, n, s, x.dtype)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.dsc_lowrank_bwd(_ptr(x), _ptr(z), _ptr(U), _ptr(dy), _ptr(dx), _ptr(dz),
                               _ptr(dU), _ptr(workspace), nbytes, B, T, D, W, H, R,
                               _dtype(x), _flags(residual, act), _stream(stream)))
    return dx, dz, dU


def dsc_lowrank_bwd_noalloc(x, z, U, dy, dx, dz, dU, W, H, residual=False, act=False,
                            stream=None):
    """dsc_lowrank_bwd with the library's own partial-sum buffer (no workspace)."""
    B, T, D = x.shape
    R = z.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("z", z, (B, T, R)), ("U", U, (R, (D // H) * W)),
                    ("dy", dy, (B, T, D)), ("dx", dx, (B, T, D)), ("dz", dz, (B, T, R)),
                    ("dU", dU, (R, (D // H) * W))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_lowrank_bwd_noalloc(_ptr(x), _ptr(z), _ptr(U), _ptr(dy), _ptr(dx), _ptr(dz),
                                       _ptr(dU), B, T, D, W, H, R, _dtype(x),
                                       _flags(residual, act), _stream(stream)))
    return dx, dz, dU


def dsc_headwise_decode(x, w, state, y, H, residual=False, act=False, stream=None):
    """One token: x (B, D), w (B, G, W); state (B, W-1, D) is advanced in place."""
    B, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, D)), ("w", w, (B, D // H, W)), ("state", state, (B, W - 1, D)),
                    ("y", y, (B, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_headwise_decode(_ptr(x), _ptr(w), _ptr(state), _ptr(y), B, D, W, H,
                                   _dtype(x), _flags(residual, act), _stream(stream)))
    return y


def dsc_lowrank_decode(x, z, U, state, y, W, H, residual=False, act=False, stream=None):
    """One token: x (B, D), z (B, R), U (R, G*W); state (B, W-1, D) advanced in place."""
    B, D = x.shape
    R = z.shape[-1]
    for n, t, s in (("x", x, (B, D)), ("z", z, (B, R)), ("U", U, (R, (D // H) * W)),
                    ("state", state, (B, W - 1, D)), ("y", y, (B, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_lowrank_decode(_ptr(x), _ptr(z), _ptr(U), _ptr(state), _ptr(y), B, D, W, H,
                                  R, _dtype(x), _flags(residual, act), _stream(stream)))
    return y


def dsc_decode_state(x, state, stream=None):
    """The (B, W-1, D) state left by a prompt x (B, T, D)."""
    B, T, D = x.shape
    W = state.shape[1] + 1
    for n, t, s in (("x", x, (B, T, D)), ("state", state, (B, W - 1, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_decode_state(_ptr(x), _ptr(state), B, T, D, W, _dtype(x), _stream(stream)))
    return state


def dsc_static_fwd(x, w, y, H, residual=False, act=False, stream=None):
    """Static filter w (G, W) for every sequence and token."""
    B, T, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("w", w, (D // H, W)), ("y", y, (B, T, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_static_fwd(_ptr(x), _ptr(w), _ptr(y), B, T, D, W, H, _dtype(x),
                              _flags(residual, act), _stream(stream)))
    return y


def dsc_static_bwd_workspace_bytes(B, T, D, W, H, dtype):
    d = DSC_BF16 if dtype == torch.bfloat16 else DSC_F32
    return int(LIB.dsc_static_bwd_workspace_bytes(B, T, D, W, H, d))


def dsc_static_bwd(x, w, dy, dx, dw, workspace, H, residual=False, act=False, stream=None):
    B, T, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("w", w, (D // H, W)), ("dy", dy, (B, T, D)),
                    ("dx", dx, (B, T, D)), ("dw", dw, (D // H, W))):
        _need(t, n, s, x.dtype)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.dsc_static_bwd(_ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(workspace),
                              nbytes, B, T, D, W, H, _dtype(x), _flags(residual, act),
                              _stream(stream)))
    return dx, dw


def _need_pos(pos, B, T):
    if pos.dtype != torch.int32:
        raise TypeError(f"pos has dtype {pos.dtype}, expected torch.int32")
    if tuple(pos.shape) != (B, T):
        raise ValueError(f"pos has shape {tuple(pos.shape)}, expected {(B, T)}")
    if not pos.is_contiguous() or not pos.is_cuda:
        raise ValueError("pos must be a contiguous device tensor")


def dsc_headwise_fwd_varlen(x, w, pos, y, H, residual=False, act=False, stream=None):
    """Packed rows: pos (B, T) int32 holds each token's index in its document."""
    B, T, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("w", w, (B, T, D // H, W)), ("y", y, (B, T, D))):
        _need(t, n, s, x.dtype)
    _need_pos(pos, B, T)
    _check(LIB.dsc_headwise_fwd_varlen(_ptr(x), _ptr(w), _ptr(pos), _ptr(y), B, T, D, W, H,
                                       _dtype(x), _flags(residual, act), _stream(stream)))
    return y


def dsc_headwise_bwd_varlen(x, w, pos, dy, dx, dw, H, residual=False, act=False, stream=None):
    B, T, D = x.shape
    W = w.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("w", w, (B, T, D // H, W)), ("dy", dy, (B, T, D)),
                    ("dx", dx, (B, T, D)), ("dw", dw, (B, T, D // H, W))):
        _need(t, n, s, x.dtype)
    _need_pos(pos, B, T)
    _check(LIB.dsc_headwise_bwd_varlen(_ptr(x), _ptr(w), _ptr(pos), _ptr(dy), _ptr(dx),
                                       _ptr(dw), B, T, D, W, H, _dtype(x), _flags(residual, act),
                                       _stream(stream)))
    return dx, dw


def dsc_lowrank_fwd_varlen(x, z, U, pos, y, W, H, residual=False, act=False, stream=None):
    B, T, D = x.shape
    R = z.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("z", z, (B, T, R)), ("U", U, (R, (D // H) * W)),
                    ("y", y, (B, T, D))):
        _need(t, n, s, x.dtype)
    _need_pos(pos, B, T)
    _check(LIB.dsc_lowrank_fwd_varlen(_ptr(x), _ptr(z), _ptr(U), _ptr(pos), _ptr(y), B, T, D,
                                      W, H, R, _dtype(x), _flags(residual, act),
                                      _stream(stream)))
    return y


def dsc_lowrank_bwd_varlen(x, z, U, pos, dy, dx, dz, dU, workspace, W, H, residual=False,
                           act=False, stream=None):
    B, T, D = x.shape
    R = z.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("z", z, (B, T, R)), ("U", U, (R, (D // H) * W)),
                    ("dy", dy, (B, T, D)), ("dx", dx, (B, T, D)), ("dz", dz, (B, T, R)),
                    ("dU", dU, (R, (D // H) * W))):
        _need(t, n, s, x.dtype)
    _need_pos(pos, B, T)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.dsc_lowrank_bwd_varlen(_ptr(x), _ptr(z), _ptr(U), _ptr(pos), _ptr(dy), _ptr(dx),
                                      _ptr(dz), _ptr(dU), _ptr(workspace), nbytes, B, T, D, W,
                                      H, R, _dtype(x), _flags(residual, act), _stream(stream)))
    return dx, dz, dU


def dsc_headwise_gen_fwd(x, xh, Mt, y, W, H, residual=False, act=False, stream=None):
    """Filters generated on chip: w = xh M with xh (B, T, Dh) and M given
    transposed, Mt (G*W, Dh) (a linear layer's weight layout)."""
    B, T, D = x.shape
    Dh = xh.shape[-1]
    for n, t, s in (("x", x, (B, T, D)), ("xh", xh, (B, T, Dh)), ("Mt", Mt, ((D // H) * W, Dh)),
                    ("y", y, (B, T, D))):
        _need(t, n, s, x.dtype)
    _check(LIB.dsc_headwise_gen_fwd(_ptr(x), _ptr(xh), _ptr(Mt), _ptr(y), B, T, D, Dh, W, H,
                                    _dtype(x), _flags(residual, act), _stream(stream)))
    return y


# --------------------------------------------------------------- allocating forms
def headwise_fwd(x, w, H, residual=False, act=False, stream=None):
    return dsc_headwise_fwd(x, w, torch.empty_like(x), H, residual, act, stream)


def headwise_bwd(x, w, dy, H, residual=False, act=False, stream=None):
    return dsc_headwise_bwd(x, w, dy, torch.empty_like(x), torch.empty_like(w), H, residual,
                            act, stream)


def lowrank_fwd(x, z, U, W, H, residual=False, act=False, stream=None):
    return dsc_lowrank_fwd(x, z, U, torch.empty_like(x), W, H, residual, act, stream)


def lowrank_workspace(x, z, W, H):
    B, T, D = x.shape
    n = dsc_lowrank_bwd_workspace_bytes(B, T, D, W, H, z.shape[-1], x.dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)


def lowrank_bwd(x, z, U, dy, W, H, residual=False, act=False, workspace=None, stream=None):
    if workspace is None:
        workspace = lowrank_workspace(x, z, W, H)
    return dsc_lowrank_bwd(x, z, U, dy, torch.empty_like(x), torch.empty_like(z),
                           torch.empty_like(U), workspace, W, H, residual, act, stream)


def decode_state(x, W, stream=None):
    B, T, D = x.shape
    return dsc_decode_state(x, torch.empty(B, W - 1, D, dtype=x.dtype, device=x.device), stream)


def headwise_decode(x, w, state, H, residual=False, act=False, stream=None):
    return dsc_headwise_decode(x, w, state, torch.empty_like(x), H, residual, act, stream)


def lowrank_decode(x, z, U, state, W, H, residual=False, act=False, stream=None):
    return dsc_lowrank_decode(x, z, U, state, torch.empty_like(x), W, H, residual, act, stream)


def static_fwd(x, w, H, residual=False, act=False, stream=None):
    return dsc_static_fwd(x, w, torch.empty_like(x), H, residual, act, stream)


def static_workspace(x, W, H):
    B, T, D = x.shape
    n = dsc_static_bwd_workspace_bytes(B, T, D, W, H, x.dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)


def static_bwd(x, w, dy, H, residual=False, act=False, workspace=None, stream=None):
    if workspace is None:
        workspace = static_workspace(x, w.shape[-1], H)
    return dsc_static_bwd(x, w, dy, torch.empty_like(x), torch.empty_like(w), workspace, H,
                          residual, act, stream)


def headwise_fwd_varlen(x, w, pos, H, residual=False, act=False, stream=None):
    return dsc_headwise_fwd_varlen(x, w, pos, torch.empty_like(x), H, residual, act, stream)


def headwise_bwd_varlen(x, w, pos, dy, H, residual=False, act=False, stream=None):
    return dsc_headwise_bwd_varlen(x, w, pos, dy, torch.empty_like(x), torch.empty_like(w), H,
                                   residual, act, stream)


def lowrank_fwd_varlen(x, z, U, pos, W, H, residual=False, act=False, stream=None):
    return dsc_lowrank_fwd_varlen(x, z, U, pos, torch.empty_like(x), W, H, residual, act, stream)


def lowrank_bwd_varlen(x, z, U, pos, dy, W, H, residual=False, act=False, workspace=None,
                       stream=None):
    if workspace is None:
        workspace = lowrank_workspace(x, z, W, H)
    return dsc_lowrank_bwd_varlen(x, z, U, pos, dy, torch.empty_like(x), torch.empty_like(z),
                                  torch.empty_like(U), workspace, W, H, residual, act, stream)


def headwise_gen_fwd(x, xh, Mt, W, H, residual=False, act=False, stream=None):
    return dsc_headwise_gen_fwd(x, xh, Mt, torch.empty_like(x), W, H, residual, act, stream)
