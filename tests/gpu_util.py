"""Helpers shared by the GPU parity tests: device transfer, fp64 views of the
exact bits the GPU saw, the tolerance rule, and windowed oracle calls for
sampled rows at full benchmark sizes.

Tolerances (the GPU against the fp64 oracle on identical input bits):
  fp32, y, dx, dz : max |gpu - oracle| <= 1e-5 (absolute)
  fp32, dw, dU    : max |gpu - oracle| <= 1e-5 * max(1, max|oracle|)
  bf16            : max |gpu - oracle| / max|oracle| <= 2e-2 for y, dx and
                    5e-2 for dw, dz, dU
y and dx are sums of at most 2W products per element, dz a sum over the
filter slots of one token.  dw is a sum over the H channels of a group (and,
for static filters, over every token of every sequence), dU a sum over every
token: their magnitudes grow with the length of the sum, and fp32 rounding of
such a sum grows with its magnitude, so their bound scales with it.
"""
import sys

import numpy as np
import torch

TOL_BF16 = {"y": 2e-2, "dx": 2e-2, "dw": 5e-2, "dz": 5e-2, "dU": 5e-2}
TOL_F32 = 1e-5
F32_RELATIVE = ("dw", "dU")   # long sums: bound scales with max|oracle| above 1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def f64(t):
    """Exact fp64 copy of a (bf16 / fp32) tensor's values, on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def err(gpu, ref):
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0, 0.0
    a = float(np.max(np.abs(g - r)))
    m = float(np.max(np.abs(r)))
    return a, m


def check(name, gpu, ref, dtype, kind):
    a, m = err(gpu, ref)
    if dtype == torch.float32:
        lim = TOL_F32 * max(1.0, m) if kind in F32_RELATIVE else TOL_F32
        ok = a <= lim
        msg = f"{name}: max abs err {a:.3e} (limit {lim:.3e}, max|ref| {m:.3e})"
    else:
        rel = a / m if m > 0 else a
        ok = rel <= TOL_BF16[kind]
        msg = f"{name}: rel err {rel:.3e} (limit {TOL_BF16[kind]:.0e}, max|ref| {m:.3e})"
    say("   ", msg)
    assert ok, msg
    assert np.all(np.isfinite(f64(gpu) if isinstance(gpu, torch.Tensor) else gpu)), name


def windows(T, W, rows_bt):
    """For sampled (b, t), the token range [s, e) of sequence b that holds every
    input the outputs at t depend on (t-2(W-1) .. t+W-1, clipped to the
    sequence), and the local index of t in it.  Causality (pinned for the
    oracle) makes the result at t independent of tokens outside the range."""
    out = []
    for b, t in rows_bt:
        s = max(0, t - 2 * (W - 1))
        e = min(T, t + W)
        out.append((b, s, e, t - s))
    return out


def sample_rows(B, T, n, seed):
    """Sampled (b, t) pairs: sequence starts and ends, chunk edges, random."""
    rng = np.random.default_rng(seed)
    fixed = [(0, 0), (0, 1), (B - 1, T - 1), (B - 1, T - 2), (0, min(T - 1, 63)),
             (0, min(T - 1, 64)), (B // 2, min(T - 1, 1023)), (B // 2, min(T - 1, 1024))]
    rnd = [(int(rng.integers(B)), int(rng.integers(T))) for _ in range(n)]
    return sorted(set(fixed + rnd))
