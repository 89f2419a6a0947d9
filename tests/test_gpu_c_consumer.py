"""The library from plain C: dynamic_short_causal_amd/examples/c_consumer
(gcc, include/dsc.h, libdsc.so, the HIP runtime; no Python in the loop) must
produce the same bits as the Python binding on the same inputs, and those
match the oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

import dsc_inputs as di
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CONSUMER = os.path.join(ROOT, "dynamic_short_causal_amd", "examples", "c_consumer")


def bits(t):
    return t.contiguous().view(torch.int16).numpy().astype(np.uint16)


def test_c_program_matches_binding(orc, tmp_path):
    import dynamic_short_causal_amd as dsc
    assert os.path.exists(CONSUMER), "build the package first (it builds the C example)"
    B, T, D, W, H, R = 2, 77, 256, 4, 8, 16
    x = di.randn((B, T, D), 1.0, 9900, "bf16")
    w = di.randn((B, T, D // H, W), 0.5, 9901, "bf16")
    dy = di.randn((B, T, D), 1.0, 9902, "bf16")
    z = di.randn((B, T, R), 1.0, 9903, "bf16")
    U = di.randn((R, D * W), 0.125, 9904, "bf16")
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array([B, T, D, W, H, R], dtype=np.int64).tobytes())
        for t in (x, w, dy, z, U):
            f.write(bits(t).tobytes())
    gu.say("  running the C consumer")
    r = subprocess.run([CONSUMER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    gu.say("  " + r.stdout.strip() + r.stderr.strip())
    assert r.returncode == 0, r.stderr
    out = np.fromfile(tmp_path / "out.bin", dtype=np.uint16)
    n_act, n_w = B * T * D, B * T * (D // H) * W
    cy, cdx = out[:n_act], out[n_act:2 * n_act]
    cdw, cyl = out[2 * n_act:2 * n_act + n_w], out[2 * n_act + n_w:]
    dev = gu.dev()
    y = dsc.headwise_fwd(x.to(dev), w.to(dev), H, residual=True)
    dx, dw = dsc.headwise_bwd(x.to(dev), w.to(dev), dy.to(dev), H, residual=True)
    yl = dsc.lowrank_fwd(x.to(dev), z.to(dev), U.to(dev), W, 1, act=True)
    torch.cuda.synchronize()
    for name, c, p in (("y", cy, y), ("dx", cdx, dx), ("dw", cdw, dw), ("lowrank y", cyl, yl)):
        assert np.array_equal(c, bits(p.cpu()).ravel()), name
    X, Wt = gu.f64(x), gu.f64(w)
    gu.check("C y", y, orc.headwise_fwd(X, Wt, H, residual=True), torch.bfloat16, "y")
    gu.check("C lowrank y", yl, orc.lowrank_fwd(X, gu.f64(z), gu.f64(U), W, 1, act=True),
             torch.bfloat16, "y")
