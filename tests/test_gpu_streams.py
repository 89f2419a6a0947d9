"""The library keeps no state between calls: calls queued on two streams at
once give the same bits as the same calls run one after another."""
import pytest
import torch

import dsc_inputs as di
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_two_streams_match_serial():
    import dynamic_short_causal_amd as dsc
    dev = gu.dev()
    x = di.randn((2, 300, 1024), 1.0, 9800, "bf16").to(dev)
    w = di.randn((2, 300, 64, 4), 0.5, 9801, "bf16").to(dev)
    z = di.randn((2, 300, 16), 1.0, 9802, "bf16").to(dev)
    U = di.randn((16, 1024 * 4), 0.125, 9803, "bf16").to(dev)
    dy = di.randn((2, 300, 1024), 1.0, 9804, "bf16").to(dev)
    ref_h = dsc.headwise_bwd(x, w, dy, 16, True, True)
    ref_l = dsc.lowrank_bwd(x, z, U, dy, 4, 1, True, False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            h = dsc.headwise_bwd(x, w, dy, 16, True, True, stream=s1)
        with torch.cuda.stream(s2):
            l = dsc.lowrank_bwd(x, z, U, dy, 4, 1, True, False, stream=s2)
        outs.append((h, l))
    torch.cuda.synchronize()
    for h, l in outs:
        assert all(torch.equal(a, b) for a, b in zip(h, ref_h))
        assert all(torch.equal(a, b) for a, b in zip(l, ref_l))
