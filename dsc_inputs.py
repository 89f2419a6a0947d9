"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds the workload shapes and the random-number recipe only; it
contains none of the convolution's arithmetic.  Every tensor is drawn on the
CPU from ``torch.Generator().manual_seed(seed)`` as float32 ``randn * std`` and
then cast to the run dtype, so the GPU and the oracle see the same bits.

Seed scheme: ``seed = 1000 * case + tensor_id + 10 * W_offset`` with tensor ids
x=0, w=1, z=2, U=3, dy=4.

The shapes are those of the pages' placements: Q,K,V before RoPE with a
residual, the all-linear placement on an MLP intermediate, and the short conv
of a linear RNN (q,k,v conv channels).  The pages train on text corpora that
are not available here; Gaussian activations of the same shapes stand in for
them.
"""
from dataclasses import dataclass, replace

import torch

X, WT, Z, U, DY = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    case: int          # seed block
    variant: str       # "headwise" or "lowrank"
    dtype: str         # "f32" or "bf16"
    B: int
    T: int
    D: int
    W: int
    H: int
    R: int = 0
    residual: bool = False
    act: bool = False
    w_var: float = 0.25   # variance of the head-wise filters
    U_var: float = 0.0    # variance of U (low-rank)

    @property
    def G(self):
        return self.D // self.H

    @property
    def N(self):
        return self.B * self.T

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    # tiny oracle check: per-channel filters, fp32, forward
    "tiny_f32": Workload("tiny_f32", 1, "headwise", "f32", 1, 64, 64, 4, 1,
                         w_var=1.0 / 4),
    # Q,K,V (3 x 2048 channels) before RoPE, head-wise tying H=16, residual
    "qkv_headwise": Workload("qkv_headwise", 2, "headwise", "bf16", 8, 2048, 6144, 4, 16,
                             residual=True, w_var=0.25),
    # Q,K,V, low-rank R=16 generated on chip, per-channel filters, residual
    "qkv_lowrank": Workload("qkv_lowrank", 3, "lowrank", "bf16", 8, 2048, 6144, 4, 1,
                            R=16, residual=True, U_var=1.0 / (16 * 4)),
    # all-linear placement on an MLP intermediate, H=64, residual
    "mlp_headwise": Workload("mlp_headwise", 4, "headwise", "bf16", 4, 4096, 8192, 4, 64,
                             residual=True, w_var=0.25),
    # linear-RNN short conv replacement: low-rank R=16 with tying H=8, SiLU
    "rnn_lowrank_silu": Workload("rnn_lowrank_silu", 5, "lowrank", "bf16", 16, 4096,
                                 4608, 4, 8, R=16, act=True, U_var=1.0 / 64),
}


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def randn(shape, std, seed, dtype):
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch_dtype(dtype) if isinstance(dtype, str) else dtype)


def make(wl: Workload, seed_offset=0, need_dy=True):
    """CPU tensors for one workload: dict with x, dy and w (head-wise) or z, U."""
    base = 1000 * wl.case + seed_offset
    out = {"x": randn((wl.B, wl.T, wl.D), 1.0, base + X, wl.dtype)}
    if wl.variant == "headwise":
        out["w"] = randn((wl.B, wl.T, wl.G, wl.W), wl.w_var ** 0.5, base + WT, wl.dtype)
    else:
        out["z"] = randn((wl.B, wl.T, wl.R), 1.0, base + Z, wl.dtype)
        out["U"] = randn((wl.R, wl.G * wl.W), wl.U_var ** 0.5, base + U, wl.dtype)
    if need_dy:
        out["dy"] = randn((wl.B, wl.T, wl.D), 1.0, base + DY, wl.dtype)
    return out
