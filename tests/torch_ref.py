"""An independent fp64 PyTorch CPU formulation of the dynamic short convolution.

Used only to cross-check the C oracle.  It shares nothing with it: the causal
window comes from ``F.pad`` + ``Tensor.unfold``, tying from
``repeat_interleave``, the low-rank filters from ``matmul`` + ``reshape`` and
every gradient from autograd.
"""
import torch
import torch.nn.functional as F


def conv(x, w, H):
    """s[b,t,c] = sum_k w[b,t,c//H,k] * x[b,t-k,c] with zero left padding."""
    W = w.shape[-1]
    xp = F.pad(x, (0, 0, W - 1, 0))            # (B, T+W-1, D)
    win = xp.unfold(1, W, 1)                   # (B, T, D, W): win[..., j] = x[t+j-W+1]
    win = win.flip(-1)                         # win[..., k] = x[t-k]
    wc = w.repeat_interleave(H, dim=2)         # (B, T, D, W)
    return (wc * win).sum(-1)


def forward(x, w, H, residual=False, act=False):
    s = conv(x, w, H)
    y = F.silu(s) if act else s
    return y + x if residual else y


def headwise_grads(x, w, dy, H, residual=False, act=False):
    x = torch.as_tensor(x, dtype=torch.float64).clone().requires_grad_(True)
    w = torch.as_tensor(w, dtype=torch.float64).clone().requires_grad_(True)
    dy = torch.as_tensor(dy, dtype=torch.float64)
    y = forward(x, w, H, residual, act)
    y.backward(dy)
    return y.detach().numpy(), x.grad.numpy(), w.grad.numpy()


def lowrank_grads(x, z, U, dy, W, H, residual=False, act=False):
    x = torch.as_tensor(x, dtype=torch.float64).clone().requires_grad_(True)
    z = torch.as_tensor(z, dtype=torch.float64).clone().requires_grad_(True)
    U = torch.as_tensor(U, dtype=torch.float64).clone().requires_grad_(True)
    dy = torch.as_tensor(dy, dtype=torch.float64)
    B, T, D = x.shape
    w = (z @ U).reshape(B, T, D // H, W)
    y = forward(x, w, H, residual, act)
    y.backward(dy)
    return y.detach().numpy(), x.grad.numpy(), z.grad.numpy(), U.grad.numpy()
