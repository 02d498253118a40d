"""Gradients of decayed linear attention (fp64, CPU): the backward pass of the
recurrence S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t (allinfo.ai.kr post on
linear attention, "Key messages": matrix state with decay gates; the recurrence
is differentiated as written).

TEST INFRASTRUCTURE ONLY, like the rest of this package. The forward is the
recurrence step by step in plain PyTorch CPU ops (float64), and the gradients
are PyTorch's reverse-mode differentiation of it: no chunking, no closed-form
backward, nothing shared with the HIP library. Pinned in tests/pins.py against
central finite differences of oracle.gla_forward (oracle.c) and against the
forward itself.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).clone()
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def gla_forward_torch(q, k, v, g) -> torch.Tensor:
    """o [B,H,N,dv] of the recurrence, token by token (differentiable)."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = torch.zeros(B, H, dk, dv, dtype=q.dtype)
    outs = []
    for t in range(N):
        S = g[:, :, t, None, None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        outs.append((S * q[:, :, t, :, None]).sum(dim=2))
    return torch.stack(outs, dim=2)


def gla_backward(q, k, v, g, do):
    """Gradients (dq, dk, dv, dg) of sum(o * do) with o = gla_forward(q, k, v, g).
    q, k [B,H,N,dk], v and do [B,H,N,dv], g [B,H,N]; returns numpy float64."""
    q, k, v, g, do = map(_t, (q, k, v, g, do))
    for x in (q, k, v, g):
        x.requires_grad_(True)
    o = gla_forward_torch(q, k, v, g)
    o.backward(do)
    return tuple(x.grad.numpy() for x in (q, k, v, g))
