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


def gla_forward_torch(q, k, v, g, state_in=None, return_state: bool = False):
    """o [B,H,N,dv] of the recurrence, token by token (differentiable), from the
    state state_in [B,H,dk,dv] (zero when None); with return_state also the
    state after the last token."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = torch.zeros(B, H, dk, dv, dtype=q.dtype) if state_in is None else state_in
    outs = []
    for t in range(N):
        S = g[:, :, t, None, None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        outs.append((S * q[:, :, t, :, None]).sum(dim=2))
    o = torch.stack(outs, dim=2)
    return (o, S) if return_state else o


def gla_backward(q, k, v, g, do, state_in=None, dstate_out=None):
    """Gradients (dq, dk, dv, dg) of sum(o * do) with o = gla_forward(q, k, v, g).
    q, k [B,H,N,dk], v and do [B,H,N,dv], g [B,H,N]; returns numpy float64.
    With a carried state: the recurrence starts from state_in [B,H,dk,dv] (zero
    when None), the loss adds sum(S_out * dstate_out) for the state S_out after
    the last token, and the gradient of state_in is returned fifth."""
    q, k, v, g, do = map(_t, (q, k, v, g, do))
    with_state = state_in is not None or dstate_out is not None
    B, H, _, dk = q.shape
    dv = v.shape[-1]
    s0 = _t(state_in) if state_in is not None else torch.zeros(B, H, dk, dv, dtype=torch.float64)
    for x in (q, k, v, g, s0):
        x.requires_grad_(True)
    o, S = gla_forward_torch(q, k, v, g, state_in=s0, return_state=True)
    loss = (o * do).sum()
    if dstate_out is not None:
        loss = loss + (S * _t(dstate_out)).sum()
    loss.backward()
    out = tuple(x.grad.numpy() for x in (q, k, v, g))
    return out + (s0.grad.numpy(),) if with_state else out


def gma_forward_torch(q, k, v, mu, log_var, logit_pi, eps, causal=True) -> torch.Tensor:
    """O [B,H,N,dv] of Gaussian Mixture Attention ("Gaussian Mixture Attention:
    Linear-Time Sequence Mixing via Probabilistic Latent Routing", method: core
    mechanism and latent memory routing), differentiable. Responsibilities are
    the diagonal-Gaussian posteriors p(z = k | x) with priors softmax(logit_pi)
    and variances exp(log_var), written directly (log 2 pi included); the causal
    form accumulates the memory token by token and reads it after the write of
    the same token."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    var = torch.exp(log_var)                                        # [H,K,d]
    log_pi = logit_pi - torch.logsumexp(logit_pi, dim=-1, keepdim=True)

    def resp(x):                                                    # x [B,H,N,d] -> [B,H,N,K]
        diff = x[:, :, :, None, :] - mu[None, :, None, :, :]
        ll = log_pi[None, :, None, :] - 0.5 * (np.log(2 * np.pi) + log_var[None, :, None] + diff * diff
                                              / var[None, :, None]).sum(dim=-1)
        return torch.softmax(ll, dim=-1)

    gq, gk = resp(q), resp(k)
    if not causal:
        vt = torch.einsum("bhnk,bhnd->bhkd", gk, v)
        z = gk.sum(dim=2)
        return torch.einsum("bhnk,bhkd->bhnd", gq, vt) / (torch.einsum("bhnk,bhk->bhn", gq, z)[..., None] + eps)
    K = mu.shape[1]
    vt = torch.zeros(B, H, K, dv, dtype=q.dtype)
    z = torch.zeros(B, H, K, dtype=q.dtype)
    outs = []
    for t in range(N):
        vt = vt + gk[:, :, t, :, None] * v[:, :, t, None, :]
        z = z + gk[:, :, t]
        num = (gq[:, :, t, :, None] * vt).sum(dim=2)
        den = (gq[:, :, t] * z).sum(dim=-1, keepdim=True) + eps
        outs.append(num / den)
    return torch.stack(outs, dim=2)


def gma_backward(q, k, v, mu, log_var, logit_pi, do, eps, causal=True):
    """Gradients (dq, dk, dv, dmu, dlog_var, dlogit_pi) of sum(O * do) with
    O = gma_forward_torch(...); returns numpy float64."""
    q, k, v, mu, log_var, logit_pi, do = map(_t, (q, k, v, mu, log_var, logit_pi, do))
    xs = (q, k, v, mu, log_var, logit_pi)
    for x in xs:
        x.requires_grad_(True)
    o = gma_forward_torch(q, k, v, mu, log_var, logit_pi, eps, causal)
    o.backward(do)
    return tuple(x.grad.numpy() for x in xs)


def ccq_forward_torch(q, k, v, g, w, b) -> torch.Tensor:
    """o [B,H,N,dv] of the curvature-conditioned read over decayed linear
    attention ("Don't Read Everything: A Curvature-Conditioned Query for Linear
    Attention", section 2 Method), token by token (differentiable): running key
    sums M = sum k k^T and m = sum k, covariance Sigma_t = M/t - (m/t)(m/t)^T,
    lambda_t = sigmoid(w . q_t + b), q_clean = q_t - lambda_t Sigma_t q_t, state
    S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_clean."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = torch.zeros(B, H, dk, dv, dtype=q.dtype)
    M = torch.zeros(B, H, dk, dk, dtype=q.dtype)
    m = torch.zeros(B, H, dk, dtype=q.dtype)
    outs = []
    for t in range(N):
        kt, qt = k[:, :, t], q[:, :, t]
        M = M + kt[..., :, None] * kt[..., None, :]
        m = m + kt
        mu = m / (t + 1)
        sigma = M / (t + 1) - mu[..., :, None] * mu[..., None, :]
        lam = torch.sigmoid((w[None] * qt).sum(-1) + b[None])
        qc = qt - lam[..., None] * (sigma * qt[..., None, :]).sum(-1)
        S = g[:, :, t, None, None] * S + kt[..., :, None] * v[:, :, t, None, :]
        outs.append((S * qc[..., :, None]).sum(dim=2))
    return torch.stack(outs, dim=2)


def ccq_backward(q, k, v, g, w, b, do):
    """Gradients (dq, dk, dv, dg, dw, db) of sum(o * do) with
    o = ccq_forward_torch(q, k, v, g, w, b); returns numpy float64."""
    q, k, v, g, w, b, do = map(_t, (q, k, v, g, w, b, do))
    xs = (q, k, v, g, w, b)
    for x in xs:
        x.requires_grad_(True)
    o = ccq_forward_torch(q, k, v, g, w, b)
    o.backward(do)
    return tuple(x.grad.numpy() for x in xs)
