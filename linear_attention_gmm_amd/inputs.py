"""Seeded synthetic inputs for the sequence-mixer forward pass.

This module only draws random numbers and shapes them into tensors; it holds
none of the mixers' arithmetic. Both the HIP library's callers (tests, bench)
and the fp64 oracle receive exactly the tensors built here.

Every tensor slice is drawn from its own counter-seeded stream,
``numpy.random.default_rng([cfg_id, tensor_id, b, h])`` (per-head parameters
use ``[cfg_id, tensor_id, h]``), in float64, then rounded to the config dtype by
torch (round-to-nearest-even). The oracle widens the rounded values back to
float64, so both sides see the same numbers.

Value distributions follow the workload descriptions the mixers are measured
on. ``N(m, s2)`` there names a mean and a *variance*.

* GMA: Q, K, V ~ N(0, 1); mu ~ N(0, 1); log sigma^2 = softplus(N(0, 0.5)) per
  dimension; mixing logits ~ N(0, 1); eps = 1e-6. Some configs scale Q and K
  by 1/sqrt(d) in float64 before rounding.
* Long-context GMA: keys come from a Gaussian mixture of ``K`` clusters
  (centres N(0, 1), within-cluster std 0.3, cluster drawn uniformly per
  token). The component means are set to the cluster centres so that
  responsibilities are peaked.
* Gated linear attention: Q, V ~ N(0, 1); K = z / ||z||_2 with z ~ N(0, 1);
  per-token scalar decay g = sigmoid(N(3, 1)) in float32.
* CCQ: as above, plus a query gate with w ~ N(0, 1/d_k) per head and bias
  b = -2.
* Gated delta rule: as gated linear attention, plus a per-token step size
  beta = sigmoid(N(0, 1)) in float32; keys always have unit norm (low-rank
  keys are normalised after they are drawn), so that the gradient step
  beta_t k_t k_t^T never amplifies the state.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

# tensor ids of the seeded streams
T_Q, T_K, T_V, T_MU, T_LOGVAR, T_LOGITPI, T_G, T_W, T_CENTRES, T_ASSIGN, T_BASIS, T_COEF, T_BETA = range(13)

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class GmaConfig:
    name: str
    cfg_id: int
    B: int
    H: int
    N: int
    d: int
    K: int
    dv: int
    dtype: str = "bf16"
    causal: bool = True
    qk_scale: bool = False  # multiply Q, K by 1/sqrt(d)
    mixture_keys: bool = False  # keys drawn from a K-cluster mixture, mu = centres
    eps: float = 1e-6

    def replace(self, **kw) -> "GmaConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class LinAttnConfig:
    name: str
    cfg_id: int
    B: int
    H: int
    N: int
    dk: int
    dv: int
    dtype: str = "bf16"
    chunk: int = 64
    g_one: bool = False  # decay identically 1
    g_logit_mean: float = 3.0  # decay g = sigmoid(N(g_logit_mean, 1))
    lowrank_keys: int = 0  # >0: keys = U z + 0.1 n with rank-r U (unnormalised)
    vector_gates: bool = False  # g [B,H,N,dk]: one decay per token and key feature
    gate_bias: float = -2.0
    delta: bool = False  # gated delta rule: beta [B,H,N], unit-norm keys

    def replace(self, **kw) -> "LinAttnConfig":
        return dataclasses.replace(self, **kw)


# The five measured workloads, plus the 16K-token GMA headline shape and the
# sensitised CCQ cases that make the curvature correction visible.
CONFIGS = {
    "gma_fp32_n256": GmaConfig("gma_fp32_n256", 1, B=1, H=1, N=256, d=32, K=16, dv=32, dtype="f32"),
    "gma_bf16_n4k": GmaConfig("gma_bf16_n4k", 2, B=4, H=8, N=4096, d=64, K=128, dv=64, qk_scale=True),
    "gla_bf16_n8k": LinAttnConfig("gla_bf16_n8k", 3, B=8, H=16, N=8192, dk=128, dv=128),
    "ccq_bf16_n16k": LinAttnConfig("ccq_bf16_n16k", 4, B=4, H=16, N=16384, dk=128, dv=128),
    "gma_bf16_n128k": GmaConfig("gma_bf16_n128k", 5, B=1, H=16, N=131072, d=128, K=256, dv=128,
                                mixture_keys=True),
    "gma_bf16_n16k": GmaConfig("gma_bf16_n16k", 6, B=4, H=8, N=16384, d=64, K=128, dv=64, qk_scale=True),
    "ccq_fp32_lowrank": LinAttnConfig("ccq_fp32_lowrank", 7, B=1, H=2, N=300, dk=32, dv=32, dtype="f32",
                                      lowrank_keys=4, gate_bias=2.0),
    "glv_bf16_n8k": LinAttnConfig("glv_bf16_n8k", 9, B=8, H=16, N=8192, dk=128, dv=128, vector_gates=True),
    "ccq_bf16_lowrank": LinAttnConfig("ccq_bf16_lowrank", 8, B=4, H=16, N=16384, dk=128, dv=128,
                                      lowrank_keys=4, gate_bias=2.0),
    # the gated delta rule on the 8K and 16K linear-attention shapes
    "deltanet_bf16_n8k": LinAttnConfig("deltanet_bf16_n8k", 10, B=8, H=16, N=8192, dk=128, dv=128, delta=True),
    "ccq_deltanet_bf16_n16k": LinAttnConfig("ccq_deltanet_bf16_n16k", 11, B=4, H=16, N=16384, dk=128, dv=128,
                                            delta=True),
    "ccq_deltanet_bf16_lowrank": LinAttnConfig("ccq_deltanet_bf16_lowrank", 12, B=4, H=16, N=16384, dk=128,
                                               dv=128, delta=True, lowrank_keys=4, gate_bias=2.0),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(x) for x in key])


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(_DTYPES[dtype])


def _softplus(x: np.ndarray) -> np.ndarray:
    # input-distribution recipe for log sigma^2 (not the mixer itself)
    return np.logaddexp(0.0, x)


def _per_slice(B: int, H: int, fn, max_workers: int = 8):
    """Runs fn(b, h) for every slice, threads across slices (numpy releases the GIL)."""
    jobs = [(b, h) for b in range(B) for h in range(H)]
    if len(jobs) == 1:
        return {jobs[0]: fn(*jobs[0])}
    with ThreadPoolExecutor(max_workers=min(max_workers, len(jobs))) as ex:
        res = list(ex.map(lambda bh: fn(*bh), jobs))
    return dict(zip(jobs, res))


def gma_params(cfg: GmaConfig) -> Dict[str, torch.Tensor]:
    """Per-head GMM parameters: mu [H,K,d], log_var [H,K,d], logit_pi [H,K], all float32."""
    H, K, d = cfg.H, cfg.K, cfg.d
    mu = np.empty((H, K, d))
    lv = np.empty((H, K, d))
    lp = np.empty((H, K))
    for h in range(H):
        if cfg.mixture_keys:
            mu[h] = _rng(cfg.cfg_id, T_CENTRES, h).standard_normal((K, d))
        else:
            mu[h] = _rng(cfg.cfg_id, T_MU, h).standard_normal((K, d))
        lv[h] = _softplus(_rng(cfg.cfg_id, T_LOGVAR, h).standard_normal((K, d)) * math.sqrt(0.5))
        lp[h] = _rng(cfg.cfg_id, T_LOGITPI, h).standard_normal(K)
    return {
        "mu": _to(mu, "f32"),
        "log_var": _to(lv, "f32"),
        "logit_pi": _to(lp, "f32"),
    }


def gma_inputs(cfg: GmaConfig, N: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """q, k [B,H,N,d] and v [B,H,N,dv] in cfg.dtype, plus the per-head parameters."""
    N = cfg.N if N is None else N
    B, H, d, dv = cfg.B, cfg.H, cfg.d, cfg.dv
    scale = 1.0 / math.sqrt(d) if cfg.qk_scale else 1.0
    params = gma_params(cfg)
    centres = params["mu"].double().numpy() if cfg.mixture_keys else None
    dt = _DTYPES[cfg.dtype]
    q = torch.empty((B, H, N, d), dtype=dt)
    k = torch.empty((B, H, N, d), dtype=dt)
    v = torch.empty((B, H, N, dv), dtype=dt)

    def one(b, h):
        qs = _rng(cfg.cfg_id, T_Q, b, h).standard_normal((N, d)) * scale
        if cfg.mixture_keys:
            m = _rng(cfg.cfg_id, T_ASSIGN, b, h).integers(0, cfg.K, size=N)
            ks = centres[h][m] + 0.3 * _rng(cfg.cfg_id, T_K, b, h).standard_normal((N, d))
        else:
            ks = _rng(cfg.cfg_id, T_K, b, h).standard_normal((N, d))
        ks = ks * scale
        vs = _rng(cfg.cfg_id, T_V, b, h).standard_normal((N, dv))
        q[b, h] = _to(qs, cfg.dtype)
        k[b, h] = _to(ks, cfg.dtype)
        v[b, h] = _to(vs, cfg.dtype)

    _per_slice(B, H, one)
    out = {"q": q, "k": k, "v": v, "eps": cfg.eps}
    out.update(params)
    return out


def linattn_inputs(cfg: LinAttnConfig, N: Optional[int] = None, ccq: bool = False) -> Dict[str, torch.Tensor]:
    """q, k [B,H,N,dk], v [B,H,N,dv] in cfg.dtype; g [B,H,N] float32 ([B,H,N,dk]
    with cfg.vector_gates, each entry drawn the same way); for CCQ also
    w_lambda [H,dk] and b_lambda [H] float32; with cfg.delta also beta [B,H,N]
    float32."""
    N = cfg.N if N is None else N
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    dt = _DTYPES[cfg.dtype]
    q = torch.empty((B, H, N, dk), dtype=dt)
    k = torch.empty((B, H, N, dk), dtype=dt)
    v = torch.empty((B, H, N, dv), dtype=dt)
    gshape = (N, dk) if cfg.vector_gates else (N,)
    g = torch.empty((B, H) + gshape, dtype=torch.float32)
    beta = torch.empty((B, H, N), dtype=torch.float32) if cfg.delta else None
    basis = None
    if cfg.lowrank_keys:
        r = cfg.lowrank_keys
        basis = [_rng(cfg.cfg_id, T_BASIS, h).standard_normal((dk, r)) / math.sqrt(dk) for h in range(H)]

    def one(b, h):
        qs = _rng(cfg.cfg_id, T_Q, b, h).standard_normal((N, dk))
        if cfg.lowrank_keys:
            z = _rng(cfg.cfg_id, T_COEF, b, h).standard_normal((N, cfg.lowrank_keys))
            ks = z @ basis[h].T + 0.1 * _rng(cfg.cfg_id, T_K, b, h).standard_normal((N, dk))
            if cfg.delta:
                ks = ks / np.linalg.norm(ks, axis=1, keepdims=True)
        else:
            z = _rng(cfg.cfg_id, T_K, b, h).standard_normal((N, dk))
            ks = z / np.linalg.norm(z, axis=1, keepdims=True)
        vs = _rng(cfg.cfg_id, T_V, b, h).standard_normal((N, dv))
        if cfg.g_one:
            gs = np.ones(gshape)
        else:
            gs = 1.0 / (1.0 + np.exp(-(cfg.g_logit_mean + _rng(cfg.cfg_id, T_G, b, h).standard_normal(gshape))))
        q[b, h] = _to(qs, cfg.dtype)
        k[b, h] = _to(ks, cfg.dtype)
        v[b, h] = _to(vs, cfg.dtype)
        g[b, h] = _to(gs, "f32")
        if cfg.delta:
            beta[b, h] = _to(1.0 / (1.0 + np.exp(-_rng(cfg.cfg_id, T_BETA, b, h).standard_normal(N))), "f32")

    _per_slice(B, H, one)
    out = {"q": q, "k": k, "v": v, "g": g}
    if cfg.delta:
        out["beta"] = beta
    if ccq:
        w = np.stack([_rng(cfg.cfg_id, T_W, h).standard_normal(dk) / math.sqrt(dk) for h in range(H)])
        out["w_lambda"] = _to(w, "f32")
        out["b_lambda"] = torch.full((H,), float(cfg.gate_bias), dtype=torch.float32)
    return out
