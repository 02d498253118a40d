"""fp64 CPU oracle for the sequence-mixer forward pass.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It wraps
``oracle.c`` (plain C loops in float64, OpenMP over independent (b, h)
slices) through ctypes. It shares no code with the HIP library.

Inputs may be torch tensors or numpy arrays of any float dtype. They are
widened to float64 exactly (bf16 and fp32 values are representable), so the
oracle sees the same numbers as the GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def compile_library(src: str, out: str) -> str:
    """gcc -O2 with OpenMP; writes atomically."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-Wno-unused-parameter", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compiles oracle.c into oracle/liboracle.so when missing or stale."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
        compile_library(SOURCE, _LIB)
    return _LIB


_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int64


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_D)


class Oracle:
    """ctypes view of one build of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_gma_responsibilities.argtypes = [_D, _I, _I, _I, _D, _D, _D, _D]
        lib.oracle_gma_forward.argtypes = [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _I,
                                           ctypes.c_int, ctypes.c_double,
                                           ctypes.POINTER(ctypes.c_uint8), _D, _D]
        lib.oracle_gma_brute.argtypes = [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _I,
                                         ctypes.c_int, ctypes.c_double, _D]
        lib.oracle_gla_forward.argtypes = [_D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _D, _D]
        lib.oracle_ccq_forward.argtypes = [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _I, _D,
                                           _D]
        lib.oracle_glv_forward.argtypes = [_D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _D, _D]
        lib.oracle_deltanet_forward.argtypes = [_D, _D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _D,
                                                _D]
        lib.oracle_ccq_deltanet_forward.argtypes = [_D, _D, _D, _D, _D, _D, _D, _D, _I, _I, _I,
                                                    _I, _I, _I, _D, _D]
        lib.oracle_gla_chunkwise.argtypes = [_D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _I]
        lib.oracle_ccq_chunkwise.argtypes = [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I, _I, _I]
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def responsibilities(self, x, mu, log_var, logit_pi) -> np.ndarray:
        """Gamma [N,K] for one head: x [N,d], mu/log_var [K,d], logit_pi [K]."""
        x, mu, lv, lp = _f64(x), _f64(mu), _f64(log_var), _f64(logit_pi)
        N, d = x.shape
        K = mu.shape[0]
        out = np.empty((N, K))
        self.lib.oracle_gma_responsibilities(_p(x), N, d, K, _p(mu), _p(lv), _p(lp), _p(out))
        return out

    def gma_forward(self, q, k, v, mu, log_var, logit_pi, causal: bool = True, eps: float = 1e-6,
                    row_mask=None, state_in=None, return_state: bool = False):
        """Associative GMA. q, k [B,H,N,d]; v [B,H,N,dv]; mu, log_var [H,K,d];
        logit_pi [H,K]. row_mask [B,H,N] (optional): rows to read, others NaN.
        Causal only: state_in [B,H,K*dv+K] (optional) is the memory [Vtil | Z]
        before the first token; return_state also returns the memory after the
        last one (same layout)."""
        q, k, v, mu, lv, lp = map(_f64, (q, k, v, mu, log_var, logit_pi))
        B, H, N, d = q.shape
        dv = v.shape[-1]
        K = mu.shape[1]
        if (state_in is not None or return_state) and not causal:
            raise ValueError("the memory is carried by the causal form only")
        out = np.full((B, H, N, dv), np.nan)
        mask_p = None
        if row_mask is not None:
            rm = np.ascontiguousarray(np.asarray(row_mask, dtype=np.uint8).reshape(B, H, N))
            mask_p = rm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        sin = None if state_in is None else _f64(state_in).reshape(B, H, K * dv + K)
        sout = np.empty((B, H, K * dv + K)) if return_state else None
        self.lib.oracle_gma_forward(_p(q), _p(k), _p(v), _p(mu), _p(lv), _p(lp), _p(out), B, H, N,
                                    d, K, dv, int(causal), float(eps), mask_p, _p(sin), _p(sout))
        return (out, sout) if return_state else out

    def gma_brute(self, q, k, v, mu, log_var, logit_pi, causal: bool = True, eps: float = 1e-6,
                  return_affinity: bool = False):
        """Materialised-affinity GMA (small N). Returns out (and the affinity of
        the last slice when return_affinity)."""
        q, k, v, mu, lv, lp = map(_f64, (q, k, v, mu, log_var, logit_pi))
        B, H, N, d = q.shape
        dv = v.shape[-1]
        K = mu.shape[1]
        out = np.empty((B, H, N, dv))
        aff = np.empty((N, N)) if return_affinity else None
        self.lib.oracle_gma_brute(_p(q), _p(k), _p(v), _p(mu), _p(lv), _p(lp), _p(out), B, H, N, d,
                                  K, dv, int(causal), float(eps), _p(aff))
        return (out, aff) if return_affinity else out

    def gla_forward(self, q, k, v, g, state_in=None, return_state: bool = False):
        """Recurrent decayed linear attention: q, k [B,H,N,dk], v [B,H,N,dv], g [B,H,N].
        state_in [B,H,dk*dv] (optional): S before the first token; return_state
        also returns S after the last one."""
        q, k, v, g = map(_f64, (q, k, v, g))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        out = np.empty((B, H, N, dv))
        sin = None if state_in is None else _f64(state_in).reshape(B, H, dk * dv)
        sout = np.empty((B, H, dk * dv)) if return_state else None
        self.lib.oracle_gla_forward(_p(q), _p(k), _p(v), _p(g), _p(out), B, H, N, dk, dv, _p(sin),
                                    _p(sout))
        return (out, sout) if return_state else out

    def ccq_forward(self, q, k, v, g, w_lambda, b_lambda, t0: int = 0, state_in=None,
                    return_state: bool = False):
        """Recurrent CCQ read over decayed linear attention; w_lambda [H,dk], b_lambda [H].
        state_in [B,H,dk*dv+dk*dk+dk] (optional): [S | M | m] after t0 earlier
        tokens; return_state also returns the state after the last token."""
        q, k, v, g, w, b = map(_f64, (q, k, v, g, w_lambda, b_lambda))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        ss = dk * dv + dk * dk + dk
        if state_in is None and t0 != 0:
            raise ValueError("t0 counts the tokens held by state_in")
        out = np.empty((B, H, N, dv))
        sin = None if state_in is None else _f64(state_in).reshape(B, H, ss)
        sout = np.empty((B, H, ss)) if return_state else None
        self.lib.oracle_ccq_forward(_p(q), _p(k), _p(v), _p(g), _p(w), _p(b), _p(out), B, H, N, dk,
                                    dv, int(t0), _p(sin), _p(sout))
        return (out, sout) if return_state else out

    def glv_forward(self, q, k, v, g, state_in=None, return_state: bool = False):
        """Recurrent linear attention with a decay per key feature: g [B,H,N,dk].
        state_in [B,H,dk*dv] (optional): S before the first token; return_state
        also returns S after the last one."""
        q, k, v, g = map(_f64, (q, k, v, g))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        out = np.empty((B, H, N, dv))
        sin = None if state_in is None else _f64(state_in).reshape(B, H, dk * dv)
        sout = np.empty((B, H, dk * dv)) if return_state else None
        self.lib.oracle_glv_forward(_p(q), _p(k), _p(v), _p(g), _p(out), B, H, N, dk, dv, _p(sin),
                                    _p(sout))
        return (out, sout) if return_state else out

    def deltanet_forward(self, q, k, v, g, beta, state_in=None, return_state: bool = False):
        """Gated delta write rule, plain read: beta [B,H,N] step sizes; other
        arguments as for gla_forward (state S [B,H,dk*dv])."""
        q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        out = np.empty((B, H, N, dv))
        sin = None if state_in is None else _f64(state_in).reshape(B, H, dk * dv)
        sout = np.empty((B, H, dk * dv)) if return_state else None
        self.lib.oracle_deltanet_forward(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(out), B, H, N,
                                         dk, dv, _p(sin), _p(sout))
        return (out, sout) if return_state else out

    def ccq_deltanet_forward(self, q, k, v, g, beta, w_lambda, b_lambda, t0: int = 0,
                             state_in=None, return_state: bool = False):
        """CCQ read over the gated delta write rule; state [S | M | m] and t0 as
        for ccq_forward."""
        q, k, v, g, beta, w, b = map(_f64, (q, k, v, g, beta, w_lambda, b_lambda))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        ss = dk * dv + dk * dk + dk
        if state_in is None and t0 != 0:
            raise ValueError("t0 counts the tokens held by state_in")
        out = np.empty((B, H, N, dv))
        sin = None if state_in is None else _f64(state_in).reshape(B, H, ss)
        sout = np.empty((B, H, ss)) if return_state else None
        self.lib.oracle_ccq_deltanet_forward(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(w), _p(b),
                                             _p(out), B, H, N, dk, dv, int(t0), _p(sin),
                                             _p(sout))
        return (out, sout) if return_state else out

    def gla_chunkwise(self, q, k, v, g, chunk: int = 64) -> np.ndarray:
        q, k, v, g = map(_f64, (q, k, v, g))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        out = np.empty((B, H, N, dv))
        self.lib.oracle_gla_chunkwise(_p(q), _p(k), _p(v), _p(g), _p(out), B, H, N, dk, dv,
                                      int(chunk))
        return out

    def ccq_chunkwise(self, q, k, v, g, w_lambda, b_lambda, chunk: int = 64) -> np.ndarray:
        q, k, v, g, w, b = map(_f64, (q, k, v, g, w_lambda, b_lambda))
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        out = np.empty((B, H, N, dv))
        self.lib.oracle_ccq_chunkwise(_p(q), _p(k), _p(v), _p(g), _p(w), _p(b), _p(out), B, H, N,
                                      dk, dv, int(chunk))
        return out


_lock = threading.Lock()
_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from oracle.c (compiled on first use)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def num_threads() -> int:
    return get().num_threads()


def responsibilities(*a, **kw):
    return get().responsibilities(*a, **kw)


def gma_forward(*a, **kw):
    return get().gma_forward(*a, **kw)


def gma_brute(*a, **kw):
    return get().gma_brute(*a, **kw)


def gla_forward(*a, **kw):
    return get().gla_forward(*a, **kw)


def ccq_forward(*a, **kw):
    return get().ccq_forward(*a, **kw)


def glv_forward(*a, **kw):
    return get().glv_forward(*a, **kw)


def deltanet_forward(*a, **kw):
    return get().deltanet_forward(*a, **kw)


def ccq_deltanet_forward(*a, **kw):
    return get().ccq_deltanet_forward(*a, **kw)


def gla_chunkwise(*a, **kw):
    return get().gla_chunkwise(*a, **kw)


def ccq_chunkwise(*a, **kw):
    return get().ccq_chunkwise(*a, **kw)
