"""Thin Python binding of liblinmix.so (the C ABI in include/linmix.h).

Argument marshalling only: tensors are checked for the layout the ABI assumes
(device, dtype, shape, contiguity), turned into raw pointers and passed with the
caller's current HIP stream. Every step of the forward pass runs in the HIP
library. If the library is missing, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinmix.so")

LM_OK, LM_EINVAL, LM_EUNSUPPORTED, LM_EWORKSPACE, LM_EHIP = range(5)
LM_F32, LM_BF16 = 0, 1

_DT = {torch.float32: LM_F32, torch.bfloat16: LM_BF16}


class LinmixError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, _status_name(status), detail))


_lock = threading.Lock()
_lib = None

_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_SIGS = {
    "lm_abi_version": ([], ctypes.c_int),
    "lm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "lm_last_error": ([], ctypes.c_char_p),
    "gma_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, ctypes.c_int, _I64], ctypes.c_size_t),
    "gma_forward": ([_P] * 7 + [_I64] * 6 + [ctypes.c_int, ctypes.c_float, ctypes.c_int, _I64, _P,
                                             ctypes.c_size_t, _P], ctypes.c_int),
    "linattn_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, _I64], ctypes.c_size_t),
    "linattn_chunk_forward": ([_P] * 5 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P],
                              ctypes.c_int),
    "ccq_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, _I64], ctypes.c_size_t),
    "ccq_forward": ([_P] * 7 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "gma_forward_noalloc": ([_P] * 7 + [_I64] * 6 + [ctypes.c_int, ctypes.c_float, ctypes.c_int, _I64, _P],
                            ctypes.c_int),
    "gma_forward_state": ([_P] * 7 + [_I64] * 6 + [ctypes.c_float, ctypes.c_int, _I64, _P, _P, _P,
                                                   ctypes.c_size_t, _P], ctypes.c_int),
    "linattn_chunk_forward_state": ([_P] * 5 + [_I64] * 6 + [ctypes.c_int, _I64, _P, _P, _P, ctypes.c_size_t, _P],
                                    ctypes.c_int),
    "ccq_forward_state": ([_P] * 7 + [_I64] * 6 + [ctypes.c_int, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P],
                          ctypes.c_int),
    "gma_decode_step": ([_P] * 8 + [_I64] * 5 + [ctypes.c_float, ctypes.c_int, _P], ctypes.c_int),
    "linattn_decode_step": ([_P] * 6 + [_I64] * 4 + [ctypes.c_int, _P], ctypes.c_int),
    "ccq_decode_step": ([_P] * 8 + [_I64] * 5 + [ctypes.c_int, _P], ctypes.c_int),
    "linattn_vec_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, _I64], ctypes.c_size_t),
    "linattn_vec_forward": ([_P] * 5 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "linattn_vec_forward_state": ([_P] * 5 + [_I64] * 6 + [ctypes.c_int, _I64, _P, _P, _P, ctypes.c_size_t, _P],
                                  ctypes.c_int),
    "linattn_vec_decode_step": ([_P] * 6 + [_I64] * 4 + [ctypes.c_int, _P], ctypes.c_int),
    "linattn_backward_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, _I64], ctypes.c_size_t),
    "linattn_chunk_backward": ([_P] * 9 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "linattn_chunk_backward_state": ([_P] * 12 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P],
                                     ctypes.c_int),
    "gma_backward_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, ctypes.c_int], ctypes.c_size_t),
    "ccq_backward_workspace_bytes": ([_I64] * 6 + [ctypes.c_int], ctypes.c_size_t),
    "ccq_backward": ([_P] * 13 + [_I64] * 6 + [ctypes.c_int, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "gma_backward": ([_P] * 13 + [_I64] * 6 + [ctypes.c_int, ctypes.c_float, ctypes.c_int, _P, ctypes.c_size_t, _P],
                     ctypes.c_int),
    "deltanet_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, _I64], ctypes.c_size_t),
    "deltanet_chunk_forward": ([_P] * 6 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "deltanet_forward_state": ([_P] * 6 + [_I64] * 6 + [ctypes.c_int, _I64, _P, _P, _P, ctypes.c_size_t, _P],
                               ctypes.c_int),
    "ccq_deltanet_workspace_bytes": ([_I64] * 6 + [ctypes.c_int, _I64], ctypes.c_size_t),
    "ccq_deltanet_forward": ([_P] * 8 + [_I64] * 6 + [ctypes.c_int, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "ccq_deltanet_forward_state": ([_P] * 8 + [_I64] * 6 + [ctypes.c_int, _I64, _I64, _P, _P, _P, ctypes.c_size_t,
                                                           _P], ctypes.c_int),
}


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("HIP library %s is missing; build it with "
                                   "`python -m linear_attention_gmm_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGS.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = res
            _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().lm_status_string(s).decode()
    except Exception:  # library unavailable while formatting an error
        return str(s)


def _check(fn: str, status: int):
    if status != LM_OK:
        raise LinmixError(fn, status, lib().lm_last_error().decode())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace holds %d bytes, %d needed" % (workspace.numel() * workspace.element_size(), nbytes))
    return workspace


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError("q must be float32 or bfloat16 (got %s)" % t.dtype)
    return _DT[t.dtype]


def gma_workspace_bytes(B, H, N, d, K, dv, causal=True, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().gma_workspace_bytes(B, H, N, d, K, dv, int(bool(causal)), _DT[dtype], segments))


def gma_forward(q, k, v, mu, log_var, logit_pi, causal: bool = True, eps: float = 1e-6, segments: int = 0,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gaussian Mixture Attention forward. q, k [B,H,N,d]; v [B,H,N,dv] (float32 or
    bfloat16, all the same); mu, log_var [H,K,d] and logit_pi [H,K] float32.
    Returns out [B,H,N,dv] in the input dtype."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    dt = _dtype_code(q)
    pq = _dev(q, "q", q.dtype, (B, H, N, d))
    pk = _dev(k, "k", q.dtype, (B, H, N, d))
    pv = _dev(v, "v", q.dtype, (B, H, N, dv))
    pmu = _dev(mu, "mu", torch.float32, (H, K, d))
    plv = _dev(log_var, "log_var", torch.float32, (H, K, d))
    plp = _dev(logit_pi, "logit_pi", torch.float32, (H, K))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", q.dtype, (B, H, N, dv))
    nbytes = gma_workspace_bytes(B, H, N, d, K, dv, causal, q.dtype, segments)
    if nbytes == 0:
        _check("gma_workspace_bytes", lib().gma_forward(None, None, None, None, None, None, None, B, H, N, d, K,
                                                        dv, int(bool(causal)), float(eps), dt, segments, None,
                                                        0, None))
    ws = _workspace(nbytes, q.device, workspace)
    st = lib().gma_forward(pq, pk, pv, pmu, plv, plp, po, B, H, N, d, K, dv, int(bool(causal)), float(eps), dt,
                           segments, ws.data_ptr(), nbytes, _stream(q.device))
    _check("gma_forward", st)
    return out


def gma_forward_noalloc(q, k, v, mu, log_var, logit_pi, causal: bool = True, eps: float = 1e-6,
                        segments: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gma_forward on the library's fixed device scratch: no workspace is
    allocated (only `out`, when the caller passes none). Calls that overlap in
    time on one GPU share that scratch and must not be issued."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    dt = _dtype_code(q)
    pq = _dev(q, "q", q.dtype, (B, H, N, d))
    pk = _dev(k, "k", q.dtype, (B, H, N, d))
    pv = _dev(v, "v", q.dtype, (B, H, N, dv))
    pmu = _dev(mu, "mu", torch.float32, (H, K, d))
    plv = _dev(log_var, "log_var", torch.float32, (H, K, d))
    plp = _dev(logit_pi, "logit_pi", torch.float32, (H, K))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", q.dtype, (B, H, N, dv))
    st = lib().gma_forward_noalloc(pq, pk, pv, pmu, plv, plp, po, B, H, N, d, K, dv, int(bool(causal)), float(eps),
                                   dt, segments, _stream(q.device))
    _check("gma_forward_noalloc", st)
    return out


def linattn_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().linattn_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype], segments))


def ccq_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().ccq_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype], segments))


def _lin_common(q, k, v, g, out):
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    ptrs = (_dev(q, "q", q.dtype, (B, H, N, dk)), _dev(k, "k", q.dtype, (B, H, N, dk)),
            _dev(v, "v", q.dtype, (B, H, N, dv)), _dev(g, "g", torch.float32, (B, H, N)))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", q.dtype, (B, H, N, dv))
    return (B, H, N, dk, dv), ptrs, out, po


def linattn_chunk_forward(q, k, v, g, chunk: int = 64, segments: int = 0, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decayed linear attention S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.
    q, k [B,H,N,dk], v [B,H,N,dv] (float32 or bfloat16); g [B,H,N] float32."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    nbytes = linattn_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().linattn_chunk_forward(pq, pk, pv, pg, po, B, H, N, dk, dv, chunk, dt, segments,
                                     ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("linattn_chunk_forward", st)
    return out


def ccq_forward(q, k, v, g, w_lambda, b_lambda, chunk: int = 64, segments: int = 0,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Curvature-conditioned-query read over decayed linear attention.
    w_lambda [H,dk], b_lambda [H] float32."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    pw = _dev(w_lambda, "w_lambda", torch.float32, (H, dk))
    pb = _dev(b_lambda, "b_lambda", torch.float32, (H,))
    nbytes = ccq_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().ccq_forward(pq, pk, pv, pg, pw, pb, po, B, H, N, dk, dv, chunk, dt, segments,
                           ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("ccq_forward", st)
    return out


# ----------------------------------------------------------------------------- gated delta rule

def deltanet_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().deltanet_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype], segments))


def ccq_deltanet_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().ccq_deltanet_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype], segments))


def _beta(beta, shape) -> int:
    return _dev(beta, "beta", torch.float32, shape)


def deltanet_chunk_forward(q, k, v, g, beta, chunk: int = 64, segments: int = 0,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gated delta rule, plain read. beta [B,H,N] float32 step sizes."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    pb = _beta(beta, (B, H, N))
    nbytes = deltanet_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib().deltanet_chunk_forward(pq, pk, pv, pg, pb, po, B, H, N, dk, dv, chunk, dt, segments, ws.data_ptr(),
                                      nbytes, _stream(q.device))
    _check("deltanet_chunk_forward", st)
    return out


def deltanet_forward_state(q, k, v, g, beta, state_in: Optional[torch.Tensor] = None, chunk: int = 64,
                           segments: int = 0, out: Optional[torch.Tensor] = None,
                           state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gated delta rule continuing from state_in [B,H,dk*dv]. Returns (out, state_out)."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    pb = _beta(beta, (B, H, N))
    shape = (B, H, linattn_state_size(dk, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    state_out = _state_out(state_out, shape, q.device)
    pso = _state(state_out, "state_out", shape, q.device)
    nbytes = deltanet_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib().deltanet_forward_state(pq, pk, pv, pg, pb, po, B, H, N, dk, dv, chunk, dt, segments, psi, pso,
                                      ws.data_ptr(), nbytes, _stream(q.device))
    _check("deltanet_forward_state", st)
    return out, state_out


def ccq_deltanet_forward(q, k, v, g, beta, w_lambda, b_lambda, chunk: int = 64, segments: int = 0,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """CCQ read over the gated delta rule."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    pb = _beta(beta, (B, H, N))
    pw = _dev(w_lambda, "w_lambda", torch.float32, (H, dk))
    pbl = _dev(b_lambda, "b_lambda", torch.float32, (H,))
    nbytes = ccq_deltanet_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib().ccq_deltanet_forward(pq, pk, pv, pg, pb, pw, pbl, po, B, H, N, dk, dv, chunk, dt, segments,
                                    ws.data_ptr(), nbytes, _stream(q.device))
    _check("ccq_deltanet_forward", st)
    return out


def ccq_deltanet_forward_state(q, k, v, g, beta, w_lambda, b_lambda, state_in: Optional[torch.Tensor] = None,
                               t_in: int = 0, chunk: int = 64, segments: int = 0, out: Optional[torch.Tensor] = None,
                               state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """CCQ over the gated delta rule continuing from state_in [B,H,dk*dv+dk*dk+dk]
    that holds t_in tokens. Returns (out, state_out)."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    pb = _beta(beta, (B, H, N))
    pw = _dev(w_lambda, "w_lambda", torch.float32, (H, dk))
    pbl = _dev(b_lambda, "b_lambda", torch.float32, (H,))
    shape = (B, H, ccq_state_size(dk, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    state_out = _state_out(state_out, shape, q.device)
    pso = _state(state_out, "state_out", shape, q.device)
    nbytes = ccq_deltanet_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace)
    st = lib().ccq_deltanet_forward_state(pq, pk, pv, pg, pb, pw, pbl, po, B, H, N, dk, dv, chunk, dt, segments,
                                          int(t_in), psi, pso, ws.data_ptr(), nbytes, _stream(q.device))
    _check("ccq_deltanet_forward_state", st)
    return out, state_out


# ----------------------------------------------------------------------------- carried state

def gma_state_size(K: int, dv: int) -> int:
    """Floats per (b,h) of the GMA memory [Vtil (K x dv) | Z (K)]."""
    return K * dv + K


def linattn_state_size(dk: int, dv: int) -> int:
    """Floats per (b,h) of the decayed state S (dk x dv)."""
    return dk * dv


def ccq_state_size(dk: int, dv: int) -> int:
    """Floats per (b,h) of the CCQ state [S (dk x dv) | M (dk x dk) | m (dk)]."""
    return dk * dv + dk * dk + dk


def _state(t: Optional[torch.Tensor], name: str, shape, dev) -> int:
    if t is None:
        return None
    if t.device != dev:
        raise ValueError("%s must be on %s (got %s)" % (name, dev, t.device))
    return _dev(t, name, torch.float32, shape)


def _state_out(state_out, shape, dev):
    if state_out is None:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    return state_out


def gma_forward_state(q, k, v, mu, log_var, logit_pi, state_in: Optional[torch.Tensor] = None, eps: float = 1e-6,
                      segments: int = 0, out: Optional[torch.Tensor] = None,
                      state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Causal GMA forward continuing from state_in [B,H,K*dv+K] (None = empty
    prefix). Returns (out, state_out): the memory after the last token.
    state_out may be state_in itself (updated in place)."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    dt = _dtype_code(q)
    pq = _dev(q, "q", q.dtype, (B, H, N, d))
    pk = _dev(k, "k", q.dtype, (B, H, N, d))
    pv = _dev(v, "v", q.dtype, (B, H, N, dv))
    pmu = _dev(mu, "mu", torch.float32, (H, K, d))
    plv = _dev(log_var, "log_var", torch.float32, (H, K, d))
    plp = _dev(logit_pi, "logit_pi", torch.float32, (H, K))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", q.dtype, (B, H, N, dv))
    shape = (B, H, gma_state_size(K, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    state_out = _state_out(state_out, shape, q.device)
    pso = _state(state_out, "state_out", shape, q.device)
    nbytes = gma_workspace_bytes(B, H, N, d, K, dv, True, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().gma_forward_state(pq, pk, pv, pmu, plv, plp, po, B, H, N, d, K, dv, float(eps), dt, segments, psi,
                                 pso, ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("gma_forward_state", st)
    return out, state_out


def linattn_chunk_forward_state(q, k, v, g, state_in: Optional[torch.Tensor] = None, chunk: int = 64,
                                segments: int = 0, out: Optional[torch.Tensor] = None,
                                state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Decayed linear attention continuing from state_in [B,H,dk*dv] (None =
    zero). Returns (out, state_out), the state after the last token."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    shape = (B, H, linattn_state_size(dk, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    state_out = _state_out(state_out, shape, q.device)
    pso = _state(state_out, "state_out", shape, q.device)
    nbytes = linattn_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().linattn_chunk_forward_state(pq, pk, pv, pg, po, B, H, N, dk, dv, chunk, dt, segments, psi, pso,
                                           ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("linattn_chunk_forward_state", st)
    return out, state_out


def ccq_forward_state(q, k, v, g, w_lambda, b_lambda, state_in: Optional[torch.Tensor] = None, t_in: int = 0,
                      chunk: int = 64, segments: int = 0, out: Optional[torch.Tensor] = None,
                      state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """CCQ forward continuing from state_in [B,H,dk*dv+dk*dk+dk] that holds t_in
    tokens. Returns (out, state_out); the new state holds t_in + N tokens."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), out, po = _lin_common(q, k, v, g, out)
    pw = _dev(w_lambda, "w_lambda", torch.float32, (H, dk))
    pb = _dev(b_lambda, "b_lambda", torch.float32, (H,))
    shape = (B, H, ccq_state_size(dk, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    state_out = _state_out(state_out, shape, q.device)
    pso = _state(state_out, "state_out", shape, q.device)
    nbytes = ccq_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().ccq_forward_state(pq, pk, pv, pg, pw, pb, po, B, H, N, dk, dv, chunk, dt, segments, int(t_in), psi,
                                 pso, ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("ccq_forward_state", st)
    return out, state_out


def _dec_common(q, k, v, out):
    B, H, d = q.shape
    dv = v.shape[-1]
    ptrs = (_dev(q, "q", q.dtype, (B, H, d)), _dev(k, "k", q.dtype, (B, H, d)), _dev(v, "v", q.dtype, (B, H, dv)))
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    return (B, H, d, dv), ptrs, out, _dev(out, "out", q.dtype, (B, H, dv))


def gma_decode_step(q, k, v, mu, log_var, logit_pi, state, eps: float = 1e-6,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One causal GMA token per (b,h): q, k [B,H,d], v [B,H,dv]; state
    [B,H,K*dv+K] advanced in place. Returns out [B,H,dv]."""
    dt = _dtype_code(q)
    (B, H, d, dv), (pq, pk, pv), out, po = _dec_common(q, k, v, out)
    K = mu.shape[1]
    pmu = _dev(mu, "mu", torch.float32, (H, K, d))
    plv = _dev(log_var, "log_var", torch.float32, (H, K, d))
    plp = _dev(logit_pi, "logit_pi", torch.float32, (H, K))
    ps = _state(state, "state", (B, H, gma_state_size(K, dv)), q.device)
    st = lib().gma_decode_step(pq, pk, pv, pmu, plv, plp, po, ps, B, H, d, K, dv, float(eps), dt, _stream(q.device))
    _check("gma_decode_step", st)
    return out


def linattn_decode_step(q, k, v, g, state, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decayed-linear-attention token per (b,h): g [B,H]; state [B,H,dk*dv]
    advanced in place. Returns out [B,H,dv]."""
    dt = _dtype_code(q)
    (B, H, dk, dv), (pq, pk, pv), out, po = _dec_common(q, k, v, out)
    pg = _dev(g, "g", torch.float32, (B, H))
    ps = _state(state, "state", (B, H, linattn_state_size(dk, dv)), q.device)
    st = lib().linattn_decode_step(pq, pk, pv, pg, po, ps, B, H, dk, dv, dt, _stream(q.device))
    _check("linattn_decode_step", st)
    return out


def ccq_decode_step(q, k, v, g, w_lambda, b_lambda, state, t_prev: int,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One CCQ token per (b,h); state [B,H,dk*dv+dk*dk+dk] holds t_prev tokens
    and is advanced in place. Returns out [B,H,dv]."""
    dt = _dtype_code(q)
    (B, H, dk, dv), (pq, pk, pv), out, po = _dec_common(q, k, v, out)
    pg = _dev(g, "g", torch.float32, (B, H))
    pw = _dev(w_lambda, "w_lambda", torch.float32, (H, dk))
    pb = _dev(b_lambda, "b_lambda", torch.float32, (H,))
    ps = _state(state, "state", (B, H, ccq_state_size(dk, dv)), q.device)
    st = lib().ccq_decode_step(pq, pk, pv, pg, pw, pb, po, ps, B, H, dk, dv, int(t_prev), dt, _stream(q.device))
    _check("ccq_decode_step", st)
    return out


# ----------------------------------------------------------------------------- per-feature decay

def linattn_vec_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().linattn_vec_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype], segments))


def linattn_vec_forward(q, k, v, g, chunk: int = 64, segments: int = 0, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decayed linear attention with one decay per key feature:
    S_t = diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t. q, k [B,H,N,dk],
    v [B,H,N,dv] (float32 or bfloat16); g [B,H,N,dk] float32."""
    dt = _dtype_code(q)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    pq = _dev(q, "q", q.dtype, (B, H, N, dk))
    pk = _dev(k, "k", q.dtype, (B, H, N, dk))
    pv = _dev(v, "v", q.dtype, (B, H, N, dv))
    pg = _dev(g, "g", torch.float32, (B, H, N, dk))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", q.dtype, (B, H, N, dv))
    nbytes = linattn_vec_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().linattn_vec_forward(pq, pk, pv, pg, po, B, H, N, dk, dv, chunk, dt, segments,
                                   ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("linattn_vec_forward", st)
    return out


def linattn_vec_forward_state(q, k, v, g, state_in: Optional[torch.Tensor] = None, chunk: int = 64,
                              segments: int = 0, out: Optional[torch.Tensor] = None,
                              state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Per-feature decay continuing from state_in [B,H,dk*dv] (None = zero).
    Returns (out, state_out), the state after the last token."""
    dt = _dtype_code(q)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    pq = _dev(q, "q", q.dtype, (B, H, N, dk))
    pk = _dev(k, "k", q.dtype, (B, H, N, dk))
    pv = _dev(v, "v", q.dtype, (B, H, N, dv))
    pg = _dev(g, "g", torch.float32, (B, H, N, dk))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", q.dtype, (B, H, N, dv))
    shape = (B, H, linattn_state_size(dk, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    state_out = _state_out(state_out, shape, q.device)
    pso = _state(state_out, "state_out", shape, q.device)
    nbytes = linattn_vec_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().linattn_vec_forward_state(pq, pk, pv, pg, po, B, H, N, dk, dv, chunk, dt, segments, psi, pso,
                                         ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("linattn_vec_forward_state", st)
    return out, state_out


def linattn_vec_decode_step(q, k, v, g, state, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per (b,h) with one decay per key feature: g [B,H,dk]; state
    [B,H,dk*dv] advanced in place. Returns out [B,H,dv]."""
    dt = _dtype_code(q)
    (B, H, dk, dv), (pq, pk, pv), out, po = _dec_common(q, k, v, out)
    pg = _dev(g, "g", torch.float32, (B, H, dk))
    ps = _state(state, "state", (B, H, linattn_state_size(dk, dv)), q.device)
    st = lib().linattn_vec_decode_step(pq, pk, pv, pg, po, ps, B, H, dk, dv, dt, _stream(q.device))
    _check("linattn_vec_decode_step", st)
    return out


# ----------------------------------------------------------------------------- backward

def linattn_backward_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib().linattn_backward_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype], segments))


def linattn_chunk_backward(q, k, v, g, dout, chunk: int = 64, segments: int = 0,
                           workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dg) of sum(out * dout) for
    out = linattn_chunk_forward(q, k, v, g); dq, dk, dv in the input dtype, dg float32."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), _, _ = _lin_common(q, k, v, g, torch.empty_like(v))
    pdo = _dev(dout, "dout", q.dtype, (B, H, N, dv))
    dq, dkt, dvt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    nbytes = linattn_backward_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().linattn_chunk_backward(pq, pk, pv, pg, pdo, dq.data_ptr(), dkt.data_ptr(), dvt.data_ptr(),
                                      dg.data_ptr(), B, H, N, dk, dv, chunk, dt, segments,
                                      ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("linattn_chunk_backward", st)
    return dq, dkt, dvt, dg


def linattn_chunk_backward_state(q, k, v, g, dout, state_in: Optional[torch.Tensor] = None,
                                 dstate_out: Optional[torch.Tensor] = None, chunk: int = 64, segments: int = 0,
                                 workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dg, dstate_in) of sum(out * dout) + sum(S_out *
    dstate_out) for (out, S_out) = linattn_chunk_forward_state(q, k, v, g,
    state_in); states [B,H,dk*dv] float32 (None = zero / no such term)."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), _, _ = _lin_common(q, k, v, g, torch.empty_like(v))
    pdo = _dev(dout, "dout", q.dtype, (B, H, N, dv))
    shape = (B, H, linattn_state_size(dk, dv))
    psi = _state(state_in, "state_in", shape, q.device)
    pdso = _state(dstate_out, "dstate_out", shape, q.device)
    dq, dkt, dvt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dsi = torch.empty(shape, dtype=torch.float32, device=q.device)
    nbytes = linattn_backward_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype, segments)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().linattn_chunk_backward_state(pq, pk, pv, pg, pdo, psi, pdso, dq.data_ptr(), dkt.data_ptr(),
                                            dvt.data_ptr(), dg.data_ptr(), dsi.data_ptr(), B, H, N, dk, dv, chunk,
                                            dt, segments, ws.data_ptr() if ws is not None else None, nbytes,
                                            _stream(q.device))
    _check("linattn_chunk_backward_state", st)
    return dq, dkt, dvt, dg, dsi


def gma_backward_workspace_bytes(B, H, N, d, K, dv, causal=True, dtype=torch.bfloat16) -> int:
    return int(lib().gma_backward_workspace_bytes(B, H, N, d, K, dv, int(bool(causal)), _DT[dtype]))


def gma_backward(q, k, v, mu, log_var, logit_pi, dout, eps: float = 1e-6, causal: bool = True,
                 workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dmu, dlog_var, dlogit_pi) of sum(out * dout) for
    out = gma_forward(q, k, v, mu, log_var, logit_pi, causal, eps); dq, dk, dv in
    the input dtype, the parameter gradients float32."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    dt = _dtype_code(q)
    pq = _dev(q, "q", q.dtype, (B, H, N, d))
    pk = _dev(k, "k", q.dtype, (B, H, N, d))
    pv = _dev(v, "v", q.dtype, (B, H, N, dv))
    pdo = _dev(dout, "dout", q.dtype, (B, H, N, dv))
    pmu = _dev(mu, "mu", torch.float32, (H, K, d))
    plv = _dev(log_var, "log_var", torch.float32, (H, K, d))
    plp = _dev(logit_pi, "logit_pi", torch.float32, (H, K))
    dq, dk, dvt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dmu, dlv, dlp = torch.empty_like(mu), torch.empty_like(log_var), torch.empty_like(logit_pi)
    nbytes = gma_backward_workspace_bytes(B, H, N, d, K, dv, causal, q.dtype)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().gma_backward(pq, pk, pv, pmu, plv, plp, pdo, dq.data_ptr(), dk.data_ptr(), dvt.data_ptr(),
                            dmu.data_ptr(), dlv.data_ptr(), dlp.data_ptr(), B, H, N, d, K, dv, int(bool(causal)),
                            float(eps), dt, ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("gma_backward", st)
    return dq, dk, dvt, dmu, dlv, dlp


def ccq_backward_workspace_bytes(B, H, N, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    return int(lib().ccq_backward_workspace_bytes(B, H, N, dk, dv, chunk, _DT[dtype]))


def ccq_backward(q, k, v, g, w_lambda, b_lambda, dout, chunk: int = 64, workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dg, dw_lambda, db_lambda) of sum(out * dout) for
    out = ccq_forward(q, k, v, g, w_lambda, b_lambda); dq, dk, dv in the input
    dtype, the rest float32."""
    dt = _dtype_code(q)
    (B, H, N, dk, dv), (pq, pk, pv, pg), _, _ = _lin_common(q, k, v, g, torch.empty_like(v))
    pw = _dev(w_lambda, "w_lambda", torch.float32, (H, dk))
    pb = _dev(b_lambda, "b_lambda", torch.float32, (H,))
    pdo = _dev(dout, "dout", q.dtype, (B, H, N, dv))
    dq, dkt, dvt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dw, db = torch.empty_like(w_lambda), torch.empty_like(b_lambda)
    nbytes = ccq_backward_workspace_bytes(B, H, N, dk, dv, chunk, q.dtype)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    st = lib().ccq_backward(pq, pk, pv, pg, pw, pb, pdo, dq.data_ptr(), dkt.data_ptr(), dvt.data_ptr(),
                            dg.data_ptr(), dw.data_ptr(), db.data_ptr(), B, H, N, dk, dv, chunk, dt,
                            ws.data_ptr() if ws is not None else None, nbytes, _stream(q.device))
    _check("ccq_backward", st)
    return dq, dkt, dvt, dg, dw, db
