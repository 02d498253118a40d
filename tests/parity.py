"""Shared helpers for the GPU parity tests: metrics, tolerances, device moves.

Metrics (the tolerances come with the method's precision targets):
  * float32 inputs: max-rel = max_i |x_i - r_i| / max_i |r_i| over an output
    tensor, <= 1e-4 (an elementwise relative error is ill-posed because outputs
    cross zero);
  * bfloat16 inputs with float32 accumulation: rel-L2 = ||x - r||_2 / ||r||_2
    over the tensor, <= 2e-2.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

TOL_F32_MAXREL = 1e-4
TOL_BF16_RELL2 = 2e-2


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def max_rel(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


def rel_l2(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm((x - r).ravel()) / max(np.linalg.norm(r.ravel()), 1e-300))


def record(what: str, metric: str, value: float, tol: float, **extra):
    """Appends one comparison to the JSON-lines file named by LM_PARITY_RECORD
    (when set), so that a test run leaves every error value and its margin."""
    path = os.environ.get("LM_PARITY_RECORD")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    row = dict(test=test, what=what, metric=metric, value=float(value), tol=float(tol))
    row.update(extra)
    with open(path, "a") as f:
        f.write(json.dumps(row) + "\n")


def assert_close(x, r, dtype: str, what: str):
    """dtype 'f32' -> max-rel <= 1e-4; 'bf16' -> rel-L2 <= 2e-2. Both finite."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "%s: non-finite output" % what
    if dtype == "f32":
        e = max_rel(x, r)
        say("  %s: max-rel %.3e (tol %.0e)" % (what, e, TOL_F32_MAXREL))
        record(what, "max-rel", e, TOL_F32_MAXREL, elements=int(x.size))
        assert e <= TOL_F32_MAXREL, "%s: max-rel %.3e > %.0e" % (what, e, TOL_F32_MAXREL)
    else:
        e = rel_l2(x, r)
        mr = max_rel(x, r)
        say("  %s: rel-L2 %.3e (tol %.0e), max-rel %.3e" % (what, e, TOL_BF16_RELL2, mr))
        record(what, "rel-L2", e, TOL_BF16_RELL2, max_rel=mr, elements=int(x.size))
        assert e <= TOL_BF16_RELL2, "%s: rel-L2 %.3e > %.0e" % (what, e, TOL_BF16_RELL2)
    return e


def cuda(d: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
