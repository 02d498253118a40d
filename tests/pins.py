"""Checks that tie the fp64 oracle to what the pages and the mathematics fix.

Each function takes an ``oracle.Oracle`` instance and raises AssertionError on
a mismatch. test_oracle_pins.py runs them against oracle.c. The mutation test
runs them against deliberately broken copies of oracle.c, so each plausible
mistake has to fail at least one pin.

Independent anchors used here, none of them the oracle's own code:
  * scipy's multivariate normal log-density and logsumexp (textbook GMM
    posterior) for the responsibilities;
  * the materialised N x N affinity written with numpy for the associative
    GMA form;
  * closed forms: K = 1 (running mean of V up to eps), identical components
    (rows of Gamma equal the priors);
  * hand-derived tiny examples (tests/golden/*.json);
  * numpy brute force with explicit decay products for gated linear attention;
  * numpy.cov(bias=True) for the running key covariance, itself checked to be
    the Hessian of the softmax log-partition at q = 0 (which fixes the 1/t);
  * reductions: lambda = 0 or constant keys turn CCQ into plain gated linear
    attention; a query orthogonal to the keys' span is not changed.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import logsumexp
from scipy.stats import multivariate_normal

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _gma_params(rng, H, K, d, spread=1.0):
    mu = rng.standard_normal((H, K, d)) * spread
    lv = np.logaddexp(0.0, rng.standard_normal((H, K, d)) * np.sqrt(0.5))
    lp = rng.standard_normal((H, K))
    return mu, lv, lp


def scipy_gamma(x, mu, lv, lp):
    """Textbook GMM posterior with scipy: log pi_k + log N(x; mu_k, diag(exp lv_k))."""
    K = mu.shape[0]
    logpi = lp - logsumexp(lp)
    cols = [multivariate_normal(mean=mu[c], cov=np.diag(np.exp(lv[c]))).logpdf(x) + logpi[c]
            for c in range(K)]
    lj = np.stack(cols, axis=-1).reshape(x.shape[0], K)
    return np.exp(lj - logsumexp(lj, axis=1, keepdims=True))


def numpy_gma_brute(q, k, v, mu, lv, lp, causal, eps):
    """Materialised affinity Gamma_Q Gamma_K^T (masked when causal), O = A V / (A 1 + eps)."""
    B, H, N, _ = q.shape
    out = np.empty(v.shape[:3] + (v.shape[-1],))
    for b in range(B):
        for h in range(H):
            gq = scipy_gamma(q[b, h], mu[h], lv[h], lp[h])
            gk = scipy_gamma(k[b, h], mu[h], lv[h], lp[h])
            a = gq @ gk.T
            if causal:
                a = np.tril(a)
            out[b, h] = (a @ v[b, h]) / (a.sum(1, keepdims=True) + eps)
    return out


def relerr(x, r):
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


# ---------------------------------------------------------------- GMA pins


def pin_gamma_scipy(orc):
    rng = _rng(101)
    for d, K in ((1, 1), (3, 5), (8, 16)):
        mu, lv, lp = _gma_params(rng, 1, K, d)
        x = rng.standard_normal((20, d)) * 1.5
        g = orc.responsibilities(x, mu[0], lv[0], lp[0])
        assert np.all(g >= 0)
        assert np.allclose(g.sum(1), 1.0, atol=1e-13, rtol=0)
        ref = scipy_gamma(x, mu[0], lv[0], lp[0])
        assert np.max(np.abs(g - ref)) < 1e-12, np.max(np.abs(g - ref))


def pin_gma_brute_numpy(orc):
    rng = _rng(102)
    B, H, N, d, K, dv = 2, 2, 33, 4, 5, 3
    mu, lv, lp = _gma_params(rng, H, K, d)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    for causal in (True, False):
        for eps in (1e-6, 0.3):
            ref = numpy_gma_brute(q, k, v, mu, lv, lp, causal, eps)
            got = orc.gma_forward(q, k, v, mu, lv, lp, causal=causal, eps=eps)
            assert relerr(got, ref) < 1e-12, (causal, eps, relerr(got, ref))
            got2 = orc.gma_brute(q, k, v, mu, lv, lp, causal=causal, eps=eps)
            assert relerr(got2, ref) < 1e-12, (causal, eps, relerr(got2, ref))


def pin_gma_k1_closed_form(orc):
    rng = _rng(103)
    B, H, N, d, dv = 1, 2, 40, 3, 4
    mu, lv, lp = _gma_params(rng, H, 1, d)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    eps = 0.25
    cnt = np.arange(1, N + 1)[:, None]
    got = orc.gma_forward(q, k, v, mu, lv, lp, causal=True, eps=eps)
    ref = np.cumsum(v, axis=2) / (cnt + eps)
    assert relerr(got, ref) < 1e-13
    got = orc.gma_forward(q, k, v, mu, lv, lp, causal=False, eps=eps)
    ref = np.broadcast_to(v.sum(2, keepdims=True) / (N + eps), v.shape)
    assert relerr(got, ref) < 1e-13


def pin_gma_identical_components(orc):
    rng = _rng(104)
    B, H, N, d, K, dv = 1, 1, 30, 3, 4, 2
    mu = np.broadcast_to(rng.standard_normal((1, 1, d)), (H, K, d)).copy()
    lv = np.broadcast_to(rng.standard_normal((1, 1, d)), (H, K, d)).copy()
    lp = rng.standard_normal((H, K))
    pi = np.exp(lp - logsumexp(lp, axis=1, keepdims=True))
    s = float((pi[0] ** 2).sum())
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    eps = 0.1
    cnt = np.arange(1, N + 1)[:, None]
    got = orc.gma_forward(q, k, v, mu, lv, lp, causal=True, eps=eps)
    ref = s * np.cumsum(v, axis=2) / (s * cnt + eps)
    assert relerr(got, ref) < 1e-12


def pin_gma_permutation(orc):
    rng = _rng(105)
    B, H, N, d, K, dv = 1, 1, 25, 3, 6, 2
    mu, lv, lp = _gma_params(rng, H, K, d)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    perm = rng.permutation(K)
    a = orc.gma_forward(q, k, v, mu, lv, lp)
    b = orc.gma_forward(q, k, v, mu[:, perm], lv[:, perm], lp[:, perm])
    assert relerr(a, b) < 1e-13


def pin_gma_prefix(orc):
    rng = _rng(106)
    B, H, N, d, K, dv = 1, 1, 40, 3, 5, 2
    mu, lv, lp = _gma_params(rng, H, K, d)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    full = orc.gma_forward(q, k, v, mu, lv, lp, causal=True)
    for i in (1, 7, 23):
        part = orc.gma_forward(q[:, :, :i], k[:, :, :i], v[:, :, :i], mu, lv, lp, causal=True)
        assert relerr(part, full[:, :, :i]) < 1e-14
    # the current token takes part in its own output (j <= i)
    v2 = v.copy()
    v2[:, :, 10] += 1.0
    changed = orc.gma_forward(q, k, v2, mu, lv, lp, causal=True)
    assert np.all(np.abs(changed[:, :, 10] - full[:, :, 10]) > 1e-9)
    assert relerr(changed[:, :, :10], full[:, :, :10]) < 1e-14


def pin_gma_affinity_structure(orc):
    rng = _rng(107)
    B, H, N, d, K, dv = 1, 1, 24, 3, 4, 2
    mu, lv, lp = _gma_params(rng, H, K, d)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    _, a = orc.gma_brute(q, k, v, mu, lv, lp, causal=False, return_affinity=True)
    assert np.all(a >= 0)
    assert np.linalg.matrix_rank(a, tol=1e-10) <= K
    # the masked causal affinity is the lower triangle of the same matrix
    _, ac = orc.gma_brute(q, k, v, mu, lv, lp, causal=True, return_affinity=True)
    assert np.max(np.abs(ac - np.tril(a))) < 1e-15


def pin_gma_golden(orc):
    with open(os.path.join(GOLDEN, "gma_two_components.json")) as f:
        case = json.load(f)
    got = orc.gma_forward(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]),
                          np.array(case["mu"]), np.array(case["log_var"]),
                          np.array(case["logit_pi"]), causal=case["causal"], eps=case["eps"])
    ref = np.array(case["expected_out"])
    assert relerr(got, ref) < 1e-12, (got, ref)


# ---------------------------------------------------------------- GLA pins


def numpy_gla_brute(q, k, v, g):
    """o_t = sum_{j<=t} (prod_{s=j+1..t} g_s) (q_t . k_j) v_j, explicit products."""
    B, H, N, _ = q.shape
    out = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            for t in range(N):
                for j in range(t + 1):
                    dec = np.prod(g[b, h, j + 1:t + 1])
                    out[b, h, t] += dec * (q[b, h, t] @ k[b, h, j]) * v[b, h, j]
    return out


def pin_gla_brute(orc):
    rng = _rng(201)
    B, H, N, dk, dv = 1, 2, 37, 5, 3
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.2, 1.0, (B, H, N))
    got = orc.gla_forward(q, k, v, g)
    assert relerr(got, numpy_gla_brute(q, k, v, g)) < 1e-12
    ones = np.ones((B, H, N))
    got = orc.gla_forward(q, k, v, ones)
    ref = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    assert relerr(got, ref) < 1e-12


def pin_gla_chunkwise(orc):
    rng = _rng(202)
    B, H, N, dk, dv = 2, 1, 70, 4, 6
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.3, 1.0, (B, H, N))
    rec = orc.gla_forward(q, k, v, g)
    for C in (1, 8, 16, 64, 128):
        assert relerr(orc.gla_chunkwise(q, k, v, g, chunk=C), rec) < 1e-12, C
    assert relerr(rec, numpy_gla_brute(q, k, v, g)) < 1e-12


# ---------------------------------------------------------------- CCQ pins


def numpy_ccq_brute(q, k, v, g, w, b):
    """o_t = S_t^T (q_t - lambda_t Cov_{<=t}[k] q_t) with np.cov(bias=True) and the
    brute-force state S_t = sum_{j<=t} prod(g_{j+1..t}) k_j v_j^T."""
    B, H, N, dk = q.shape
    out = np.zeros(v.shape)
    for bb in range(B):
        for h in range(H):
            for t in range(N):
                kk = k[bb, h, :t + 1]
                sig = np.cov(kk.T, bias=True).reshape(dk, dk) if t > 0 else np.zeros((dk, dk))
                lam = 1.0 / (1.0 + np.exp(-(w[h] @ q[bb, h, t] + b[h])))
                qc = q[bb, h, t] - lam * sig @ q[bb, h, t]
                S = np.zeros((dk, v.shape[-1]))
                for j in range(t + 1):
                    S += np.prod(g[bb, h, j + 1:t + 1]) * np.outer(kk[j], v[bb, h, j])
                out[bb, h, t] = S.T @ qc
    return out


def _ccq_case(rng, B=1, H=2, N=30, dk=4, dv=3, bias=1.0, center=0.0):
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk)) + center
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.3, 1.0, (B, H, N))
    w = rng.standard_normal((H, dk)) / np.sqrt(dk)
    b = np.full(H, bias)
    return q, k, v, g, w, b


def pin_ccq_numpy_cov(orc):
    rng = _rng(301)
    for center in (0.0, 2.0):
        q, k, v, g, w, b = _ccq_case(rng, center=center)
        got = orc.ccq_forward(q, k, v, g, w, b)
        ref = numpy_ccq_brute(q, k, v, g, w, b)
        assert relerr(got, ref) < 1e-11, (center, relerr(got, ref))
        # the correction is not negligible in this case
        assert relerr(orc.gla_forward(q, k, v, g), ref) > 1e-2


def pin_cov_is_logpartition_hessian(orc):
    """The pages state that the Hessian at q = 0 of log sum_{j<=t} exp(k_j^T q) is
    the running key covariance; numpy.cov(bias=True), used above, must be it."""
    rng = _rng(302)
    dk, t = 4, 9
    kk = rng.standard_normal((t, dk)) + 0.5
    f = lambda qq: logsumexp(kk @ qq)
    h = 1e-4
    hess = np.empty((dk, dk))
    for a in range(dk):
        for c in range(dk):
            ea = np.eye(dk)[a] * h
            ec = np.eye(dk)[c] * h
            hess[a, c] = (f(ea + ec) - f(ea - ec) - f(-ea + ec) + f(-ea - ec)) / (4 * h * h)
    assert np.max(np.abs(hess - np.cov(kk.T, bias=True))) < 1e-6
    assert np.max(np.abs(hess - np.cov(kk.T, bias=False))) > 1e-2


def pin_ccq_reductions(orc):
    rng = _rng(303)
    q, k, v, g, w, b = _ccq_case(rng)
    gla = orc.gla_forward(q, k, v, g)
    # gate closed: lambda = sigmoid(-1e4) = 0 exactly
    assert relerr(orc.ccq_forward(q, k, v, g, w, np.full(2, -1e4)), gla) < 1e-14
    # constant keys: covariance is zero
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()
    assert relerr(orc.ccq_forward(q, kc, v, g, w, b), orc.gla_forward(q, kc, v, g)) < 1e-12
    # query orthogonal to the span of the keys: Sigma q = 0, q unchanged
    k2 = k.copy()
    k2[..., 2:] = 0.0
    q2 = q.copy()
    q2[..., :2] = 0.0
    assert relerr(orc.ccq_forward(q2, k2, v, g, w, np.full(2, 3.0)),
                  orc.gla_forward(q2, k2, v, g)) < 1e-12


def pin_ccq_chunkwise(orc):
    rng = _rng(304)
    q, k, v, g, w, b = _ccq_case(rng, N=45, bias=0.5)
    rec = orc.ccq_forward(q, k, v, g, w, b)
    for C in (1, 4, 16, 64):
        assert relerr(orc.ccq_chunkwise(q, k, v, g, w, b, chunk=C), rec) < 1e-11, C


def pin_ccq_golden(orc):
    with open(os.path.join(GOLDEN, "ccq_two_keys.json")) as f:
        case = json.load(f)
    args = [np.array(case[x]) for x in ("q", "k", "v", "g", "w_lambda", "b_lambda")]
    got = orc.ccq_forward(*args)
    ref = np.array(case["expected_out"])
    assert relerr(got, ref) < 1e-14, (got, ref)


def pin_gma_state(orc):
    """The causal memory after a prefix is Gamma_K^T [V | 1] over that prefix
    (scipy posterior), and reading on from it gives the rows of the whole
    sequence (numpy brute force), one token at a time included."""
    rng = _rng(401)
    B, H, N, d, K, dv, eps = 1, 2, 23, 4, 3, 2, 1e-3
    mu, lv, lp = _gma_params(rng, H, K, d)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    ref = numpy_gma_brute(q, k, v, mu, lv, lp, True, eps)
    for a in (9, N - 1):
        o1, st = orc.gma_forward(q[:, :, :a], k[:, :, :a], v[:, :, :a], mu, lv, lp, True, eps,
                                 return_state=True)
        for h in range(H):
            gam = scipy_gamma(k[0, h, :a], mu[h], lv[h], lp[h])
            want = np.concatenate([(gam.T @ v[0, h, :a]).ravel(), gam.sum(0)])
            assert relerr(st[0, h], want) < 1e-12
        o2, st2 = orc.gma_forward(q[:, :, a:], k[:, :, a:], v[:, :, a:], mu, lv, lp, True, eps,
                                  state_in=st, return_state=True)
        assert relerr(np.concatenate([o1, o2], 2), ref) < 1e-12
        # every responsibility row sums to 1: the normaliser mass is the token count
        assert abs(st2[0, 0, K * dv:].sum() - N) < 1e-12


def pin_gla_state(orc):
    """S after a prefix is sum_j prod(g_{j+1..a}) k_j v_j^T; continuing from it
    (also one token at a time) gives the brute-force rows of the whole sequence."""
    rng = _rng(402)
    B, H, N, dk, dv = 1, 2, 21, 4, 3
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.2, 1.0, (B, H, N))
    ref = numpy_gla_brute(q, k, v, g)
    for a in (8, N - 1):
        o1, st = orc.gla_forward(q[:, :, :a], k[:, :, :a], v[:, :, :a], g[:, :, :a], return_state=True)
        for h in range(H):
            want = sum(np.prod(g[0, h, j + 1:a]) * np.outer(k[0, h, j], v[0, h, j]) for j in range(a))
            assert relerr(st[0, h], want.ravel()) < 1e-12
        o2 = orc.gla_forward(q[:, :, a:], k[:, :, a:], v[:, :, a:], g[:, :, a:], state_in=st)
        assert relerr(np.concatenate([o1, o2], 2), ref) < 1e-12


def pin_ccq_state(orc):
    """The CCQ state after a prefix holds S (as for plain decay), M = K^T K and
    m = K^T 1 of that prefix; continuing from it with the token count gives the
    brute-force rows (np.cov over the whole prefix) of the whole sequence."""
    rng = _rng(403)
    q, k, v, g, w, b = _ccq_case(rng, N=19, center=0.7)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    ref = numpy_ccq_brute(q, k, v, g, w, b)
    for a in (7, N - 1):
        o1, st = orc.ccq_forward(q[:, :, :a], k[:, :, :a], v[:, :, :a], g[:, :, :a], w, b,
                                 return_state=True)
        for h in range(H):
            kk = k[0, h, :a]
            S = sum(np.prod(g[0, h, j + 1:a]) * np.outer(kk[j], v[0, h, j]) for j in range(a))
            want = np.concatenate([S.ravel(), (kk.T @ kk).ravel(), kk.sum(0)])
            assert relerr(st[0, h], want) < 1e-12
        o2 = orc.ccq_forward(q[:, :, a:], k[:, :, a:], v[:, :, a:], g[:, :, a:], w, b, t0=a,
                             state_in=st)
        assert relerr(np.concatenate([o1, o2], 2), ref) < 1e-12
    assert dk * dv + dk * dk + dk == st.shape[-1]


def numpy_glv_brute(q, k, v, g):
    """o_t = sum_{j<=t} sum_a q_ta k_ja (prod_{s=j+1..t} g_sa) v_j, explicit products."""
    B, H, N, _ = q.shape
    out = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            for t in range(N):
                for j in range(t + 1):
                    dec = np.prod(g[b, h, j + 1:t + 1], axis=0)  # per key feature
                    out[b, h, t] += np.sum(q[b, h, t] * k[b, h, j] * dec) * v[b, h, j]
    return out


def pin_glv(orc):
    """Per-feature decay: explicit products; a decay equal across features is the
    scalar form (numpy brute force); g = 1 is tril(Q K^T) V; a feature with
    g = 0 forgets all earlier keys in that feature only."""
    rng = _rng(501)
    B, H, N, dk, dv = 1, 2, 23, 4, 3
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.2, 1.0, (B, H, N, dk))
    assert relerr(orc.glv_forward(q, k, v, g), numpy_glv_brute(q, k, v, g)) < 1e-12
    gs = rng.uniform(0.2, 1.0, (B, H, N))
    got = orc.glv_forward(q, k, v, np.repeat(gs[..., None], dk, axis=-1))
    assert relerr(got, numpy_gla_brute(q, k, v, gs)) < 1e-12
    got = orc.glv_forward(q, k, v, np.ones((B, H, N, dk)))
    assert relerr(got, np.tril(q @ np.swapaxes(k, -1, -2)) @ v) < 1e-12
    g0 = np.ones((B, H, N, dk))
    g0[..., 1] = 0.0  # feature 1 keeps only the current key
    got = orc.glv_forward(q, k, v, g0)
    keep = np.ones(dk, dtype=bool)
    keep[1] = False
    ref = np.tril(q[..., keep] @ np.swapaxes(k[..., keep], -1, -2)) @ v
    ref += (q[..., 1] * k[..., 1])[..., None] * v
    assert relerr(got, ref) < 1e-12
    # carried state: S after a prefix is sum_j diag(prod g) k_j v_j^T, and
    # continuing from it (also one token at a time) gives the brute-force rows
    ref = numpy_glv_brute(q, k, v, g)
    for a in (9, N - 1):
        o1, st = orc.glv_forward(q[:, :, :a], k[:, :, :a], v[:, :, :a], g[:, :, :a], return_state=True)
        for h in range(H):
            want = sum(np.prod(g[0, h, j + 1:a], axis=0)[:, None] * np.outer(k[0, h, j], v[0, h, j])
                       for j in range(a))
            assert relerr(st[0, h], want.ravel()) < 1e-12
        o2 = orc.glv_forward(q[:, :, a:], k[:, :, a:], v[:, :, a:], g[:, :, a:], state_in=st)
        assert relerr(np.concatenate([o1, o2], 2), ref) < 1e-12


def pin_gla_backward(orc):
    """Gradients of the decayed linear attention: the autograd oracle's forward
    equals oracle.c's recurrence, and every gradient (q, k, v and the gates)
    equals central finite differences of oracle.c's forward."""
    from oracle import grad
    rng = _rng(601)
    B, H, N, dk, dv = 1, 2, 6, 3, 2
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.3, 1.0, (B, H, N))
    do = rng.standard_normal((B, H, N, dv))
    fw = grad.gla_forward_torch(*[grad._t(x) for x in (q, k, v, g)]).numpy()
    assert relerr(fw, orc.gla_forward(q, k, v, g)) < 1e-12
    dq, dk_, dv_, dg = grad.gla_backward(q, k, v, g, do)
    loss = lambda q_, k_, v_, g_: float(np.sum(orc.gla_forward(q_, k_, v_, g_) * do))
    h = 1e-6
    for idx, (x, gx) in enumerate(((q, dq), (k, dk_), (v, dv_), (g, dg))):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += h
            xm = x.copy(); xm[pos] -= h
            args_p = [q, k, v, g]; args_p[idx] = xp
            args_m = [q, k, v, g]; args_m[idx] = xm
            num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert relerr(gx, num) < 1e-7, ("gradient", idx, relerr(gx, num))


def pin_gla_backward_state(orc):
    """Gradients of the decayed linear attention with a carried state: from a
    state_in, with the loss sum(o * do) + sum(S_out * dS_out), every gradient
    (q, k, v, the gates and state_in) equals central finite differences of
    oracle.c's forward with a carried state."""
    from oracle import grad
    rng = _rng(605)
    B, H, N, dk, dv = 1, 2, 5, 3, 2
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.3, 1.0, (B, H, N))
    do = rng.standard_normal((B, H, N, dv))
    s0 = rng.standard_normal((B, H, dk, dv))
    dso = rng.standard_normal((B, H, dk, dv))
    gs = grad.gla_backward(q, k, v, g, do, state_in=s0, dstate_out=dso)
    assert len(gs) == 5

    def loss(q_, k_, v_, g_, s_):
        o, so = orc.gla_forward(q_, k_, v_, g_, state_in=s_.reshape(B, H, dk * dv), return_state=True)
        return float(np.sum(o * do) + np.sum(so.reshape(B, H, dk, dv) * dso))

    h = 1e-6
    args = [q, k, v, g, s0]
    for idx, gx in enumerate(gs):
        x = args[idx]
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += h
            xm = x.copy(); xm[pos] -= h
            ap = list(args); ap[idx] = xp
            am = list(args); am[idx] = xm
            num[pos] = (loss(*ap) - loss(*am)) / (2 * h)
        assert relerr(gx, num) < 1e-7, ("gradient", idx, relerr(gx, num))
    # without the state terms the extra output is the plain state gradient and
    # the others equal the stateless backward's
    g0 = grad.gla_backward(q, k, v, g, do)
    gz = grad.gla_backward(q, k, v, g, do, state_in=np.zeros_like(s0))
    for a_, b_ in zip(g0, gz[:4]):
        assert relerr(a_, b_) < 1e-12


def pin_gma_backward(orc):
    """Gradients of GMA (causal and bidirectional): the autograd oracle's forward
    equals oracle.c's, and every gradient (q, k, v, mu, log_var, logit_pi)
    equals central finite differences of oracle.c's forward."""
    from oracle import grad
    rng = _rng(602)
    B, H, N, d, K, dv, eps = 1, 2, 5, 3, 4, 2, 1e-3
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, dv))
    mu = rng.standard_normal((H, K, d))
    lv = rng.normal(0.0, 0.5, (H, K, d))
    lp = rng.standard_normal((H, K))
    do = rng.standard_normal((B, H, N, dv))
    for causal in (True, False):
        fw = grad.gma_forward_torch(*[grad._t(x) for x in (q, k, v, mu, lv, lp)], eps, causal).numpy()
        assert relerr(fw, orc.gma_forward(q, k, v, mu, lv, lp, causal=causal, eps=eps)) < 1e-12
        gs = grad.gma_backward(q, k, v, mu, lv, lp, do, eps, causal)
        base = [q, k, v, mu, lv, lp]
        loss = lambda a: float(np.sum(orc.gma_forward(*a, causal=causal, eps=eps) * do))
        h = 1e-6
        for idx, gx in enumerate(gs):
            x = base[idx]
            num = np.zeros_like(x)
            for pos in np.ndindex(x.shape):
                xp = x.copy(); xp[pos] += h
                xm = x.copy(); xm[pos] -= h
                ap = list(base); ap[idx] = xp
                am = list(base); am[idx] = xm
                num[pos] = (loss(ap) - loss(am)) / (2 * h)
            assert relerr(gx, num) < 1e-7, ("gradient", causal, idx, relerr(gx, num))


def pin_ccq_backward(orc):
    """Gradients of the CCQ read: the autograd oracle's forward equals oracle.c's
    recurrence, and every gradient (q, k, v, g, w, b) equals central finite
    differences of oracle.c's forward (keys with a common offset and a strong
    gate, so that the covariance term carries weight)."""
    from oracle import grad
    rng = _rng(603)
    B, H, N, dk = 1, 2, 6, 3
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk)) + 0.5
    v = rng.standard_normal((B, H, N, dk))
    g = rng.uniform(0.3, 1.0, (B, H, N))
    w = rng.standard_normal((H, dk))
    b = np.array([1.0, -0.5])
    do = rng.standard_normal((B, H, N, dk))
    fw = grad.ccq_forward_torch(*[grad._t(x) for x in (q, k, v, g, w, b)]).numpy()
    assert relerr(fw, orc.ccq_forward(q, k, v, g, w, b)) < 1e-12
    gs = grad.ccq_backward(q, k, v, g, w, b, do)
    base = [q, k, v, g, w, b]
    loss = lambda a: float(np.sum(orc.ccq_forward(*a) * do))
    h = 1e-6
    for idx, gx in enumerate(gs):
        x = base[idx]
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += h
            xm = x.copy(); xm[pos] -= h
            ap = list(base); ap[idx] = xp
            am = list(base); am[idx] = xm
            num[pos] = (loss(ap) - loss(am)) / (2 * h)
        assert relerr(gx, num) < 1e-7, ("gradient", idx, relerr(gx, num))


# ---------------------------------------------------------- gated delta rule


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _deltanet_case(rng, B=1, H=2, N=30, dk=5, dv=3, unit=True):
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    k = _unit(k) if unit else k
    v = rng.standard_normal((B, H, N, dv))
    g = rng.uniform(0.3, 1.0, (B, H, N))
    beta = rng.uniform(0.0, 1.0, (B, H, N))
    return q, k, v, g, beta


def pin_deltanet_gradient_step(orc):
    """One token from a random state: the new state is the decayed state minus
    beta times the gradient of 1/2 ||S^T k - v||^2 there. The gradient is
    taken by central differences of that loss (exact for a quadratic up to
    rounding), with dk != dv and a key of arbitrary norm."""
    rng = _rng(401)
    dk, dv = 5, 3
    for trial in range(3):
        s_in = rng.standard_normal((1, 1, dk * dv))
        q = rng.standard_normal((1, 1, 1, dk))
        k = rng.standard_normal((1, 1, 1, dk)) * (0.5 + trial)
        v = rng.standard_normal((1, 1, 1, dv))
        g = rng.uniform(0.2, 1.0, (1, 1, 1))
        beta = rng.uniform(0.1, 1.0, (1, 1, 1))
        out, s_out = orc.deltanet_forward(q, k, v, g, beta, state_in=s_in, return_state=True)
        kk, vv = k[0, 0, 0], v[0, 0, 0]
        loss = lambda S: 0.5 * np.sum((S.T @ kk - vv) ** 2)
        S1 = g[0, 0, 0] * s_in.reshape(dk, dv)
        grad = np.empty((dk, dv))
        h = 1e-3
        for a in range(dk):
            for e in range(dv):
                E = np.zeros((dk, dv))
                E[a, e] = h
                grad[a, e] = (loss(S1 + E) - loss(S1 - E)) / (2 * h)
        expect = S1 - beta[0, 0, 0] * grad
        assert relerr(s_out.reshape(dk, dv), expect) < 1e-9, trial
        assert relerr(out[0, 0, 0], expect.T @ q[0, 0, 0]) < 1e-9, trial


def pin_deltanet_orthogonal_keys(orc):
    """Orthonormal keys never interfere: the error term S^T k_t is zero, so the
    delta rule writes beta_t v_t, which is gated linear attention with values
    beta v. CCQ on it likewise equals CCQ on gated linear attention."""
    rng = _rng(402)
    B, H, N, dk, dv = 1, 2, 6, 8, 3
    q, _, v, g, beta = _deltanet_case(rng, B, H, N, dk, dv)
    k = np.empty((B, H, N, dk))
    for h in range(H):
        basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k[0, h] = basis[:N]
    bv = beta[..., None] * v
    assert relerr(orc.deltanet_forward(q, k, v, g, beta), orc.gla_forward(q, k, bv, g)) < 1e-12
    w = rng.standard_normal((H, dk)) / np.sqrt(dk)
    b = np.array([1.0, -0.5])
    assert relerr(orc.ccq_deltanet_forward(q, k, v, g, beta, w, b),
                  orc.ccq_forward(q, k, bv, g, w, b)) < 1e-12
    # non-orthogonal keys: the two differ
    q, k, v, g, beta = _deltanet_case(rng, B, H, N, dk, dv)
    assert relerr(orc.deltanet_forward(q, k, v, g, beta),
                  orc.gla_forward(q, k, beta[..., None] * v, g)) > 1e-2


def pin_deltanet_exact_recall(orc):
    """With a unit key and beta = 1 the step overwrites exactly: right after the
    write, reading with q = k returns v, whatever the history and decay."""
    rng = _rng(403)
    B, H, N, dk, dv = 1, 1, 40, 6, 4
    q, k, v, g, beta = _deltanet_case(rng, B, H, N, dk, dv)
    s_in = rng.standard_normal((B, H, dk * dv))
    sel = [3, 17, 18, 39]
    for t in sel:
        beta[0, 0, t] = 1.0
        q[0, 0, t] = k[0, 0, t]
    out = orc.deltanet_forward(q, k, v, g, beta, state_in=s_in)
    for t in sel:
        assert np.max(np.abs(out[0, 0, t] - v[0, 0, t])) < 1e-12, t
    # and with beta < 1 the recall is only partial
    beta[0, 0, sel] = 0.5
    out = orc.deltanet_forward(q, k, v, g, beta, state_in=s_in)
    assert np.max(np.abs(out[0, 0, sel] - v[0, 0, sel])) > 1e-2


def pin_deltanet_beta_zero(orc):
    """beta = 0 writes nothing: the state only decays, o_t = (prod_{s<=t} g_s) S_0^T q_t."""
    rng = _rng(404)
    B, H, N, dk, dv = 1, 2, 12, 4, 5
    q, k, v, g, _ = _deltanet_case(rng, B, H, N, dk, dv)
    s_in = rng.standard_normal((B, H, dk * dv))
    out, s_out = orc.deltanet_forward(q, k, v, g, np.zeros((B, H, N)), state_in=s_in, return_state=True)
    for h in range(H):
        S0 = s_in[0, h].reshape(dk, dv)
        dec = np.cumprod(g[0, h])
        assert relerr(out[0, h], dec[:, None] * (q[0, h] @ S0)) < 1e-13
        assert relerr(s_out[0, h], dec[-1] * s_in[0, h]) < 1e-13
    assert np.all(orc.deltanet_forward(q, k, v, g, np.zeros((B, H, N))) == 0.0)


def numpy_deltanet_chunkwise(q, k, v, g, beta, C):
    """The chunk form used by the GPU kernel, derived from the recurrence. The
    step is S_r = g_r S_{r-1} + k_r u_r^T with the pseudo-value u_r = beta_r (v_r
    - g_r S_{r-1}^T k_r), so a chunk is decayed linear attention with values U;
    unrolling g_r S_{r-1} inside the chunk gives (I + A) U = diag(beta) V
    - diag(beta gamma) K S_0, A_rj = beta_r (gamma_r / gamma_j) (k_r . k_j) for
    j < r, gamma the running product of g inside the chunk, S_0 the state at the
    chunk start."""
    N, dk = k.shape
    S = np.zeros((dk, v.shape[1]))
    out = np.zeros(v.shape)
    for c0 in range(0, N, C):
        sl = slice(c0, min(c0 + C, N))
        Q, K, V, bb = q[sl], k[sl], v[sl], beta[sl]
        gam = np.cumprod(g[sl])
        ratio = gam[:, None] / gam[None, :]
        L = len(gam)
        A = np.tril(bb[:, None] * ratio * (K @ K.T), -1)
        T = np.linalg.inv(np.eye(L) + A)
        W = T @ ((bb * gam)[:, None] * K)
        U = T @ (bb[:, None] * V) - W @ S
        P = np.tril(ratio * (Q @ K.T))
        out[sl] = gam[:, None] * (Q @ S) + P @ U
        S = gam[-1] * S + K.T @ ((gam[-1] / gam)[:, None] * U)
    return out


def pin_deltanet_chunkwise(orc):
    rng = _rng(405)
    q, k, v, g, beta = _deltanet_case(rng, 1, 2, 70, 6, 4)
    rec = orc.deltanet_forward(q, k, v, g, beta)
    for h in range(2):
        for C in (1, 7, 16, 64):
            got = numpy_deltanet_chunkwise(q[0, h], k[0, h], v[0, h], g[0, h], beta[0, h], C)
            assert relerr(got, rec[0, h]) < 1e-11, (h, C)


def pin_deltanet_state(orc):
    """Continuing from the state after a prefix gives the rows of the whole
    sequence (plain and CCQ read; the CCQ count t0 carried)."""
    rng = _rng(406)
    B, H, N, dk, dv, n1 = 1, 2, 33, 4, 3, 14
    q, k, v, g, beta = _deltanet_case(rng, B, H, N, dk, dv)
    full = orc.deltanet_forward(q, k, v, g, beta)
    a, st = orc.deltanet_forward(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], g[:, :, :n1], beta[:, :, :n1],
                                 return_state=True)
    b = orc.deltanet_forward(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], g[:, :, n1:], beta[:, :, n1:],
                             state_in=st)
    assert relerr(np.concatenate([a, b], axis=2), full) < 1e-12
    w = rng.standard_normal((H, dk)) / np.sqrt(dk)
    bl = np.array([0.5, 2.0])
    full = orc.ccq_deltanet_forward(q, k, v, g, beta, w, bl)
    a, st = orc.ccq_deltanet_forward(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], g[:, :, :n1],
                                     beta[:, :, :n1], w, bl, return_state=True)
    b = orc.ccq_deltanet_forward(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], g[:, :, n1:], beta[:, :, n1:],
                                 w, bl, t0=n1, state_in=st)
    assert relerr(np.concatenate([a, b], axis=2), full) < 1e-12


def pin_ccq_deltanet_reductions(orc):
    """Gate closed (lambda = 0): CCQ over the delta rule is the plain delta
    rule. The read's correction is the CCQ one: with the delta rule's state
    S_t taken from the oracle's own plain run, o_t = S_t^T (q_t - lambda_t
    Cov_{<=t}[k] q_t) with numpy.cov(bias=True)."""
    rng = _rng(407)
    B, H, N, dk, dv = 1, 2, 20, 4, 3
    q, k, v, g, beta = _deltanet_case(rng, B, H, N, dk, dv, unit=False)
    k = k * 0.5 + 0.3
    w = rng.standard_normal((H, dk)) / np.sqrt(dk)
    plain = orc.deltanet_forward(q, k, v, g, beta)
    assert relerr(orc.ccq_deltanet_forward(q, k, v, g, beta, w, np.full(H, -1e4)), plain) < 1e-14
    bl = np.array([1.0, 2.5])
    got = orc.ccq_deltanet_forward(q, k, v, g, beta, w, bl)
    for h in range(H):
        for t in range(N):
            _, st = orc.deltanet_forward(q[:, h:h + 1, :t + 1], k[:, h:h + 1, :t + 1], v[:, h:h + 1, :t + 1],
                                         g[:, h:h + 1, :t + 1], beta[:, h:h + 1, :t + 1], return_state=True)
            S = st.reshape(dk, dv)
            kk = k[0, h, :t + 1]
            sig = np.cov(kk.T, bias=True).reshape(dk, dk) if t > 0 else np.zeros((dk, dk))
            lam = 1.0 / (1.0 + np.exp(-(w[h] @ q[0, h, t] + bl[h])))
            ref = S.T @ (q[0, h, t] - lam * sig @ q[0, h, t])
            assert relerr(got[0, h, t], ref) < 1e-11, (h, t)
    assert relerr(got, plain) > 1e-2


ALL_PINS = [
    pin_gamma_scipy, pin_gma_brute_numpy, pin_gma_k1_closed_form, pin_gma_identical_components,
    pin_gma_permutation, pin_gma_prefix, pin_gma_affinity_structure, pin_gma_golden,
    pin_gla_brute, pin_gla_chunkwise, pin_ccq_numpy_cov, pin_cov_is_logpartition_hessian,
    pin_ccq_reductions, pin_ccq_chunkwise, pin_ccq_golden, pin_gma_state, pin_gla_state,
    pin_ccq_state, pin_glv, pin_gla_backward, pin_gla_backward_state, pin_gma_backward, pin_ccq_backward,
    pin_deltanet_gradient_step, pin_deltanet_orthogonal_keys, pin_deltanet_exact_recall,
    pin_deltanet_beta_zero, pin_deltanet_chunkwise, pin_deltanet_state, pin_ccq_deltanet_reductions,
]
