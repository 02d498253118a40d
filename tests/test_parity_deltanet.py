"""The gated delta rule (plain and CCQ read) on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_gmm_amd import (ccq_deltanet_forward, ccq_deltanet_forward_state, deltanet_chunk_forward,
                                      deltanet_forward_state, inputs)
from parity import assert_close, cuda, host, rel_l2, say

pytestmark = pytest.mark.gpu


def _worst_slice(got, ref):
    g = got.reshape(-1, *got.shape[2:])
    r = ref.reshape(-1, *ref.shape[2:])
    w = max(rel_l2(g[i], r[i]) for i in range(g.shape[0]))
    say("  worst (b,h) slice rel-L2 %.3e" % w)
    return w


def _run(cfg, ccq, N=None, segments=0, beta=None, with_plain=False):
    x = inputs.linattn_inputs(cfg, N=N, ccq=ccq)
    if beta is not None:
        x["beta"] = torch.full_like(x["beta"], float(beta))
    say("%s: %s N=%d segments=%d dtype=%s" % ("ccq_deltanet" if ccq else "deltanet", cfg.name, x["q"].shape[2],
                                              segments, cfg.dtype))
    d = cuda(x)
    if ccq:
        got = host(ccq_deltanet_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w_lambda"], d["b_lambda"],
                                        segments=segments))
        ref = oracle.ccq_deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w_lambda"], x["b_lambda"])
        if with_plain:
            plain = oracle.deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
            say("  oracle |O_ccq - O_plain| / |O_ccq| = %.3e" % rel_l2(plain, ref))
    else:
        got = host(deltanet_chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], segments=segments))
        ref = oracle.deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
        if with_plain:
            gla = oracle.gla_forward(x["q"], x["k"], x["beta"][..., None].double() * x["v"].double(), x["g"])
            say("  oracle |O_delta - O_gla(beta v)| / |O_delta| = %.3e" % rel_l2(gla, ref))
    return got, ref


@pytest.mark.parametrize("dk", [32, 64])
@pytest.mark.parametrize("ccq", [False, True])
def test_deltanet_fp32(dk, ccq):
    # 300 tokens: four whole chunks and a ragged tail
    cfg = inputs.LinAttnConfig("deltanet_fp32", 401, B=2, H=2, N=300, dk=dk, dv=dk, dtype="f32", delta=True,
                               lowrank_keys=4 if ccq else 0, gate_bias=2.0)
    got, ref = _run(cfg, ccq, segments=3, with_plain=True)
    assert_close(got, ref, "f32", "%s fp32 dk=%d" % ("ccq_deltanet" if ccq else "deltanet", dk))


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 129])
def test_deltanet_short_fp32(N):
    cfg = inputs.LinAttnConfig("deltanet_short", 402, B=1, H=2, N=N, dk=32, dv=32, dtype="f32", delta=True)
    got, ref = _run(cfg, False)
    assert_close(got, ref, "f32", "deltanet N=%d" % N)


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_deltanet_beta_extremes_fp32(beta):
    # beta = 1 overwrites the value of each (unit) key exactly; beta = 0 writes nothing
    cfg = inputs.LinAttnConfig("deltanet_beta", 403, B=1, H=2, N=200, dk=64, dv=64, dtype="f32", delta=True)
    got, ref = _run(cfg, False, beta=beta)
    if beta == 0.0:
        assert np.all(got == 0.0)
    else:
        assert_close(got, ref, "f32", "deltanet beta=1")


@pytest.mark.parametrize("g_logit_mean", [1.0, -1.0, -30.0])
def test_deltanet_strong_decay_fp32(g_logit_mean):
    # g ~ 0.7, 0.3 and 1e-13 per token: decay ratios inside a chunk far below
    # the float range in the last case
    cfg = inputs.LinAttnConfig("deltanet_decay", 404, B=1, H=2, N=400, dk=64, dv=64, dtype="f32", delta=True,
                               g_logit_mean=g_logit_mean)
    got, ref = _run(cfg, False)
    assert_close(got, ref, "f32", "deltanet g logit mean %g" % g_logit_mean)


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("ccq", [False, True])
def test_deltanet_bf16_ragged(dk, ccq):
    cfg = inputs.LinAttnConfig("deltanet_bf16", 405, B=2, H=3, N=1000, dk=dk, dv=dk, delta=True,
                               lowrank_keys=4 if ccq else 0, gate_bias=2.0)
    got, ref = _run(cfg, ccq, segments=2)
    assert_close(got, ref, "bf16", "%s bf16 dk=%d N=1000" % ("ccq_deltanet" if ccq else "deltanet", dk))


def test_deltanet_bf16_n8k():
    # the gated delta rule on the 8K-token shape (B=8, H=16), every slice
    cfg = inputs.CONFIGS["deltanet_bf16_n8k"]
    got, ref = _run(cfg, False, with_plain=True)
    assert_close(got, ref, "bf16", "deltanet bf16 B8 H16 N=8192, whole tensor")
    assert _worst_slice(got, ref) <= 2e-2


@pytest.mark.parametrize("name", ["ccq_deltanet_bf16_n16k", "ccq_deltanet_bf16_lowrank"])
def test_ccq_deltanet_bf16_n16k(name):
    # CCQ over the gated delta rule on the 16K-token shape (B=4, H=16) in the
    # launch the bench times, every slice; isotropic and low-rank keys
    cfg = inputs.CONFIGS[name]
    got, ref = _run(cfg, True, with_plain=True)
    assert_close(got, ref, "bf16", "ccq_deltanet bf16 %s B4 H16 N=16384, whole tensor" % name)
    assert _worst_slice(got, ref) <= 2e-2


def test_deltanet_bf16_n16k_plain():
    # the plain read at the 16K-token shape, every slice
    cfg = inputs.CONFIGS["ccq_deltanet_bf16_n16k"]
    got, ref = _run(cfg, False)
    assert_close(got, ref, "bf16", "deltanet bf16 B4 H16 N=16384, whole tensor")
    assert _worst_slice(got, ref) <= 2e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ccq", [False, True])
def test_deltanet_state_continuation(dtype, ccq):
    # prefill N1 tokens, continue with the rest from the carried state; both
    # halves against the oracle on the whole sequence, and the final state
    dk = 64
    cfg = inputs.LinAttnConfig("deltanet_state", 406, B=2, H=2, N=500, dk=dk, dv=dk, dtype=dtype, delta=True,
                               lowrank_keys=4, gate_bias=2.0)
    x = inputs.linattn_inputs(cfg, ccq=True)
    n1 = 190
    d = cuda(x)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    args = ("q", "k", "v", "g", "beta")
    first = [sl(d[n], 0, n1) for n in args]
    second = [sl(d[n], n1, cfg.N) for n in args]
    if ccq:
        o1, s1 = ccq_deltanet_forward_state(*first, d["w_lambda"], d["b_lambda"])
        o2, s2 = ccq_deltanet_forward_state(*second, d["w_lambda"], d["b_lambda"], state_in=s1, t_in=n1)
        ref, sref = oracle.ccq_deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w_lambda"],
                                                x["b_lambda"], return_state=True)
    else:
        o1, s1 = deltanet_forward_state(*first)
        o2, s2 = deltanet_forward_state(*second, state_in=s1)
        ref, sref = oracle.deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], return_state=True)
    got = np.concatenate([host(o1), host(o2)], axis=2)
    assert_close(got, ref, dtype, "deltanet state continuation out (%s, ccq=%d)" % (dtype, ccq))
    assert_close(host(s2), sref, dtype, "deltanet state after the sequence (%s, ccq=%d)" % (dtype, ccq))


def test_deltanet_state_in_place():
    # state_in and state_out the same buffer
    cfg = inputs.LinAttnConfig("deltanet_inplace", 407, B=1, H=2, N=300, dk=64, dv=64, dtype="f32", delta=True,
                               lowrank_keys=4, gate_bias=2.0)
    x = inputs.linattn_inputs(cfg, ccq=True)
    d = cuda(x)
    st = torch.zeros((1, 2, 64 * 64 + 64 * 64 + 64), dtype=torch.float32, device="cuda")
    ccq_deltanet_forward_state(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w_lambda"], d["b_lambda"],
                               state_in=st, state_out=st, segments=3)
    _, sref = oracle.ccq_deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w_lambda"], x["b_lambda"],
                                          return_state=True)
    assert_close(host(st), sref, "f32", "ccq_deltanet state updated in place")


def test_deltanet_deterministic():
    cfg = inputs.CONFIGS["ccq_deltanet_bf16_n16k"].replace(B=1, H=2, N=4096)
    x = cuda(inputs.linattn_inputs(cfg, ccq=True))
    a = ccq_deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w_lambda"], x["b_lambda"])
    b = ccq_deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w_lambda"], x["b_lambda"])
    assert torch.equal(a, b)
    a = deltanet_chunk_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    b = deltanet_chunk_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    assert torch.equal(a, b)
