"""Chunks of 32 tokens (the plain and CCQ forwards of decayed linear attention)
on the GPU: against the fp64 oracle, and invariance of the result under the
chunk length (32 against the 64-token kernels)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_gmm_amd import binding, ccq_forward, inputs, linattn_chunk_forward
from parity import assert_close, cuda, host, max_rel, record, say

pytestmark = pytest.mark.gpu


def _cfg(dtype, d, N, ccq, **kw):
    extra = dict(lowrank_keys=4, gate_bias=2.0) if ccq else {}
    extra.update(kw)
    return inputs.LinAttnConfig("chunk32", 601, B=2, H=2, N=N, dk=d, dv=d, dtype=dtype, **extra)


def _fwd(d, ccq, chunk, **kw):
    if ccq:
        return ccq_forward(d["q"], d["k"], d["v"], d["g"], d["w_lambda"], d["b_lambda"], chunk=chunk, **kw)
    return linattn_chunk_forward(d["q"], d["k"], d["v"], d["g"], chunk=chunk, **kw)


def _ref(x, ccq):
    if ccq:
        return oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"])
    return oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("ccq", [False, True])
def test_chunk32_fp32(d, ccq):
    # 300 tokens: nine whole chunks of 32 and a ragged tail
    cfg = _cfg("f32", d, 300, ccq)
    x = inputs.linattn_inputs(cfg, ccq=ccq)
    say("chunk 32: %s d=%d fp32" % ("ccq" if ccq else "gla", d))
    got = host(_fwd(cuda(x), ccq, 32))
    assert_close(got, _ref(x, ccq), "f32", "%s chunk 32 fp32 d=%d" % ("ccq" if ccq else "gla", d))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ccq", [False, True])
def test_chunk32_bf16(d, ccq):
    cfg = _cfg("bf16", d, 1000, ccq)
    x = inputs.linattn_inputs(cfg, ccq=ccq)
    say("chunk 32: %s d=%d bf16" % ("ccq" if ccq else "gla", d))
    got = host(_fwd(cuda(x), ccq, 32))
    assert_close(got, _ref(x, ccq), "bf16", "%s chunk 32 bf16 d=%d" % ("ccq" if ccq else "gla", d))


@pytest.mark.parametrize("N", [1, 31, 32, 33, 95])
def test_chunk32_short(N):
    cfg = _cfg("f32", 64, N, True)
    x = inputs.linattn_inputs(cfg, ccq=True)
    got = host(_fwd(cuda(x), True, 32))
    assert_close(got, _ref(x, True), "f32", "ccq chunk 32 N=%d" % N)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("ccq", [False, True])
@pytest.mark.parametrize("g_logit_mean", [3.0, -1.0])
def test_chunk_length_invariance(d, ccq, g_logit_mean):
    # float32: the 32-token schedule and the 64-token kernels agree to 1e-5
    # relative (max |a - b| / max |b|); also against several segments
    cfg = _cfg("f32", d, 1000, ccq, g_logit_mean=g_logit_mean)
    x = cuda(inputs.linattn_inputs(cfg, ccq=ccq))
    a = host(_fwd(x, ccq, 32))
    b1 = host(_fwd(x, ccq, 64, segments=1))
    b8 = host(_fwd(x, ccq, 64, segments=8))
    for name, b in (("P=1", b1), ("P=8", b8)):
        e = max_rel(a, b)
        what = "%s d=%d g logit mean %g: chunk 32 against chunk 64 %s" % ("ccq" if ccq else "gla", d, g_logit_mean,
                                                                            name)
        say("  %s: max-rel %.3e" % (what, e))
        record(what, "max-rel", e, 1e-5, elements=int(a.size))
        assert e <= 1e-5, what


@pytest.mark.parametrize("ccq", [False, True])
def test_chunk32_state_continuation(ccq):
    # prefill 150 tokens with chunks of 32, continue from the state; both
    # halves and the final state against the oracle on the whole sequence
    cfg = _cfg("f32", 64, 400, ccq)
    x = inputs.linattn_inputs(cfg, ccq=ccq)
    d = cuda(x)
    n1 = 150
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    first = [sl(d[n], 0, n1) for n in "qkvg"]
    second = [sl(d[n], n1, cfg.N) for n in "qkvg"]
    if ccq:
        par = (d["w_lambda"], d["b_lambda"])
        o1, s1 = binding.ccq_forward_state(*first, *par, chunk=32)
        o2, s2 = binding.ccq_forward_state(*second, *par, state_in=s1, t_in=n1, chunk=32)
        ref, sref = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"],
                                       return_state=True)
    else:
        o1, s1 = binding.linattn_chunk_forward_state(*first, chunk=32)
        o2, s2 = binding.linattn_chunk_forward_state(*second, state_in=s1, chunk=32)
        ref, sref = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"], return_state=True)
    got = np.concatenate([host(o1), host(o2)], axis=2)
    assert_close(got, ref, "f32", "chunk 32 continuation out (ccq=%d)" % ccq)
    assert_close(host(s2), sref, "f32", "chunk 32 state after the sequence (ccq=%d)" % ccq)


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 64)])
def test_chunk32_padded(dk, dv):
    cfg = inputs.LinAttnConfig("chunk32_pad", 602, B=2, H=2, N=200, dk=dk, dv=dv, dtype="f32", lowrank_keys=4,
                               gate_bias=2.0)
    x = inputs.linattn_inputs(cfg, ccq=True)
    got = host(_fwd(cuda(x), True, 32))
    assert_close(got, _ref(x, True), "f32", "ccq chunk 32 dk=%d dv=%d" % (dk, dv))


def test_chunk32_deterministic():
    cfg = _cfg("bf16", 128, 777, True)
    x = cuda(inputs.linattn_inputs(cfg, ccq=True))
    assert torch.equal(_fwd(x, True, 32), _fwd(x, True, 32))
