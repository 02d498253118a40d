"""Feature widths of 16 and d != dv (run on the kernels of the next wider width
after zero padding of the feature axis), on the GPU against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from linear_attention_gmm_amd import (binding, ccq_deltanet_forward, ccq_forward, deltanet_chunk_forward, gma_forward,
                                      inputs, linattn_chunk_forward)
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,dv,causal", [("f32", 16, 16, True), ("f32", 64, 32, True), ("f32", 32, 64, False),
                                               ("f32", 16, 128, True), ("bf16", 64, 32, True), ("bf16", 16, 64, False)])
def test_gma_padded(dtype, d, dv, causal):
    N = 300 if dtype == "f32" else 1000
    cfg = inputs.GmaConfig("gma_pad", 501, B=2, H=2, N=N, d=d, K=24, dv=dv, dtype=dtype, causal=causal,
                           qk_scale=True)
    x = inputs.gma_inputs(cfg)
    say("gma padded: d=%d dv=%d %s causal=%d" % (d, dv, dtype, causal))
    g = cuda(x)
    got = host(gma_forward(g["q"], g["k"], g["v"], g["mu"], g["log_var"], g["logit_pi"], causal=causal,
                           eps=cfg.eps, segments=3))
    ref = oracle.gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], causal=causal,
                             eps=cfg.eps)
    assert got.shape == ref.shape
    assert_close(got, ref, dtype, "gma d=%d dv=%d %s causal=%d" % (d, dv, dtype, causal))


def _lin(dtype, dk, dv, **kw):
    N = 300 if dtype == "f32" else 1000
    return inputs.LinAttnConfig("lin_pad", 502, B=2, H=2, N=N, dk=dk, dv=dv, dtype=dtype, **kw)


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 16, 16), ("f32", 64, 32), ("f32", 32, 128), ("bf16", 16, 64)])
def test_gla_padded(dtype, dk, dv):
    cfg = _lin(dtype, dk, dv)
    x = inputs.linattn_inputs(cfg)
    d = cuda(x)
    got = host(linattn_chunk_forward(d["q"], d["k"], d["v"], d["g"], segments=2))
    ref = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])
    assert_close(got, ref, dtype, "gla dk=%d dv=%d %s" % (dk, dv, dtype))


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 16, 16), ("f32", 32, 64), ("bf16", 64, 32)])
def test_ccq_padded(dtype, dk, dv):
    cfg = _lin(dtype, dk, dv, lowrank_keys=4, gate_bias=2.0)
    x = inputs.linattn_inputs(cfg, ccq=True)
    d = cuda(x)
    got = host(ccq_forward(d["q"], d["k"], d["v"], d["g"], d["w_lambda"], d["b_lambda"], segments=3))
    ref = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"])
    assert_close(got, ref, dtype, "ccq dk=%d dv=%d %s" % (dk, dv, dtype))


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 16, 16), ("bf16", 32, 64)])
def test_vec_padded(dtype, dk, dv):
    cfg = _lin(dtype, dk, dv, vector_gates=True)
    x = inputs.linattn_inputs(cfg)
    d = cuda(x)
    got = host(binding.linattn_vec_forward(d["q"], d["k"], d["v"], d["g"], segments=2))
    ref = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"])
    assert_close(got, ref, dtype, "per-feature decay dk=%d dv=%d %s" % (dk, dv, dtype))


@pytest.mark.parametrize("dtype,dk,dv,ccq", [("f32", 16, 16, False), ("f32", 64, 32, False), ("bf16", 16, 128, False),
                                             ("f32", 16, 32, True), ("bf16", 32, 64, True)])
def test_deltanet_padded(dtype, dk, dv, ccq):
    cfg = _lin(dtype, dk, dv, delta=True, lowrank_keys=4 if ccq else 0, gate_bias=2.0)
    x = inputs.linattn_inputs(cfg, ccq=ccq)
    d = cuda(x)
    if ccq:
        got = host(ccq_deltanet_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["w_lambda"], d["b_lambda"]))
        ref = oracle.ccq_deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w_lambda"], x["b_lambda"])
    else:
        got = host(deltanet_chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"]))
        ref = oracle.deltanet_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    assert_close(got, ref, dtype, "%s dk=%d dv=%d %s" % ("ccq_deltanet" if ccq else "deltanet", dk, dv, dtype))


def test_padded_equals_native_on_zero_features():
    # a width-16 call equals the width-32 call on the same rows with 16 zero
    # features appended (both run the same kernel; the padding is exact)
    import torch
    cfg = _lin("f32", 16, 16)
    x = cuda(inputs.linattn_inputs(cfg))
    z = lambda t: torch.cat([t, torch.zeros_like(t)], dim=-1).contiguous()
    a = linattn_chunk_forward(x["q"], x["k"], x["v"], x["g"])
    b = linattn_chunk_forward(z(x["q"]), z(x["k"]), z(x["v"]), x["g"])[..., :16]
    assert torch.equal(a, b)
