"""Decayed linear attention and CCQ on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_gmm_amd import ccq_forward, inputs, linattn_chunk_forward
from parity import assert_close, cuda, host, record, rel_l2, say

pytestmark = pytest.mark.gpu


def _gla(cfg, N=None, segments=0, sl=None):
    x = inputs.linattn_inputs(cfg, N=N)
    say("gla: %s N=%d segments=%d dtype=%s g_one=%s" % (cfg.name, x["q"].shape[2], segments, cfg.dtype, cfg.g_one))
    d = cuda(x)
    got = host(linattn_chunk_forward(d["q"], d["k"], d["v"], d["g"], segments=segments))
    if sl is None:
        return got, oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])
    gs, rs = [], []
    for b, h in sl:
        r = oracle.gla_forward(x["q"][b:b + 1, h:h + 1], x["k"][b:b + 1, h:h + 1], x["v"][b:b + 1, h:h + 1],
                               x["g"][b:b + 1, h:h + 1])
        gs.append(got[b, h])
        rs.append(r[0, 0])
    return np.stack(gs), np.stack(rs)


def _ccq(cfg, N=None, segments=0, sl=None, with_gla=False):
    x = inputs.linattn_inputs(cfg, N=N, ccq=True)
    say("ccq: %s N=%d segments=%d dtype=%s" % (cfg.name, x["q"].shape[2], segments, cfg.dtype))
    d = cuda(x)
    got = host(ccq_forward(d["q"], d["k"], d["v"], d["g"], d["w_lambda"], d["b_lambda"], segments=segments))
    if sl is None:
        # whole tensor: one oracle call over every slice (threads over (b, h))
        ref = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"])
        if with_gla:
            gl = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])
            e = rel_l2(gl, ref)
            say("  oracle |O_ccq - O_gla| / |O_ccq| = %.3e" % e)
            record("oracle CCQ vs GLA at %s" % cfg.name, "rel-L2 (sensitivity)", e, float("nan"))
        return got.reshape(-1, *got.shape[2:]), ref.reshape(-1, *ref.shape[2:])
    gs, rs, gl = [], [], []
    for b, h in sl:
        sel = lambda t: t[b:b + 1, h:h + 1]
        r = oracle.ccq_forward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["g"]), x["w_lambda"][h:h + 1],
                               x["b_lambda"][h:h + 1])
        gs.append(got[b, h])
        rs.append(r[0, 0])
        if with_gla:
            gl.append(oracle.gla_forward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["g"]))[0, 0])
    if with_gla:
        e = rel_l2(np.stack(gl), np.stack(rs))
        say("  oracle |O_ccq - O_gla| / |O_ccq| = %.3e" % e)
        record("oracle CCQ vs GLA at %s" % cfg.name, "rel-L2 (sensitivity)", e, float("nan"))
    return np.stack(gs), np.stack(rs)


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("segments", [1, 3])
def test_gla_fp32(dk, segments):
    cfg = inputs.LinAttnConfig("gla_fp32", 201, B=2, H=2, N=300, dk=dk, dv=dk, dtype="f32")
    got, ref = _gla(cfg, segments=segments)
    assert_close(got, ref, "f32", "gla fp32 dk=%d P=%d" % (dk, segments))


@pytest.mark.parametrize("g_logit_mean", [1.0, -1.0, -30.0])
@pytest.mark.parametrize("ccq", [False, True])
def test_strong_decay_fp32(g_logit_mean, ccq):
    # g ~ 0.7 and g ~ 0.3 per token: the decay of the carried state is applied
    # both lazily (folded into later weights) and eagerly within a few chunks;
    # g ~ 1e-13: decay ratios across a chunk far beyond the float range
    cfg = inputs.LinAttnConfig("decay_fp32", 205, B=1, H=2, N=700, dk=64, dv=64, dtype="f32",
                               g_logit_mean=g_logit_mean, lowrank_keys=4 if ccq else 0, gate_bias=2.0)
    got, ref = (_ccq(cfg, segments=3) if ccq else _gla(cfg, segments=3))
    assert_close(got, ref, "f32", "%s fp32 g logit mean %g" % ("ccq" if ccq else "gla", g_logit_mean))


@pytest.mark.parametrize("N", [1, 63, 64, 65, 200])
def test_gla_short(N):
    cfg = inputs.LinAttnConfig("gla_short", 202, B=1, H=2, N=N, dk=32, dv=32, dtype="f32")
    got, ref = _gla(cfg)
    assert_close(got, ref, "f32", "gla N=%d" % N)


def test_gla_g_one_fp32():
    cfg = inputs.LinAttnConfig("gla_g1", 203, B=1, H=2, N=700, dk=64, dv=64, dtype="f32", g_one=True)
    got, ref = _gla(cfg, segments=4)
    assert_close(got, ref, "f32", "gla g=1 fp32")


def _worst_slice(got, ref):
    w = max(rel_l2(got[i], ref[i]) for i in range(got.shape[0]))
    say("  worst (b,h) slice rel-L2 %.3e" % w)
    return w


def test_gla_bf16_n8k():
    # the 8K-token GLA workload (B=8, H=16), every slice
    cfg = inputs.CONFIGS["gla_bf16_n8k"]
    got, ref = _gla(cfg)
    assert_close(got, ref, "bf16", "gla bf16 B8 H16 N=8192, whole tensor")
    assert _worst_slice(got.reshape(-1, *got.shape[2:]), ref.reshape(-1, *ref.shape[2:])) <= 2e-2


def test_gla_bf16_g_one_sampled():
    cfg = inputs.CONFIGS["gla_bf16_n8k"].replace(name="gla_bf16_g1", B=2, H=2, N=4096, g_one=True)
    got, ref = _gla(cfg, segments=4, sl=[(0, 0), (1, 1)])
    assert_close(got, ref, "bf16", "gla bf16 g=1")


def test_gla_segment_invariance_fp32():
    cfg = inputs.LinAttnConfig("gla_seg", 204, B=1, H=2, N=2048, dk=64, dv=64, dtype="f32", g_one=True)
    x = cuda(inputs.linattn_inputs(cfg))
    outs = [host(linattn_chunk_forward(x["q"], x["k"], x["v"], x["g"], segments=s)) for s in (1, 8)]
    e = float(np.max(np.abs(outs[0] - outs[1])) / np.max(np.abs(outs[0])))
    say("  gla P=1 vs P=8 max-rel %.3e" % e)
    assert e <= 1e-5


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("segments", [1, 3])
def test_ccq_fp32(dk, segments):
    cfg = inputs.LinAttnConfig("ccq_fp32", 301, B=1, H=2, N=300, dk=dk, dv=dk, dtype="f32", lowrank_keys=4,
                               gate_bias=2.0)
    got, ref = _ccq(cfg, segments=segments, with_gla=True)
    assert_close(got, ref, "f32", "ccq fp32 dk=%d P=%d" % (dk, segments))


def test_ccq_fp32_lowrank_config():
    cfg = inputs.CONFIGS["ccq_fp32_lowrank"]
    got, ref = _ccq(cfg, with_gla=True)
    assert_close(got, ref, "f32", "ccq fp32 low-rank keys")


@pytest.mark.parametrize("N", [1, 65, 130])
def test_ccq_short(N):
    cfg = inputs.LinAttnConfig("ccq_short", 302, B=1, H=1, N=N, dk=32, dv=32, dtype="f32", lowrank_keys=4,
                               gate_bias=2.0)
    got, ref = _ccq(cfg)
    assert_close(got, ref, "f32", "ccq N=%d" % N)


def test_ccq_bf16_n16k():
    # the 16K-token CCQ workload (B=4, H=16) in the launch the bench times,
    # every slice
    cfg = inputs.CONFIGS["ccq_bf16_n16k"]
    got, ref = _ccq(cfg, with_gla=True)
    assert_close(got, ref, "bf16", "ccq bf16 B4 H16 N=16384, whole tensor")
    assert _worst_slice(got, ref) <= 2e-2


def test_ccq_bf16_lowrank():
    # the same shapes with low-rank keys and gate bias +2, where the CCQ
    # correction is large: every slice
    cfg = inputs.CONFIGS["ccq_bf16_lowrank"]
    got, ref = _ccq(cfg, with_gla=True)
    assert_close(got, ref, "bf16", "ccq bf16 low-rank keys B4 H16 N=16384, whole tensor")
    assert _worst_slice(got, ref) <= 2e-2


@pytest.mark.parametrize("N,segments", [(1, 0), (63, 0), (65, 0), (1000, 1), (1000, 3), (777, 2)])
@pytest.mark.parametrize("lowrank", [False, True])
def test_ccq_bf16_d128_ragged(N, segments, lowrank):
    # the bf16 dk = 128 chunk pass at ragged lengths, one and several segments
    name = "ccq_bf16_lowrank" if lowrank else "ccq_bf16_n16k"
    cfg = inputs.CONFIGS[name].replace(name=name + "_ragged", cfg_id=304, B=2, H=2, N=N)
    got, ref = _ccq(cfg, segments=segments, with_gla=True)
    assert_close(got, ref, "bf16", "ccq bf16 dk=128 N=%d P=%d lowrank=%d" % (N, segments, lowrank))


@pytest.mark.parametrize("segments", [3, 4])
def test_ccq_bf16_sub_segments(segments):
    # N = 768 is 12 chunks: 3 segments of 4 chunks (two sub-segments each in the
    # segment-state pass) and 4 segments of 3 chunks (one each)
    cfg = inputs.CONFIGS["ccq_bf16_n16k"].replace(name="ccq_bf16_sub", B=1, H=2, N=768)
    got, ref = _ccq(cfg, segments=segments)
    assert_close(got, ref, "bf16", "ccq bf16 N=768 P=%d" % segments)


def test_ccq_segment_invariance_fp32():
    cfg = inputs.LinAttnConfig("ccq_seg", 303, B=1, H=2, N=2048, dk=64, dv=64, dtype="f32", lowrank_keys=4,
                               gate_bias=2.0)
    x = cuda(inputs.linattn_inputs(cfg, ccq=True))
    outs = [host(ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"], segments=s))
            for s in (1, 8)]
    e = float(np.max(np.abs(outs[0] - outs[1])) / np.max(np.abs(outs[0])))
    say("  ccq P=1 vs P=8 max-rel %.3e" % e)
    assert e <= 1e-5


def test_linattn_deterministic():
    cfg = inputs.CONFIGS["ccq_bf16_n16k"].replace(B=1, H=2, N=4096)
    x = cuda(inputs.linattn_inputs(cfg, ccq=True))
    a = ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"])
    b = ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"])
    assert torch.equal(a, b)
    a = linattn_chunk_forward(x["q"], x["k"], x["v"], x["g"])
    b = linattn_chunk_forward(x["q"], x["k"], x["v"], x["g"])
    assert torch.equal(a, b)
