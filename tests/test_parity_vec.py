"""Decayed linear attention with one decay per key feature, on the GPU against
the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_gmm_amd import binding, inputs
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu


def _run(cfg, segments=0, N=None, sl=None):
    x = inputs.linattn_inputs(cfg, N=N)
    say("glv: %s N=%d dk=%d dtype=%s segments=%d g_mean=%s g_one=%s" % (
        cfg.name, x["q"].shape[2], cfg.dk, cfg.dtype, segments, cfg.g_logit_mean, cfg.g_one))
    d = cuda(x)
    got = host(binding.linattn_vec_forward(d["q"], d["k"], d["v"], d["g"], segments=segments))
    if sl is None:
        return got, oracle.glv_forward(x["q"], x["k"], x["v"], x["g"])
    gs, rs = [], []
    for b, h in sl:
        sel = lambda t: t[b:b + 1, h:h + 1]
        rs.append(oracle.glv_forward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["g"]))[0, 0])
        gs.append(got[b, h])
    return np.stack(gs), np.stack(rs)


def _cfg(dk, dtype, **kw):
    return inputs.LinAttnConfig("glv_small", 401, B=2, H=2, N=300, dk=dk, dv=dk, dtype=dtype, vector_gates=True,
                                **kw)


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("segments", [1, 3])
def test_glv_fp32(dk, segments):
    got, ref = _run(_cfg(dk, "f32"), segments)
    assert_close(got, ref, "f32", "glv fp32 dk=%d P=%d" % (dk, segments))


@pytest.mark.parametrize("dk", [64, 128])
def test_glv_bf16(dk):
    got, ref = _run(_cfg(dk, "bf16"), 3)
    assert_close(got, ref, "bf16", "glv bf16 dk=%d" % dk)


@pytest.mark.parametrize("g_logit_mean", [-1.0, -6.0])
def test_glv_strong_decay_fp32(g_logit_mean):
    # g ~ 0.27 and g ~ 0.0025 per token and feature: whole sub-chunks decay by
    # many powers of two, which the scaled operands of the diagonal products
    # and the carried state must survive
    got, ref = _run(_cfg(64, "f32", g_logit_mean=g_logit_mean), 2)
    assert_close(got, ref, "f32", "glv fp32 strong decay %.0f" % g_logit_mean)


def test_glv_no_decay_fp32():
    cfg = _cfg(64, "f32", g_one=True)
    x = inputs.linattn_inputs(cfg)
    d = cuda(x)
    got = host(binding.linattn_vec_forward(d["q"], d["k"], d["v"], d["g"], segments=2))
    q, k, v = (x[n].double().numpy() for n in "qkv")
    assert_close(got, np.tril(q @ np.swapaxes(k, -1, -2)) @ v, "f32", "glv g=1 vs tril(QK^T)V")


@pytest.mark.parametrize("N", [1, 17, 64, 65])
def test_glv_short_and_ragged(N):
    got, ref = _run(_cfg(32, "f32"), 0, N=N)
    assert_close(got, ref, "f32", "glv fp32 N=%d" % N)


def test_glv_equal_gates_match_the_scalar_kernel():
    # a decay equal across features is the scalar form: both kernels against the
    # same oracle rows
    cfg = inputs.LinAttnConfig("glv_eq", 402, B=1, H=2, N=200, dk=64, dv=64, dtype="f32")
    x = inputs.linattn_inputs(cfg)
    d = cuda(x)
    gv = d["g"][..., None].expand(-1, -1, -1, 64).contiguous()
    got_v = host(binding.linattn_vec_forward(d["q"], d["k"], d["v"], gv))
    got_s = host(binding.linattn_chunk_forward(d["q"], d["k"], d["v"], d["g"]))
    ref = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])
    assert_close(got_v, ref, "f32", "glv with equal gates")
    assert_close(got_s, ref, "f32", "scalar kernel")


def test_glv_full_size_sampled():
    cfg = inputs.CONFIGS["glv_bf16_n8k"]
    got, ref = _run(cfg, sl=[(0, 0), (7, 15)])
    assert_close(got, ref, "bf16", "glv bf16 8K workload, slices (0,0) and (7,15)")


@pytest.mark.parametrize("dtype,dk,segments", [("f32", 64, 1), ("f32", 128, 3), ("bf16", 128, 3), ("f32", 32, 2)])
def test_glv_state_prefill_continue_decode(dtype, dk, segments):
    # prefill 300 tokens with the state handed back, continue for 77 from it,
    # then decode 5 one at a time; every row against the oracle's rows of the
    # whole sequence, the state against the oracle's state
    from test_parity_state import cmp_state
    c1, c2, n = 300, 377, 382
    cfg = inputs.LinAttnConfig("glv_state", 403, B=2, H=2, N=n, dk=dk, dv=dk, dtype=dtype, vector_gates=True)
    x = inputs.linattn_inputs(cfg)
    say("glv state: dk=%d dtype=%s segments=%d" % (dk, dtype, segments))
    d = cuda(x)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    ref = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"])
    _, rs1 = oracle.glv_forward(*[sl(x[m], 0, c1) for m in "qkvg"], return_state=True)
    _, rs3 = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"], return_state=True)
    o1, s1 = binding.linattn_vec_forward_state(*[sl(d[m], 0, c1) for m in "qkvg"], segments=segments)
    assert_close(host(o1), ref[:, :, :c1], dtype, "prefill out")
    cmp_state(host(s1), rs1, "gla", dk, dtype, "prefill state")
    o2, s2 = binding.linattn_vec_forward_state(*[sl(d[m], c1, c2) for m in "qkvg"], state_in=s1, state_out=s1,
                                               segments=segments)
    assert s2.data_ptr() == s1.data_ptr()
    assert_close(host(o2), ref[:, :, c1:c2], dtype, "continuation out")
    outs = [host(binding.linattn_vec_decode_step(*[d[m][:, :, i].contiguous() for m in "qkvg"], s2))
            for i in range(c2, n)]
    assert_close(np.stack(outs, axis=2), ref[:, :, c2:], dtype, "decode out")
    cmp_state(host(s2), rs3, "gla", dk, dtype, "state after decode")


def _with_tiny_decays(x, seed):
    """Decays near 1 (a large state builds up), then about 3% of the (token,
    feature) decays set to 1e-7 and 1% to exactly 0; the second chunk of every
    sequence keeps its ordinary decays, so the exact and the fast chunk paths
    alternate."""
    g = x["g"].clone()
    m = torch.from_numpy(np.random.default_rng(seed).random(tuple(g.shape)))
    g[m < 0.03] = 1e-7
    g[m > 0.99] = 0.0
    g[:, :, 64:128] = x["g"][:, :, 64:128]
    x = dict(x)
    x["g"] = g
    return x


@pytest.mark.parametrize("dtype,dk,segments", [("f32", 64, 1), ("f32", 64, 3), ("f32", 32, 2), ("bf16", 128, 3)])
def test_glv_tiny_and_zero_decays(dtype, dk, segments):
    # decays of 1e-7 and 0 are honoured exactly (no floor on g)
    cfg = inputs.LinAttnConfig("glv_tiny", 404, B=2, H=2, N=450, dk=dk, dv=dk, dtype=dtype, vector_gates=True,
                               g_logit_mean=6.0)
    x = _with_tiny_decays(inputs.linattn_inputs(cfg), 4040 + dk)
    say("glv tiny decays: dk=%d dtype=%s segments=%d" % (dk, dtype, segments))
    d = cuda(x)
    got = host(binding.linattn_vec_forward(d["q"], d["k"], d["v"], d["g"], segments=segments))
    ref = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"])
    assert_close(got, ref, dtype, "glv %s dk=%d P=%d with decays 1e-7 and 0" % (dtype, dk, segments))


@pytest.mark.parametrize("segments", [1, 2])
def test_glv_zero_decay_resets_the_state(segments):
    # a huge state is built without being read (q = 0, values x 1000, no
    # decay), then a decay of 0 on every feature at token 200 and 1e-7 on half
    # of them at token 230: the rows after must not see the old state at all
    # (a floor of 2^-15 on g would leave 3e-5 of it, far above the tolerance)
    cfg = inputs.LinAttnConfig("glv_reset", 406, B=1, H=2, N=260, dk=64, dv=64, dtype="f32", vector_gates=True,
                               g_one=True)
    x = inputs.linattn_inputs(cfg)
    x["q"][:, :, :200] = 0.0
    x["v"][:, :, :200] *= 1000.0
    x["g"][:, :, 200] = 0.0
    x["g"][:, :, 230, :32] = 1e-7
    d = cuda(x)
    got = host(binding.linattn_vec_forward(d["q"], d["k"], d["v"], d["g"], segments=segments))
    ref = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"])
    assert_close(got, ref, "f32", "glv state reset by g = 0, P=%d" % segments)
    floored = oracle.glv_forward(x["q"], x["k"], x["v"], torch.clamp(x["g"], min=2.0 ** -15))
    assert np.max(np.abs(floored - ref)) / np.max(np.abs(ref)) > 1e-2


@pytest.mark.parametrize("dtype,dk", [("f32", 64), ("bf16", 128)])
def test_glv_tiny_decays_prefill_continue_decode(dtype, dk):
    # prefill, continuation from the carried state and one-token steps agree
    # with the recurrence on the whole sequence when decays reach 1e-7 and 0
    from test_parity_state import cmp_state
    c1, c2, n = 300, 377, 382
    cfg = inputs.LinAttnConfig("glv_tiny_state", 405, B=2, H=2, N=n, dk=dk, dv=dk, dtype=dtype, vector_gates=True,
                               g_logit_mean=6.0)
    x = _with_tiny_decays(inputs.linattn_inputs(cfg), 4050 + dk)
    # a tiny decay on the decode tokens too
    x["g"][:, :, c2 + 1, :dk // 2] = 0.0
    say("glv tiny-decay state: dk=%d dtype=%s" % (dk, dtype))
    d = cuda(x)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    ref = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"])
    _, rs1 = oracle.glv_forward(*[sl(x[m], 0, c1) for m in "qkvg"], return_state=True)
    _, rs3 = oracle.glv_forward(x["q"], x["k"], x["v"], x["g"], return_state=True)
    o1, s1 = binding.linattn_vec_forward_state(*[sl(d[m], 0, c1) for m in "qkvg"], segments=3)
    assert_close(host(o1), ref[:, :, :c1], dtype, "tiny-decay prefill out")
    cmp_state(host(s1), rs1, "gla", dk, dtype, "tiny-decay prefill state")
    o2, s2 = binding.linattn_vec_forward_state(*[sl(d[m], c1, c2) for m in "qkvg"], state_in=s1, state_out=s1,
                                               segments=2)
    assert_close(host(o2), ref[:, :, c1:c2], dtype, "tiny-decay continuation out")
    outs = [host(binding.linattn_vec_decode_step(*[d[m][:, :, i].contiguous() for m in "qkvg"], s2))
            for i in range(c2, n)]
    assert_close(np.stack(outs, axis=2), ref[:, :, c2:], dtype, "tiny-decay decode out")
    cmp_state(host(s2), rs3, "gla", dk, dtype, "tiny-decay state after decode")
