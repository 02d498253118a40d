"""Backward pass of decayed linear attention on the GPU against the fp64
reverse-mode oracle (oracle/grad.py)."""
import numpy as np
import pytest
import torch

from linear_attention_gmm_amd import binding, inputs
from oracle import grad
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu


def _case(cfg, N=None, segments=0, sl=None):
    x = inputs.linattn_inputs(cfg, N=N)
    n = x["q"].shape[2]
    do = torch.from_numpy(np.random.default_rng([cfg.cfg_id, 99]).standard_normal(x["v"].shape)).to(x["v"].dtype)
    say("gla backward: %s N=%d dk=%d dtype=%s segments=%d" % (cfg.name, n, cfg.dk, cfg.dtype, segments))
    d = cuda(x)
    got = [host(t) for t in binding.linattn_chunk_backward(d["q"], d["k"], d["v"], d["g"], do.cuda(),
                                                           segments=segments)]
    sl = sl if sl is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    gs = [[], [], [], []]
    rs = [[], [], [], []]
    for b, h in sl:
        sel = lambda t: t[b:b + 1, h:h + 1]
        ref = grad.gla_backward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["g"]), sel(do))
        for i in range(4):
            gs[i].append(got[i][b, h])
            rs[i].append(ref[i][0, 0])
    return [np.stack(t) for t in gs], [np.stack(t) for t in rs]


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("segments", [1, 3])
def test_gla_backward_fp32(dk, segments):
    cfg = inputs.LinAttnConfig("gla_bwd", 501, B=2, H=2, N=300, dk=dk, dv=dk, dtype="f32")
    got, ref = _case(cfg, segments=segments)
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(a, r, "f32", "%s fp32 dk=%d P=%d" % (name, dk, segments))


@pytest.mark.parametrize("dk", [64, 128])
def test_gla_backward_bf16(dk):
    cfg = inputs.LinAttnConfig("gla_bwd", 502, B=2, H=2, N=300, dk=dk, dv=dk, dtype="bf16")
    got, ref = _case(cfg, segments=3)
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(a, r, "bf16", "%s bf16 dk=%d" % (name, dk))


@pytest.mark.parametrize("N", [1, 64, 65])
def test_gla_backward_short(N):
    cfg = inputs.LinAttnConfig("gla_bwd", 503, B=1, H=2, N=N, dk=32, dv=32, dtype="f32")
    got, ref = _case(cfg)
    for name, a, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(a, r, "f32", "%s fp32 N=%d" % (name, N))
    # the first token's gate multiplies the empty state: its gradient is zero
    # (up to rounding of q.dq - k.dk, which cancel), so dg is checked on the
    # scale of those terms
    scale = np.max(np.abs(got[0])) * 1.0 + 1e-30
    assert np.max(np.abs(got[3][:, 0])) <= 1e-4 * scale * 32
    if N > 1:
        assert_close(got[3][:, 1:], ref[3][:, 1:], "f32", "dg fp32 N=%d (tokens 1..)" % N)


def test_gla_backward_full_size_sampled():
    # the 8K-token GLA workload (B=8, H=16, d=128, bf16), checked on one slice
    cfg = inputs.CONFIGS["gla_bf16_n8k"]
    got, ref = _case(cfg, sl=[(5, 9)])
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(a, r, "bf16", "%s bf16 8K workload, slice (5,9)" % name)


# the dedicated bf16 d = 128 kernel runs from 32 sequences on (B=2, H=16 here);
# its cases are checked on four of the 32 slices, the last one included
SL32 = [(0, 0), (0, 9), (1, 4), (1, 15)]


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 200])
def test_gla_backward_bf16_d128_ragged(N):
    # bf16 with d = 128 (its own kernel): inside one chunk, whole chunks and a
    # ragged last chunk
    cfg = inputs.LinAttnConfig("gla_bwd128", 504, B=2, H=16, N=N, dk=128, dv=128, dtype="bf16")
    got, ref = _case(cfg, sl=SL32)
    for name, a, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(a, r, "bf16", "%s bf16 d=128 N=%d" % (name, N))
    # the first token's gate gradient is rounding of q.dq - k.dk (see above)
    scale = np.max(np.abs(got[0].astype(np.float32))) + 1e-30
    assert np.max(np.abs(got[3][:, 0])) <= 1e-3 * scale * 128
    if N > 1:
        assert_close(got[3][:, 1:], ref[3][:, 1:], "bf16", "dg bf16 d=128 N=%d (tokens 1..)" % N)


@pytest.mark.parametrize("N", [1100, 2600])
def test_gla_backward_bf16_d128_gate_slices(N):
    # several 1024-token slices of the gate gradient's suffix sums, the last
    # one ragged (2600 = 1024 + 1024 + 552, 1100 = 1024 + 76); dg on every token
    cfg = inputs.LinAttnConfig("gla_bwd128", 510, B=2, H=16, N=N, dk=128, dv=128, dtype="bf16")
    got, ref = _case(cfg, sl=[(0, 3), (1, 15)])
    for name, a, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(a, r, "bf16", "%s bf16 d=128 N=%d" % (name, N))
    assert_close(got[3][:, 1:], ref[3][:, 1:], "bf16", "dg bf16 d=128 N=%d (tokens 1..)" % N)


@pytest.mark.parametrize("g_logit_mean", [0.0, -1.0])
def test_gla_backward_bf16_d128_strong_decay(g_logit_mean):
    # gates around 0.5 and 0.27 per token: states forget within a few tokens
    cfg = inputs.LinAttnConfig("gla_bwd128", 505, B=2, H=16, N=300, dk=128, dv=128, dtype="bf16",
                               g_logit_mean=g_logit_mean)
    got, ref = _case(cfg, sl=SL32)
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(a, r, "bf16", "%s bf16 d=128 g logit mean %g" % (name, g_logit_mean))


def test_gla_backward_full_size_last_slice():
    # the 8K-token GLA workload, the last (b, h) block of the tensors
    cfg = inputs.CONFIGS["gla_bf16_n8k"]
    got, ref = _case(cfg, sl=[(7, 15)])
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(a, r, "bf16", "%s bf16 8K workload, slice (7,15)" % name)


def test_gla_backward_bf16_deterministic():
    cfg = inputs.LinAttnConfig("gla_bwd128", 506, B=2, H=16, N=777, dk=128, dv=128, dtype="bf16")
    x = cuda(inputs.linattn_inputs(cfg))
    do = torch.randn(x["v"].shape, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).cuda()
    a = binding.linattn_chunk_backward(x["q"], x["k"], x["v"], x["g"], do)
    b = binding.linattn_chunk_backward(x["q"], x["k"], x["v"], x["g"], do)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def _state_case(cfg, x, do, st_in, dst_out):
    d = cuda(x)
    got = binding.linattn_chunk_backward_state(d["q"], d["k"], d["v"], d["g"], do.cuda(),
                                               state_in=None if st_in is None else st_in.cuda(),
                                               dstate_out=None if dst_out is None else dst_out.cuda())
    B, H, D = cfg.B, cfg.H, cfg.dk
    r4 = lambda t: None if t is None else t.reshape(B, H, D, D).double().numpy()
    ref = grad.gla_backward(x["q"], x["k"], x["v"], x["g"], do, state_in=r4(st_in), dstate_out=r4(dst_out))
    return [host(t) for t in got], ref


@pytest.mark.parametrize("with_in,with_out", [(True, True), (True, False), (False, True)])
def test_gla_backward_state_bf16(with_in, with_out):
    # a carried state into the call and a gradient for the state after it;
    # gates near 1 (g ~ sigmoid(N(6, 1))) so that both states reach every token
    cfg = inputs.LinAttnConfig("gla_bwd_state", 507, B=2, H=2, N=200, dk=128, dv=128, dtype="bf16",
                               g_logit_mean=6.0)
    x = inputs.linattn_inputs(cfg)
    rng = np.random.default_rng([cfg.cfg_id, 97])
    do = torch.from_numpy(rng.standard_normal(x["v"].shape)).to(torch.bfloat16)
    shape = (cfg.B, cfg.H, cfg.dk * cfg.dv)
    st_in = torch.from_numpy(rng.standard_normal(shape) * 0.3).float() if with_in else None
    dst_out = torch.from_numpy(rng.standard_normal(shape) * 0.3).float() if with_out else None
    say("gla backward with state: in=%d out=%d" % (with_in, with_out))
    got, ref = _state_case(cfg, x, do, st_in, dst_out)
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got[:4], ref[:4]):
        assert_close(a, r, "bf16", "%s bf16 with state (in=%d out=%d)" % (name, with_in, with_out))
    assert_close(got[4].reshape(ref[4].shape), ref[4], "f32" if not with_in and not with_out else "bf16",
                 "dstate_in (in=%d out=%d)" % (with_in, with_out))


def test_gla_backward_state_chaining():
    # the gradients of a 300-token sequence from two calls: the second half
    # from the state after the first (the forward's carried state), its
    # dstate_in as the first half's dstate_out; against the oracle on the
    # whole sequence
    cfg = inputs.LinAttnConfig("gla_bwd_chain", 508, B=2, H=2, N=300, dk=128, dv=128, dtype="bf16")
    x = inputs.linattn_inputs(cfg)
    do = torch.from_numpy(np.random.default_rng([cfg.cfg_id, 96]).standard_normal(x["v"].shape)).to(torch.bfloat16)
    d = cuda(x)
    n1 = 130
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    _, s1 = binding.linattn_chunk_forward_state(*[sl(d[n], 0, n1) for n in "qkvg"])
    g2 = binding.linattn_chunk_backward_state(*[sl(d[n], n1, cfg.N) for n in "qkvg"], sl(do.cuda(), n1, cfg.N),
                                              state_in=s1)
    g1 = binding.linattn_chunk_backward_state(*[sl(d[n], 0, n1) for n in "qkvg"], sl(do.cuda(), 0, n1),
                                              dstate_out=g2[4])
    ref = grad.gla_backward(x["q"], x["k"], x["v"], x["g"], do)
    for i, name in enumerate(("dq", "dk", "dv", "dg")):
        got = np.concatenate([host(g1[i]), host(g2[i])], axis=2)
        assert_close(got, ref[i], "bf16", "%s of the whole sequence from two chained calls" % name)


def test_gla_backward_bf16_d128_few_sequences():
    # fewer than 32 sequences: the chunk passes over segments (the dedicated
    # kernel would leave most CUs idle); the same gradients
    cfg = inputs.LinAttnConfig("gla_bwd128_few", 509, B=1, H=4, N=700, dk=128, dv=128, dtype="bf16")
    got, ref = _case(cfg, segments=4)
    for name, a, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(a, r, "bf16", "%s bf16 d=128, 4 sequences" % name)
