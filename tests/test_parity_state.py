"""Carried state on the GPU against the fp64 oracle: a prefill that returns the
state after its last token, a continuation from that state, and one-token
decode steps, for causal GMA, decayed linear attention and CCQ.

Every output row is compared with the oracle's rows of the WHOLE sequence
(prefix + continuation + decoded tokens), so a state that is wrong in any part
(decay, key sums, token count, normaliser) shows up in the rows that read it.
The states themselves are compared with the oracle's states at each cut."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_gmm_amd import binding, inputs
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu

CUT1, CUT2, STEPS = 300, 377, 5  # prefill, continuation, decode steps
NTOT = CUT2 + STEPS


def _sl(t, a, b):
    return t[:, :, a:b].contiguous()


def _tok(t, i):
    return t[:, :, i].contiguous()


def _parts(kind, d):
    """(name, start, stop) of the pieces of one state block."""
    if kind == "gma":
        dv, K = d
        return [("Vtil", 0, K * dv), ("Z", K * dv, K * dv + K)]
    dk = d
    p = [("S", 0, dk * dk)]
    if kind == "ccq":
        p += [("M", dk * dk, 2 * dk * dk), ("m", 2 * dk * dk, 2 * dk * dk + dk)]
    return p


def cmp_state(got, ref, kind, d, dtype, what):
    """Each piece of the state on its own scale (M and m dwarf S)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    for name, a, b in _parts(kind, d):
        assert_close(got[..., a:b], ref[..., a:b], dtype, "%s %s" % (what, name))


def _lin_case(dk, dtype, ccq, segments, inplace=False, cfg_id=301):
    # CCQ on low-rank keys with gate bias +2, where the covariance correction is
    # a large part of q_clean: a state with a wrong count or key sum shows
    cfg = inputs.LinAttnConfig("state_lin", cfg_id, B=2, H=2, N=NTOT, dk=dk, dv=dk, dtype=dtype,
                               lowrank_keys=4 if ccq else 0, gate_bias=2.0 if ccq else -2.0)
    x = inputs.linattn_inputs(cfg, ccq=ccq)
    say("state %s: dk=%d dtype=%s segments=%d inplace=%s" % ("ccq" if ccq else "gla", dk, dtype, segments, inplace))
    d = cuda(x)
    if ccq:
        par = (x["w_lambda"], x["b_lambda"])
        ref = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], *par)
        _, rs1 = oracle.ccq_forward(*[_sl(x[n], 0, CUT1) for n in "qkvg"], *par, return_state=True)
        _, rs2 = oracle.ccq_forward(*[_sl(x[n], CUT1, CUT2) for n in "qkvg"], *par, t0=CUT1, state_in=rs1,
                                    return_state=True)
        _, rs3 = oracle.ccq_forward(*[_sl(x[n], CUT2, NTOT) for n in "qkvg"], *par, t0=CUT2, state_in=rs2,
                                    return_state=True)
        gpar = (d["w_lambda"], d["b_lambda"])
        fwd = lambda a, b, st, t: binding.ccq_forward_state(*[_sl(d[n], a, b) for n in "qkvg"], *gpar, state_in=st,
                                                            t_in=t, segments=segments,
                                                            state_out=st if (inplace and st is not None) else None)
        step = lambda i, st: binding.ccq_decode_step(*[_tok(d[n], i) for n in "qkvg"], *gpar, st, t_prev=i)
    else:
        ref = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])
        _, rs1 = oracle.gla_forward(*[_sl(x[n], 0, CUT1) for n in "qkvg"], return_state=True)
        _, rs2 = oracle.gla_forward(*[_sl(x[n], CUT1, CUT2) for n in "qkvg"], state_in=rs1, return_state=True)
        _, rs3 = oracle.gla_forward(*[_sl(x[n], CUT2, NTOT) for n in "qkvg"], state_in=rs2, return_state=True)
        fwd = lambda a, b, st, t: binding.linattn_chunk_forward_state(
            *[_sl(d[n], a, b) for n in "qkvg"], state_in=st, segments=segments,
            state_out=st if (inplace and st is not None) else None)
        step = lambda i, st: binding.linattn_decode_step(*[_tok(d[n], i) for n in "qkvg"], st)
    return ref, (rs1, rs2, rs3), fwd, step


def _run_lin(dk, dtype, ccq, segments, inplace=False):
    ref, (rs1, rs2, rs3), fwd, step = _lin_case(dk, dtype, ccq, segments, inplace)
    kind = "ccq" if ccq else "gla"
    o1, s1 = fwd(0, CUT1, None, 0)
    assert_close(host(o1), ref[:, :, :CUT1], dtype, "prefill out")
    cmp_state(host(s1), rs1, kind, dk, dtype, "prefill state")
    o2, s2 = fwd(CUT1, CUT2, s1, CUT1)
    if inplace:
        assert s2.data_ptr() == s1.data_ptr()
    assert_close(host(o2), ref[:, :, CUT1:CUT2], dtype, "continuation out")
    cmp_state(host(s2), rs2, kind, dk, dtype, "continuation state")
    outs = [host(step(i, s2)) for i in range(CUT2, NTOT)]
    assert_close(np.stack(outs, axis=2), ref[:, :, CUT2:], dtype, "decode out")
    cmp_state(host(s2), rs3, kind, dk, dtype, "decode state")


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("segments", [1, 3])
@pytest.mark.parametrize("ccq", [False, True])
def test_lin_state_fp32(dk, segments, ccq):
    _run_lin(dk, "f32", ccq, segments)


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("ccq", [False, True])
def test_lin_state_bf16(dk, ccq):
    _run_lin(dk, "bf16", ccq, 3)


@pytest.mark.parametrize("ccq", [False, True])
def test_lin_state_in_place(ccq):
    _run_lin(64, "f32", ccq, 2, inplace=True)


@pytest.mark.parametrize("ccq", [False, True])
def test_lin_decode_from_empty_state(ccq):
    # decoding every token from a zero state is the recurrent form itself
    cfg = inputs.LinAttnConfig("state_lin_empty", 302, B=2, H=3, N=9, dk=32, dv=32, dtype="f32")
    x = inputs.linattn_inputs(cfg, ccq=ccq)
    d = cuda(x)
    st = torch.zeros((2, 3, (binding.ccq_state_size if ccq else binding.linattn_state_size)(32, 32)),
                     dtype=torch.float32, device="cuda")
    outs = []
    for i in range(cfg.N):
        if ccq:
            outs.append(host(binding.ccq_decode_step(*[_tok(d[n], i) for n in "qkvg"], d["w_lambda"], d["b_lambda"],
                                                     st, t_prev=i)))
        else:
            outs.append(host(binding.linattn_decode_step(*[_tok(d[n], i) for n in "qkvg"], st)))
    if ccq:
        ref, rs = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"], return_state=True)
    else:
        ref, rs = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"], return_state=True)
    assert_close(np.stack(outs, axis=2), ref, "f32", "decode-only out")
    cmp_state(host(st), rs, "ccq" if ccq else "gla", 32, "f32", "decode-only state")


def _gma_case(d, K, dtype, segments, qk_scale=False, inplace=False):
    cfg = inputs.GmaConfig("state_gma", 303, B=2, H=2, N=NTOT, d=d, K=K, dv=d, dtype=dtype, qk_scale=qk_scale,
                           eps=1e-6)
    x = inputs.gma_inputs(cfg)
    say("state gma: d=%d K=%d dtype=%s segments=%d inplace=%s" % (d, K, dtype, segments, inplace))
    dd = cuda(x)
    par = (x["mu"], x["log_var"], x["logit_pi"])
    gpar = (dd["mu"], dd["log_var"], dd["logit_pi"])
    ref = oracle.gma_forward(x["q"], x["k"], x["v"], *par, True, cfg.eps)
    _, rs1 = oracle.gma_forward(*[_sl(x[n], 0, CUT1) for n in "qkv"], *par, True, cfg.eps, return_state=True)
    _, rs2 = oracle.gma_forward(*[_sl(x[n], CUT1, CUT2) for n in "qkv"], *par, True, cfg.eps, state_in=rs1,
                                return_state=True)
    _, rs3 = oracle.gma_forward(*[_sl(x[n], CUT2, NTOT) for n in "qkv"], *par, True, cfg.eps, state_in=rs2,
                                return_state=True)

    def fwd(a, b, st):
        return binding.gma_forward_state(*[_sl(dd[n], a, b) for n in "qkv"], *gpar, state_in=st, eps=cfg.eps,
                                         segments=segments,
                                         state_out=st if (inplace and st is not None) else None)

    o1, s1 = fwd(0, CUT1, None)
    assert_close(host(o1), ref[:, :, :CUT1], dtype, "prefill out")
    cmp_state(host(s1), rs1, "gma", (d, K), dtype, "prefill memory")
    o2, s2 = fwd(CUT1, CUT2, s1)
    if inplace:
        assert s2.data_ptr() == s1.data_ptr()
    assert_close(host(o2), ref[:, :, CUT1:CUT2], dtype, "continuation out")
    cmp_state(host(s2), rs2, "gma", (d, K), dtype, "continuation memory")
    outs = [host(binding.gma_decode_step(*[_tok(dd[n], i) for n in "qkv"], *gpar, s2, eps=cfg.eps))
            for i in range(CUT2, NTOT)]
    assert_close(np.stack(outs, axis=2), ref[:, :, CUT2:], dtype, "decode out")
    cmp_state(host(s2), rs3, "gma", (d, K), dtype, "decode memory")


@pytest.mark.parametrize("segments", [1, 3])
@pytest.mark.parametrize("d,K", [(32, 16), (64, 64)])
def test_gma_state_fp32(d, K, segments):
    _gma_case(d, K, "f32", segments)


@pytest.mark.parametrize("d,K", [(64, 128), (128, 256), (32, 100)])
def test_gma_state_bf16(d, K):
    _gma_case(d, K, "bf16", 3, qk_scale=d == 64)


def test_gma_state_in_place():
    _gma_case(64, 32, "f32", 2, inplace=True)


@pytest.mark.parametrize("name", ["ccq_bf16_n16k", "ccq_bf16_lowrank"])
def test_ccq_full_size_prefill_then_decode(name):
    # the 16K-token CCQ workload (B=4, H=16, d=128, bf16; also with low-rank
    # keys and gate bias +2) as a prefill, then two decode steps; every slice
    cfg = inputs.CONFIGS[name]
    N = cfg.N
    x = inputs.linattn_inputs(cfg, N=N + 2, ccq=True)
    say("state ccq full size (%s): N=%d + 2 steps" % (name, N))
    d = cuda(x)
    out, st = binding.ccq_forward_state(*[_sl(d[n], 0, N) for n in "qkvg"], d["w_lambda"], d["b_lambda"])
    outs = [host(binding.ccq_decode_step(*[_tok(d[n], i) for n in "qkvg"], d["w_lambda"], d["b_lambda"], st,
                                         t_prev=i)) for i in (N, N + 1)]
    stg = host(st)
    ref, rs = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"], return_state=True)
    assert_close(host(out), ref[:, :, :N], "bf16", "prefill out (%s)" % name)
    assert_close(np.stack(outs, axis=2), ref[:, :, N:], "bf16", "decode out (%s)" % name)
    cmp_state(stg, rs, "ccq", 128, "bf16", "state after decode (%s)" % name)


@pytest.mark.parametrize("B", [2, 5, 11])
def test_gma_decode_from_empty_state(B):
    # the decode kernel serves 1, 4 or 8 batch entries of one head per
    # workgroup; 5 and 11 leave the last group partly filled
    cfg = inputs.GmaConfig("state_gma_empty", 304, B=B, H=3, N=7, d=32, K=20, dv=32, dtype="f32", eps=1e-6)
    x = inputs.gma_inputs(cfg)
    dd = cuda(x)
    st = torch.zeros((B, 3, binding.gma_state_size(20, 32)), dtype=torch.float32, device="cuda")
    outs = [host(binding.gma_decode_step(*[_tok(dd[n], i) for n in "qkv"], dd["mu"], dd["log_var"], dd["logit_pi"],
                                         st, eps=cfg.eps)) for i in range(cfg.N)]
    ref, rs = oracle.gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], True, cfg.eps,
                                 return_state=True)
    assert_close(np.stack(outs, axis=2), ref, "f32", "decode-only out")
    cmp_state(host(st), rs, "gma", (32, 20), "f32", "decode-only memory")


@pytest.mark.parametrize("kind", ["gla", "ccq", "gma"])
@pytest.mark.parametrize("n2", [1, 64])
def test_continuation_lengths_and_no_state_out(kind, n2):
    # a continuation of one token and of exactly one chunk, through the raw ABI
    # with state_out = NULL (the binding always asks for the state)
    n1 = 130
    if kind == "gma":
        cfg = inputs.GmaConfig("state_len", 305, B=1, H=3, N=n1 + n2, d=32, K=12, dv=32, dtype="f32", eps=1e-6)
        x = inputs.gma_inputs(cfg)
    else:
        cfg = inputs.LinAttnConfig("state_len", 305, B=1, H=3, N=n1 + n2, dk=32, dv=32, dtype="f32")
        x = inputs.linattn_inputs(cfg, ccq=kind == "ccq")
    d = cuda(x)
    say("continuation %s n1=%d n2=%d" % (kind, n1, n2))
    pre = {m: _sl(d[m], 0, n1) for m in ("qkvg" if kind != "gma" else "qkv")}
    post = {m: _sl(d[m], n1, n1 + n2) for m in ("qkvg" if kind != "gma" else "qkv")}
    L = binding.lib()
    out = torch.empty_like(post["v"])
    if kind == "gma":
        _, st = binding.gma_forward_state(pre["q"], pre["k"], pre["v"], d["mu"], d["log_var"], d["logit_pi"],
                                          eps=cfg.eps, segments=2)
        nb = binding.gma_workspace_bytes(1, 3, n2, 32, 12, 32, True, torch.float32, 0)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        rc = L.gma_forward_state(post["q"].data_ptr(), post["k"].data_ptr(), post["v"].data_ptr(),
                                 d["mu"].data_ptr(), d["log_var"].data_ptr(), d["logit_pi"].data_ptr(),
                                 out.data_ptr(), 1, 3, n2, 32, 12, 32, cfg.eps, binding.LM_F32, 0, st.data_ptr(),
                                 None, ws.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
        ref = oracle.gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], True, cfg.eps)
    elif kind == "gla":
        _, st = binding.linattn_chunk_forward_state(pre["q"], pre["k"], pre["v"], pre["g"], segments=2)
        nb = binding.linattn_workspace_bytes(1, 3, n2, 32, 32, 64, torch.float32, 0)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        rc = L.linattn_chunk_forward_state(post["q"].data_ptr(), post["k"].data_ptr(), post["v"].data_ptr(),
                                           post["g"].data_ptr(), out.data_ptr(), 1, 3, n2, 32, 32, 64,
                                           binding.LM_F32, 0, st.data_ptr(), None, ws.data_ptr(), nb,
                                           torch.cuda.current_stream().cuda_stream)
        ref = oracle.gla_forward(x["q"], x["k"], x["v"], x["g"])
    else:
        _, st = binding.ccq_forward_state(pre["q"], pre["k"], pre["v"], pre["g"], d["w_lambda"], d["b_lambda"],
                                          segments=2)
        nb = binding.ccq_workspace_bytes(1, 3, n2, 32, 32, 64, torch.float32, 0)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        rc = L.ccq_forward_state(post["q"].data_ptr(), post["k"].data_ptr(), post["v"].data_ptr(),
                                 post["g"].data_ptr(), d["w_lambda"].data_ptr(), d["b_lambda"].data_ptr(),
                                 out.data_ptr(), 1, 3, n2, 32, 32, 64, binding.LM_F32, 0, n1, st.data_ptr(), None,
                                 ws.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
        ref = oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"])
    assert rc == binding.LM_OK, L.lm_last_error().decode()
    assert_close(host(out), ref[:, :, n1:], "f32", "continuation of %d token(s)" % n2)
