"""The segment-state pass and scan for bf16 at dk = dv = 128 on the GPU against
the fp64 oracle, over many segments: two sub-segments per segment, a scan over
up to 20 sub-segment states, and a scan that starts from a carried state.
Outputs and the state after the last token are compared."""
import numpy as np
import pytest

import oracle
from linear_attention_gmm_amd import binding, inputs
from parity import assert_close, cuda, host, say
from test_parity_state import cmp_state

pytestmark = pytest.mark.gpu


def _cfg(ccq, N, cfg_id=611):
    return inputs.LinAttnConfig("segpass", cfg_id, B=1, H=4, N=N, dk=128, dv=128, dtype="bf16",
                                lowrank_keys=4 if ccq else 0, gate_bias=2.0 if ccq else -2.0)


def _sl(t, a, b):
    return t[:, :, a:b].contiguous()


def _fwd(d, ccq, a, b, segments, state_in=None, t_in=0):
    args = [_sl(d[n], a, b) for n in "qkvg"]
    if ccq:
        return binding.ccq_forward_state(*args, d["w_lambda"], d["b_lambda"], state_in=state_in, t_in=t_in,
                                         segments=segments)
    return binding.linattn_chunk_forward_state(*args, state_in=state_in, segments=segments)


def _ref(x, ccq):
    if ccq:
        return oracle.ccq_forward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"], return_state=True)
    return oracle.gla_forward(x["q"], x["k"], x["v"], x["g"], return_state=True)


# 4133 tokens = 64 whole chunks and a tail of 37: 3 segments of 22 chunks, 7 of
# 10, 9 of 8 and 11 of 6, each cut into two sub-segments by the segment pass
@pytest.mark.parametrize("segments", [3, 7, 9, 11])
@pytest.mark.parametrize("ccq", [False, True])
def test_many_segments(ccq, segments):
    x = inputs.linattn_inputs(_cfg(ccq, 4133), ccq=ccq)
    say("segment pass: %s bf16 d=128 N=4133 segments=%d" % ("ccq" if ccq else "gla", segments))
    o, s = _fwd(cuda(x), ccq, 0, 4133, segments)
    ref, rs = _ref(x, ccq)
    kind = "ccq" if ccq else "gla"
    assert_close(host(o), ref, "bf16", "%s P=%d out" % (kind, segments))
    cmp_state(host(s), rs, kind, 128, "bf16", "%s P=%d state" % (kind, segments))


@pytest.mark.parametrize("ccq", [False, True])
def test_many_segments_state_in(ccq):
    # a prefill of 1000 tokens, then 3000 more in 5 segments of 10 chunks
    # starting from its state: the scan starts from the carried state
    x = inputs.linattn_inputs(_cfg(ccq, 4000, 612), ccq=ccq)
    d = cuda(x)
    o1, s1 = _fwd(d, ccq, 0, 1000, 1)
    o2, s2 = _fwd(d, ccq, 1000, 4000, 5, state_in=s1, t_in=1000)
    ref, rs = _ref(x, ccq)
    kind = "ccq" if ccq else "gla"
    got = np.concatenate([host(o1), host(o2)], axis=2)
    assert_close(got, ref, "bf16", "%s continuation over 5 segments out" % kind)
    cmp_state(host(s2), rs, kind, 128, "bf16", "%s continuation over 5 segments state" % kind)
