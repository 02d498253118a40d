"""Backward pass of the CCQ read on the GPU against the fp64 reverse-mode oracle
(oracle/grad.py) on the same seeded inputs. Low-rank keys with a strong gate
(bias +2) make the covariance term large, so that a mistake in its gradient
shows."""
import numpy as np
import pytest
import torch

from linear_attention_gmm_amd import binding, inputs
from oracle import grad
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dw", "db")


def _case(cfg, N=None, heads=None):
    """GPU gradients of the whole config and the oracle's for the heads listed
    (all batch entries of a head: dw and db sum over them)."""
    x = inputs.linattn_inputs(cfg, N=N, ccq=True)
    n = x["q"].shape[2]
    do = torch.from_numpy(np.random.default_rng([cfg.cfg_id, 97]).standard_normal(x["v"].shape)).to(x["v"].dtype)
    say("ccq backward: %s N=%d dk=%d dtype=%s" % (cfg.name, n, cfg.dk, cfg.dtype))
    d = cuda(x)
    got = binding.ccq_backward(d["q"], d["k"], d["v"], d["g"], d["w_lambda"], d["b_lambda"], do.cuda())
    torch.cuda.synchronize()
    got = [host(t) for t in got]
    heads = list(range(cfg.H)) if heads is None else heads
    gs = [[] for _ in NAMES]
    rs = [[] for _ in NAMES]
    for h in heads:
        hs = slice(h, h + 1)
        ref = grad.ccq_backward(x["q"][:, hs], x["k"][:, hs], x["v"][:, hs], x["g"][:, hs], x["w_lambda"][hs],
                                x["b_lambda"][hs], do[:, hs])
        for i in range(4):
            gs[i].append(got[i][:, h])
            rs[i].append(ref[i][:, 0])
        for i in range(4, 6):
            gs[i].append(got[i][h])
            rs[i].append(ref[i][0])
    return [np.stack(t) for t in gs], [np.stack(t) for t in rs]


def _check(got, ref, dtype, what):
    for name, a, r in zip(NAMES, got, ref):
        if name == "dg":
            # the first token's gate multiplies the empty state: its gradient is
            # zero in exact arithmetic and the rounding of q.dq - k.dk (which
            # cancel) otherwise; checked on the other tokens
            a, r = a[..., 1:], r[..., 1:]
        assert_close(a, r, dtype, "%s %s" % (name, what))


def test_ccq_backward_fp32_lowrank():
    # the low-rank fp32 CCQ case (B=1, H=2, N=300, dk=32)
    cfg = inputs.CONFIGS["ccq_fp32_lowrank"]
    got, ref = _case(cfg)
    _check(got, ref, "f32", "fp32 low-rank keys dk=32 N=300")


@pytest.mark.parametrize("dk,N", [(64, 200), (128, 130)])
def test_ccq_backward_fp32(dk, N):
    cfg = inputs.CONFIGS["ccq_fp32_lowrank"].replace(name="ccq_bwd", cfg_id=801, B=2, H=2, N=N, dk=dk, dv=dk)
    got, ref = _case(cfg)
    _check(got, ref, "f32", "fp32 low-rank keys dk=%d N=%d" % (dk, N))


@pytest.mark.parametrize("N", [1, 2, 65])
def test_ccq_backward_short(N):
    cfg = inputs.CONFIGS["ccq_fp32_lowrank"].replace(name="ccq_bwd_short", cfg_id=802, N=N)
    got, ref = _case(cfg)
    if N == 1:
        # one token: Sigma_1 = 0, so dw and db are zero (the rounding of
        # k k^T - m m^T in float32 leaves them at that level) and dg has no
        # token after the first
        for name, a, r in zip(NAMES[:3], got[:3], ref[:3]):
            assert_close(a, r, "f32", "%s fp32 N=1" % name)
        scale = np.max(np.abs(ref[0])) * np.max(np.abs(inputs.linattn_inputs(cfg, ccq=True)["q"].numpy()))
        assert np.max(np.abs(got[4])) <= 1e-5 * scale and np.max(np.abs(got[5])) <= 1e-5 * scale
    else:
        _check(got, ref, "f32", "fp32 N=%d" % N)


def test_ccq_backward_bf16():
    # the CCQ workload's distribution (unit-norm keys, gate bias -2) and the
    # low-rank one, bf16, on a ragged sequence
    for base, cid in (("ccq_bf16_n16k", 803), ("ccq_bf16_lowrank", 804)):
        cfg = inputs.CONFIGS[base].replace(name="ccq_bwd_bf16", cfg_id=cid, B=2, H=2, N=300)
        got, ref = _case(cfg)
        _check(got, ref, "bf16", "bf16 %s N=300" % base)


@pytest.mark.parametrize("dk", [32, 64])
def test_ccq_backward_bf16_narrow(dk):
    # bf16 at the narrower widths (the chunk passes of the decayed read, the
    # scans reading bf16 keys), low-rank keys, a ragged length
    cfg = inputs.CONFIGS["ccq_bf16_lowrank"].replace(name="ccq_bwd_bf16_narrow", cfg_id=807, B=2, H=2, N=333, dk=dk,
                                                     dv=dk)
    got, ref = _case(cfg)
    _check(got, ref, "bf16", "bf16 low-rank keys dk=%d N=333" % dk)


def test_ccq_backward_workload_shape_sampled():
    # the CCQ workload's shape (B=4, H=16, dk=dv=128, bf16) at N=2048 (the
    # autograd oracle keeps every step's state; at 16K tokens it would need
    # tens of GB), checked on one head over the four batch entries
    cfg = inputs.CONFIGS["ccq_bf16_n16k"]
    got, ref = _case(cfg, N=2048, heads=[9])
    _check(got, ref, "bf16", "bf16 CCQ workload shape N=2048, head 9")


def test_ccq_backward_lowrank_many_heads():
    # low-rank keys with gate bias +2 (a large covariance correction) at
    # B*H = 32, a ragged length, dk = dv = 128 in bf16: the decayed read's
    # gradients come from the fused bf16 backward kernel; two heads checked
    cfg = inputs.CONFIGS["ccq_bf16_lowrank"].replace(name="ccq_bwd_lowrank_fused", cfg_id=806, B=2, H=16, N=1000)
    got, ref = _case(cfg, heads=[3, 12])
    _check(got, ref, "bf16", "bf16 low-rank keys B2 H16 N=1000, heads 3 and 12")


def test_ccq_backward_deterministic():
    # fixed-order reductions: two calls give bit-identical gradients
    cfg = inputs.CONFIGS["ccq_bf16_lowrank"].replace(name="ccq_bwd_det", cfg_id=805, B=2, H=2, N=777)
    x = cuda(inputs.linattn_inputs(cfg, ccq=True))
    do = torch.randn_like(x["v"])
    a = binding.ccq_backward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"], do)
    b = binding.ccq_backward(x["q"], x["k"], x["v"], x["g"], x["w_lambda"], x["b_lambda"], do)
    for name, u, w in zip(NAMES, a, b):
        assert torch.equal(u, w), name
