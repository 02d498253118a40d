"""Backward pass of GMA (causal and bidirectional) on the GPU against the fp64
reverse-mode oracle (oracle/grad.py) on the same seeded inputs."""
import numpy as np
import pytest
import torch

from linear_attention_gmm_amd import binding, inputs
from oracle import grad
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dmu", "dlog_var", "dlogit_pi")


def _case(cfg, N=None, heads=None, eps=None, causal=True):
    """GPU gradients of the whole config and the oracle's for the heads listed
    (all batch entries of a head: the parameter gradients sum over them)."""
    x = inputs.gma_inputs(cfg, N=N)
    eps = cfg.eps if eps is None else eps
    n = x["q"].shape[2]
    do = torch.from_numpy(np.random.default_rng([cfg.cfg_id, 98]).standard_normal(x["v"].shape)).to(x["v"].dtype)
    say("gma backward: %s N=%d d=%d K=%d dtype=%s causal=%d" % (cfg.name, n, cfg.d, cfg.K, cfg.dtype, causal))
    d = cuda(x)
    got = binding.gma_backward(d["q"], d["k"], d["v"], d["mu"], d["log_var"], d["logit_pi"], do.cuda(), eps=eps,
                               causal=causal)
    torch.cuda.synchronize()
    got = [host(t) for t in got]
    heads = list(range(cfg.H)) if heads is None else heads
    gs = [[] for _ in NAMES]
    rs = [[] for _ in NAMES]
    for h in heads:
        hs = slice(h, h + 1)
        ref = grad.gma_backward(x["q"][:, hs], x["k"][:, hs], x["v"][:, hs], x["mu"][hs], x["log_var"][hs],
                                x["logit_pi"][hs], do[:, hs], eps, causal)
        for i in range(3):
            gs[i].append(got[i][:, h])
            rs[i].append(ref[i][:, 0])
        for i in range(3, 6):
            gs[i].append(got[i][h])
            rs[i].append(ref[i][0])
    return [np.stack(t) for t in gs], [np.stack(t) for t in rs]


@pytest.mark.parametrize("d,K,N", [(32, 16, 200), (32, 40, 130), (64, 128, 97), (64, 63, 300)])
def test_gma_backward_fp32(d, K, N):
    cfg = inputs.GmaConfig("gma_bwd", 701, B=2, H=2, N=N, d=d, K=K, dv=d, dtype="f32")
    got, ref = _case(cfg)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "f32", "%s fp32 d=%d K=%d N=%d" % (name, d, K, N))


@pytest.mark.parametrize("N", [1, 16, 17])
def test_gma_backward_short(N):
    # As eps -> 0 the first token's output stops depending on the routing
    # (O_1 = v_1 A / (A + eps)): its routing gradients are O(eps) differences
    # of O(1) terms, which float32 resolves only to about 1e-2 relative at
    # eps = 1e-6. A larger eps keeps them well conditioned, so that these short
    # sequences (where the first tokens set the scale of the tensor) are checked
    # at the float32 bar.
    cfg = inputs.GmaConfig("gma_bwd_short", 702, B=1, H=2, N=N, d=32, K=16, dv=32, dtype="f32", eps=0.25)
    got, ref = _case(cfg)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "f32", "%s fp32 N=%d" % (name, N))


def test_gma_backward_bf16():
    # the 4K-token GMA shapes (d = dv = 64, K = 128, Q and K scaled by 1/8) on a
    # short ragged sequence
    cfg = inputs.CONFIGS["gma_bf16_n4k"].replace(name="gma_bwd_bf16", cfg_id=703, B=2, H=2, N=300)
    got, ref = _case(cfg)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "bf16", "%s bf16 N=300" % name)


def test_gma_backward_full_size_sampled():
    # the 4K-token GMA workload (B=4, H=8, bf16): the gradients of one head
    # (all four batch entries) against the oracle
    cfg = inputs.CONFIGS["gma_bf16_n4k"]
    got, ref = _case(cfg, heads=[5])
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "bf16", "%s bf16 4K workload, head 5" % name)


@pytest.mark.parametrize("d,K,N", [(32, 16, 200), (64, 63, 300)])
def test_gma_backward_bidirectional_fp32(d, K, N):
    cfg = inputs.GmaConfig("gma_bwd_bidir", 704, B=2, H=2, N=N, d=d, K=K, dv=d, dtype="f32")
    got, ref = _case(cfg, causal=False)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "f32", "%s fp32 bidirectional d=%d K=%d N=%d" % (name, d, K, N))


@pytest.mark.parametrize("N", [1, 17])
def test_gma_backward_bidirectional_short(N):
    # eps as in the causal short test: a one-token sequence is the same function
    cfg = inputs.GmaConfig("gma_bwd_bidir_short", 705, B=1, H=2, N=N, d=32, K=16, dv=32, dtype="f32", eps=0.25)
    got, ref = _case(cfg, causal=False)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "f32", "%s fp32 bidirectional N=%d" % (name, N))


def test_gma_backward_bidirectional_bf16():
    cfg = inputs.CONFIGS["gma_bf16_n4k"].replace(name="gma_bwd_bidir_bf16", cfg_id=706, B=2, H=2, N=300)
    got, ref = _case(cfg, causal=False)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "bf16", "%s bf16 bidirectional N=300" % name)


def test_gma_backward_deterministic():
    # fixed-order reductions: two calls give bit-identical gradients
    cfg = inputs.CONFIGS["gma_bf16_n4k"].replace(name="gma_bwd_det", cfg_id=707, B=2, H=2, N=777)
    x = cuda(inputs.gma_inputs(cfg))
    do = torch.randn_like(x["v"])
    a = binding.gma_backward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], do)
    b = binding.gma_backward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], do)
    for name, u, w in zip(NAMES, a, b):
        assert torch.equal(u, w), name


@pytest.mark.parametrize("d,K,N", [(128, 64, 150), (64, 200, 130), (128, 256, 100), (32, 129, 70)])
def test_gma_backward_wide_fp32(d, K, N):
    # d = 128 or more than 128 components: the inner linear attention on blocks
    # of 128 feature / value columns
    cfg = inputs.GmaConfig("gma_bwd_wide", 708, B=2, H=2, N=N, d=d, K=K, dv=d, dtype="f32")
    got, ref = _case(cfg)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "f32", "%s fp32 wide d=%d K=%d N=%d" % (name, d, K, N))


def test_gma_backward_wide_bidirectional_fp32():
    cfg = inputs.GmaConfig("gma_bwd_wide_bidir", 709, B=1, H=2, N=90, d=128, K=256, dv=128, dtype="f32")
    got, ref = _case(cfg, causal=False)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "f32", "%s fp32 wide bidirectional" % name)


@pytest.mark.parametrize("heads", [2, 16])
def test_gma_backward_long_context_shape(heads):
    # the long-context GMA shapes (d = dv = 128, K = 256, keys drawn from a
    # 256-cluster mixture, bf16) on a short ragged sequence; all 16 heads in
    # the second case
    cfg = inputs.CONFIGS["gma_bf16_n128k"].replace(name="gma_bwd_long", cfg_id=710, B=1, H=heads, N=200)
    got, ref = _case(cfg)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, "bf16", "%s bf16 long-context shapes, %d heads, N=200" % (name, heads))
