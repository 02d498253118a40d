"""GMA forward on the GPU against the fp64 oracle (same seeded inputs)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_gmm_amd import gma_forward, inputs
from parity import assert_close, cuda, host, rel_l2, say

pytestmark = pytest.mark.gpu


def _run(cfg, N=None, causal=True, segments=0, eps=None, sl=None):
    """Runs the GPU path and the oracle on cfg; sl = list of (b, h) slices the
    oracle checks (None = all)."""
    x = inputs.gma_inputs(cfg, N=N)
    eps = cfg.eps if eps is None else eps
    say("gma: %s N=%d causal=%d segments=%d dtype=%s" % (cfg.name, x["q"].shape[2], causal, segments, cfg.dtype))
    d = cuda(x)
    out = gma_forward(d["q"], d["k"], d["v"], d["mu"], d["log_var"], d["logit_pi"], causal=causal, eps=eps,
                      segments=segments)
    torch.cuda.synchronize()
    got = host(out)
    if sl is None:
        ref = oracle.gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], causal=causal,
                                 eps=eps)
        return got, ref
    gs, rs = [], []
    for b, h in sl:
        ref = oracle.gma_forward(x["q"][b:b + 1, h:h + 1], x["k"][b:b + 1, h:h + 1], x["v"][b:b + 1, h:h + 1],
                                 x["mu"][h:h + 1], x["log_var"][h:h + 1], x["logit_pi"][h:h + 1], causal=causal,
                                 eps=eps)
        gs.append(got[b, h])
        rs.append(ref[0, 0])
    return np.stack(gs), np.stack(rs)


def test_gma_fp32_n256_causal():
    cfg = inputs.CONFIGS["gma_fp32_n256"]
    got, ref = _run(cfg)
    assert_close(got, ref, "f32", "gma fp32 N=256 causal")
    x = inputs.gma_inputs(cfg)
    brute = oracle.gma_brute(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], causal=True,
                             eps=cfg.eps)
    assert_close(got, brute, "f32", "gma fp32 N=256 vs materialised affinity")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("segments", [1, 3])
def test_gma_fp32_ragged(causal, segments):
    cfg = inputs.CONFIGS["gma_fp32_n256"].replace(name="gma_fp32_ragged", B=2, H=3, cfg_id=101)
    got, ref = _run(cfg, N=300, causal=causal, segments=segments)
    assert_close(got, ref, "f32", "gma fp32 N=300 causal=%d P=%d" % (causal, segments))


@pytest.mark.parametrize("K", [1, 5, 33, 64, 100, 200])
@pytest.mark.parametrize("d", [32, 64])
def test_gma_fp32_components(K, d):
    cfg = inputs.GmaConfig("gma_fp32_k", 102, B=1, H=2, N=130, d=d, K=K, dv=d, dtype="f32")
    for causal in (True, False):
        got, ref = _run(cfg, causal=causal, segments=2)
        assert_close(got, ref, "f32", "gma fp32 d=%d K=%d causal=%d" % (d, K, causal))


def test_gma_fp32_d128():
    cfg = inputs.GmaConfig("gma_fp32_d128", 103, B=1, H=2, N=200, d=128, K=100, dv=128, dtype="f32",
                           qk_scale=True)
    for causal in (True, False):
        got, ref = _run(cfg, causal=causal, segments=2)
        assert_close(got, ref, "f32", "gma fp32 d=128 causal=%d" % causal)


def test_gma_k1_is_running_mean():
    cfg = inputs.GmaConfig("gma_k1", 104, B=1, H=1, N=100, d=32, K=1, dv=32, dtype="f32", eps=0.5)
    x = inputs.gma_inputs(cfg)
    d = cuda(x)
    out = host(gma_forward(d["q"], d["k"], d["v"], d["mu"], d["log_var"], d["logit_pi"], causal=True, eps=0.5))
    v = x["v"].double().numpy()
    ref = np.cumsum(v, axis=2) / (np.arange(1, 101)[:, None] + 0.5)
    assert_close(out, ref, "f32", "gma K=1 running mean")


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 129])
def test_gma_short_sequences(N):
    cfg = inputs.GmaConfig("gma_short", 105, B=2, H=1, N=N, d=32, K=20, dv=32, dtype="f32")
    for causal in (True, False):
        got, ref = _run(cfg, causal=causal)
        assert_close(got, ref, "f32", "gma N=%d causal=%d" % (N, causal))


@pytest.mark.parametrize("causal", [True, False])
def test_gma_bf16_n4k(causal):
    cfg = inputs.CONFIGS["gma_bf16_n4k"]
    got, ref = _run(cfg, causal=causal)
    assert_close(got, ref, "bf16", "gma bf16 N=4096 causal=%d" % causal)


@pytest.mark.parametrize("causal", [True, False])
def test_gma_bf16_n16k(causal):
    # the 16K-token GMA workload (B=4, H=8) in the launch the bench times, every
    # (b, h) slice against the oracle
    cfg = inputs.CONFIGS["gma_bf16_n16k"]
    got, ref = _run(cfg, causal=causal)
    assert_close(got, ref, "bf16", "gma bf16 B4 H8 N=16384 causal=%d, whole tensor" % causal)
    worst = max(rel_l2(got[b, h], ref[b, h]) for b in range(cfg.B) for h in range(cfg.H))
    say("  worst (b,h) slice rel-L2 %.3e" % worst)
    assert worst <= 2e-2


@pytest.mark.parametrize("causal", [True, False])
def test_gma_bf16_d128_k256_ragged(causal):
    # the long-context shape (d = dv = 128, 256 components, mixture keys) at a
    # small, ragged N over several segments
    cfg = inputs.CONFIGS["gma_bf16_n128k"].replace(name="gma_bf16_wide", cfg_id=108, B=1, H=2, N=1000)
    for seg in (1, 5):
        got, ref = _run(cfg, causal=causal, segments=seg)
        assert_close(got, ref, "bf16", "gma bf16 d=128 K=256 N=1000 causal=%d P=%d" % (causal, seg))


def test_gma_bf16_n128k():
    # the long-context workload at full size (B=1, H=16, N=131072): every head,
    # every row against the oracle
    cfg = inputs.CONFIGS["gma_bf16_n128k"]
    got, ref = _run(cfg, causal=True)
    assert_close(got, ref, "bf16", "gma bf16 B1 H16 N=131072 causal, whole tensor")
    worst = max(rel_l2(got[0, h], ref[0, h]) for h in range(cfg.H))
    say("  worst head rel-L2 %.3e" % worst)
    assert worst <= 2e-2


def test_gma_bf16_ragged_multiseg():
    cfg = inputs.GmaConfig("gma_bf16_ragged", 106, B=2, H=2, N=1000, d=64, K=128, dv=64, qk_scale=True)
    for causal in (True, False):
        for seg in (1, 5):
            got, ref = _run(cfg, causal=causal, segments=seg)
            assert_close(got, ref, "bf16", "gma bf16 N=1000 causal=%d P=%d" % (causal, seg))


@pytest.mark.parametrize("d,K", [(32, 40), (64, 64), (32, 128)])
def test_gma_bf16_causal_stored_key_responsibilities(d, K):
    # the causal bf16 kernel over several segments, where the segment pass
    # stores every chunk's key responsibilities and the causal pass loads them:
    # both padded widths (64 and 128 components) and a ragged last chunk
    cfg = inputs.GmaConfig("gma_bf16_gk", 108, B=2, H=2, N=777, d=d, K=K, dv=d, qk_scale=d == 64)
    for seg in (2, 7):
        got, ref = _run(cfg, causal=True, segments=seg)
        assert_close(got, ref, "bf16", "gma bf16 d=%d K=%d N=777 causal P=%d" % (d, K, seg))


def test_gma_segment_invariance_fp32():
    cfg = inputs.GmaConfig("gma_seg", 107, B=1, H=2, N=1024, d=64, K=128, dv=64, dtype="f32", qk_scale=True)
    x = cuda(inputs.gma_inputs(cfg))
    outs = [host(gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], causal=True,
                             segments=s)) for s in (1, 8)]
    e = float(np.max(np.abs(outs[0] - outs[1])) / np.max(np.abs(outs[0])))
    say("  gma P=1 vs P=8 max-rel %.3e" % e)
    assert e <= 1e-5


def test_gma_deterministic():
    cfg = inputs.CONFIGS["gma_bf16_n4k"].replace(B=1, H=2)
    x = cuda(inputs.gma_inputs(cfg))
    a = gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"])
    b = gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"])
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,N", [("gma_bf16_n16k", 4096), ("gma_bf16_n16k", 16384), ("gma_bf16_n128k", 8010),
                                    ("gma_bf16_n128k", 32768)])
def test_stored_key_responsibilities_are_bit_identical(name, N):
    # the causal bf16 pass over several segments loads each chunk's key
    # responsibilities stored by the segment pass; the entry point that
    # allocates nothing routes the keys again in the causal pass, with the same
    # segment plan: the outputs must agree bit for bit (d = 64 with 128
    # components, and d = 128 with 256)
    import torch
    from linear_attention_gmm_amd import binding
    cfg = inputs.CONFIGS[name].replace(B=2, H=4, N=N) if name == "gma_bf16_n128k" else \
        inputs.CONFIGS[name].replace(B=2, N=N)
    x = cuda(inputs.gma_inputs(cfg))
    a = binding.gma_forward(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], causal=True, eps=cfg.eps)
    b = binding.gma_forward_noalloc(x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"], causal=True,
                                    eps=cfg.eps)
    torch.cuda.synchronize()
    say("  stored vs routed key responsibilities, N=%d: max |diff| %.3e" % (N, float((a.float() - b.float()).abs().max())))
    assert torch.equal(a, b)
