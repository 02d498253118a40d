"""gma_forward_noalloc (the GMA forward on the library's fixed device scratch)
against gma_forward on the same inputs, through the C ABI: two calls in a row
on one GPU, the second with a smaller input, each held to the parity bar of its
dtype (bf16: rel-L2 <= 2e-2; float32: max-rel <= 1e-4)."""
import numpy as np
import pytest
import torch

from linear_attention_gmm_amd import binding, inputs
from parity import assert_close, cuda, host, say

pytestmark = pytest.mark.gpu


def _pair(cfg, causal, N=None):
    x = cuda(inputs.gma_inputs(cfg, N=N))
    args = (x["q"], x["k"], x["v"], x["mu"], x["log_var"], x["logit_pi"])
    say("noalloc: %s N=%d causal=%d dtype=%s" % (cfg.name, x["q"].shape[2], causal, cfg.dtype))
    ref = binding.gma_forward(*args, causal=causal, eps=cfg.eps)
    got = binding.gma_forward_noalloc(*args, causal=causal, eps=cfg.eps)
    torch.cuda.synchronize()
    g, r = host(got), host(ref)
    say("  max |noalloc - gma_forward| = %.3e" % float(np.max(np.abs(g - r))))
    return g, r


def test_noalloc_matches_gma_forward_two_calls():
    # first call: the 4096-token bf16 GMA workload, causal (several segments)
    big = inputs.CONFIGS["gma_bf16_n4k"]
    g, r = _pair(big, True)
    assert_close(g, r, "bf16", "noalloc vs gma_forward, bf16 B4 H8 N4096 causal")
    # second call, smaller: float32, ragged length, over the scratch the first
    # call left behind
    small = inputs.CONFIGS["gma_fp32_n256"].replace(name="gma_fp32_noalloc", B=2, H=3, cfg_id=109)
    g, r = _pair(small, True, N=300)
    assert_close(g, r, "f32", "noalloc vs gma_forward, fp32 B2 H3 N300 causal")
    g, r = _pair(small, False, N=300)
    assert_close(g, r, "f32", "noalloc vs gma_forward, fp32 B2 H3 N300 bidirectional")
