"""Benchmark: forward head-tokens/s of causal GMA and CCQ at 16K tokens on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--secondary] [--decode]

One step is one forward of each headline path on its own synthetic batch:
  * causal Gaussian Mixture Attention, bf16 in / fp32 accumulate:
    B=4, H=8, N=16384, d=dv=64, K=128 components;
  * CCQ read over gated linear attention, bf16 in / fp32 accumulate:
    B=4, H=16, N=16384, dk=dv=128, chunk 64.
value = (head-tokens of both batches) x steps / wall time of the timed region,
where a head-token is one (b, h, n) row. Inputs are resident in HBM before
timing starts. Each path rotates through copies of its inputs totalling more
than the 256 MB last-level cache, so no step reads a previous step's inputs
from cache.

The JSON line also holds:
  * roofline: the entry point that takes longer per step (its kernels measured
    with HIP events on the stream they run on), as algorithmic HBM bytes per
    call / average call time, against MI355X's 8 TB/s. traffic is the measured
    HBM bytes per call of that entry point (rocprofv3 FETCH_SIZE + WRITE_SIZE
    runs, scaled by the same counters on a copy of known size), read from
    profiles/traffic.json when it was taken on the current kernel sources,
    else null;
  * cpu_baseline: the fp64 oracle on a bounded sample of the same workload
    (one (b, h) slice per host thread at full length, repeated until at least
    10 s of work) on the host cores;
  * parts: per-path rates;
  * secondary (--secondary): the bidirectional 16K GMA, the 8K-token GLA
    forward and backward, the per-feature-decay forward, the long-context GMA,
    the causal GMA backward at the 16K GMA shapes, the CCQ backward at the
    CCQ workload, the gated delta rule at the 8K-token GLA shape and the CCQ
    read over it at the CCQ workload, each against 8 TB/s of
    its algorithmic bytes (and, for the long-context GMA, the bf16 MFMA peak);
  * decode (--decode): the one-token steps at the model shapes of the two
    workloads, batched so that the states (about 0.5 GB) exceed the cache,
    against the same 8 TB/s (the state is read and written once per step).

    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR

turns the counter collections of two runs of this bench under
`rocprofv3 --pmc FETCH_SIZE` and `rocprofv3 --pmc WRITE_SIZE` (csv output)
into profiles/traffic.json and prints a summary table. Each run of the bench
first copies a 384 MiB buffer once; that copy's counters give the scale.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
LLC_BYTES = 256 << 20
METRIC = "fwd tokens/s per head at N=16K (causal GMA, CCQ-GLA) + % MFMA/HBM roofline"
CALIB_BYTES = 384 << 20  # differs from every input tensor size
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# kernels launched by each entry point (name fragments as rocprofv3 reports them)
ENTRY_KERNELS = {
    "gma_forward": ("gma4fast6kernel", "lm::gma::fast::kernel", "gma_kernel", "prep_kernel", "lm::gma::scan_kernel"),
    "ccq_forward": ("lin_kernelIDF16bLi128ELb1", "lm::lin::scan_kernel", "lm::ccqp::chunk_kernel"),
}


# Sources of the two measured entry points (their kernels, launchers and the
# ABI layer that plans their segments). The one-token steps and the
# per-feature-decay kernel are not part of the measured step.
DIGEST_SOURCES = ("abi.cpp", "launch.hpp", "mfma.hpp", "gma.hip", "gma.hpp", "gma_bf16.hip", "gma_generic.hpp",
                  "gma_wide.hip", "linattn.hip", "ccq_pipe.hip")


def sources_digest():
    """Hash of the measured entry points' sources and of the build script that
    sets their compile flags (identifies the code the counters were taken on).
    Lines that hold only a comment (// in C++, # in Python) are left out, so
    that editing such a comment keeps the digest. Only --summarize-pmc, which
    reads fresh counters, records it in profiles/traffic.json."""
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "linear_attention_gmm_amd", "csrc", f) for f in DIGEST_SOURCES]
    files.append(os.path.join(ROOT, "linear_attention_gmm_amd", "build.py"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            for line in fh.read().splitlines(keepends=True):
                if not line.lstrip().startswith((b"//", b"#")):
                    h.update(line)
    return h.hexdigest()[:16]


def host_cpu():
    """(model name, logical CPUs this process may run on, logical CPUs of the host)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 0
    return model, avail, os.cpu_count() or 0


def gma_bytes_per_head_token(cfg, esize=2):
    # q, k, v read + out written
    return (2 * cfg.d + 2 * cfg.dv) * esize


def gma_flops_per_head_token(cfg):
    # routing of q and k (8 K d), write + read (4 K (dv + 1))
    return 8 * cfg.K * cfg.d + 4 * cfg.K * (cfg.dv + 1)


def ccq_bytes_per_head_token(cfg, esize=2):
    # q, k, v read + out written + the fp32 decay
    return (2 * cfg.dk + 2 * cfg.dv) * esize + 4


def ccq_flops_per_head_token(cfg):
    return 4 * cfg.dk * cfg.dv + 4 * cfg.dk * cfg.dk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps (the GPU's clocks rise over the first "
                         "tens of ms of sustained work; 0 times that rise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", action="store_true",
                    help="also time bidirectional GMA, GLA (forward and backward), per-feature decay and long GMA")
    ap.add_argument("--decode", action="store_true",
                    help="also time the one-token decode steps on states larger than the last-level cache")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs of this bench into profiles/traffic.json")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(every (b, h) slice is independent, so data or head parallelism would need no exchange). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_gmm_amd import ccq_forward, gma_forward, inputs, linattn_chunk_forward

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gcfg = inputs.CONFIGS["gma_bf16_n16k"]
    ccfg = inputs.CONFIGS["ccq_bf16_n16k"]

    t_gen = time.perf_counter()
    gx = inputs.gma_inputs(gcfg)
    cx = inputs.linattn_inputs(ccfg, ccq=True)
    print("inputs generated in %.1f s" % (time.perf_counter() - t_gen), file=sys.stderr, flush=True)

    def copies(x, keys, nbytes):
        n = max(2, math.ceil(2 * LLC_BYTES / nbytes))
        base = {k: v.to(dev) for k, v in x.items() if isinstance(v, torch.Tensor)}
        out = [base]
        for _ in range(n - 1):
            out.append({k: (v.clone() if k in keys else v) for k, v in base.items()})
        return out

    g_in_bytes = sum(gx[k].numel() * gx[k].element_size() for k in ("q", "k", "v"))
    c_in_bytes = sum(cx[k].numel() * cx[k].element_size() for k in ("q", "k", "v", "g"))
    gset = copies(gx, ("q", "k", "v"), g_in_bytes)
    cset = copies(cx, ("q", "k", "v", "g"), c_in_bytes)
    gout = torch.empty_like(gset[0]["v"])
    cout = torch.empty_like(cset[0]["v"])
    gws = torch.empty(max(16, __import__("linear_attention_gmm_amd").gma_workspace_bytes(
        gcfg.B, gcfg.H, gcfg.N, gcfg.d, gcfg.K, gcfg.dv, True, torch.bfloat16)), dtype=torch.uint8, device=dev)
    cws = torch.empty(max(16, __import__("linear_attention_gmm_amd").ccq_workspace_bytes(
        ccfg.B, ccfg.H, ccfg.N, ccfg.dk, ccfg.dv, 64, torch.bfloat16)), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        a = gset[i % len(gset)]
        b = cset[i % len(cset)]
        if ev is not None:
            ev[0].record()
        gma_forward(a["q"], a["k"], a["v"], a["mu"], a["log_var"], a["logit_pi"], causal=True, eps=gcfg.eps,
                    out=gout, workspace=gws)
        if ev is not None:
            ev[1].record()
        ccq_forward(b["q"], b["k"], b["v"], b["g"], b["w_lambda"], b["b_lambda"], out=cout, workspace=cws)
        if ev is not None:
            ev[2].record()

    # one copy of known size: its HBM counters scale the kernels' counters
    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    # The GPU's clocks rise over the first tens of milliseconds of sustained
    # work. Untimed steps for args.settle seconds first, so that the warm-up
    # and the timed steps run at the steady clock (with 5 warm-up steps and no
    # settle the timed steps caught the rise: about 0.66 against 0.59 ms per step).
    n_settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(8):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(n_settle + i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(n_settle + args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0

    g_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    c_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    g_tok = gcfg.B * gcfg.H * gcfg.N
    c_tok = ccfg.B * ccfg.H * ccfg.N
    value = (g_tok + c_tok) * args.steps / wall

    g_bytes = g_tok * gma_bytes_per_head_token(gcfg)
    c_bytes = c_tok * ccq_bytes_per_head_token(ccfg)
    parts = {
        "gma_causal": {"head_tokens_per_s": g_tok / (g_ms * 1e-3), "ms_per_call": g_ms,
                       "alg_GBps": g_bytes / (g_ms * 1e-3) / 1e9,
                       "hbm_frac": g_bytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "alg_TFLOPs": g_tok * gma_flops_per_head_token(gcfg) / (g_ms * 1e-3) / 1e12,
                       "alg_bytes_per_call": g_bytes},
        "ccq": {"head_tokens_per_s": c_tok / (c_ms * 1e-3), "ms_per_call": c_ms,
                "alg_GBps": c_bytes / (c_ms * 1e-3) / 1e9,
                "hbm_frac": c_bytes / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "alg_TFLOPs": c_tok * ccq_flops_per_head_token(ccfg) / (c_ms * 1e-3) / 1e12,
                "alg_bytes_per_call": c_bytes},
    }
    dom = "ccq" if c_ms >= g_ms else "gma_causal"
    achieved = parts[dom]["alg_GBps"]
    traffic = None
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as fh:
            tj = json.load(fh)
        entry = "ccq_forward" if dom == "ccq" else "gma_forward"
        if tj.get("sources") == sources_digest() and entry in tj.get("bytes_per_call", {}):
            traffic = tj["bytes_per_call"][entry]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": "ccq_forward (segment-state + chunk kernels)" if dom == "ccq"
                else "gma_forward (prep + segment-state + chunk kernels)",
                "alg_bytes_per_call": parts[dom]["alg_bytes_per_call"], "avg_call_ms": parts[dom]["ms_per_call"]}

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; distributions of the GMA and CCQ workloads)",
        "config": {"workload": "causal GMA B4 H8 N16384 d64 K128 dv64 + CCQ-GLA B4 H16 N16384 dk=dv=128, "
                               "bf16 inputs, fp32 accumulation, chunk 64",
                   "head_tokens_per_step": g_tok + c_tok},
        "roofline": roofline,
        "parts": parts,
    }

    if args.secondary:
        sec = {}
        for name, fn in (("gma_bidir_n16k", "bidir"), ("gla_bf16_n8k", "gla"), ("gla_backward_bf16_n8k", "glab"),
                         ("glv_bf16_n8k", "glv"), ("gma_bf16_n128k", "gma5"), ("gma_backward_bf16_n16k", "gmab"),
                         ("ccq_backward_bf16_n16k", "ccqb"), ("deltanet_bf16_n8k", "gdn"),
                         ("ccq_deltanet_bf16_n16k", "ccqgdn"), ("gma_backward_bf16_n128k", "gmab5")):
            if fn == "bidir":
                a = gset[0]
                call = lambda: gma_forward(a["q"], a["k"], a["v"], a["mu"], a["log_var"], a["logit_pi"],
                                           causal=False, out=gout, workspace=gws)
                tok, byt = g_tok, g_bytes
            elif fn == "gla":
                cfg = inputs.CONFIGS["gla_bf16_n8k"]
                x = {k: v.to(dev) for k, v in inputs.linattn_inputs(cfg).items()}
                call = lambda: linattn_chunk_forward(x["q"], x["k"], x["v"], x["g"])
                tok = cfg.B * cfg.H * cfg.N
                byt = tok * ccq_bytes_per_head_token(cfg)
            elif fn == "glab":
                from linear_attention_gmm_amd import linattn_backward_workspace_bytes, linattn_chunk_backward
                cfg = inputs.CONFIGS["gla_bf16_n8k"]
                xb = {k: v.to(dev) for k, v in inputs.linattn_inputs(cfg).items()}
                dout = torch.randn_like(xb["v"])
                wsb = torch.empty(linattn_backward_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.dk, cfg.dv, 64,
                                                                   torch.bfloat16), dtype=torch.uint8, device=dev)
                call = lambda: linattn_chunk_backward(xb["q"], xb["k"], xb["v"], xb["g"], dout, workspace=wsb)
                tok = cfg.B * cfg.H * cfg.N
                # read Q, K, V, dO (bf16) and g; write dQ, dK, dV (bf16) and dg (fp32)
                byt = tok * (7 * cfg.dk * 2 + 8)
            elif fn == "glv":
                from linear_attention_gmm_amd import linattn_vec_forward
                cfg = inputs.CONFIGS["glv_bf16_n8k"]
                xv = {k: v.to(dev) for k, v in inputs.linattn_inputs(cfg).items()}
                call = lambda: linattn_vec_forward(xv["q"], xv["k"], xv["v"], xv["g"])
                tok = cfg.B * cfg.H * cfg.N
                # Q, K, V, O in bf16 plus one fp32 decay per key feature
                byt = tok * (4 * cfg.dk * 2 + 4 * cfg.dk)
            elif fn == "gmab":
                from linear_attention_gmm_amd import gma_backward, gma_backward_workspace_bytes
                a = gset[0]
                gdo = torch.randn_like(a["v"])
                wsg = torch.empty(gma_backward_workspace_bytes(gcfg.B, gcfg.H, gcfg.N, gcfg.d, gcfg.K, gcfg.dv),
                                  dtype=torch.uint8, device=dev)
                call = lambda: gma_backward(a["q"], a["k"], a["v"], a["mu"], a["log_var"], a["logit_pi"], gdo,
                                            eps=gcfg.eps, workspace=wsg)
                tok = g_tok
                # read Q, K, V, dO and write dQ, dK, dV (bf16); parameters are negligible
                byt = tok * 7 * gcfg.d * 2
            elif fn == "gmab5":
                from linear_attention_gmm_amd import gma_backward, gma_backward_workspace_bytes
                cfg = inputs.CONFIGS["gma_bf16_n128k"]
                y5 = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inputs.gma_inputs(cfg).items()}
                g5do = torch.randn_like(y5["v"])
                ws5 = torch.empty(gma_backward_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d, cfg.K, cfg.dv),
                                  dtype=torch.uint8, device=dev)
                call = lambda: gma_backward(y5["q"], y5["k"], y5["v"], y5["mu"], y5["log_var"], y5["logit_pi"], g5do,
                                            eps=cfg.eps, workspace=ws5)
                tok = cfg.B * cfg.H * cfg.N
                # read Q, K, V, dO and write dQ, dK, dV (bf16); parameters are negligible
                byt = tok * 7 * cfg.d * 2
            elif fn == "ccqb":
                from linear_attention_gmm_amd import ccq_backward, ccq_backward_workspace_bytes
                b_ = cset[0]
                cdo = torch.randn_like(b_["v"])
                wsc = torch.empty(ccq_backward_workspace_bytes(ccfg.B, ccfg.H, ccfg.N, ccfg.dk, ccfg.dv),
                                  dtype=torch.uint8, device=dev)
                call = lambda: ccq_backward(b_["q"], b_["k"], b_["v"], b_["g"], b_["w_lambda"], b_["b_lambda"], cdo,
                                            workspace=wsc)
                tok = c_tok
                # read Q, K, V, dO (bf16) and g; write dQ, dK, dV (bf16) and dg (fp32)
                byt = tok * (7 * ccfg.dk * 2 + 8)
            elif fn in ("gdn", "ccqgdn"):
                from linear_attention_gmm_amd import (ccq_deltanet_forward, ccq_deltanet_workspace_bytes,
                                                      deltanet_chunk_forward)
                cfg = inputs.CONFIGS["deltanet_bf16_n8k" if fn == "gdn" else "ccq_deltanet_bf16_n16k"]
                xd = {k: v.to(dev) for k, v in inputs.linattn_inputs(cfg, ccq=fn == "ccqgdn").items()}
                dout_ = torch.empty_like(xd["v"])
                if fn == "gdn":
                    call = lambda: deltanet_chunk_forward(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], out=dout_)
                else:
                    wsd = torch.empty(ccq_deltanet_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.dk, cfg.dv),
                                      dtype=torch.uint8, device=dev)
                    call = lambda: ccq_deltanet_forward(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"],
                                                        xd["w_lambda"], xd["b_lambda"], out=dout_, workspace=wsd)
                tok = cfg.B * cfg.H * cfg.N
                # Q, K, V read and O written (bf16), decay and step size (fp32)
                byt = tok * ((2 * cfg.dk + 2 * cfg.dv) * 2 + 8)
            else:
                cfg = inputs.CONFIGS["gma_bf16_n128k"]
                y = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inputs.gma_inputs(cfg).items()}
                call = lambda: gma_forward(y["q"], y["k"], y["v"], y["mu"], y["log_var"], y["logit_pi"], causal=True)
                tok = cfg.B * cfg.H * cfg.N
                byt = tok * gma_bytes_per_head_token(cfg)
            for _ in range(2):
                call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            n = 5
            for _ in range(n):
                call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            sec[name] = {"ms_per_call": ms, "head_tokens_per_s": tok / (ms * 1e-3),
                         "alg_GBps": byt / (ms * 1e-3) / 1e9, "hbm_frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            if fn == "gma5":
                sec[name]["alg_TFLOPs"] = tok * gma_flops_per_head_token(cfg) / (ms * 1e-3) / 1e12
                sec[name]["mfma_frac"] = sec[name]["alg_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
        result["secondary"] = sec

    if args.decode:
        result["decode"] = decode_steps(torch, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(gx, cx, gcfg, ccfg)
    print(json.dumps(result), flush=True)


def decode_steps(torch, dev, steps=20):
    """One-token steps of the mixers at the model shapes of the 8K- and 16K-token
    workloads, with batches whose states (about 0.5 GB) exceed the 256 MB
    last-level cache. Algorithmic bytes per step: the state read and written
    once, plus q, k, v, out (and g) in bf16."""
    import numpy as np

    import linear_attention_gmm_amd as lm

    res = {}
    gen = torch.Generator(device=dev).manual_seed(7)
    for name, kind, B, H, d, K in (("gma_decode_b2048_h8_d64_k128", "gma", 2048, 8, 64, 128),
                                   ("gla_decode_b512_h16_d128", "gla", 512, 16, 128, 0),
                                   ("glv_decode_b512_h16_d128", "glv", 512, 16, 128, 0),
                                   ("ccq_decode_b256_h16_d128", "ccq", 256, 16, 128, 0)):
        rnd = lambda *shape: torch.randn(*shape, generator=gen, device=dev)
        q, k, v = (rnd(B, H, d).bfloat16() for _ in range(3))
        out = torch.empty_like(v)
        if kind == "gma":
            sf = lm.gma_state_size(K, d)
            mu, lv, lp = rnd(H, K, d), torch.nn.functional.softplus(rnd(H, K, d)), rnd(H, K)
            call = lambda st: lm.gma_decode_step(q, k, v, mu, lv, lp, st, out=out)
        else:
            sf = lm.ccq_state_size(d, d) if kind == "ccq" else lm.linattn_state_size(d, d)
            g = torch.sigmoid(rnd(B, H, d) + 3.0) if kind == "glv" else torch.sigmoid(rnd(B, H) + 3.0)
            if kind == "glv":
                call = lambda st: lm.linattn_vec_decode_step(q, k, v, g, st, out=out)
            elif kind == "ccq":
                w, b = rnd(H, d) / d ** 0.5, torch.full((H,), -2.0, device=dev)
                call = lambda st: lm.ccq_decode_step(q, k, v, g, w, b, st, t_prev=16384, out=out)
            else:
                call = lambda st: lm.linattn_decode_step(q, k, v, g, st, out=out)
        st = rnd(B, H, sf) * 0.01
        io = B * H * (4 * d * 2 + {"gma": 0, "glv": 4 * d}.get(kind, 4))
        nbytes = 2 * st.numel() * 4 + io
        for _ in range(3):
            call(st)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(steps):
            call(st)
            evs[i + 1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]))
        res[name] = {"ms_per_step": ms, "tokens_per_s": B * H / (ms * 1e-3), "state_MB": st.numel() * 4 / 1e6,
                     "alg_bytes_per_step": nbytes, "alg_GBps": nbytes / (ms * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del st, q, k, v, out
    return res


def cpu_baseline(gx, cx, gcfg, ccfg, min_seconds=10.0, max_rounds=20):
    """The fp64 oracle (as it is) on a bounded sample of the step's workload:
    the first S (b, h) slices of each path at full length, S = host threads
    (at most the slice count), so every thread has one slice of each; the
    sample is run again until at least min_seconds of work are timed."""
    import numpy as np

    import oracle

    threads = oracle.num_threads()
    sg = min(threads, gcfg.B * gcfg.H)
    sc = min(threads, ccfg.B * ccfg.H)

    def head_slices(n, H):
        return [(i // H, i % H) for i in range(n)]

    t0 = time.perf_counter()
    gidx = head_slices(sg, gcfg.H)
    gsel = lambda t: np.stack([t[b, h].float().numpy() for b, h in gidx])[None]
    q, k, v = gsel(gx["q"]), gsel(gx["k"]), gsel(gx["v"])
    # every slice keeps its own head's parameters: the sample is passed as B = 1, H = slices
    mu = np.stack([gx["mu"][h].numpy() for _, h in gidx])
    lv = np.stack([gx["log_var"][h].numpy() for _, h in gidx])
    lp = np.stack([gx["logit_pi"][h].numpy() for _, h in gidx])
    cidx = head_slices(sc, ccfg.H)
    sel = lambda t: np.stack([t[b, h].float().numpy() for b, h in cidx])[None]
    cq, ck, cv, cg = sel(cx["q"]), sel(cx["k"]), sel(cx["v"]), sel(cx["g"])
    w = np.stack([cx["w_lambda"][h].numpy() for _, h in cidx])
    bb = np.stack([cx["b_lambda"][h].numpy() for _, h in cidx])
    tg = tc = 0.0
    rounds = 0
    while rounds < max_rounds and (rounds == 0 or tg + tc < min_seconds):
        tg0 = time.perf_counter()
        oracle.gma_forward(q, k, v, mu, lv, lp, causal=True, eps=gcfg.eps)
        tg += time.perf_counter() - tg0
        tc0 = time.perf_counter()
        oracle.ccq_forward(cq, ck, cv, cg, w, bb)
        tc += time.perf_counter() - tc0
        rounds += 1
    toks = rounds * (sg * gcfg.N + sc * ccfg.N)
    model, avail, ncpu = host_cpu()
    # cores: the OpenMP threads that had work (one (b, h) slice each)
    return {"value": toks / (tg + tc), "unit": "head-tokens/s", "cores": max(sg, sc), "kind": "oracle",
            "sample": "%d round(s) of %d causal-GMA + %d CCQ slices at N=16384 (one slice per thread per path), "
                      "fp64; GMA %.1f s, CCQ %.1f s" % (rounds, sg, sc, tg, tc),
            "host_threads": threads, "cpu_model": model, "nproc": avail, "host_cpus": ncpu,
            "wall_s": time.perf_counter() - t0}


def summarize_pmc(fetch_dir, write_dir):
    """Per-dispatch HBM bytes of each kernel from two rocprofv3 --pmc runs of
    this bench (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), scaled so that the
    calibration copy reads and writes exactly its size. Writes
    profiles/traffic.json and prints a markdown table."""

    def load(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit("no counter_collection.csv under %s" % d)
        rows = []
        with open(f[0]) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0))
        rows.sort()
        return [(name, b) for _, name, b in rows]

    fetch = load(fetch_dir, "FETCH_SIZE")
    write = load(write_dir, "WRITE_SIZE")

    # the calibration copy: the last copy dispatched before the library's first kernel
    def calib(rows):
        last = None
        for name, b in rows:
            if "lm::" in name or "_ZN2lm" in name:
                break
            if "copy" in name.lower():
                last = b
        if not last:
            raise SystemExit("calibration copy not found")
        return last

    fs, ws = CALIB_BYTES / calib(fetch), CALIB_BYTES / calib(write)

    def per_kernel(rows, scale):
        acc = {}
        for name, b in rows:
            n, t = acc.get(name, (0, 0.0))
            acc[name] = (n + 1, t + b * scale)
        return {k: (n, t / n) for k, (n, t) in acc.items()}

    fk, wk = per_kernel(fetch, fs), per_kernel(write, ws)
    out = {"sources": sources_digest(), "fetch_scale": fs, "write_scale": ws, "kernels": {}, "bytes_per_call": {}}
    print("| kernel | dispatches | read MB/dispatch | written MB/dispatch |")
    print("|---|---|---|---|")
    for k in sorted(fk, key=lambda k: -fk[k][1]):
        n, fb = fk[k]
        wb = wk.get(k, (0, 0.0))[1]
        out["kernels"][k] = {"dispatches": n, "read_bytes": fb, "write_bytes": wb}
        print("| %s | %d | %.1f | %.1f |" % (k[:70], n, fb / 1e6, wb / 1e6))
    for entry, frags in ENTRY_KERNELS.items():
        total = 0.0
        for k, v in out["kernels"].items():
            if any(f in k for f in frags):
                total += v["read_bytes"] + v["write_bytes"]
        out["bytes_per_call"][entry] = total
    print("\nscale factors: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f (%d MiB copy)" % (fs, ws, CALIB_BYTES >> 20))
    for entry, b in out["bytes_per_call"].items():
        print("%s: %.1f MB of HBM traffic per call" % (entry, b / 1e6))
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)


if __name__ == "__main__":
    main()
