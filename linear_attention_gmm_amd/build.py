"""Builds liblinmix.so (the HIP library) in-tree for gfx950.

    python -m linear_attention_gmm_amd.build [--jobs N]

Each csrc/*.hip|*.cpp file is compiled to an object under _build/ in parallel.
The objects are then linked into linear_attention_gmm_amd/liblinmix.so. Every
call compiles from scratch, so a stale library is never kept.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblinmix.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are kept out of the generated code (the host pass warns
# that it does not know the feature, which is harmless). MFMA accumulators are
# kept in VGPRs where possible, which avoids AGPR<->VGPR copies around the VALU
# work on accumulators.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The generic GMA kernel file crashes the compiler's AGPR rewrite pass under
# the VGPR-form option (fp32 d = 128 instantiations), so it is built without it.
NO_VGPR_FORM = {"gma.hip"}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = [] if os.path.basename(src) in NO_VGPR_FORM else VGPR_FORM
    cmd = [HIPCC] + FLAGS + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    _check_symbols(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_symbols(path: str) -> None:
    """Fails the build when the library references its own code it does not define
    (e.g. a kernel stub that was never instantiated)."""
    r = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True)
    bad = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN2lm" in l]
    if bad:
        raise RuntimeError("undefined library symbols: " + ", ".join(bad))


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    args = ap.parse_args()
    print(build(args.jobs))
