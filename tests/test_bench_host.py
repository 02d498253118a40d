"""Host logic of bench.py that needs no GPU: the multi-GPU refusal and the
source digest that decides whether recorded HBM counters still describe the
kernels."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_digest_ignores_comment_lines_and_tracks_code(tmp_path, monkeypatch):
    csrc = tmp_path / "linear_attention_gmm_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.DIGEST_SOURCES:
        shutil.copy(os.path.join(ROOT, "linear_attention_gmm_amd", "csrc", f), csrc / f)
    shutil.copy(os.path.join(ROOT, "linear_attention_gmm_amd", "build.py"), csrc.parent / "build.py")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.sources_digest()
    assert base == bench.sources_digest()
    p = csrc / "gma_bf16.hip"
    text = p.read_text()
    p.write_text("// an added comment line\n" + text.replace("\n", "\n    // indented comment\n", 1))
    assert bench.sources_digest() == base
    p.write_text(text + "\nstatic int added_code_line;\n")
    assert bench.sources_digest() != base
    p.write_text(text)
    assert bench.sources_digest() == base
    # a change of compile flags in the build script also changes the digest
    b = csrc.parent / "build.py"
    btext = b.read_text()
    b.write_text(btext.replace('"-O3"', '"-O2"'))
    assert bench.sources_digest() != base


def test_host_cpu_reports_model_and_counts():
    model, avail, ncpu = bench.host_cpu()
    assert isinstance(model, str) and model
    assert 1 <= avail <= ncpu
