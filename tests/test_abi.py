"""The C ABI library on the host: it loads without a GPU, exports every function
include/linmix.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from linear_attention_gmm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linmix.h")

needs_lib = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH), reason="liblinmix.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gma_forward", "linattn_chunk_forward", "ccq_forward", "gma_workspace_bytes",
              "linattn_workspace_bytes", "ccq_workspace_bytes", "lm_abi_version", "lm_status_string",
              "lm_last_error"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@needs_lib
def test_version_and_status_strings():
    L = binding.lib()
    assert L.lm_abi_version() == 6
    for code, name in enumerate(["LM_OK", "LM_EINVAL", "LM_EUNSUPPORTED", "LM_EWORKSPACE", "LM_EHIP"]):
        assert L.lm_status_string(code).decode() == name
    assert L.lm_status_string(99).decode() == "LM_UNKNOWN"


FAKE = 1 << 40  # an aligned address that is never dereferenced (calls fail before any HIP call)


def _gma(L, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), mu=FAKE + (3 << 30), lv=FAKE + (4 << 30),
             lp=FAKE + (5 << 30), out=FAKE + (6 << 30), B=1, H=2, N=100, d=64, K=16, dv=64, causal=1,
             eps=1e-6, dt=binding.LM_BF16, seg=0, ws=FAKE + (7 << 30), wsb=0)
    a.update(kw)
    if a["wsb"] == 0 and "wsb" not in kw:
        a["wsb"] = L.gma_workspace_bytes(a["B"], a["H"], a["N"], a["d"], a["K"], a["dv"], a["causal"], a["dt"], a["seg"])
    st = L.gma_forward(a["q"], a["k"], a["v"], a["mu"], a["lv"], a["lp"], a["out"], a["B"], a["H"], a["N"], a["d"],
                       a["K"], a["dv"], a["causal"], a["eps"], a["dt"], a["seg"], a["ws"], a["wsb"], None)
    return st, L.lm_last_error().decode()


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.LM_EINVAL),
    (dict(out=FAKE + (6 << 30) + 2), binding.LM_EINVAL),  # misaligned
    (dict(N=0), binding.LM_EINVAL),
    (dict(eps=-1.0), binding.LM_EINVAL),
    (dict(eps=float("nan")), binding.LM_EINVAL),
    (dict(causal=2), binding.LM_EINVAL),
    (dict(dt=7), binding.LM_EINVAL),
    (dict(seg=-1), binding.LM_EINVAL),
    (dict(d=48, dv=48), binding.LM_EUNSUPPORTED),
    (dict(d=64, dv=48), binding.LM_EUNSUPPORTED),
    (dict(d=16, dv=8), binding.LM_EUNSUPPORTED),
    (dict(K=257), binding.LM_EUNSUPPORTED),
    (dict(d=16, dv=128, K=200, dt=binding.LM_F32), binding.LM_EUNSUPPORTED),  # padded to d = 128
    (dict(d=128, dv=128, K=200, dt=binding.LM_F32), binding.LM_EUNSUPPORTED),
    (dict(wsb=16), binding.LM_EWORKSPACE),
    (dict(out=FAKE + 16), binding.LM_EINVAL),  # overlaps q
    (dict(N=(1 << 30) + 1), binding.LM_EUNSUPPORTED),  # beyond the largest sequence
    (dict(B=256, H=256), binding.LM_EUNSUPPORTED),  # beyond the largest B*H
])
def test_gma_errors(kw, code):
    st, msg = _gma(binding.lib(), **kw)
    assert st == code, (st, msg)
    assert msg


def _lin(L, fn, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30), w=FAKE + (4 << 30),
             b=FAKE + (5 << 30), out=FAKE + (6 << 30), B=1, H=2, N=100, dk=64, dv=64, chunk=64,
             dt=binding.LM_BF16, seg=0, ws=FAKE + (7 << 30), wsb=None)
    a.update(kw)
    ccq = fn == "ccq_forward"
    if a["wsb"] is None:
        wsf = L.ccq_workspace_bytes if ccq else L.linattn_workspace_bytes
        a["wsb"] = wsf(a["B"], a["H"], a["N"], a["dk"], a["dv"], a["chunk"], a["dt"], a["seg"])
    if ccq:
        st = L.ccq_forward(a["q"], a["k"], a["v"], a["g"], a["w"], a["b"], a["out"], a["B"], a["H"], a["N"], a["dk"],
                           a["dv"], a["chunk"], a["dt"], a["seg"], a["ws"], a["wsb"], None)
    else:
        st = L.linattn_chunk_forward(a["q"], a["k"], a["v"], a["g"], a["out"], a["B"], a["H"], a["N"], a["dk"],
                                     a["dv"], a["chunk"], a["dt"], a["seg"], a["ws"], a["wsb"], None)
    return st, L.lm_last_error().decode()


@needs_lib
@pytest.mark.parametrize("fn", ["linattn_chunk_forward", "ccq_forward"])
@pytest.mark.parametrize("kw,code", [
    (dict(k=None), binding.LM_EINVAL),
    (dict(g=FAKE + (3 << 30) + 2), binding.LM_EINVAL),
    (dict(H=0), binding.LM_EINVAL),
    (dict(chunk=48), binding.LM_EUNSUPPORTED),
    (dict(chunk=128), binding.LM_EUNSUPPORTED),
    (dict(dk=96, dv=96), binding.LM_EUNSUPPORTED),
    (dict(dk=64, dv=96), binding.LM_EUNSUPPORTED),
    (dict(wsb=8), binding.LM_EWORKSPACE),
    (dict(chunk=32, wsb=8), binding.LM_EWORKSPACE),  # chunk 32 runs (needs the same workspace)
    (dict(dk=16, dv=64, wsb=8), binding.LM_EWORKSPACE),  # padded shape
    (dict(dk=16, dv=64, out=FAKE + (2 << 30) + 64), binding.LM_EINVAL),  # padded shape, out overlaps v
    (dict(dk=32, dv=64, ws=FAKE + (3 << 30)), binding.LM_EINVAL),  # padded shape, g inside the workspace
    (dict(out=FAKE + (2 << 30) + 64), binding.LM_EINVAL),  # overlaps v
    (dict(N=(1 << 30) + 1), binding.LM_EUNSUPPORTED),  # beyond the largest sequence
    (dict(B=256, H=256), binding.LM_EUNSUPPORTED),  # beyond the largest B*H
])
def test_linattn_errors(fn, kw, code):
    st, msg = _lin(binding.lib(), fn, **kw)
    assert st == code, (st, msg)
    assert msg


def _delta(L, fn, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30), beta=FAKE + (10 << 30),
             w=FAKE + (4 << 30), b=FAKE + (5 << 30), out=FAKE + (6 << 30), B=1, H=2, N=100, dk=64, dv=64,
             chunk=64, dt=binding.LM_BF16, seg=0, ws=FAKE + (7 << 30), wsb=None)
    a.update(kw)
    ccq = fn == "ccq_deltanet_forward"
    if a["wsb"] is None:
        wsf = L.ccq_deltanet_workspace_bytes if ccq else L.deltanet_workspace_bytes
        a["wsb"] = wsf(a["B"], a["H"], a["N"], a["dk"], a["dv"], a["chunk"], a["dt"], a["seg"])
    if ccq:
        st = L.ccq_deltanet_forward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["w"], a["b"], a["out"], a["B"],
                                    a["H"], a["N"], a["dk"], a["dv"], a["chunk"], a["dt"], a["seg"], a["ws"],
                                    a["wsb"], None)
    else:
        st = L.deltanet_chunk_forward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["out"], a["B"], a["H"], a["N"],
                                      a["dk"], a["dv"], a["chunk"], a["dt"], a["seg"], a["ws"], a["wsb"], None)
    return st, L.lm_last_error().decode()


@needs_lib
@pytest.mark.parametrize("fn", ["deltanet_chunk_forward", "ccq_deltanet_forward"])
@pytest.mark.parametrize("kw,code", [
    (dict(beta=None), binding.LM_EINVAL),
    (dict(beta=FAKE + (10 << 30) + 2), binding.LM_EINVAL),  # misaligned
    (dict(N=0), binding.LM_EINVAL),
    (dict(chunk=32), binding.LM_EUNSUPPORTED),
    (dict(dk=64, dv=96), binding.LM_EUNSUPPORTED),
    (dict(dk=128, dv=128, dt=binding.LM_F32), binding.LM_EUNSUPPORTED),
    (dict(dk=16, dv=128, dt=binding.LM_F32), binding.LM_EUNSUPPORTED),  # padded to 128 in float32
    (dict(dk=16, dv=32, wsb=16), binding.LM_EWORKSPACE),
    (dict(out=FAKE + (10 << 30)), binding.LM_EINVAL),  # overlaps beta
    (dict(B=256, H=256), binding.LM_EUNSUPPORTED),
])
def test_deltanet_errors(fn, kw, code):
    st, msg = _delta(binding.lib(), fn, **kw)
    assert st == code, (st, msg)
    assert msg


@needs_lib
def test_deltanet_workspaces():
    L = binding.lib()
    # W and Ut of every chunk (the shapes of K and V); the CCQ read also holds
    # the clean queries
    tensor = 4 * 16 * 16384 * 128 * 2
    assert L.deltanet_workspace_bytes(4, 16, 16384, 128, 128, 64, binding.LM_BF16, 0) == 2 * tensor
    n = L.ccq_deltanet_workspace_bytes(4, 16, 16384, 128, 128, 64, binding.LM_BF16, 0)
    assert n >= 3 * tensor
    st, _ = _delta(L, "ccq_deltanet_forward", wsb=16)
    assert st == binding.LM_EWORKSPACE
    for fn in ("deltanet_chunk_forward", "ccq_deltanet_forward"):
        st, _ = _delta(L, fn, ws=None)
        assert st == binding.LM_EINVAL
    st, _ = _delta(L, "ccq_deltanet_forward", w=None)
    assert st == binding.LM_EINVAL


@needs_lib
def test_padded_shapes_workspace_and_native_only_entry_points():
    L = binding.lib()
    # d = 16 and d != dv run padded: the workspace holds the padded tensors too
    assert L.linattn_workspace_bytes(2, 4, 1000, 16, 16, 64, binding.LM_BF16, 0) > \
        L.linattn_workspace_bytes(2, 4, 1000, 32, 32, 64, binding.LM_BF16, 0)
    assert L.gma_workspace_bytes(2, 4, 1000, 64, 16, 32, 1, binding.LM_BF16, 0) > \
        L.gma_workspace_bytes(2, 4, 1000, 64, 16, 64, 1, binding.LM_BF16, 0)
    for fn in ("ccq_workspace_bytes", "linattn_vec_workspace_bytes", "deltanet_workspace_bytes",
               "ccq_deltanet_workspace_bytes"):
        assert getattr(L, fn)(2, 4, 1000, 16, 64, 64, binding.LM_BF16, 0) > 0, fn
        assert getattr(L, fn)(2, 4, 1000, 24, 64, 64, binding.LM_BF16, 0) == 0, fn
    # the carried-state entry points and the backward take the native widths only
    st, _ = _ccq_state(L, dk=16, dv=16)
    assert st == binding.LM_EUNSUPPORTED
    st, _ = _ccq_state(L, dk=32, dv=64)
    assert st == binding.LM_EUNSUPPORTED
    st, _ = _gma_state(L, d=16, dv=16)
    assert st == binding.LM_EUNSUPPORTED


@needs_lib
def test_ccq_needs_gate_parameters():
    st, _ = _lin(binding.lib(), "ccq_forward", w=None)
    assert st == binding.LM_EINVAL


@needs_lib
def test_workspace_sizes_are_deterministic_and_grow_with_segments():
    L = binding.lib()
    a = L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 1, binding.LM_BF16, 0)
    assert a == L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 1, binding.LM_BF16, 0) and a > 0
    assert L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 1, binding.LM_BF16, 16) > \
        L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 1, binding.LM_BF16, 2)
    assert L.gma_workspace_bytes(4, 8, 16384, 48, 128, 48, 1, binding.LM_BF16, 0) == 0
    # the causal bf16 kernel over several segments also keeps every chunk's key
    # responsibilities (64 x 128 bf16 per chunk); one segment, float32 and the
    # bidirectional form do not
    tiles = 4 * 8 * (16384 // 64) * 64 * 128 * 2
    assert a - L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 0, binding.LM_BF16, 0) == tiles
    assert L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 1, binding.LM_BF16, 1) == \
        L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 0, binding.LM_BF16, 1)
    assert L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 1, binding.LM_F32, 0) == \
        L.gma_workspace_bytes(4, 8, 16384, 64, 128, 64, 0, binding.LM_F32, 0)
    assert L.ccq_workspace_bytes(4, 16, 16384, 128, 128, 64, binding.LM_BF16, 0) > \
        L.linattn_workspace_bytes(4, 16, 16384, 128, 128, 64, binding.LM_BF16, 0)


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 32)
    with pytest.raises((ValueError, RuntimeError)):
        binding.gma_forward(q, q, q, torch.zeros(1, 4, 32), torch.zeros(1, 4, 32), torch.zeros(1, 4))


# ----------------------------------------------------------------------------- carried state and decode steps

def _ccq_state(L, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30), w=FAKE + (4 << 30),
             b=FAKE + (5 << 30), out=FAKE + (6 << 30), B=1, H=2, N=100, dk=64, dv=64, chunk=64,
             dt=binding.LM_BF16, seg=0, t_in=0, sin=FAKE + (8 << 30), sout=FAKE + (9 << 30),
             ws=FAKE + (7 << 30), wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.ccq_workspace_bytes(a["B"], a["H"], a["N"], a["dk"], a["dv"], a["chunk"], a["dt"], a["seg"])
    st = L.ccq_forward_state(a["q"], a["k"], a["v"], a["g"], a["w"], a["b"], a["out"], a["B"], a["H"], a["N"],
                             a["dk"], a["dv"], a["chunk"], a["dt"], a["seg"], a["t_in"], a["sin"], a["sout"],
                             a["ws"], a["wsb"], None)
    return st, L.lm_last_error().decode()


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(sin=None, t_in=5), binding.LM_EINVAL),  # a token count without a state
    (dict(t_in=-1), binding.LM_EINVAL),
    (dict(sin=FAKE + (8 << 30) + 4), binding.LM_EINVAL),  # misaligned state
    (dict(sout=FAKE + (8 << 30) + 256), binding.LM_EINVAL),  # partial overlap of the two states
    (dict(sout=FAKE + (6 << 30)), binding.LM_EINVAL),  # state_out overlaps out
    (dict(dk=48, dv=48), binding.LM_EUNSUPPORTED),
])
def test_ccq_state_errors(kw, code):
    st, msg = _ccq_state(binding.lib(), **kw)
    assert st == code, (st, msg)
    assert msg


def _gma_state(L, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), mu=FAKE + (3 << 30), lv=FAKE + (4 << 30),
             lp=FAKE + (5 << 30), out=FAKE + (6 << 30), B=1, H=2, N=100, d=64, K=16, dv=64, eps=1e-6,
             dt=binding.LM_BF16, seg=0, sin=FAKE + (8 << 30), sout=FAKE + (9 << 30), ws=FAKE + (7 << 30), wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.gma_workspace_bytes(a["B"], a["H"], a["N"], a["d"], a["K"], a["dv"], 1, a["dt"], a["seg"])
    st = L.gma_forward_state(a["q"], a["k"], a["v"], a["mu"], a["lv"], a["lp"], a["out"], a["B"], a["H"], a["N"],
                             a["d"], a["K"], a["dv"], a["eps"], a["dt"], a["seg"], a["sin"], a["sout"], a["ws"],
                             a["wsb"], None)
    return st, L.lm_last_error().decode()


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(sin=FAKE + (8 << 30) + 8), binding.LM_EINVAL),
    (dict(sout=FAKE + (7 << 30)), binding.LM_EINVAL),  # state_out overlaps the workspace
    (dict(sout=FAKE + (8 << 30) + 16), binding.LM_EINVAL),  # partial overlap of the two states
    (dict(K=300), binding.LM_EUNSUPPORTED),
])
def test_gma_state_errors(kw, code):
    st, msg = _gma_state(binding.lib(), **kw)
    assert st == code, (st, msg)
    assert msg


@needs_lib
def test_decode_step_errors():
    L = binding.lib()
    q, k, v, g, w, b, out, s = (FAKE + (i << 30) for i in range(8))
    bf = binding.LM_BF16
    assert L.linattn_decode_step(q, k, v, g, out, s, 2, 2, 48, 48, bf, None) == binding.LM_EUNSUPPORTED
    assert L.linattn_decode_step(q, k, v, g, out, None, 2, 2, 64, 64, bf, None) == binding.LM_EINVAL
    assert L.linattn_decode_step(q, k, v, g, out + 4, s, 2, 2, 64, 64, bf, None) == binding.LM_EINVAL
    assert L.linattn_decode_step(q, k, v, g, q, s, 2, 2, 64, 64, bf, None) == binding.LM_EINVAL  # out is q
    assert L.linattn_decode_step(q, k, v, g, out, s, 0, 2, 64, 64, bf, None) == binding.LM_EINVAL
    assert L.ccq_decode_step(q, k, v, g, w, b, out, s, 2, 2, 64, 64, -1, bf, None) == binding.LM_EINVAL
    assert L.ccq_decode_step(q, k, v, g, None, b, out, s, 2, 2, 64, 64, 3, bf, None) == binding.LM_EINVAL
    assert L.ccq_decode_step(q, k, v, g, w, b, out, k, 2, 2, 64, 64, 3, bf, None) == binding.LM_EINVAL  # state is k
    assert L.gma_decode_step(q, k, v, g, w, b, out, s, 2, 2, 64, 257, 64, 1e-6, bf, None) == binding.LM_EUNSUPPORTED
    assert L.gma_decode_step(q, k, v, g, w, b, out, s, 2, 2, 64, 16, 64, -1.0, bf, None) == binding.LM_EINVAL
    assert L.gma_decode_step(q, k, v, g, w, b, out, s, 2, 2, 64, 16, 32, 1e-6, bf, None) == binding.LM_EUNSUPPORTED
    assert L.lm_last_error().decode()


@needs_lib
def test_vec_forward_errors():
    L = binding.lib()
    q, k, v, g, out, ws = (FAKE + (i << 30) for i in range(6))
    bf = binding.LM_BF16
    wsb = L.linattn_vec_workspace_bytes(1, 2, 100, 64, 64, 64, bf, 0)
    assert wsb > 0
    call = lambda **kw: L.linattn_vec_forward(kw.get("q", q), k, v, kw.get("g", g), kw.get("out", out), 1, 2,
                                              kw.get("N", 100), kw.get("dk", 64), kw.get("dv", 64), kw.get("ch", 64),
                                              bf, 0, ws, kw.get("wsb", wsb), None)
    assert call(g=g + 4) == binding.LM_EINVAL  # g is read in 16-byte transfers
    assert call(q=None) == binding.LM_EINVAL
    assert call(out=g + 64) == binding.LM_EINVAL  # out overlaps g
    assert call(wsb=16) == binding.LM_EWORKSPACE
    assert call(dk=48, dv=48) == binding.LM_EUNSUPPORTED
    assert call(ch=32) == binding.LM_EUNSUPPORTED
    assert call(N=0) == binding.LM_EINVAL
    assert L.lm_last_error().decode()


@needs_lib
def test_vec_state_and_decode_errors():
    L = binding.lib()
    q, k, v, g, out, ws, s0, s1 = (FAKE + (i << 30) for i in range(8))
    bf = binding.LM_BF16
    wsb = L.linattn_vec_workspace_bytes(1, 2, 100, 64, 64, 64, bf, 0)
    fwd = lambda sin, sout: L.linattn_vec_forward_state(q, k, v, g, out, 1, 2, 100, 64, 64, 64, bf, 0, sin, sout, ws,
                                                        wsb, None)
    assert fwd(s0 + 8, None) == binding.LM_EINVAL  # misaligned state
    assert fwd(s0, s0 + 64) == binding.LM_EINVAL  # partial overlap of the two states
    assert fwd(None, out) == binding.LM_EINVAL  # state_out overlaps out
    assert L.linattn_vec_decode_step(q, k, v, None, out, s0, 2, 2, 64, 64, bf, None) == binding.LM_EINVAL
    assert L.linattn_vec_decode_step(q, k, v, g, out, s0, 2, 2, 48, 48, bf, None) == binding.LM_EUNSUPPORTED
    assert L.linattn_vec_decode_step(q, k, v, g, out, q, 2, 2, 64, 64, bf, None) == binding.LM_EINVAL  # state is q


@needs_lib
def test_backward_errors():
    L = binding.lib()
    q, k, v, g, do, dq, dk, dv, dg, ws = (FAKE + (i << 30) for i in range(10))
    bf = binding.LM_BF16
    wsb = L.linattn_backward_workspace_bytes(1, 2, 100, 64, 64, 64, bf, 0)
    assert wsb > L.linattn_workspace_bytes(1, 2, 100, 64, 64, 64, bf, 0)
    call = lambda **kw: L.linattn_chunk_backward(q, k, v, g, do, kw.get("dq", dq), dk, dv, kw.get("dg", dg), 1, 2,
                                                 100, kw.get("d", 64), kw.get("d", 64), 64, bf, 0, ws,
                                                 kw.get("wsb", wsb), None)
    assert call(wsb=wsb - 1) == binding.LM_EWORKSPACE
    assert call(dq=dk) == binding.LM_EINVAL  # two outputs in one buffer
    assert call(dq=q + 64) == binding.LM_EINVAL  # output overlaps an input
    assert call(dg=dg + 2) == binding.LM_EINVAL  # misaligned
    assert call(dq=None) == binding.LM_EINVAL
    assert call(d=48) == binding.LM_EUNSUPPORTED
    assert L.lm_last_error().decode()


@needs_lib
def test_gma_backward_errors():
    L = binding.lib()
    (q, k, v, mu, lv, lp, do, dq, dk, dv, dmu, dlv, dlp, ws) = (FAKE + (i << 30) for i in range(14))
    bf, f32 = binding.LM_BF16, binding.LM_F32
    wsb = L.gma_backward_workspace_bytes(2, 2, 300, 64, 128, 64, 1, bf)
    assert wsb > 0
    assert L.gma_backward_workspace_bytes(2, 2, 300, 64, 128, 64, 0, bf) > wsb  # bidirectional: 2N inner rows
    # d = 128 or K > 128: the inner tensors in two blocks of 128 columns
    assert L.gma_backward_workspace_bytes(2, 2, 300, 128, 256, 128, 1, bf) > wsb
    assert L.gma_backward_workspace_bytes(2, 2, 300, 64, 129, 64, 1, f32) > 0
    assert L.gma_backward_workspace_bytes(2, 2, 300, 64, 257, 64, 1, f32) == 0  # K > 256: not implemented
    assert L.gma_backward_workspace_bytes(2, 2, 300, 96, 64, 96, 1, f32) == 0  # d = 96: not implemented
    assert L.gma_backward_workspace_bytes(2, 2, 300, 32, 16, 32, 1, f32) > 0

    def call(**kw):
        a = dict(dq=dq, dk=dk, dmu=dmu, d=64, K=128, causal=1, eps=1e-6, wsb=wsb)
        a.update(kw)
        return L.gma_backward(q, k, v, mu, lv, lp, do, a["dq"], a["dk"], dv, a["dmu"], dlv, dlp, 2, 2, 300, a["d"],
                              a["K"], a["d"], a["causal"], a["eps"], bf, ws, a["wsb"], None)

    assert call(wsb=wsb - 1) == binding.LM_EWORKSPACE
    assert call(dq=dk) == binding.LM_EINVAL  # two outputs in one buffer
    assert call(dq=q + 64) == binding.LM_EINVAL  # output overlaps an input
    assert call(dmu=dmu + 2) == binding.LM_EINVAL  # misaligned
    assert call(dq=None) == binding.LM_EINVAL
    assert call(eps=-1.0) == binding.LM_EINVAL
    assert call(causal=2) == binding.LM_EINVAL
    assert call(d=16) == binding.LM_EUNSUPPORTED
    assert call(K=300) == binding.LM_EUNSUPPORTED
    assert L.lm_last_error().decode()


@needs_lib
def test_ccq_backward_errors():
    L = binding.lib()
    (q, k, v, g, w, b, do, dq, dk, dv, dg, dw, db, ws) = (FAKE + (i << 30) for i in range(14))
    bf = binding.LM_BF16
    wsb = L.ccq_backward_workspace_bytes(1, 2, 100, 64, 64, 64, bf)
    assert wsb > L.linattn_backward_workspace_bytes(1, 2, 100, 64, 64, 64, bf, 0)
    assert L.ccq_backward_workspace_bytes(1, 2, 100, 48, 48, 64, bf) == 0
    assert L.ccq_backward_workspace_bytes(1, 2, 100, 64, 64, 32, bf) == 0

    def call(**kw):
        a = dict(dq=dq, dg=dg, db=db, d=64, chunk=64, wsb=wsb)
        a.update(kw)
        return L.ccq_backward(q, k, v, g, w, b, do, a["dq"], dk, dv, a["dg"], dw, a["db"], 1, 2, 100, a["d"],
                              a["d"], a["chunk"], bf, ws, a["wsb"], None)

    assert call(wsb=wsb - 1) == binding.LM_EWORKSPACE
    assert call(dq=dk) == binding.LM_EINVAL  # two outputs in one buffer
    assert call(dq=q + 64) == binding.LM_EINVAL  # output overlaps an input
    assert call(db=db + 2) == binding.LM_EINVAL  # misaligned
    assert call(dg=None) == binding.LM_EINVAL
    assert call(d=48) == binding.LM_EUNSUPPORTED
    assert call(chunk=32) == binding.LM_EUNSUPPORTED
    assert L.lm_last_error().decode()


@needs_lib
def test_noalloc_checks_before_any_hip_call():
    # gma_forward_noalloc: argument errors and a shape beyond its fixed scratch
    # are reported before the scratch is looked up (no GPU needed)
    L = binding.lib()
    G = 1 << 30
    p = [FAKE + i * G for i in range(7)]

    def call(ptrs, B=1, H=16, N=131072, d=128, K=256, seg=64, eps=1e-6):
        st = L.gma_forward_noalloc(*ptrs, B, H, N, d, K, d, 1, eps, binding.LM_BF16, seg, None)
        return st, L.lm_last_error().decode()

    # 64 segments of the long-context shapes: 16 * 64 * 256 * 129 * 4 bytes > 64 MiB
    st, msg = call(p)
    assert st == binding.LM_EWORKSPACE and "scratch" in msg, msg
    assert call([None] + p[1:], seg=1)[0] == binding.LM_EINVAL
    assert call(p[:6] + [p[6] + 2], seg=1)[0] == binding.LM_EINVAL  # misaligned out
    assert call(p, seg=1, eps=-1.0)[0] == binding.LM_EINVAL
    assert call(p, d=48, seg=1)[0] == binding.LM_EUNSUPPORTED


@needs_lib
@pytest.mark.parametrize("fn", ["linattn_workspace_bytes", "ccq_workspace_bytes"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (16, 64), (128, 128)])
def test_chunk32_accepted(fn, dk, dv):
    # chunks of 32 tokens are implemented for the plain and CCQ forwards
    L = binding.lib()
    assert getattr(L, fn)(2, 3, 500, dk, dv, 32, binding.LM_F32, 0) > 0
    assert getattr(L, fn)(2, 3, 500, dk, dv, 32, binding.LM_BF16, 0) > 0
    assert getattr(L, fn)(2, 3, 500, dk, dv, 48, binding.LM_F32, 0) == 0


@needs_lib
@pytest.mark.parametrize("fn", ["deltanet_workspace_bytes", "ccq_deltanet_workspace_bytes",
                                "linattn_vec_workspace_bytes", "linattn_backward_workspace_bytes"])
def test_chunk32_not_elsewhere(fn):
    # the other chunked calls run chunks of 64 only
    L = binding.lib()
    assert getattr(L, fn)(2, 3, 500, 64, 64, 64, binding.LM_F32, 0) > 0
    assert getattr(L, fn)(2, 3, 500, 64, 64, 32, binding.LM_F32, 0) == 0


@needs_lib
def test_backward_state_errors():
    L = binding.lib()
    (q, k, v, g, do, si, dso, dq, dk, dv, dg, dsi, ws) = (FAKE + (i << 30) for i in range(13))
    bf, f32 = binding.LM_BF16, binding.LM_F32

    def call(**kw):
        a = dict(si=si, dso=dso, dq=dq, dsi=dsi, d=128, dt=bf, ws=ws, wsb=1 << 30)
        a.update(kw)
        return L.linattn_chunk_backward_state(q, k, v, g, do, a["si"], a["dso"], a["dq"], dk, dv, dg, a["dsi"], 2, 2,
                                              300, a["d"], a["d"], 64, a["dt"], 0, a["ws"], a["wsb"], None)

    assert call(d=64) == binding.LM_EUNSUPPORTED  # a carried state: bf16, d = 128 only
    assert call(dt=f32) == binding.LM_EUNSUPPORTED
    assert call(si=si + 4) == binding.LM_EINVAL  # misaligned
    assert call(dsi=dq + 64) == binding.LM_EINVAL  # dstate_in overlaps dq
    assert call(dsi=si) == binding.LM_EINVAL  # dstate_in overlaps state_in
    assert call(dq=dso) == binding.LM_EINVAL  # an output overlaps a state input
    assert call(wsb=8) == binding.LM_EWORKSPACE
    assert L.lm_last_error().decode()
