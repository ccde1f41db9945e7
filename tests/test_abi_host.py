"""Host-side checks of libgdn.so (CPU only, no kernel is ever launched).

The library must load without a GPU, export every function include/gdn.h
declares, and reject bad arguments on the host with the documented status
codes before enqueueing anything."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_58_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4
P = ctypes.c_void_p(4096)          # stand-in device pointers: never dereferenced
P2 = ctypes.c_void_p(8192)
MIS = ctypes.c_void_p(4096 + 4)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_matches_binding():
    assert declared_functions() == sorted(B.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version():
    assert B.version().startswith("gdn-mi355x")


def shape(**kw):
    d = dict(B=2, T=100, H=4, d_k=128, d_v=128, chunk=64, n_seqs=0, io_dtype=1, o_dtype=0,
             prologue=0)
    d.update(kw)
    return B.GdnShape(**d)


def ws_size(s):
    out = ctypes.c_size_t(123)
    rc = B.lib().gdn_chunk_fwd_workspace_size(ctypes.byref(s) if s is not None else None,
                                               ctypes.byref(out))
    return rc, out.value


def fwd(s, q=P, k=P, v=P, la=P, be=P, S0=None, cu=None, o=P2, ST=None, ws=None, wsb=0):
    return B.lib().gdn_chunk_fwd(ctypes.byref(s), q, k, v, la, be, S0, cu, o, ST, ws, wsb, None)


def err():
    return B.lib().gdn_last_error().decode()


@pytest.mark.parametrize("kw", [dict(d_k=128, d_v=128, io_dtype=1),
                                dict(d_k=64, d_v=64, io_dtype=1),
                                dict(d_k=16, d_v=16, chunk=16, io_dtype=0),
                                dict(d_k=64, d_v=64, chunk=32, io_dtype=0, o_dtype=1)])
def test_workspace_query_supported(kw):
    rc, n = ws_size(shape(**kw))
    assert rc == OK and n == 0 and err() == ""


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(T=-1), INVALID),
    (dict(d_k=0), INVALID), (dict(chunk=0), INVALID), (dict(n_seqs=-1), INVALID),
    (dict(n_seqs=3, B=2), INVALID), (dict(io_dtype=7), INVALID), (dict(o_dtype=-1), INVALID),
    (dict(d_k=96, d_v=96), UNSUPPORTED), (dict(d_k=128, d_v=64), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED), (dict(d_k=128, d_v=128, io_dtype=0), UNSUPPORTED),
    (dict(d_k=16, d_v=16, chunk=8, io_dtype=0), UNSUPPORTED),
    (dict(B=1, T=1, H=32769), UNSUPPORTED),
])
def test_workspace_query_rejects(kw, code):
    rc, _ = ws_size(shape(**kw))
    assert rc == code
    assert err() != ""


def test_null_shape():
    assert ws_size(None)[0] == INVALID


def test_fwd_rejects_before_launch():
    s = shape()
    assert fwd(s, q=None) == INVALID and "required" in err()
    assert fwd(s, o=None) == INVALID
    assert fwd(s, k=MIS) == ALIGN and "k=" in err()
    assert fwd(s, S0=MIS) == ALIGN
    assert fwd(s, o=P) == INVALID and "alias" in err()
    assert fwd(s, cu=P) == INVALID and "n_seqs" in err()
    sv = shape(B=1, n_seqs=3)
    assert fwd(sv, cu=None) == INVALID and "cu_seqlens" in err()
    assert fwd(shape(d_k=96, d_v=96)) == UNSUPPORTED


def test_fwd_empty_without_state_is_a_noop():
    # T = 0 and no final state requested: nothing to do, nothing launched.
    assert fwd(shape(T=0), q=None, k=None, v=None, la=None, be=None, o=None) == OK
    assert err() == ""


def step(Bn=2, H=3, dk=128, dv=128, io=1, od=0, q=P, k=P, v=P, la=P, be=P, S=P2, o=P, pro=0):
    return B.lib().gdn_step(Bn, H, dk, dv, io, od, pro, q, k, v, la, be, S, o, None)


def test_step_rejects_before_launch():
    assert step(Bn=0) == INVALID
    assert step(dv=-3) == INVALID
    assert step(io=5) == INVALID
    assert step(dk=32) == UNSUPPORTED and "d_k" in err()
    assert step(S=None) == INVALID
    assert step(q=MIS) == ALIGN
    assert step(o=P2) == INVALID and "alias" in err()


def test_prologue_flags_are_validated():
    # bits 0 and 1 are the only prologue flags; anything else is rejected
    for bad in (4, 8, -1, 1 << 30):
        assert ws_size(shape(prologue=bad))[0] == INVALID and "prologue" in err()
        assert fwd(shape(prologue=bad)) == INVALID
        assert step(pro=bad) == INVALID and "prologue" in err()
    for good in (0, 1, 2, 3):
        assert ws_size(shape(prologue=good)) == (OK, 0)
        assert ws_size(shape(prologue=good, io_dtype=0, d_k=32, d_v=32, chunk=32)) == (OK, 0)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        B.lib()


def bws(s):
    out = ctypes.c_size_t(123)
    rc = B.lib().gdn_chunk_bwd_workspace_size(ctypes.byref(s), ctypes.byref(out))
    return rc, out.value


def bwd(s, ws=P, wsb=1 << 40, **kw):
    a = dict(q=P, k=P, v=P, la=P, be=P, S0=None, cu=None, dO=P, dST=None, dq=P2, dk=P2, dv=P2,
             dla=P2, dbe=P2, dS0=None)
    a.update(kw)
    return B.lib().gdn_chunk_bwd(ctypes.byref(s), a["q"], a["k"], a["v"], a["la"], a["be"],
                                 a["S0"], a["cu"], a["dO"], a["dST"], a["dq"], a["dk"], a["dv"],
                                 a["dla"], a["dbe"], a["dS0"], ws, wsb, None)


def test_bwd_workspace_size_formula():
    # per (chunk, head): T and P (64x64), state and its gradient (d x d), five 64 x d blocks, 1
    for d, io in ((128, 1), (64, 1), (64, 0)):
        rc, n = bws(shape(T=130, d_k=d, d_v=d, io_dtype=io))
        nch = 2 * 3 * 4                                 # B * ceil(130/64) * H
        assert rc == OK and n == 4 * nch * (2 * 64 * 64 + 2 * d * d + 5 * 64 * d + 1)
    # packed: floor(T/64) + n_seqs + 1 slots per head
    rc, n = bws(shape(B=1, T=300, n_seqs=5))
    assert rc == OK and n == 4 * (300 // 64 + 5 + 1) * 4 * (2 * 4096 + 2 * 16384 + 5 * 8192 + 1)


def test_bwd_rejects_before_launch():
    assert bws(shape(prologue=1))[0] == UNSUPPORTED and "prologue" in err()
    assert bws(shape(prologue=8))[0] == INVALID
    assert bws(shape(chunk=32))[0] == UNSUPPORTED
    assert bws(shape(io_dtype=0))[0] == UNSUPPORTED          # fp32 inputs: d = 64 only
    assert bws(shape(io_dtype=0, d_k=64, d_v=64))[0] == OK
    assert bws(shape(d_k=128, d_v=64))[0] == UNSUPPORTED
    assert bws(shape(B=0))[0] == INVALID
    s = shape()
    assert bwd(s, dq=None) == INVALID
    assert bwd(s, dO=None) == INVALID
    assert bwd(s, dq=MIS) == ALIGN and "dq" in err()
    assert bwd(s, dv=P) == INVALID and "alias" in err()
    assert bwd(s, wsb=16) == WORKSPACE
    assert bwd(shape(n_seqs=2, B=1)) == INVALID and "cu_seqlens" in err()


def test_kda_workspace_and_rejects():
    def kws(s):
        out = ctypes.c_size_t(7)
        return B.lib().gdn_kda_fwd_workspace_size(ctypes.byref(s), ctypes.byref(out)), out.value
    rc, nb = kws(shape(T=130))
    nch = 2 * 3 * 4
    # per chunk and head, bf16 hi + lo pairs with dense rows: K o e^G and
    # Q o e^G (64 x d each), T diag(beta) and P (64 x 64 each),
    # (K o e^{G_n - G})^T (d x 64), then e^{G_n} (d floats)
    d = 128
    per = 2 * 2 * 64 * d + 2 * 2 * 64 * 64 + 2 * d * 64 + 2 * d
    assert rc == OK and nb == 2 * nch * per
    assert kws(shape(prologue=2))[0] == UNSUPPORTED
    assert kws(shape(io_dtype=0))[0] == UNSUPPORTED
    assert kws(shape(chunk=16))[0] == UNSUPPORTED
    assert kws(shape(B=1, T=1, H=32769))[0] == UNSUPPORTED   # 32-bit store offsets
    s = shape()
    call = lambda **kw: B.lib().gdn_kda_fwd(
        ctypes.byref(s), kw.get("q", P), P, P, P, P, None, None, kw.get("o", P2), None,
        kw.get("ws", P), kw.get("wsb", 16), None)
    assert call(wsb=16) == WORKSPACE
    assert call(q=None, wsb=1 << 40) == INVALID
    assert call(o=P, wsb=1 << 40) == INVALID and "alias" in err()


def test_gdn2_workspace_and_rejects():
    def gws(s):
        out = ctypes.c_size_t(7)
        return B.lib().gdn_gdn2_fwd_workspace_size(ctypes.byref(s), ctypes.byref(out)), out.value
    rc, nb = gws(shape(T=130))
    # per chunk and head, bf16 hi + lo pairs with dense rows: F1 and Qh
    # (64 x d each), (E o e^{G_n - G})^T (d x 64), e^{G_n} (d floats),
    # (K o e^{G_n - G})^T (d x 64), N1 and N2 (64 x 64 each)
    d = 128
    per = 2 * 2 * 64 * d + 2 * d * 64 + 2 * d + 2 * d * 64 + 2 * 2 * 64 * 64
    assert rc == OK and nb == 2 * 2 * 3 * 4 * per
    assert gws(shape(prologue=1))[0] == UNSUPPORTED
    assert gws(shape(io_dtype=0))[0] == UNSUPPORTED
    assert gws(shape(B=1, T=1, H=32769))[0] == UNSUPPORTED
    s = shape()
    call = lambda **kw: B.lib().gdn_gdn2_fwd(
        ctypes.byref(s), P, P, P, P, kw.get("erase", P), P, None, None, kw.get("o", P2), None,
        kw.get("ws", P), kw.get("wsb", 16), None)
    assert call(wsb=16) == WORKSPACE
    assert call(erase=None, wsb=1 << 40) == INVALID
    assert call(erase=MIS, wsb=1 << 40) == ALIGN


def test_kda_noalloc_rejects_before_launch():
    """The no-allocation KDA entry point checks its arguments and its array
    size on the host: nothing here reaches the GPU."""
    L = B.lib()
    cap = L.gdn_kda_fwd_noalloc_max_workspace()
    assert cap == 64 << 20
    shape = B.GdnShape(1, 8192, 16, 128, 128, 64, 0, B.GDN_BF16, B.GDN_F32, 0)
    need = ctypes.c_size_t(0)
    assert L.gdn_kda_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(need)) == 0
    assert need.value > cap
    fake = ctypes.c_void_p(1 << 20)
    out = ctypes.c_void_p(1 << 21)
    rc = L.gdn_kda_fwd_noalloc(ctypes.byref(shape), fake, fake, fake, fake, fake, None, None,
                               out, None, None)
    assert rc == 4 and b"scratch" in L.gdn_last_error()
    bad = B.GdnShape(1, 64, 2, 128, 96, 64, 0, B.GDN_BF16, B.GDN_F32, 0)
    rc = L.gdn_kda_fwd_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, None, None,
                               out, None, None)
    assert rc == 2   # GDN_ERR_UNSUPPORTED (d_k != d_v)
