"""ctypes binding of libgdn.so (argument marshalling only).

Every computation happens in the library's HIP kernels; this module only
checks torch tensor shapes/dtypes, allocates outputs with torch (device
memory is PyTorch's job) and passes raw device pointers and the current
HIP stream to the C ABI declared in include/gdn.h.  If the library is not
built, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
PROLOGUE_NORM_QK, PROLOGUE_GATES = 1, 2
_DTYPE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}

# symbol -> (restype, argtypes); this is the whole exported surface of gdn.h
_c_int, _vp, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t


class GdnShape(ctypes.Structure):
    _fields_ = [("B", _c_int), ("T", _c_int), ("H", _c_int), ("d_k", _c_int),
                ("d_v", _c_int), ("chunk", _c_int), ("n_seqs", _c_int),
                ("io_dtype", _c_int), ("o_dtype", _c_int), ("prologue", _c_int)]


SYMBOLS = {
    "gdn_chunk_fwd_workspace_size": (_c_int, [ctypes.POINTER(GdnShape),
                                              ctypes.POINTER(_sz)]),
    "gdn_chunk_fwd": (_c_int, [ctypes.POINTER(GdnShape), _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gdn_chunk_bwd_workspace_size": (_c_int, [ctypes.POINTER(GdnShape),
                                              ctypes.POINTER(_sz)]),
    "gdn_chunk_bwd": (_c_int, [ctypes.POINTER(GdnShape)] + [_vp] * 16 + [_sz, _vp]),
    "gdn_kda_fwd_workspace_size": (_c_int, [ctypes.POINTER(GdnShape),
                                            ctypes.POINTER(_sz)]),
    "gdn_kda_fwd": (_c_int, [ctypes.POINTER(GdnShape)] + [_vp] * 10 + [_sz, _vp]),
    "gdn_kda_fwd_noalloc": (_c_int, [ctypes.POINTER(GdnShape)] + [_vp] * 9 + [_vp]),
    "gdn_kda_fwd_noalloc_max_workspace": (_sz, []),
    "gdn_gdn2_fwd_workspace_size": (_c_int, [ctypes.POINTER(GdnShape),
                                             ctypes.POINTER(_sz)]),
    "gdn_gdn2_fwd": (_c_int, [ctypes.POINTER(GdnShape)] + [_vp] * 11 + [_sz, _vp]),
    "gdn_step": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gdn_last_error": (ctypes.c_char_p, []),
    "gdn_version": (ctypes.c_char_p, []),
}

_lib = None


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gdn error {code}: {msg}")
        self.code = code


def lib():
    """Load libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_delta_rule_58_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def version() -> str:
    return lib().gdn_version().decode()


def _check(rc: int):
    if rc != 0:
        raise GdnError(rc, lib().gdn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_cuda(name, t, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _need_shape(name, t, shape, dtype=None, device=None):
    """t must be a contiguous GPU tensor of exactly `shape` (and dtype, and on
    `device`): the C ABI only sees pointers, so a smaller buffer would be read
    or written out of bounds by the kernels."""
    _need_cuda(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _state_or_new(name, t, shape, device, want):
    """Caller-supplied fp32 state buffer (checked), or a new one, or None."""
    if t is not None:
        _need_shape(name, t, shape, torch.float32, device)
        return t
    return torch.empty(shape, device=device, dtype=torch.float32) if want else None


def _out_or_new(t, shape, device, dtype):
    """Caller-supplied output buffer (checked: fp32 or bf16), or a new one."""
    if t is None:
        return torch.empty(shape, device=device, dtype=dtype)
    if t.dtype not in _DTYPE:
        raise ValueError(f"o must be float32 or bfloat16, got {t.dtype}")
    _need_shape("o", t, shape, None, device)
    return t


def _prologue(norm_qk: bool, gates: bool) -> int:
    return (PROLOGUE_NORM_QK if norm_qk else 0) | (PROLOGUE_GATES if gates else 0)


def chunk_fwd_workspace_size(B, T, H, d_k, d_v, chunk=64, n_seqs=0,
                             io_dtype=torch.bfloat16, o_dtype=torch.float32,
                             prologue=0) -> int:
    shape = GdnShape(B, T, H, d_k, d_v, chunk, n_seqs, _DTYPE[io_dtype], _DTYPE[o_dtype],
                     prologue)
    out = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, chunk=64,
              o_dtype=torch.float32, o=None, S_T=None, want_state=True,
              norm_qk=False, gates=False):
    """Chunkwise forward.  q,k [B,T,H,dk]; v [B,T,H,dv]; log_alpha, beta
    [B,T,H] fp32; S0 [U,H,dv,dk] fp32 or None; cu_seqlens int32 [N+1] (device)
    or None.  norm_qk / gates turn on the fused input prologue (q, k
    L2-normalised in the kernel; log_alpha, beta passed as pre-activations a,
    b with log alpha = -softplus(a), beta = sigmoid(b)).  Returns (o, S_T)
    (S_T is None when want_state is False)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, io)
    for name, t in (("log_alpha", log_alpha), ("beta", beta)):
        _need_cuda(name, t, torch.float32)
        if tuple(t.shape) != (B, T, H):
            raise ValueError(f"{name} must be [B,T,H]")
    if tuple(k.shape) != (B, T, H, dk) or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("q, k, v shapes disagree")
    n_seqs = 0
    if cu_seqlens is not None:
        _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.shape[0] - 1
    units = n_seqs if n_seqs > 0 else B
    st_shape = (units, H, dv, dk)
    if S0 is not None:
        _need_shape("S0", S0, st_shape, torch.float32, q.device)
    o = _out_or_new(o, (B, T, H, dv), q.device, o_dtype)
    S_T = _state_or_new("S_T", S_T, st_shape, q.device, want_state)
    shape = GdnShape(B, T, H, dk, dv, chunk, n_seqs, _DTYPE[io], _DTYPE[o.dtype],
                     _prologue(norm_qk, gates))
    ws_bytes = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(ws_bytes)))
    ws = None
    if ws_bytes.value:
        ws = torch.empty(ws_bytes.value, device=q.device, dtype=torch.uint8)
    _check(lib().gdn_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
                               _ptr(o), _ptr(S_T), _ptr(ws), ws_bytes.value,
                               _stream(q.device)))
    return o, S_T


def chunk_bwd_workspace_size(B, T, H, d_k, d_v, chunk=64, n_seqs=0,
                             io_dtype=torch.bfloat16, o_dtype=torch.float32) -> int:
    shape = GdnShape(B, T, H, d_k, d_v, chunk, n_seqs, _DTYPE[io_dtype], _DTYPE[o_dtype], 0)
    out = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def chunk_bwd(q, k, v, log_alpha, beta, dO, S0=None, cu_seqlens=None, dS_T=None, chunk=64,
              want_dS0=True, workspace=None, out=None):
    """Backward of chunk_fwd: gradients of <dO, o> + <dS_T, S_T>.  dO
    [B,T,H,dv] (fp32 or bf16; the q/k/v gradients take its dtype); dS_T
    [U,H,dv,dk] fp32 or None.  `out` optionally supplies the six gradient
    buffers (checked like every other output).  Returns (dq, dk, dv,
    dlog_alpha, dbeta, dS0) (dS0 is None when want_dS0 is False)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, io)
    for name, t in (("log_alpha", log_alpha), ("beta", beta)):
        _need_cuda(name, t, torch.float32)
        if tuple(t.shape) != (B, T, H):
            raise ValueError(f"{name} must be [B,T,H]")
    _need_cuda("dO", dO)
    if tuple(dO.shape) != (B, T, H, dv) or dO.dtype not in _DTYPE:
        raise ValueError("dO must be [B,T,H,dv] fp32 or bf16")
    n_seqs = 0
    if cu_seqlens is not None:
        _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.shape[0] - 1
    units = n_seqs if n_seqs > 0 else B
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _need_cuda(name, t, torch.float32)
            if tuple(t.shape) != (units, H, dv, dk):
                raise ValueError(f"{name} must be [{units},{H},{dv},{dk}]")
    gd = dO.dtype
    shapes = (((B, T, H, dk), gd), ((B, T, H, dk), gd), ((B, T, H, dv), gd),
              ((B, T, H), torch.float32), ((B, T, H), torch.float32),
              ((units, H, dv, dk), torch.float32))
    if out is None:
        out = [torch.empty(sh, device=q.device, dtype=dt) for sh, dt in shapes]
        if not want_dS0:
            out[5] = None
    else:
        out = list(out)
        if len(out) != 6:
            raise ValueError("out must hold six gradient buffers (dS0 may be None)")
        for name, t, (sh, dt) in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"),
                                     out, shapes):
            if t is not None or name != "dS0":
                _need_shape(name, t, sh, dt, q.device)
    dq, dk_, dv_, dla, dbe, dS0 = out
    shape = GdnShape(B, T, H, dk, dv, chunk, n_seqs, _DTYPE[io], _DTYPE[gd], 0)
    need = ctypes.c_size_t(0)
    _check(lib().gdn_chunk_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), device=q.device, dtype=torch.uint8)
    _check(lib().gdn_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                               _ptr(beta), _ptr(S0), _ptr(cu_seqlens), _ptr(dO), _ptr(dS_T),
                               _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dbe), _ptr(dS0),
                               _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk_, dv_, dla, dbe, dS0


def kda_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, chunk=64,
            o_dtype=torch.float32, o=None, S_T=None, want_state=True, workspace=None):
    """Forward with channel-wise decay: log_alpha [B,T,H,dk] fp32, other
    arguments as in chunk_fwd.  Returns (o, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_shape(name, t, (B, T, H, dk if name != "v" else dv), io, q.device)
    _need_shape("log_alpha", log_alpha, (B, T, H, dk), torch.float32, q.device)
    _need_shape("beta", beta, (B, T, H), torch.float32, q.device)
    n_seqs = 0
    if cu_seqlens is not None:
        _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.shape[0] - 1
    units = n_seqs if n_seqs > 0 else B
    st_shape = (units, H, dv, dk)
    if S0 is not None:
        _need_shape("S0", S0, st_shape, torch.float32, q.device)
    o = _out_or_new(o, (B, T, H, dv), q.device, o_dtype)
    S_T = _state_or_new("S_T", S_T, st_shape, q.device, want_state)
    shape = GdnShape(B, T, H, dk, dv, chunk, n_seqs, _DTYPE[io], _DTYPE[o.dtype], 0)
    need = ctypes.c_size_t(0)
    _check(lib().gdn_kda_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), device=q.device, dtype=torch.uint8)
    _check(lib().gdn_kda_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                             _ptr(beta), _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(S_T),
                             _ptr(workspace), workspace.numel(), _stream(q.device)))
    return o, S_T


def kda_fwd_noalloc(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, chunk=64,
                    o_dtype=torch.float32, o=None, S_T=None, want_state=True):
    """kda_fwd with the workspace taken from the library's device array
    (gdn_kda_fwd_noalloc): no workspace argument and no device allocation in
    the library.  Outputs are allocated here (torch) unless o / S_T are
    given, so a caller that must not allocate passes both.  Returns (o, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_shape(name, t, (B, T, H, dk if name != "v" else dv), io, q.device)
    _need_shape("log_alpha", log_alpha, (B, T, H, dk), torch.float32, q.device)
    _need_shape("beta", beta, (B, T, H), torch.float32, q.device)
    n_seqs = 0
    if cu_seqlens is not None:
        _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.shape[0] - 1
    units = n_seqs if n_seqs > 0 else B
    st_shape = (units, H, dv, dk)
    if S0 is not None:
        _need_shape("S0", S0, st_shape, torch.float32, q.device)
    o = _out_or_new(o, (B, T, H, dv), q.device, o_dtype)
    S_T = _state_or_new("S_T", S_T, st_shape, q.device, want_state)
    shape = GdnShape(B, T, H, dk, dv, chunk, n_seqs, _DTYPE[io], _DTYPE[o.dtype], 0)
    _check(lib().gdn_kda_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
                                     _ptr(o), _ptr(S_T), _stream(q.device)))
    return o, S_T


def kda_fwd_noalloc_max_workspace() -> int:
    """Bytes of the library's device array behind kda_fwd_noalloc."""
    return int(lib().gdn_kda_fwd_noalloc_max_workspace())


def gdn2_fwd(q, k, v, log_alpha, erase, write, S0=None, cu_seqlens=None, chunk=64,
             o_dtype=torch.float32, o=None, S_T=None, want_state=True, workspace=None):
    """Gated DeltaNet-2 forward: log_alpha, erase [B,T,H,dk], write [B,T,H,dv]
    fp32; other arguments as in chunk_fwd.  Returns (o, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, io)
    if tuple(k.shape) != (B, T, H, dk) or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("q, k, v shapes disagree")
    for name, t, last in (("log_alpha", log_alpha, dk), ("erase", erase, dk),
                          ("write", write, dv)):
        _need_cuda(name, t, torch.float32)
        if tuple(t.shape) != (B, T, H, last):
            raise ValueError(f"{name} must be [B,T,H,{last}]")
    n_seqs = 0
    if cu_seqlens is not None:
        _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
        n_seqs = cu_seqlens.shape[0] - 1
    units = n_seqs if n_seqs > 0 else B
    st_shape = (units, H, dv, dk)
    if S0 is not None:
        _need_shape("S0", S0, st_shape, torch.float32, q.device)
    o = _out_or_new(o, (B, T, H, dv), q.device, o_dtype)
    S_T = _state_or_new("S_T", S_T, st_shape, q.device, want_state)
    shape = GdnShape(B, T, H, dk, dv, chunk, n_seqs, _DTYPE[io], _DTYPE[o.dtype], 0)
    need = ctypes.c_size_t(0)
    _check(lib().gdn_gdn2_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), device=q.device, dtype=torch.uint8)
    _check(lib().gdn_gdn2_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                              _ptr(erase), _ptr(write), _ptr(S0), _ptr(cu_seqlens), _ptr(o),
                              _ptr(S_T), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return o, S_T


def gdn2_fwd_workspace_size(B, T, H, d_k, d_v, chunk=64, n_seqs=0, io_dtype=torch.bfloat16,
                            o_dtype=torch.float32) -> int:
    shape = GdnShape(B, T, H, d_k, d_v, chunk, n_seqs, _DTYPE[io_dtype], _DTYPE[o_dtype], 0)
    out = ctypes.c_size_t(0)
    _check(lib().gdn_gdn2_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def kda_fwd_workspace_size(B, T, H, d_k, d_v, chunk=64, n_seqs=0, io_dtype=torch.bfloat16,
                           o_dtype=torch.float32) -> int:
    shape = GdnShape(B, T, H, d_k, d_v, chunk, n_seqs, _DTYPE[io_dtype], _DTYPE[o_dtype], 0)
    out = ctypes.c_size_t(0)
    _check(lib().gdn_kda_fwd_workspace_size(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def step(q, k, v, log_alpha, beta, S, o_dtype=torch.float32, o=None, norm_qk=False,
         gates=False):
    """One decode step.  q,k [B,H,dk]; v [B,H,dv]; gates [B,H] fp32; S
    [B,H,dv,dk] fp32, updated in place; norm_qk / gates as in chunk_fwd.
    Returns o [B,H,dv]."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [B,H,dk] and v [B,H,dv]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    _need_shape("q", q, (B, H, dk), io)
    _need_shape("k", k, (B, H, dk), io, q.device)
    _need_shape("v", v, (B, H, dv), io, q.device)
    for name, t in (("log_alpha", log_alpha), ("beta", beta)):
        _need_shape(name, t, (B, H), torch.float32, q.device)
    _need_shape("S", S, (B, H, dv, dk), torch.float32, q.device)
    o = _out_or_new(o, (B, H, dv), q.device, o_dtype)
    _check(lib().gdn_step(B, H, dk, dv, _DTYPE[io], _DTYPE[o.dtype],
                          _prologue(norm_qk, gates), _ptr(q), _ptr(k),
                          _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(o),
                          _stream(q.device)))
    return o
