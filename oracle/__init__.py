"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never loads it and
shares no code with it.

Two independent CPU forms live here:

* ``fwd`` / ``step``: the plain definition, a token-by-token fp64 recurrence
  in C (``gdn_oracle.c``), OpenMP over independent (sequence, head) units.
  It follows the recurrence of "Gated Delta Networks: Improving Mamba2 with
  Delta Rule" (research-map summary, section "Approach") with the read-out
  o_t = S_t q_t on the post-update state (the pages print no read-out).
* ``chunk_form``: the chunkwise WY/UT form in NumPy fp64, used to check that
  the chunk algorithm reaches the recurrence's result for every chunk size,
  forward and backward.
* ``bwd``: reverse-mode gradients through the fp64 token recurrence (C).
* ``kda_fwd``: the recurrence with channel-wise decay (C).
* ``gdn2_fwd``: the recurrence with channel-wise decay and separate erase
  and write gates (C).

Neither form has values printed on the pages to compare against; both are
pinned by the closed forms and invariants in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the .so path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB_PATH):
    """Load a compiled oracle library (building the default one if it is
    absent or older than its source)."""
    if path == LIB_PATH and (not os.path.exists(path)
                             or os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.gdn_oracle_fwd.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ip,
                                   dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.gdn_oracle_fwd.restype = ctypes.c_int
    lib.gdn_oracle_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, dp, dp, dp, dp, dp, dp, dp,
                                    ctypes.c_int]
    lib.gdn_oracle_step.restype = ctypes.c_int
    if hasattr(lib, "gdn_oracle_kda_fwd"):
        lib.gdn_oracle_kda_fwd.argtypes = lib.gdn_oracle_fwd.argtypes
        lib.gdn_oracle_kda_fwd.restype = ctypes.c_int
    if hasattr(lib, "gdn_oracle_gdn2_fwd"):
        lib.gdn_oracle_gdn2_fwd.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int, ip,
                                            dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.gdn_oracle_gdn2_fwd.restype = ctypes.c_int
    if hasattr(lib, "gdn_oracle_bwd"):
        lib.gdn_oracle_bwd.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ip,
                                       dp, dp, dp, dp, dp, dp, dp, dp,
                                       dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
    return lib


def _lib_default():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a (CPU) torch tensor to C-contiguous fp64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, threads: int = 0,
        lib=None, want_o: bool = True):
    """Token-by-token fp64 forward.

    q,k [B,T,H,dk]; v [B,T,H,dv]; log_alpha, beta [B,T,H]; S0 [U,H,dv,dk] or
    None (zeros); cu_seqlens int [n_seqs+1] or None.  Returns (o, S_T) as fp64
    numpy arrays (o is None when want_o is False).
    """
    lib = lib or _lib_default()
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, be = as_f64(log_alpha), as_f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int32))
        n_seqs = cu.shape[0] - 1
        units = n_seqs
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        n_seqs, units, cu_p = 0, B, None
    s0 = as_f64(S0) if S0 is not None else None
    o = np.zeros((B, T, H, dv), dtype=np.float64) if want_o else None
    st = np.zeros((units, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_fwd(B, T, H, dk, dv, n_seqs, cu_p,
                            _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be),
                            _ptr(s0), _ptr(o), _ptr(st), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return o, st


def bwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, dO=None, dS_T=None,
        threads: int = 0, lib=None):
    """Reverse-mode gradients of L = <dO, o> + <dS_T, S_T> through the fp64
    token recurrence (same layouts as ``fwd``; dS_T None means zero).

    Returns (dq, dk, dv, dlog_alpha, dbeta, dS0) as fp64 numpy arrays.
    """
    lib = lib or _lib_default()
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, be = as_f64(log_alpha), as_f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int32))
        n_seqs = cu.shape[0] - 1
        units = n_seqs
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        n_seqs, units, cu_p = 0, B, None
    s0 = as_f64(S0) if S0 is not None else None
    do = as_f64(dO)
    dst = as_f64(dS_T) if dS_T is not None else None
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dla, dbe = np.zeros_like(la), np.zeros_like(be)
    ds0 = np.zeros((units, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_bwd(B, T, H, dk, dv, n_seqs, cu_p,
                            _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0),
                            _ptr(do), _ptr(dst), _ptr(dq), _ptr(dk_), _ptr(dv_),
                            _ptr(dla), _ptr(dbe), _ptr(ds0), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return dq, dk_, dv_, dla, dbe, ds0


def kda_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, threads: int = 0, lib=None):
    """Token-by-token fp64 forward with channel-wise decay (log_alpha
    [B,T,H,dk]); other layouts as in ``fwd``.  Returns (o, S_T)."""
    lib = lib or _lib_default()
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, be = as_f64(log_alpha), as_f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if la.shape != (B, T, H, dk):
        raise ValueError("log_alpha must be [B,T,H,dk]")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int32))
        n_seqs = cu.shape[0] - 1
        units = n_seqs
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        n_seqs, units, cu_p = 0, B, None
    s0 = as_f64(S0) if S0 is not None else None
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    st = np.zeros((units, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_kda_fwd(B, T, H, dk, dv, n_seqs, cu_p, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(la), _ptr(be), _ptr(s0), _ptr(o), _ptr(st), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return o, st


def gdn2_fwd(q, k, v, log_alpha, erase, write, S0=None, cu_seqlens=None, threads: int = 0,
             lib=None):
    """Token-by-token fp64 Gated DeltaNet-2 forward: log_alpha and erase
    [B,T,H,dk], write [B,T,H,dv]; other layouts as in ``fwd``.  Returns
    (o, S_T)."""
    lib = lib or _lib_default()
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, eb, wg = as_f64(log_alpha), as_f64(erase), as_f64(write)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if la.shape != (B, T, H, dk) or eb.shape != (B, T, H, dk) or wg.shape != (B, T, H, dv):
        raise ValueError("log_alpha, erase must be [B,T,H,dk] and write [B,T,H,dv]")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int32))
        n_seqs = cu.shape[0] - 1
        units = n_seqs
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        n_seqs, units, cu_p = 0, B, None
    s0 = as_f64(S0) if S0 is not None else None
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    st = np.zeros((units, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_gdn2_fwd(B, T, H, dk, dv, n_seqs, cu_p, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(la), _ptr(eb), _ptr(wg), _ptr(s0), _ptr(o), _ptr(st),
                                 int(threads))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return o, st


def step(q, k, v, log_alpha, beta, S, threads: int = 0, lib=None):
    """One decode step.  q,k [B,H,dk]; v [B,H,dv]; gates [B,H]; S [B,H,dv,dk].

    Returns (o, S_new); the input S is not modified.
    """
    lib = lib or _lib_default()
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, be = as_f64(log_alpha), as_f64(beta)
    s = as_f64(S).copy()
    B, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, dv), dtype=np.float64)
    rc = lib.gdn_oracle_step(B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                             _ptr(be), _ptr(s), _ptr(o), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return o, s
