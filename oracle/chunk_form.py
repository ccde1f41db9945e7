"""Chunkwise WY/UT form of the gated delta rule in NumPy fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages only name the method: an extended WY/UT chunkwise algorithm
("Gated Delta Networks: Improving Mamba2 with Delta Rule", research-map
summary, section "Approach"), i.e. the WY representation extended to gating
so the recurrence runs in chunks on matrix units (blog "Gated DeltaNet:
Harmonizing Gating and the Delta Rule for Superior Linear RNNs", section
"Hardware-Efficient Training").  The steps below are that algorithm written
out for one chunk of n <= C tokens, state S (d_v x d_k) entering the chunk:

  1. gate prefix        g_r = sum_{s<=r} log alpha_s            (chunk-local)
  2. UT transform       A[r,i] = beta_r exp(g_r - g_i) (k_r . k_i), i < r
                        T = (I + A)^{-1}   (unit lower, forward substitution)
  3. WY factors         U = T diag(beta) V,   W = T diag(beta e^g) K
  4. corrected values   Delta = U - W S^T
  5. output             O = diag(e^g) Q S^T + (tril(Q K^T) o E) Delta,
                        E[r,i] = exp(g_r - g_i) for i <= r (diagonal kept)
  6. next state         S' = e^{g_n} S + Delta^T diag(e^{g_n - g}) K

Step 1-3 do not depend on S.  Only exponentials of non-positive arguments are
formed (masked entries are set to -inf before exp).  This form is an exact
rewrite of the token recurrence; the tests check that it reaches the C
oracle's result for every chunk size, including ragged last chunks.
"""
from __future__ import annotations

import numpy as np

from . import as_f64


def unit_lower_inverse(L: np.ndarray) -> np.ndarray:
    """Inverse of a unit lower-triangular matrix by forward substitution.

    Row r of X = L^{-1} satisfies X[r] = e_r - sum_{i<r} L[r,i] X[i].
    """
    n = L.shape[0]
    X = np.eye(n)
    for r in range(1, n):
        X[r, :] -= L[r, :r] @ X[:r, :]
    return X


def chunk_step(Q, K, V, la, beta, S, want_parts: bool = False):
    """One chunk (n tokens).  Q,K [n,dk]; V [n,dv]; la, beta [n]; S [dv,dk].

    Returns (O [n,dv], S' [dv,dk]) and, if want_parts, a dict of the
    intermediates g, A, T, W, U, Delta and the chunk's affine map (M, R) with
    S' = S M + R.
    """
    n = Q.shape[0]
    g = np.cumsum(la)                                   # step 1
    diff = g[:, None] - g[None, :]                      # g_r - g_i
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    lower = np.tril(np.ones((n, n), dtype=bool), 0)
    A = beta[:, None] * np.exp(np.where(strict, diff, -np.inf)) * (K @ K.T)
    T = unit_lower_inverse(np.eye(n) + A)               # step 2
    U = T @ (beta[:, None] * V)                         # step 3
    W = T @ ((beta * np.exp(g))[:, None] * K)
    D = U - W @ S.T                                     # step 4
    E = np.exp(np.where(lower, diff, -np.inf))
    O = np.exp(g)[:, None] * (Q @ S.T) + ((Q @ K.T) * E) @ D   # step 5
    Kt = np.exp(g[-1] - g)[:, None] * K
    S_next = np.exp(g[-1]) * S + D.T @ Kt               # step 6
    if not want_parts:
        return O, S_next
    M = np.exp(g[-1]) * np.eye(K.shape[1]) - W.T @ Kt
    R = U.T @ Kt
    return O, S_next, dict(g=g, A=A, T=T, W=W, U=U, Delta=D, M=M, R=R)


def unit_fwd(Q, K, V, la, beta, S0, C: int, want_parts: bool = False):
    """All chunks of one (sequence, head) unit, chunk grid starting at token 0."""
    L = Q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((L, V.shape[1]))
    parts = []
    for s in range(0, L, C):
        e = min(s + C, L)
        res = chunk_step(Q[s:e], K[s:e], V[s:e], la[s:e], beta[s:e], S,
                         want_parts)
        O[s:e], S = res[0], res[1]
        if want_parts:
            parts.append(res[2])
    return (O, S, parts) if want_parts else (O, S)


def fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, chunk: int = 64):
    """Chunkwise forward over the same layouts as ``oracle.fwd``."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, be = as_f64(log_alpha), as_f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu")
                        else cu_seqlens, dtype=np.int64)
        spans = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    else:
        spans = [(b, 0, T) for b in range(B)]
    s0 = as_f64(S0) if S0 is not None else None
    o = np.zeros((B, T, H, dv))
    st = np.zeros((len(spans), H, dv, dk))
    for u, (b, t0, t1) in enumerate(spans):
        for h in range(H):
            init = s0[u, h] if s0 is not None else np.zeros((dv, dk))
            O, S = unit_fwd(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                            la[b, t0:t1, h], be[b, t0:t1, h], init, chunk)
            o[b, t0:t1, h] = O
            st[u, h] = S
    return o, st
