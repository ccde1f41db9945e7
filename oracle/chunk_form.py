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


# ---------------------------------------------------------------------------
# Backward of the chunk form (reverse mode, fp64).
#
# The pages name a gate-aware backward pass for the chunkwise algorithm
# ("Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
# abstract) but print none; this is the chain rule taken through steps 1-6
# above, one chunk at a time.  With S the state entering a chunk, dS' the
# gradient of the state leaving it, dO the output gradient, and
# P = tril(Q K^T) o E, K~ = diag(e^{g_n - g}) K:
#
#   dDelta = P^T dO + K~ dS'^T
#   dS     = e^{g_n} dS' + dO^T diag(e^g) Q - dDelta^T W     (to the previous chunk)
#
# so the state gradients run over the chunks in reverse order, and every
# other gradient of a chunk needs only its (S, dS'):
#
#   dP   = tril(dO Delta^T),  dQK = dP o E
#   dQ   = diag(e^g) dO S + dQK K
#   dW   = -dDelta S,  dU = dDelta,  dV = diag(beta) T^T dU
#   dK   = dQK^T Q + diag(e^{g_n - g}) Delta dS' + diag(beta e^g) T^T dW + dG K + dG^T K
#   dT   = dU V^T diag(beta) + dW K^T diag(beta e^g),  dA = -strict(T^T dT T^T)
#   dG   = dA o beta_r E  (strictly lower)
#   dbeta = rows(T^T dU . V) + e^g rows(T^T dW . K) + rowsum(dA o E o K K^T)
#   dg   = e^g rows(dO . Q S^T) + rowsum(dP o P) - colsum(dP o P)
#          + beta e^g rows(T^T dW . K) + rowsum(dA o A) - colsum(dA o A)
#          - s + [last] (sum(s) + e^{g_n} <dS', S>),   s_r = rows(Delta dS' . K~)_r
#   dlog_alpha = reverse cumulative sum of dg within the chunk.
# ---------------------------------------------------------------------------
def chunk_grads(Q, K, V, la, beta, S, dO, dSn):
    """Gradients of one chunk given the entering state S and the gradient dSn
    of the leaving state.  Returns (dQ, dK, dV, dla, dbeta, dS)."""
    n = Q.shape[0]
    g = np.cumsum(la)
    eg = np.exp(g)
    diff = g[:, None] - g[None, :]
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    lower = np.tril(np.ones((n, n), dtype=bool), 0)
    E = np.exp(np.where(lower, diff, -np.inf))
    KK = K @ K.T
    A = beta[:, None] * np.where(strict, E, 0.0) * KK
    T = unit_lower_inverse(np.eye(n) + A)
    U = T @ (beta[:, None] * V)
    W = T @ ((beta * eg)[:, None] * K)
    D = U - W @ S.T
    P = (Q @ K.T) * E
    Kt = np.exp(g[-1] - g)[:, None] * K
    dD = P.T @ dO + Kt @ dSn.T
    dS = np.exp(g[-1]) * dSn + dO.T @ (eg[:, None] * Q) - dD.T @ W
    dP = np.where(lower, dO @ D.T, 0.0)
    dQK = dP * E
    dQ = eg[:, None] * (dO @ S) + dQK @ K
    dW = -dD @ S
    TdU, TdW = T.T @ dD, T.T @ dW
    dV = beta[:, None] * TdU
    dKt = D @ dSn
    dT = dD @ (beta[:, None] * V).T + dW @ ((beta * eg)[:, None] * K).T
    dA = np.where(strict, -(T.T @ dT @ T.T), 0.0)
    dG = dA * beta[:, None] * E
    dK = (dQK.T @ Q + np.exp(g[-1] - g)[:, None] * dKt
          + (beta * eg)[:, None] * TdW + dG @ K + dG.T @ K)
    rw = np.sum(TdW * K, axis=1)
    dbeta = np.sum(TdU * V, axis=1) + eg * rw + np.sum(dA * E * KK, axis=1)
    s = np.sum(dKt * Kt, axis=1)
    dg = (eg * np.sum(dO * (Q @ S.T), axis=1)
          + np.sum(dP * P, axis=1) - np.sum(dP * P, axis=0)
          + beta * eg * rw
          + np.sum(dA * A, axis=1) - np.sum(dA * A, axis=0)
          - s)
    dg[-1] += np.sum(s) + np.exp(g[-1]) * np.sum(dSn * S)
    dla = np.cumsum(dg[::-1])[::-1]
    return dQ, dK, dV, dla, dbeta, dS


def unit_bwd(Q, K, V, la, beta, S0, dO, dST, C: int):
    """Backward of ``unit_fwd``: forward states per chunk, reverse state
    gradients, then each chunk's gradients."""
    L = Q.shape[0]
    starts = list(range(0, L, C))
    states = []
    S = np.array(S0, dtype=np.float64, copy=True)
    for s in starts:
        e = min(s + C, L)
        states.append(S)
        S = chunk_step(Q[s:e], K[s:e], V[s:e], la[s:e], beta[s:e], S)[1]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dla, dbeta = np.zeros_like(la), np.zeros_like(beta)
    G = np.array(dST, dtype=np.float64, copy=True)
    for ci in range(len(starts) - 1, -1, -1):
        s, e = starts[ci], min(starts[ci] + C, L)
        r = chunk_grads(Q[s:e], K[s:e], V[s:e], la[s:e], beta[s:e], states[ci], dO[s:e], G)
        dQ[s:e], dK[s:e], dV[s:e], dla[s:e], dbeta[s:e], G = r
    return dQ, dK, dV, dla, dbeta, G


def bwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, dO=None, dS_T=None,
        chunk: int = 64):
    """Chunkwise backward over the same layouts as ``oracle.bwd``."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, be = as_f64(log_alpha), as_f64(beta)
    do = as_f64(dO)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu")
                        else cu_seqlens, dtype=np.int64)
        spans = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    else:
        spans = [(b, 0, T) for b in range(B)]
    s0 = as_f64(S0) if S0 is not None else None
    dst = as_f64(dS_T) if dS_T is not None else None
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(la),
           np.zeros_like(be), np.zeros((len(spans), H, dv, dk))]
    for u, (b, t0, t1) in enumerate(spans):
        for h in range(H):
            init = s0[u, h] if s0 is not None else np.zeros((dv, dk))
            gS = dst[u, h] if dst is not None else np.zeros((dv, dk))
            r = unit_bwd(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], la[b, t0:t1, h],
                         be[b, t0:t1, h], init, do[b, t0:t1, h], gS, chunk)
            for i in range(5):
                out[i][b, t0:t1, h] = r[i]
            out[5][u, h] = r[5]
    return tuple(out)


# ---------------------------------------------------------------------------
# Channel-wise decay (KDA) in chunk form, fp64.
#
# With the decay acting on the key channels, G_r = sum_{s<=r} log alpha_s is
# a vector (d_k) and every e^{g_r - g_i} of the scalar form becomes the
# channel-wise weight Diag(e^{G_r - G_i}) inside the key products:
#
#   A[r,i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic}   (i < r),  T = (I + A)^{-1}
#   Delta  = T diag(beta) (V - (K o e^G) S^T)
#   O      = (Q o e^G) S^T + P Delta,  P[r,i] = sum_c q_rc k_ic e^{G_rc - G_ic} (i <= r)
#   S'     = S Diag(e^{G_n}) + Delta^T (K o e^{G_n - G})
#
# (the same unrolling as the scalar steps above, with Diag(e^{G}) in place
# of e^g).  Only exponentials of non-positive arguments are formed.
# ---------------------------------------------------------------------------
def kda_chunk_step(Q, K, V, LA, beta, S):
    """One chunk: Q,K [n,dk]; V [n,dv]; LA [n,dk] log alpha; beta [n]; S [dv,dk]."""
    n = Q.shape[0]
    G = np.cumsum(LA, axis=0)
    diff = G[:, None, :] - G[None, :, :]                  # [r, i, c]
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    lower = np.tril(np.ones((n, n), dtype=bool), 0)
    W = np.exp(np.where(lower[:, :, None], diff, -np.inf))
    A = beta[:, None] * np.einsum("rc,ic,ric->ri", K, K, W) * strict
    T = unit_lower_inverse(np.eye(n) + A)
    Z = beta[:, None] * (V - (K * np.exp(G)) @ S.T)
    D = T @ Z
    P = np.einsum("rc,ic,ric->ri", Q, K, W)
    O = (Q * np.exp(G)) @ S.T + P @ D
    S_next = S * np.exp(G[-1])[None, :] + D.T @ (K * np.exp(G[-1][None, :] - G))
    return O, S_next


def kda_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, chunk: int = 64):
    """Chunkwise forward with channel-wise decay, layouts as ``oracle.kda_fwd``."""
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
            S = s0[u, h].copy() if s0 is not None else np.zeros((dv, dk))
            for s in range(t0, t1, chunk):
                e = min(s + chunk, t1)
                o[b, s:e, h], S = kda_chunk_step(q[b, s:e, h], k[b, s:e, h], v[b, s:e, h],
                                                 la[b, s:e, h], be[b, s:e, h], S)
            st[u, h] = S
    return o, st


# ---------------------------------------------------------------------------
# Gated DeltaNet-2 in chunk form, fp64.
#
# Step: S~ = S Diag(alpha_r), S_r = S~ - (S~ k_r)(b_r o k_r)^T + (w_r o v_r) k_r^T.
# With x_r = -S~_r k_r (the erased read), e_r = b_r o k_r, z_r = w_r o v_r and
# the channel-wise prefix G, the state inside a chunk is
#   S_r = S Diag(e^{G_r}) + sum_{i<=r} (x_i e_i^T + z_i k_i^T) Diag(e^{G_r - G_i}),
# so the reads solve a unit lower triangular system with asymmetric factors:
#   A_e[r,i] = sum_c k_rc e_ic e^{G_rc - G_ic},  A_k[r,i] = sum_c k_rc k_ic e^{...}  (i < r)
#   X  = -(I + A_e)^{-1} ((K o e^G) S^T + A_k Z)
#   O  = (Q o e^G) S^T + P_e X + P_k Z,  P_e, P_k as A_e, A_k with q_r, i <= r
#   S' = S Diag(e^{G_n}) + X^T (E o e^{G_n - G}) + Z^T (K o e^{G_n - G})
# ---------------------------------------------------------------------------
def gdn2_chunk_step(Q, K, V, LA, Bg, Wg, S):
    """One chunk: Q,K,Bg,LA [n,dk]; V,Wg [n,dv]; S [dv,dk]."""
    n = Q.shape[0]
    G = np.cumsum(LA, axis=0)
    diff = G[:, None, :] - G[None, :, :]
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    lower = np.tril(np.ones((n, n), dtype=bool), 0)
    W = np.exp(np.where(lower[:, :, None], diff, -np.inf))
    E = Bg * K
    Z = Wg * V
    Ae = np.einsum("rc,ic,ric->ri", K, E, W) * strict
    Ak = np.einsum("rc,ic,ric->ri", K, K, W) * strict
    Pe = np.einsum("rc,ic,ric->ri", Q, E, W)
    Pk = np.einsum("rc,ic,ric->ri", Q, K, W)
    Te = unit_lower_inverse(np.eye(n) + Ae)
    X = -Te @ ((K * np.exp(G)) @ S.T + Ak @ Z)
    O = (Q * np.exp(G)) @ S.T + Pe @ X + Pk @ Z
    tail = np.exp(G[-1][None, :] - G)
    S_next = S * np.exp(G[-1])[None, :] + X.T @ (E * tail) + Z.T @ (K * tail)
    return O, S_next


def gdn2_fwd(q, k, v, log_alpha, erase, write, S0=None, cu_seqlens=None, chunk: int = 64):
    """Chunkwise Gated DeltaNet-2 forward, layouts as ``oracle.gdn2_fwd``."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    la, eb, wg = as_f64(log_alpha), as_f64(erase), as_f64(write)
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
            S = s0[u, h].copy() if s0 is not None else np.zeros((dv, dk))
            for s in range(t0, t1, chunk):
                e = min(s + chunk, t1)
                o[b, s:e, h], S = gdn2_chunk_step(q[b, s:e, h], k[b, s:e, h], v[b, s:e, h],
                                                  la[b, s:e, h], eb[b, s:e, h], wg[b, s:e, h], S)
            st[u, h] = S
    return o, st
