"""CPU model of the bf16 MFMA chunk kernel's operand precision (test helper).

Runs the chunkwise WY/UT form ("Gated Delta Networks: Improving Mamba2 with
Delta Rule", research-map summary, section "Approach") in fp64 while rounding
each intermediate the way the kernel does: bf16 operands ("bf16"), hi + lo
bf16 pairs ("split", about 16 mantissa bits: x = hi + lo with hi = bf16(x),
lo = bf16(x - hi)), fp32 storage ("f32"), with fp32 accumulation treated as
exact.  The UT inverse is modelled block by block as the kernel forms it:
16 x 16 diagonal blocks inverted in fp32, off-diagonal blocks
T_ij = -T_ii sum_k A_ik T_kj from the rounded A blocks and the rounded
T blocks.  `SCHEMES` names the kernel's scheme and the earlier all-bf16 one.

This is a model of the kernel's arithmetic, not an oracle: tests compare it
with the fp64 oracle to show which operand formats keep the parity bar.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def split(x):
    hi = bf16(x)
    return hi + bf16(x - hi)


ROUND = {"bf16": bf16, "split": split, "f32": f32}

# A: off-diagonal blocks of A; T: T blocks entering the block products;
# TU, TW: the factors (T - I) diag(beta) and T diag(beta e^g); Y: K S^T
SCHEMES = {
    "kernel": dict(A="split", T="split", TU="split", TW="split", Y="bf16"),
    "all-bf16 factors": dict(A="bf16", T="bf16", TU="bf16", TW="bf16", Y="bf16"),
}


def ut_blocked(k, b, g, scheme, C=64):
    """T = (I + A)^{-1} of one chunk (n <= C rows, zero-padded to C), formed
    as the kernel forms it."""
    n, rA, rT = k.shape[0], ROUND[scheme["A"]], ROUND[scheme["T"]]
    kp = np.zeros((C, k.shape[1]))
    kp[:n] = k
    bp = np.zeros(C)
    bp[:n] = b
    gp = np.full(C, g[-1])
    gp[:n] = g
    strict = np.tril(np.ones((C, C), bool), -1)
    dec = f32(np.exp(np.where(strict, gp[:, None] - gp[None, :], -np.inf)))
    A = f32(bp[:, None] * dec * f32(kp @ kp.T))
    Ar = rA(A)
    T = np.zeros((C, C))
    diag = []
    for i in range(4):
        s = slice(16 * i, 16 * i + 16)
        diag.append(f32(np.linalg.inv(np.eye(16) + A[s, s])))
        T[s, s] = diag[-1]
    for j in range(3):
        col = {j: rT(diag[j])}
        for i in range(j + 1, 4):
            y = sum(Ar[16 * i:16 * i + 16, 16 * m:16 * m + 16] @ col[m] for m in range(j, i))
            t = -f32(rT(diag[i]) @ rT(y))
            col[i] = rT(t)
            T[16 * i:16 * i + 16, 16 * j:16 * j + 16] = t
    return T[:n, :n]


def forward_unit(Q, K, V, la, be, S0, scheme, C=64):
    """o [L, d_v] and the final state of one (sequence, head) under `scheme`.
    Operands that the kernel always carries as hi + lo pairs (S^T where it
    multiplies Q, Delta, Delta~, P) are split here too."""
    L = Q.shape[0]
    S = S0.copy()
    O = np.zeros((L, V.shape[1]))
    rTU, rTW, rY = ROUND[scheme["TU"]], ROUND[scheme["TW"]], ROUND[scheme["Y"]]
    for s in range(0, L, C):
        e = min(s + C, L)
        n = e - s
        q, k, v, b = Q[s:e], K[s:e], V[s:e], be[s:e]
        g = f32(np.cumsum(la[s:e]))
        lower = np.tril(np.ones((n, n), bool))
        T = ut_blocked(k, b, g, scheme, C)
        TU = rTU((T - np.eye(n)) * b[None, :])
        TW = rTW(T * (b * f32(np.exp(g)))[None, :])
        Y = rY(k @ bf16(S.T))
        D = b[:, None] * v + TU @ v - TW @ Y
        P = split(f32((q @ k.T) * np.exp(np.where(lower, g[:, None] - g[None, :], -np.inf))))
        O[s:e] = np.exp(g)[:, None] * (q @ split(S.T)) + P @ split(D)
        Dt = split(np.exp(g[-1] - g)[:, None] * D)
        S = f32(np.exp(g[-1]) * S + (k.T @ Dt).T)
    return O, S
