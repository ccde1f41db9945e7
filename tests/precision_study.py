"""Precision study behind the MFMA kernel's operand formats (not a test).

    python -m tests.precision_study [T] [H]

Runs the chunkwise WY/UT form in fp64 while rounding chosen intermediates the
way a bf16-operand / fp32-accumulate kernel would, and reports the parity
statistic max|x - oracle| / RMS(oracle) for o and for the final state on the
1.3B-layer-shaped input distribution.  "bf16" rounds an operand to bfloat16,
"split" keeps it as a hi + lo pair of bfloat16 (about 16 mantissa bits),
"fp32" rounds to float, "diag" keeps the diagonal of the beta-scaled T in
full precision (the kernel forms beta V exactly and only the strictly lower
part of T diag(beta) goes through bf16).  The last variant is the kernel's
scheme: the state is split only where it multiplies Q; K S^T uses the hi
part alone and is rounded once to bf16 before T diag(beta e^g) multiplies
it (that product's left factor is bf16 anyway, so the extra bits do not
show in o or the state).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import gdn_inputs as gi
import oracle


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _split(x):
    hi = _bf(x)
    return hi + _bf(x - hi)


ROUND = {"bf16": _bf, "split": _split, "exact": lambda x: x,
         "fp32": lambda x: x.astype(np.float32).astype(np.float64)}


def _r(mode, x, keep_diag=False):
    if keep_diag:
        d = np.diag(np.diag(x))
        return ROUND[mode](x - d) + d
    return ROUND[mode](x)


def emulate_unit(Q, K, V, la, be, S0, cfg, C=64):
    L = Q.shape[0]
    S = S0.copy()
    O = np.zeros((L, V.shape[1]))
    for s in range(0, L, C):
        e = min(s + C, L)
        n = e - s
        q, k, v, b = Q[s:e], K[s:e], V[s:e], be[s:e]
        g = np.cumsum(la[s:e])
        diff = g[:, None] - g[None, :]
        strict = np.tril(np.ones((n, n), bool), -1)
        lower = np.tril(np.ones((n, n), bool))
        A = b[:, None] * np.exp(np.where(strict, diff, -np.inf)) * (k @ k.T)
        T = _bf(np.linalg.inv(np.eye(n) + A) - np.eye(n)) + np.eye(n)
        TU = _r(cfg["TU"], T * b[None, :], cfg["TU_diag"])
        TW = _bf(T * (b * np.exp(g))[None, :])
        ST = _r(cfg["S"], S.T)
        Y = k @ _r(cfg.get("SY", cfg["S"]), S.T)
        D = TU @ v - TW @ _r(cfg["Y"], Y)
        P = _r(cfg["P"], (q @ k.T) * np.exp(np.where(lower, diff, -np.inf)))
        O[s:e] = _r(cfg["O"], np.exp(g)[:, None] * (q @ ST) + P @ _r(cfg["D"], D))
        Dt = _r(cfg["D"], np.exp(g[-1] - g)[:, None] * D)
        S = np.exp(g[-1]) * S + (k.T @ Dt).T
    return O, S


VARIANTS = {
    "all operands bf16, o bf16": dict(TU="bf16", TU_diag=False, S="bf16", Y="bf16", P="bf16", D="bf16", O="bf16"),
    "all operands bf16, o fp32": dict(TU="bf16", TU_diag=False, S="bf16", Y="bf16", P="bf16", D="bf16", O="fp32"),
    "+ beta diagonal exact": dict(TU="bf16", TU_diag=True, S="bf16", Y="bf16", P="bf16", D="bf16", O="fp32"),
    "+ Delta split": dict(TU="bf16", TU_diag=True, S="bf16", Y="bf16", P="bf16", D="split", O="fp32"),
    "+ P split": dict(TU="bf16", TU_diag=True, S="bf16", Y="bf16", P="split", D="split", O="fp32"),
    "+ S^T, Y split": dict(TU="bf16", TU_diag=True, S="split", Y="split", P="split", D="split", O="fp32"),
    "S^T split for Q S^T only (kernel)": dict(TU="bf16", TU_diag=True, S="split", SY="bf16", Y="bf16", P="split", D="split", O="fp32"),
}


def main(T=2048, H=4):
    w = gi.WORKLOADS[2]
    inp = gi.chunk_inputs(1, T, H, w["dk"], w["dv"], "bf16", w["alpha_mu"], 0.0, seed=3)
    a = {k: oracle.as_f64(x) for k, x in inp.items() if x is not None and k != "cu_seqlens"}
    o, st = oracle.fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], None)
    ro, rs = np.sqrt(np.mean(o ** 2)), np.sqrt(np.mean(st ** 2))
    print(f"T={T} H={H} d=128, max|o|/RMS(o) = {np.abs(o).max() / ro:.1f}")
    for name, cfg in VARIANTS.items():
        eo = es = 0.0
        for h in range(H):
            O, S = emulate_unit(a["q"][0, :, h], a["k"][0, :, h], a["v"][0, :, h],
                                a["log_alpha"][0, :, h], a["beta"][0, :, h],
                                np.zeros((w["dv"], w["dk"])), cfg)
            eo = max(eo, np.max(np.abs(O - o[0, :, h])) / ro)
            es = max(es, np.max(np.abs(S - st[0, h])) / rs)
        print(f"{name:32s} o {eo:.4f}  S {es:.4f}", flush=True)


if __name__ == "__main__":
    main(*(int(x) for x in sys.argv[1:3]))
