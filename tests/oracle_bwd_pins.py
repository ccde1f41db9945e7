"""Pins of the oracle's backward pass (CPU only, fp64).

A backward pass is fixed by its forward: these checks compare the oracle's
reverse-mode gradients with central finite differences of the oracle's own
forward (whose pins are in ``oracle_pins.py``), with two identities that
hold for the exact gradient, and with the closed form of the beta = 0 case.
``failing_bwd_pins`` runs them all and names the ones that fail, so the
mutant test can run the same suite against a planted mistake.
"""
from __future__ import annotations

import numpy as np


def _inputs(rng, B, T, H, dk, dv, units=None, s0=True):
    u = B if units is None else units
    return dict(
        q=rng.standard_normal((B, T, H, dk)),
        k=rng.standard_normal((B, T, H, dk)) / np.sqrt(dk),
        v=rng.standard_normal((B, T, H, dv)),
        la=-np.log1p(np.exp(rng.normal(0.5, 1.0, (B, T, H)))),
        be=1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
        S0=rng.standard_normal((u, H, dv, dk)) * 0.5 if s0 else None,
        dO=rng.standard_normal((B, T, H, dv)),
        dS_T=rng.standard_normal((u, H, dv, dk)),
    )


def _loss(fwd, x, cu):
    o, st = fwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], cu)
    return float(np.sum(o * x["dO"]) + np.sum(st * x["dS_T"]))


def finite_difference_error(fwd, bwd, x, cu=None, h=1e-6):
    """max |reverse mode - central difference| / max |central difference|
    over every element of every differentiable input."""
    g = bwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], cu, x["dO"], x["dS_T"])
    worst = 0.0
    for name, gi in zip(("q", "k", "v", "la", "be", "S0"), g):
        if x[name] is None:
            continue
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            keep = x[name][idx]
            x[name][idx] = keep + h
            lp = _loss(fwd, x, cu)
            x[name][idx] = keep - h
            lm = _loss(fwd, x, cu)
            x[name][idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        scale = max(np.max(np.abs(num)), 1e-12)
        worst = max(worst, float(np.max(np.abs(num - gi)) / scale))
    return worst


def pin_fd_dense(fwd, bwd):
    # T = 70 spans three recompute segments of the oracle (32 tokens each)
    x = _inputs(np.random.default_rng(11), 1, 70, 1, 3, 2)
    return finite_difference_error(fwd, bwd, x) < 1e-6


def pin_fd_varlen(fwd, bwd):
    cu = np.array([0, 5, 5, 12], dtype=np.int32)   # includes an empty sequence
    x = _inputs(np.random.default_rng(12), 1, 12, 2, 3, 4, units=3)
    return finite_difference_error(fwd, bwd, x, cu) < 1e-6


def pin_fd_no_state(fwd, bwd):
    x = _inputs(np.random.default_rng(13), 2, 9, 1, 4, 3, s0=False)
    return finite_difference_error(fwd, bwd, x) < 1e-6


def pin_homogeneity(fwd, bwd):
    """o and S_T are jointly linear in (V, S0), and o is linear in Q with S_T
    independent of Q, so the exact gradient satisfies (Euler)
    <dV, V> + <dS0, S0> = L  and  <dQ, Q> = <dO, o>."""
    x = _inputs(np.random.default_rng(14), 2, 100, 2, 8, 6)
    o, st = fwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], None)
    L = np.sum(o * x["dO"]) + np.sum(st * x["dS_T"])
    dq, dk, dv, dla, dbe, ds0 = bwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], None,
                                    x["dO"], x["dS_T"])
    ok1 = abs(np.sum(dv * x["v"]) + np.sum(ds0 * x["S0"]) - L) <= 1e-9 * max(1.0, abs(L))
    lo = np.sum(o * x["dO"])
    ok2 = abs(np.sum(dq * x["q"]) - lo) <= 1e-9 * max(1.0, abs(lo))
    return bool(ok1 and ok2)


def pin_beta_zero_closed_form(fwd, bwd):
    """beta = 0: S_t = e^{g_t} S0 (pure decay), so o_t = e^{g_t} S0 q_t and
    dq_t = e^{g_t} S0^T dO_t, dS0 = sum_t e^{g_t} dO_t q_t^T + e^{g_T} dS_T,
    dlog_alpha_s = sum_{t >= s} e^{g_t} dO_t . S0 q_t + e^{g_T} <dS_T, S0>,
    dv = dk = 0, and dbeta_t = (G_t k_t) . (v_t - e^{g_t} S0 k_t) with
    G_t = sum_{s >= t} e^{g_s - g_t} dO_s q_s^T + e^{g_T - g_t} dS_T."""
    rng = np.random.default_rng(15)
    x = _inputs(rng, 1, 40, 1, 5, 4)
    x["be"] = np.zeros_like(x["be"])
    dq, dk, dv, dla, dbe, ds0 = bwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], None,
                                    x["dO"], x["dS_T"])
    q, k, v, dO = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["dO"][0, :, 0]
    S0, dST = x["S0"][0, 0], x["dS_T"][0, 0]
    g = np.cumsum(x["la"][0, :, 0])
    T = q.shape[0]
    e = np.exp(g)
    want_dq = e[:, None] * (dO @ S0)
    want_ds0 = (e[:, None] * dO).T @ q + e[-1] * dST
    c = e * np.einsum("ti,ij,tj->t", dO, S0, q)
    want_dla = np.cumsum(c[::-1])[::-1] + e[-1] * np.sum(dST * S0)
    want_dbe = np.zeros(T)
    for t in range(T):
        G = e[-1] / e[t] * dST
        for s in range(t, T):
            G = G + (e[s] / e[t]) * np.outer(dO[s], q[s])
        want_dbe[t] = (G @ k[t]) @ (v[t] - e[t] * (S0 @ k[t]))
    tol = 1e-10
    return bool(np.allclose(dq[0, :, 0], want_dq, atol=tol, rtol=tol)
                and np.allclose(ds0[0, 0], want_ds0, atol=tol, rtol=tol)
                and np.allclose(dla[0, :, 0], want_dla, atol=tol, rtol=tol)
                and np.allclose(dbe[0, :, 0], want_dbe, atol=tol, rtol=tol)
                and np.all(dv == 0) and np.all(dk == 0))


PINS = {
    "fd_dense": pin_fd_dense,
    "fd_varlen": pin_fd_varlen,
    "fd_no_state": pin_fd_no_state,
    "homogeneity": pin_homogeneity,
    "beta_zero_closed_form": pin_beta_zero_closed_form,
}


def failing_bwd_pins(fwd, bwd):
    bad = []
    for name, pin in PINS.items():
        try:
            ok = pin(fwd, bwd)
        except Exception:   # a crash or a shape error counts as a failure
            ok = False
        if not ok:
            bad.append(name)
    return bad
