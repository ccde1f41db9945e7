"""Pins for the CPU oracle: closed forms and invariants the recurrence must
satisfy, independent of how the oracle computes it.

Each ``pin_*`` takes a forward function
    fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None) -> (o, S_T)
over fp64 numpy arrays in the library's layouts (q,k [B,T,H,dk], v [B,T,H,dv],
gates [B,T,H], states [U,H,dv,dk]) and raises AssertionError on a mismatch.
They are run against the C oracle, against the NumPy chunk form at several
chunk sizes, and against deliberately broken copies of the C oracle (which
must each fail at least one pin).

The recurrence is that of "Gated Delta Networks: Improving Mamba2 with Delta
Rule" (research-map summary, section "Approach"); the special cases are the
ones the blog "Gated DeltaNet: Harmonizing Gating and the Delta Rule for
Superior Linear RNNs" describes in "Problem & Motivation" (Mamba2's scalar
decay that dims the whole state, DeltaNet's rank-one overwrite) and the
online-regression reading S_t k_t ~ v_t of its "Critical Insight".
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-11


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(seed, B=2, T=9, H=2, dk=4, dv=3, s0=True, unit_keys=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_keys:
        k = _unit(k)
    v = rng.standard_normal((B, T, H, dv))
    la = -rng.uniform(0.0, 1.5, (B, T, H))
    be = rng.uniform(0.0, 1.0, (B, T, H))
    S0 = rng.standard_normal((B, H, dv, dk)) if s0 else None
    return q, k, v, la, be, S0


def orthonormal_keys(seed, T, dk):
    """T <= dk orthonormal rows (numpy's QR of a Gaussian matrix)."""
    rng = np.random.default_rng(seed)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    return Qm[:T]


# --------------------------------------------------------------------------
def pin_worked_example(fwd):
    """Hand-derived 2x2 example (tests/golden/worked_example_2x2.json)."""
    with open(os.path.join(GOLDEN, "worked_example_2x2.json")) as f:
        g = json.load(f)
    q = np.array(g["q"])[None, :, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    la = np.log(np.array(g["alpha"]))[None, :, None]
    be = np.array(g["beta"])[None, :, None]
    S0 = np.array(g["S0"])[None, None]
    o, st = fwd(q, k, v, la, be, S0)
    _close(o[0, :, 0], g["o"], 1e-12, "worked example o")
    _close(st[0, 0], g["S_T"], 1e-12, "worked example S_T")


def pin_frozen_state(fwd):
    """alpha=1, beta=0: nothing is erased or written, S_T = S0, o_t = S0 q_t."""
    q, k, v, la, be, S0 = rand_case(1, unit_keys=False)
    la[:] = 0.0
    be[:] = 0.0
    o, st = fwd(q, k, v, la, be, S0)
    _close(st, S0, what="frozen S_T")
    _close(o, np.einsum("bhvk,bthk->bthv", S0, q), what="frozen o")


def pin_pure_decay(fwd):
    """beta=0 (Mamba2-style scalar gating): S_t = exp(g_t) S0, o_t = exp(g_t) S0 q_t."""
    q, k, v, la, be, S0 = rand_case(2, unit_keys=False)
    be[:] = 0.0
    g = np.cumsum(la, axis=1)                       # [B,T,H]
    o, st = fwd(q, k, v, la, be, S0)
    _close(st, np.exp(g[:, -1])[:, :, None, None] * S0, what="decay S_T")
    ref = np.exp(g)[..., None] * np.einsum("bhvk,bthk->bthv", S0, q)
    _close(o, ref, what="decay o")


def pin_deltanet_exact_write(fwd):
    """alpha=1, beta=1, S0=0, orthonormal keys (DeltaNet overwrite):
    S_T k_j = v_j for every j, o_t = sum_{j<=t} (k_j . q_t) v_j."""
    T, dk, dv = 5, 6, 3
    K = orthonormal_keys(3, T, dk)
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    q, k, v = Q[None, :, None], K[None, :, None], V[None, :, None]
    la = np.zeros((1, T, 1))
    be = np.ones((1, T, 1))
    o, st = fwd(q, k, v, la, be, None)
    _close(st[0, 0] @ K.T, V.T, what="exact write S_T k_j = v_j")
    ref = np.array([sum((K[j] @ Q[t]) * V[j] for j in range(t + 1))
                    for t in range(T)])
    _close(o[0, :, 0], ref, what="exact write o")


def pin_orthonormal_closed_form(fwd):
    """Orthonormal keys, any gates: the erase projections commute, so
    S_t = e^{g_t} S0 (I - sum_{j<=t} b_j k_j k_j^T) + sum_{j<=t} e^{g_t-g_j} b_j v_j k_j^T."""
    T, dk, dv = 6, 7, 4
    K = orthonormal_keys(5, T, dk)
    rng = np.random.default_rng(6)
    Q = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    la = -rng.uniform(0.0, 2.0, T)
    be = rng.uniform(0.0, 1.0, T)
    S0 = rng.standard_normal((dv, dk))
    o, st = fwd(Q[None, :, None], K[None, :, None], V[None, :, None],
                la[None, :, None], be[None, :, None], S0[None, None])
    g = np.cumsum(la)
    for t in range(T):
        proj = sum(be[j] * np.outer(K[j], K[j]) for j in range(t + 1))
        St = np.exp(g[t]) * S0 @ (np.eye(dk) - proj)
        St = St + sum(np.exp(g[t] - g[j]) * be[j] * np.outer(V[j], K[j])
                      for j in range(t + 1))
        _close(o[0, t, 0], St @ Q[t], what=f"orthonormal o_{t}")
        if t == T - 1:
            _close(st[0, 0], St, what="orthonormal S_T")


def product_form_states(K, V, la, be, S0):
    """Explicit closed form of the linear recurrence, with d_k x d_k matrices:
    S_t = S0 P_{1:t} + sum_{j<=t} b_j v_j k_j^T P_{j+1:t},
    P_{a:b} = prod_{s=a..b} alpha_s (I - b_s k_s k_s^T)   (left to right)."""
    T, dk = K.shape
    M = [np.exp(la[s]) * (np.eye(dk) - be[s] * np.outer(K[s], K[s]))
         for s in range(T)]

    def P(a, b):
        out = np.eye(dk)
        for s in range(a, b + 1):
            out = out @ M[s]
        return out

    states = []
    for t in range(T):
        St = S0 @ P(0, t)
        for j in range(t + 1):
            St = St + be[j] * np.outer(V[j], K[j]) @ P(j + 1, t)
        states.append(St)
    return states


def pin_product_form(fwd):
    """Random (non-unit) keys, d_k != d_v: matches the explicit product form."""
    rng = np.random.default_rng(7)
    T, dk, dv = 7, 3, 5
    K = rng.standard_normal((T, dk)) * 0.7
    Q = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    la = -rng.uniform(0.0, 1.0, T)
    be = rng.uniform(0.0, 1.5, T)
    S0 = rng.standard_normal((dv, dk))
    o, st = fwd(Q[None, :, None], K[None, :, None], V[None, :, None],
                la[None, :, None], be[None, :, None], S0[None, None])
    states = product_form_states(K, V, la, be, S0)
    for t in range(T):
        _close(o[0, t, 0], states[t] @ Q[t], what=f"product form o_{t}")
    _close(st[0, 0], states[-1], what="product form S_T")


def pin_regression_identity(fwd):
    """Unit keys: S_t k_t = alpha_t (1 - beta_t) S_{t-1} k_t + beta_t v_t
    (the delta rule moves the read at k_t towards v_t); with beta_t = 1 the
    read equals v_t exactly."""
    q, k, v, la, be, S0 = rand_case(8, B=1, T=8, H=1, dk=5, dv=4)
    be[0, 3, 0] = 1.0
    prev = S0[0, 0]
    for t in range(q.shape[1]):
        _, st = fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], la[:, :t + 1],
                    be[:, :t + 1], S0)
        St = st[0, 0]
        kt = k[0, t, 0]
        a, b = np.exp(la[0, t, 0]), be[0, t, 0]
        _close(St @ kt, a * (1 - b) * (prev @ kt) + b * v[0, t, 0],
               what=f"regression identity t={t}")
        prev = St
    _, st = fwd(q[:, :4], k[:, :4], v[:, :4], la[:, :4], be[:, :4], S0)
    _close(st[0, 0] @ k[0, 3, 0], v[0, 3, 0], what="beta=1 exact read")


def pin_linearity(fwd):
    """(o, S_T) are linear in (V, S0) jointly; o is linear in Q; S_T does not
    depend on Q."""
    q, k, v, la, be, S0 = rand_case(9)
    _, _, v2, _, _, S02 = rand_case(10)
    q2 = rand_case(11)[0]
    c = -1.75
    o1, s1 = fwd(q, k, v, la, be, S0)
    o2, s2 = fwd(q, k, v2, la, be, S02)
    o3, s3 = fwd(q, k, v + c * v2, la, be, S0 + c * S02)
    _close(o3, o1 + c * o2, what="linear in (V,S0): o")
    _close(s3, s1 + c * s2, what="linear in (V,S0): S_T")
    o4, s4 = fwd(q2, k, v, la, be, S0)
    o5, _ = fwd(q + c * q2, k, v, la, be, S0)
    _close(o5, o1 + c * o4, what="linear in Q")
    _close(s4, s1, what="S_T independent of Q")


def pin_split_resume(fwd):
    """Running tokens [0,T1) then [T1,T) from the carried state equals one run."""
    q, k, v, la, be, S0 = rand_case(12, T=11)
    o, st = fwd(q, k, v, la, be, S0)
    for t1 in (0, 4, 11):
        oa, sa = fwd(q[:, :t1], k[:, :t1], v[:, :t1], la[:, :t1], be[:, :t1], S0)
        ob, sb = fwd(q[:, t1:], k[:, t1:], v[:, t1:], la[:, t1:], be[:, t1:], sa)
        _close(np.concatenate([oa, ob], axis=1), o, what=f"split {t1}: o")
        _close(sb, st, what=f"split {t1}: S_T")


def pin_varlen_equals_separate(fwd):
    """Packed sequences (one of them empty) with cu_seqlens equal separate runs;
    the state restarts at every sequence start."""
    lens = [5, 0, 7, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt = int(cu[-1])
    q, k, v, la, be, _ = rand_case(13, B=1, T=Tt, H=2)
    rng = np.random.default_rng(14)
    S0 = rng.standard_normal((len(lens), 2, v.shape[-1], q.shape[-1]))
    o, st = fwd(q, k, v, la, be, S0, cu)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        oi, si = fwd(q[:, a:b], k[:, a:b], v[:, a:b], la[:, a:b], be[:, a:b],
                     S0[i:i + 1])
        _close(o[:, a:b], oi, what=f"varlen seq {i} o")
        _close(st[i:i + 1], si, what=f"varlen seq {i} S_T")


def pin_unit_permutation(fwd):
    """Units are independent: permuting batch and heads permutes the outputs."""
    q, k, v, la, be, S0 = rand_case(15, B=3, H=4)
    o, st = fwd(q, k, v, la, be, S0)
    pb, ph = np.array([2, 0, 1]), np.array([3, 1, 0, 2])
    P = lambda x: x[pb][:, :, ph] if x.ndim >= 3 else x  # noqa: E731
    o2, st2 = fwd(P(q), P(k), P(v), la[pb][:, :, ph], be[pb][:, :, ph],
                  S0[pb][:, ph])
    _close(o2, o[pb][:, :, ph], what="permuted o")
    _close(st2, st[pb][:, ph], what="permuted S_T")


def pin_empty_and_single(fwd):
    """T=0 writes no output and returns S0 (zeros when S0 is absent)."""
    q, k, v, la, be, S0 = rand_case(16, T=0)
    o, st = fwd(q, k, v, la, be, S0)
    assert o.shape[1] == 0
    _close(st, S0, what="empty S_T")
    _, st = fwd(q, k, v, la, be, None)
    _close(st, np.zeros_like(S0), what="empty S_T, no S0")


ALL_PINS = [pin_worked_example, pin_frozen_state, pin_pure_decay,
            pin_deltanet_exact_write, pin_orthonormal_closed_form,
            pin_product_form, pin_regression_identity, pin_linearity,
            pin_split_resume, pin_varlen_equals_separate,
            pin_unit_permutation, pin_empty_and_single]


def failing_pins(fwd) -> list[str]:
    """Names of the pins that fail (an exception of any kind counts)."""
    bad = []
    for p in ALL_PINS:
        try:
            p(fwd)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            bad.append(p.__name__)
    return bad
