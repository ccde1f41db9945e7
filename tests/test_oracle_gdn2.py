"""The oracle's Gated DeltaNet-2 forward against what fixes it (CPU).

The pages state that the rule generalises KDA and reduces to it when the
erase and write gates collapse to one scalar.  The oracle's reading (erase
gate on the key side of the erase term, write gate on the value side of the
write term) is pinned by that reduction to the pinned KDA oracle, by two
closed forms (no erase: a linear recurrence; axis-aligned keys: one scalar
recurrence per channel), by the chunk form reaching the same result, and by
planted mistakes that these pins catch.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import chunk_form

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")


def _inputs(rng, B, T, H, dk, dv, units=None):
    u = B if units is None else units
    k = rng.standard_normal((B, T, H, dk))
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    return dict(q=rng.standard_normal((B, T, H, dk)),
                k=k / np.linalg.norm(k, axis=-1, keepdims=True),
                v=rng.standard_normal((B, T, H, dv)),
                la=-np.log1p(np.exp(rng.normal(0.5, 1.0, (B, T, H, dk)))),
                b=sig(rng.standard_normal((B, T, H, dk))),
                w=sig(rng.standard_normal((B, T, H, dv))),
                S0=rng.standard_normal((u, H, dv, dk)))


def pin_scalar_gates_are_kda(g2):
    x = _inputs(np.random.default_rng(1), 2, 50, 2, 8, 5)
    beta = x["b"][..., 0]
    o1, s1 = oracle.kda_fwd(x["q"], x["k"], x["v"], x["la"], beta, x["S0"])
    o2, s2 = g2(x["q"], x["k"], x["v"], x["la"], np.repeat(beta[..., None], 8, -1),
                np.repeat(beta[..., None], 5, -1), x["S0"])
    return np.allclose(o1, o2, atol=1e-12) and np.allclose(s1, s2, atol=1e-12)


def pin_no_erase_is_linear(g2):
    """b = 0: S_t = S0 Diag(e^{G_t}) + sum_{i<=t} (w_i o v_i) k_i^T Diag(e^{G_t - G_i})."""
    x = _inputs(np.random.default_rng(2), 1, 25, 1, 6, 4)
    b = np.zeros_like(x["b"])
    o, st = g2(x["q"], x["k"], x["v"], x["la"], b, x["w"], x["S0"])
    G = np.cumsum(x["la"][0, :, 0], axis=0)
    k, z = x["k"][0, :, 0], (x["w"] * x["v"])[0, :, 0]
    S0 = x["S0"][0, 0]
    ok = True
    for t in range(25):
        S = S0 * np.exp(G[t])[None, :]
        for i in range(t + 1):
            S = S + np.outer(z[i], k[i] * np.exp(G[t] - G[i]))
        ok &= np.allclose(o[0, t, 0], S @ x["q"][0, t, 0], atol=1e-12)
    return bool(ok and np.allclose(st[0, 0], S, atol=1e-12))


def pin_axis_keys_decouple(g2):
    """k_t = e_{c_t}: column c_t becomes (1 - b_c) alpha_c S[:, c] + w o v and the
    other columns only decay."""
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 5, 3
    x = _inputs(rng, 1, T, 1, dk, dv)
    ch = rng.integers(0, dk, T)
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, ch] = 1.0
    o, st = g2(x["q"], k, x["v"], x["la"], x["b"], x["w"], x["S0"])
    S = x["S0"][0, 0].copy()
    outs = []
    for t in range(T):
        a = np.exp(x["la"][0, t, 0])
        for c in range(dk):
            if c == ch[t]:
                S[:, c] = (1 - x["b"][0, t, 0, c]) * a[c] * S[:, c] + x["w"][0, t, 0] * x["v"][0, t, 0]
            else:
                S[:, c] = a[c] * S[:, c]
        outs.append(S @ x["q"][0, t, 0])
    return np.allclose(o[0, :, 0], np.stack(outs), atol=1e-12) and np.allclose(st[0, 0], S,
                                                                                atol=1e-12)


PINS = {"scalar_gates_are_kda": pin_scalar_gates_are_kda,
        "no_erase_is_linear": pin_no_erase_is_linear,
        "axis_keys_decouple": pin_axis_keys_decouple}


def _g2(q, k, v, la, b, w, S0=None, cu=None):
    return oracle.gdn2_fwd(q, k, v, la, b, w, S0, cu)


@pytest.mark.parametrize("name", sorted(PINS))
def test_gdn2_pin(name):
    assert PINS[name](_g2)


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_gdn2_chunk_form_equals_recurrence(C):
    rng = np.random.default_rng(20 + C)
    cu = np.array([0, 70, 70, 131, 200], dtype=np.int32)
    for c in (None, cu):
        x = _inputs(rng, 1 if c is not None else 2, 200 if c is not None else 150, 2, 8, 6,
                    units=4 if c is not None else None)
        a = oracle.gdn2_fwd(x["q"], x["k"], x["v"], x["la"], x["b"], x["w"], x["S0"], c)
        b = chunk_form.gdn2_fwd(x["q"], x["k"], x["v"], x["la"], x["b"], x["w"], x["S0"], c,
                                chunk=C)
        for ga, gb in zip(a, b):
            assert np.max(np.abs(ga - gb)) <= 1e-10 * max(1.0, np.max(np.abs(ga)))


MUTANTS = {
    "erase_ungated": ("ek[c] = bt[c] * kt[c];                   /* erase direction b o k */",
                      "ek[c] = kt[c];"),
    "write_ungated": ("const double wv = wt[r] * vt[r];", "const double wv = vt[r];"),
    "read_undecayed": ("Sr[c] *= decay[c];\n                    rd += Sr[c] * kt[c];                 /* read (S~ k)_r */",
                       "rd += Sr[c] * kt[c];\n                    Sr[c] *= decay[c];"),
    "erase_sign": ("Sr[c] += wv * kt[c] - rd * ek[c];", "Sr[c] += wv * kt[c] + rd * ek[c];"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import test_oracle_gdn2 as t
lib = oracle.load({lib!r})
g2 = lambda q, k, v, la, b, w, S0=None, cu=None: oracle.gdn2_fwd(q, k, v, la, b, w, S0, cu,
                                                                  lib=lib)
bad = [n for n, p in t.PINS.items() if not p(g2)]
print(",".join(bad))
sys.exit(1 if bad else 0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_gdn2_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not found: {old}"
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(text.replace(old, new))
    oracle.build(str(c), str(so))
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(so))],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught the planted mistake {name!r}"
