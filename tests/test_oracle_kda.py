"""The oracle's channel-wise decay (KDA) forward against what fixes it (CPU).

The pages state that KDA is the delta rule with channel-wise decay and that
it reduces to Gated DeltaNet when the decay collapses to a scalar; the
oracle's reading (decay on the key channels, before the delta update) is
pinned by that reduction, by two closed forms (beta = 0: pure channel
decay; axis-aligned keys: one scalar recurrence per channel), by the chunk
form reaching the same result for several chunk sizes, and by planted
mistakes that these pins catch.
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
    return dict(q=rng.standard_normal((B, T, H, dk)),
                k=k / np.linalg.norm(k, axis=-1, keepdims=True),
                v=rng.standard_normal((B, T, H, dv)),
                la=-np.log1p(np.exp(rng.normal(0.5, 1.0, (B, T, H, dk)))),
                be=1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
                S0=rng.standard_normal((u, H, dv, dk)))


def pin_scalar_decay_is_gdn(kda):
    x = _inputs(np.random.default_rng(1), 2, 50, 2, 8, 5)
    la = x["la"][..., 0]
    o1, s1 = oracle.fwd(x["q"], x["k"], x["v"], la, x["be"], x["S0"])
    o2, s2 = kda(x["q"], x["k"], x["v"], np.repeat(la[..., None], 8, -1), x["be"], x["S0"])
    return np.allclose(o1, o2, atol=1e-12) and np.allclose(s1, s2, atol=1e-12)


def pin_beta_zero_pure_decay(kda):
    """beta = 0: S_t = S0 Diag(e^{G_t}), o_t = S_t q_t."""
    x = _inputs(np.random.default_rng(2), 1, 30, 1, 6, 4)
    be = np.zeros_like(x["be"])
    o, st = kda(x["q"], x["k"], x["v"], x["la"], be, x["S0"])
    G = np.cumsum(x["la"][0, :, 0], axis=0)
    S0 = x["S0"][0, 0]
    want_o = np.stack([(S0 * np.exp(G[t])[None, :]) @ x["q"][0, t, 0] for t in range(30)])
    return (np.allclose(o[0, :, 0], want_o, atol=1e-12)
            and np.allclose(st[0, 0], S0 * np.exp(G[-1])[None, :], atol=1e-12))


def pin_axis_keys_decouple(kda):
    """k_t = e_{c_t}: column c_t becomes (1 - beta) alpha_c S[:, c] + beta v and
    every other column only decays, so each column is a scalar recurrence."""
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 5, 3
    x = _inputs(rng, 1, T, 1, dk, dv)
    ch = rng.integers(0, dk, T)
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, ch] = 1.0
    o, st = kda(x["q"], k, x["v"], x["la"], x["be"], x["S0"])
    S = x["S0"][0, 0].copy()
    outs = []
    for t in range(T):
        a = np.exp(x["la"][0, t, 0])
        b = x["be"][0, t, 0]
        for c in range(dk):
            if c == ch[t]:
                S[:, c] = (1 - b) * a[c] * S[:, c] + b * x["v"][0, t, 0]
            else:
                S[:, c] = a[c] * S[:, c]
        outs.append(S @ x["q"][0, t, 0])
    return np.allclose(o[0, :, 0], np.stack(outs), atol=1e-12) and np.allclose(st[0, 0], S,
                                                                                atol=1e-12)


PINS = {"scalar_decay_is_gdn": pin_scalar_decay_is_gdn,
        "beta_zero_pure_decay": pin_beta_zero_pure_decay,
        "axis_keys_decouple": pin_axis_keys_decouple}


def _kda(q, k, v, la, be, S0=None, cu=None):
    return oracle.kda_fwd(q, k, v, la, be, S0, cu)


@pytest.mark.parametrize("name", sorted(PINS))
def test_kda_pin(name):
    assert PINS[name](_kda)


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_kda_chunk_form_equals_recurrence(C):
    rng = np.random.default_rng(10 + C)
    cu = np.array([0, 70, 70, 131, 200], dtype=np.int32)
    for c in (None, cu):
        x = _inputs(rng, 1 if c is not None else 2, 200 if c is not None else 150, 2, 8, 6,
                    units=4 if c is not None else None)
        a = oracle.kda_fwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], c)
        b = chunk_form.kda_fwd(x["q"], x["k"], x["v"], x["la"], x["be"], x["S0"], c, chunk=C)
        for ga, gb in zip(a, b):
            assert np.max(np.abs(ga - gb)) <= 1e-10 * max(1.0, np.max(np.abs(ga)))


MUTANTS = {
    "decay_dropped": ("Sr[c] *= decay[c];                   /* S~ = S Diag(alpha) */",
                           "Sr[c] *= 1.0;"),
    "decay_not_exponentiated": ("for (int c = 0; c < dk; ++c) decay[c] = exp(lat[c]);",
                                "for (int c = 0; c < dk; ++c) decay[c] = 1.0 + lat[c];"),
    "decay_on_values": ("Sr[c] *= decay[c];                   /* S~ = S Diag(alpha) */",
                        "Sr[c] *= exp(lat[r % dk]);"),
    "write_without_beta": ("const double wr = b * (vt[r] - read);",
                           "const double wr = vt[r] - b * read;"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import test_oracle_kda as t
lib = oracle.load({lib!r})
kda = lambda q, k, v, la, be, S0=None, cu=None: oracle.kda_fwd(q, k, v, la, be, S0, cu, lib=lib)
bad = [n for n, p in t.PINS.items() if not p(kda)]
print(",".join(bad))
sys.exit(1 if bad else 0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_kda_mistake_is_caught(tmp_path, name):
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
