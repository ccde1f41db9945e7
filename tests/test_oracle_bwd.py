"""The oracle's backward pass against its pins, and planted mistakes in it
(CPU only).

The pins (``tests/oracle_bwd_pins.py``) compare the reverse-mode gradients
with central finite differences of the pinned forward, with the Euler
identities of the two linear parts of the map, and with the closed form at
beta = 0.  Each mutant copies ``oracle/gdn_oracle.c``, plants one plausible
mistake in the backward by a textual substitution, compiles the copy and runs
the pins in a child process; every mutant must fail at least one of them.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_bwd_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")


def _fwd(q, k, v, la, be, S0=None, cu=None):
    return oracle.fwd(q, k, v, la, be, S0, cu)


def _bwd(q, k, v, la, be, S0, cu, dO, dS_T):
    return oracle.bwd(q, k, v, la, be, S0, cu, dO, dS_T)


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_bwd_pin(name):
    assert pins.PINS[name](_fwd, _bwd), name


MUTANTS = {
    "readout_term_dropped": ("G[(long)r * dk + c] += dot[r] * qt[c];",
                             "G[(long)r * dk + c] += 0.0 * dot[r] * qt[c];"),
    "dq_from_old_state": ("acc += Sn[(long)r * dk + c] * dot[r];",
                          "acc += Sp[(long)r * dk + c] * dot[r];"),
    "dk_read_term_dropped": (
        "acc += G[(long)r * dk + c] * b * (vt[r] - a * p[r]) + Sp[(long)r * dk + c] * dp[r];",
        "acc += G[(long)r * dk + c] * b * (vt[r] - a * p[r]);"),
    "dalpha_read_term_dropped": ("dla[t * ts_g] = a * (gs - b * dup);",
                                 "dla[t * ts_g] = a * gs;"),
    "dlog_alpha_not_chained": ("dla[t * ts_g] = a * (gs - b * dup);",
                               "dla[t * ts_g] = gs - b * dup;"),
    "dbeta_without_erase": ("db += du[r] * (vt[r] - a * p[r]);", "db += du[r] * vt[r];"),
    "dp_sign": ("dp[r] = -a * b * du[r];", "dp[r] = a * b * du[r];"),
    "state_grad_undecayed": ("G[(long)r * dk + c] = a * G[(long)r * dk + c] + dp[r] * kt[c];",
                             "G[(long)r * dk + c] = G[(long)r * dk + c] + dp[r] * kt[c];"),
    "state_grad_erase_dropped": (
        "G[(long)r * dk + c] = a * G[(long)r * dk + c] + dp[r] * kt[c];",
        "G[(long)r * dk + c] = a * G[(long)r * dk + c];"),
    "dv_without_beta": ("dvt[r] = b * du[r];", "dvt[r] = du[r];"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_bwd_pins as pins
lib = oracle.load({lib!r})
fwd = lambda q, k, v, la, be, S0=None, cu=None: oracle.fwd(q, k, v, la, be, S0, cu, lib=lib)
bwd = lambda q, k, v, la, be, S0, cu, dO, dS_T: oracle.bwd(q, k, v, la, be, S0, cu, dO, dS_T,
                                                         lib=lib)
bad = pins.failing_bwd_pins(fwd, bwd)
print(",".join(bad))
sys.exit(1 if bad else 0)
"""


def _run_pins(tmp_path, name, src_text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src_text)
    oracle.build(str(c), str(so))
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(so))],
                       capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout.strip()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_bwd_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor not found: {old}"
    rc, out = _run_pins(tmp_path, name, text.replace(old, new))
    assert rc != 0, f"no pin caught the planted mistake {name!r}"


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_chunk_form_backward_equals_recurrence_backward(C):
    """The chunkwise backward (reverse state gradients across chunks, then
    each chunk's gradients) reaches the token recurrence's gradients."""
    import numpy as np
    from oracle import chunk_form
    rng = np.random.default_rng(40 + C)
    cu = np.array([0, 70, 70, 131, 200], dtype=np.int32)
    x = pins._inputs(rng, 1, 200, 2, 8, 6, units=4)
    x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)
    for c in (None, cu):
        if c is None:
            y = pins._inputs(rng, 2, 150, 2, 8, 6)
        else:
            y = x
        a = oracle.bwd(y["q"], y["k"], y["v"], y["la"], y["be"], y["S0"], c, y["dO"], y["dS_T"])
        b = chunk_form.bwd(y["q"], y["k"], y["v"], y["la"], y["be"], y["S0"], c, y["dO"],
                           y["dS_T"], chunk=C)
        for ga, gb in zip(a, b):
            assert np.max(np.abs(ga - gb)) <= 1e-11 * max(1.0, np.max(np.abs(ga)))
