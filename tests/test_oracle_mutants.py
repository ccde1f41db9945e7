"""The pins catch plausible mistakes in the oracle (CPU only).

Each case below copies ``oracle/gdn_oracle.c``, plants one plausible mistake
by a textual substitution, compiles the copy into a temporary directory and
runs the pin suite against it in a child process (so an out-of-bounds
mistake cannot take down the test runner).  Every planted mistake must make
at least one pin fail; the unmodified source must pass all of them.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

WRITE = "const double w = b * vt[r] - a * b * p[r];"
GATE = "const double a = exp(log_alpha[t * ts_g]);"
READ_P = "acc += S[(long)r * dk + c] * kt[c];"
READ_O = "acc += S[(long)r * dk + c] * qt[c];"
INIT = "S[e] = S0 ? S0[e] : 0.0;"

MUTANTS = {
    "gate_on_write": (WRITE, "const double w = a * b * vt[r] - a * b * p[r];"),
    "erase_sign": (WRITE, "const double w = b * vt[r] + a * b * p[r];"),
    "erase_undecayed": (WRITE, "const double w = b * vt[r] - b * p[r];"),
    "erase_dropped": (WRITE, "const double w = b * vt[r];"),
    "erase_without_beta": (WRITE, "const double w = b * vt[r] - a * p[r];"),
    "gate_not_exponentiated": (GATE, "const double a = 1.0 + log_alpha[t * ts_g];"),
    "gate_next_token": (GATE, "const double a = exp(log_alpha[(t + 1 < L ? t + 1 : t) * ts_g]);"),
    "read_transposed_state": (READ_P, "acc += S[(long)(c % dv) * dk + (r % dk)] * kt[c];"),
    "readout_with_key": (READ_O, "acc += S[(long)r * dk + c] * kt[c];"),
    "initial_state_ignored": (INIT, "S[e] = 0.0;"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins as pins
lib = oracle.load({lib!r})
fwd = lambda q, k, v, la, be, S0=None, cu=None: oracle.fwd(q, k, v, la, be, S0, cu, lib=lib)
bad = pins.failing_pins(fwd)
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


def test_unmodified_source_passes(tmp_path):
    with open(SRC) as f:
        text = f.read()
    rc, out = _run_pins(tmp_path, "clean", text)
    assert rc == 0, f"pins failed on the unmodified oracle: {out}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor not found: {old}"
    rc, out = _run_pins(tmp_path, name, text.replace(old, new))
    assert rc != 0, f"no pin caught the planted mistake {name!r}"
