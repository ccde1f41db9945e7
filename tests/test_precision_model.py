"""The MFMA kernel's operand formats keep the 2e-2 parity bar, in a CPU model.

`tests/precision_model.py` runs the chunk form with the kernel's roundings.
On random keys both the kernel's scheme and a plain all-bf16-factor scheme
are within the bar; with keys repeated inside a chunk, or nearly collinear,
under weak decay only the kernel's scheme (A, the T blocks and the factors
(T - I) diag(beta), T diag(beta e^g) carried as hi + lo pairs) stays within
it.  The GPU tests in test_gpu_hard_keys.py check the kernel itself on the
same kinds of inputs.
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from tests import precision_model as pm

TAU = 2e-2


def errors(inp, scheme):
    a = {k: oracle.as_f64(x) for k, x in inp.items() if x is not None and k != "cu_seqlens"}
    o, st = oracle.fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["S0"])
    ro, rs = np.sqrt(np.mean(o ** 2)), np.sqrt(np.mean(st ** 2))
    eo = es = 0.0
    for h in range(a["q"].shape[2]):
        O, S = pm.forward_unit(a["q"][0, :, h], a["k"][0, :, h], a["v"][0, :, h],
                               a["log_alpha"][0, :, h], a["beta"][0, :, h],
                               a["S0"][0, h], pm.SCHEMES[scheme])
        eo = max(eo, np.abs(O - o[0, :, h]).max() / ro)
        es = max(es, np.abs(S - st[0, h]).max() / rs)
    return eo, es


def test_model_rounding_helpers():
    x = np.array([1.0 + 2 ** -12, np.pi, -1e-3])
    assert np.all(np.abs(pm.bf16(x) - x) <= 2 ** -9 * np.abs(x))
    assert np.all(np.abs(pm.split(x) - x) <= 2 ** -16 * np.abs(x))
    assert pm.f32(np.array([1.0 + 2 ** -30]))[0] == 1.0


def test_blocked_inverse_matches_inverse_in_fp64():
    """With every rounding turned off the blocked UT inverse is the inverse."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal((50, 32))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    b = rng.uniform(0, 1, 50)
    g = np.cumsum(-rng.uniform(0, 0.5, 50))
    exact = {"A": "f32", "T": "f32"}
    T = pm.ut_blocked(k, b, g, exact)
    A = np.tril(b[:, None] * np.exp(g[:, None] - g[None, :]) * (k @ k.T), -1)
    assert np.allclose(T, np.linalg.inv(np.eye(50) + A), atol=1e-5)


@pytest.mark.parametrize("scheme", ["kernel", "all-bf16 factors"])
def test_random_keys_within_bar(scheme):
    inp = gi.chunk_inputs(1, 256, 1, 128, 128, "bf16", alpha_mu=1.0, s0_std=0.1, seed=3)
    eo, es = errors(inp, scheme)
    assert eo <= TAU and es <= TAU


@pytest.mark.parametrize("mode,param,shift", [("repeat", 16, 0.0), ("cluster", 1, 0.0),
                                              ("cluster", 4, 1.0)])
def test_structured_keys_need_the_split_factors(mode, param, shift):
    inp = gi.structured_chunk_inputs(1, 320, 1, 128, 128, mode, param, "bf16",
                                     alpha_mu=-4.0, s0_std=0.1, beta_shift=shift, seed=4)
    eo, es = errors(inp, "kernel")
    assert eo <= TAU / 3 and es <= TAU / 3, (eo, es)
    bo, bs = errors(inp, "all-bf16 factors")
    assert max(bo, bs) > TAU, (bo, bs)
