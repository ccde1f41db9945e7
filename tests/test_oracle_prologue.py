"""The oracle's input prologue against closed forms and torch (CPU only).

The prologue turns raw projections into the rule's inputs: q, k are
L2-normalised per token, beta = sigmoid(b), log alpha = -softplus(a).  The
pages are silent on this step; the definitions follow the workloads' input
recipe.  Pins: unit norms and scale invariance, the clamp on all-zero rows,
closed forms of sigmoid and softplus (sigmoid(0) = 1/2, sigmoid(x) +
sigmoid(-x) = 1, softplus(0) = log 2, softplus(x) - softplus(-x) = x and the
asymptotes), torch's own normalize / sigmoid / softplus, and a planted
mistake for each function that one of these pins catches."""
import math

import numpy as np
import pytest
import torch

from oracle import prologue as pro

RNG = np.random.default_rng(5801)


def test_l2_normalize_unit_and_scale_invariant():
    x = RNG.standard_normal((3, 7, 2, 32))
    y = pro.l2_normalize(x)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(pro.l2_normalize(4.5 * x), y, atol=1e-15)
    # direction kept: y is a positive multiple of x
    assert np.all(np.sum(x * y, axis=-1) > 0)


def test_l2_normalize_matches_torch():
    x = RNG.standard_normal((5, 128))
    ref = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy()
    assert np.allclose(pro.l2_normalize(x), ref, atol=1e-15)


def test_l2_normalize_zero_row_and_clamp():
    x = np.zeros((2, 16))
    x[1, 3] = 1e-9           # norm below the 1e-6 floor
    y = pro.l2_normalize(x)
    assert np.all(y[0] == 0.0)
    assert math.isclose(y[1, 3], 1e-9 / 1e-6, rel_tol=1e-12)


def test_sigmoid_closed_forms():
    assert pro.sigmoid(0.0) == 0.5
    b = RNG.standard_normal(1000) * 5
    assert np.allclose(pro.sigmoid(b) + pro.sigmoid(-b), 1.0, atol=1e-15)
    assert np.allclose(pro.sigmoid(b), torch.sigmoid(torch.from_numpy(b)).numpy(), atol=1e-15)
    assert math.isclose(float(pro.sigmoid(np.log(3.0))), 0.75, rel_tol=1e-15)


def test_neg_softplus_closed_forms():
    assert math.isclose(float(pro.neg_softplus(0.0)), -math.log(2.0), rel_tol=1e-15)
    a = RNG.standard_normal(1000) * 5
    # softplus(x) - softplus(-x) = x
    assert np.allclose(-pro.neg_softplus(a) + pro.neg_softplus(-a), a, atol=1e-13)
    assert np.allclose(pro.neg_softplus(a),
                       -torch.nn.functional.softplus(torch.from_numpy(a), threshold=1e9).numpy(),
                       atol=1e-14)
    # asymptotes, without overflow: -softplus(x) -> -x (x >> 0), -> -e^x (x << 0)
    assert math.isclose(float(pro.neg_softplus(800.0)), -800.0, rel_tol=1e-15)
    assert math.isclose(float(pro.neg_softplus(-40.0)), -math.exp(-40.0), rel_tol=1e-12)
    assert np.all(pro.neg_softplus(a) < 0)


def test_apply_flags():
    q = RNG.standard_normal((2, 3, 8))
    k = RNG.standard_normal((2, 3, 8))
    a = RNG.standard_normal((2, 3))
    b = RNG.standard_normal((2, 3))
    q1, k1, la, be = pro.apply(q, k, a, b)
    assert np.allclose(np.linalg.norm(q1, axis=-1), 1.0)
    assert np.all(la < 0) and np.all((be > 0) & (be < 1))
    q2, k2, la2, be2 = pro.apply(q, k, a, b, norm_qk=False, gates=False)
    assert np.array_equal(q2, q) and np.array_equal(la2, a) and np.array_equal(be2, b)


def _mutants():
    """Plausible mistakes, each of which a pin above must catch."""
    return {
        "norm without sqrt": lambda x: x / np.maximum(np.sum(x * x, -1, keepdims=True), 1e-12),
        "sigmoid sign": lambda b: 1.0 / (1.0 + np.exp(b)),
        "softplus as log(e^a)": lambda a: -a,
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_mistake_is_caught(name):
    f = _mutants()[name]
    x = RNG.standard_normal((4, 16))
    if name.startswith("norm"):
        assert not np.allclose(np.linalg.norm(f(x), axis=-1), 1.0)
    elif name.startswith("sigmoid"):
        assert f(0.0) == 0.5 and not np.allclose(f(np.log(3.0)), 0.75)
    else:
        assert not math.isclose(float(f(0.0)), -math.log(2.0))
