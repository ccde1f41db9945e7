"""Input prologue of the path, in fp64 -- TEST INFRASTRUCTURE ONLY.

The step just before the recurrence: each token's query and key are
L2-normalised over d_k, beta is the logistic sigmoid of a pre-activation
b, and log alpha = -softplus(a) of a pre-activation a, so alpha is in (0,1).
The pages are silent on this step; the definitions follow the input recipe
of the workloads (q, k L2-normalised per token; beta = sigmoid(.); log alpha
= -softplus(.)).  The norm is clamped below at 1e-6 (its square at 1e-12),
so an all-zero row stays zero instead of dividing by zero.

Written as the definitions themselves, in numpy fp64; pinned in
``tests/test_oracle_pins.py`` against closed forms and torch's own
normalize / sigmoid / softplus.
"""
from __future__ import annotations

import numpy as np

NORM_SQ_FLOOR = 1e-12


def l2_normalize(x) -> np.ndarray:
    """x / sqrt(max(sum x^2, 1e-12)) over the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    ss = np.sum(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(np.maximum(ss, NORM_SQ_FLOOR))


def sigmoid(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-b))


def neg_softplus(a) -> np.ndarray:
    """-log(1 + e^a), evaluated as -(max(a, 0) + log1p(e^-|a|))."""
    a = np.asarray(a, dtype=np.float64)
    return -(np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))))


def apply(q, k, a, b, norm_qk: bool = True, gates: bool = True):
    """(q, k, log_alpha, beta) from raw (q, k, a, b), all fp64 arrays.
    With norm_qk False q, k pass through; with gates False a and b are taken
    as log alpha and beta already."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if norm_qk:
        q, k = l2_normalize(q), l2_normalize(k)
    if gates:
        return q, k, neg_softplus(a), sigmoid(b)
    return q, k, np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
