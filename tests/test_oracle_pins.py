"""The CPU oracle against closed forms and invariants (CPU only).

The token recurrence is pinned by the closed forms of ``oracle_pins``; the
chunkwise WY/UT form is pinned by the same closed forms and by agreement with
the token recurrence for every chunk size (the chunk form is an exact rewrite,
so the two agree to fp64 rounding)."""
import functools

import numpy as np
import pytest

import oracle
from oracle import chunk_form
from tests import oracle_pins as pins


def c_oracle(q, k, v, la, be, S0=None, cu=None):
    return oracle.fwd(q, k, v, la, be, S0, cu)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_token_oracle_pins(pin):
    pin(c_oracle)


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 16, 64])
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_chunk_form_pins(pin, chunk):
    def fwd(q, k, v, la, be, S0=None, cu=None):
        return chunk_form.fwd(q, k, v, la, be, S0, cu, chunk=chunk)
    pin(fwd)


@pytest.mark.parametrize("chunk", [1, 3, 8, 16, 64, 100])
def test_chunk_form_equals_recurrence(chunk):
    """Chunk-size invariance: ragged last chunks (T=100 is not a multiple of
    3, 8, 16 or 64) and a chunk longer than the sequence."""
    q, k, v, la, be, S0 = pins.rand_case(20, B=2, T=100, H=2, dk=16, dv=12)
    o1, s1 = oracle.fwd(q, k, v, la, be, S0)
    o2, s2 = chunk_form.fwd(q, k, v, la, be, S0, chunk=chunk)
    pins._close(o2, o1, 1e-10, "chunk form o")
    pins._close(s2, s1, 1e-10, "chunk form S_T")


def test_chunk_form_strong_decay():
    """Decays that underflow exp(g) inside a chunk (log alpha ~ -4 per token,
    g reaches ~ -250 over 64 tokens) stay finite and exact."""
    q, k, v, la, be, S0 = pins.rand_case(21, B=1, T=130, H=1, dk=8, dv=8)
    la = la * 0 - 4.0
    o1, s1 = oracle.fwd(q, k, v, la, be, S0)
    o2, s2 = chunk_form.fwd(q, k, v, la, be, S0, chunk=64)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(s2))
    pins._close(o2, o1, 1e-10, "strong decay o")
    pins._close(s2, s1, 1e-10, "strong decay S_T")


def test_ut_inverse_is_textbook_inverse():
    """The forward-substitution inverse equals numpy.linalg.inv(I + A)."""
    rng = np.random.default_rng(22)
    n = 64
    A = np.tril(rng.standard_normal((n, n)) * 0.1, -1)
    T = chunk_form.unit_lower_inverse(np.eye(n) + A)
    pins._close(T, np.linalg.inv(np.eye(n) + A), 1e-12, "UT inverse")
    assert np.allclose(np.triu(T, 1), 0.0) and np.allclose(np.diag(T), 1.0)


def test_chunk_intermediates_and_affine_maps():
    """Per-chunk intermediates: (I+A) T = I, A strictly lower; W and U solve
    the triangular systems; the chunk maps S' = S M + R compose to the
    explicit product form of the recurrence."""
    rng = np.random.default_rng(23)
    L, dk, dv, C = 21, 5, 4, 8
    K = rng.standard_normal((L, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((L, dk))
    V = rng.standard_normal((L, dv))
    la = -rng.uniform(0.0, 1.0, L)
    be = rng.uniform(0.0, 1.0, L)
    S0 = rng.standard_normal((dv, dk))
    _, S_end, parts = chunk_form.unit_fwd(Q, K, V, la, be, S0, C, want_parts=True)
    Mtot, Rtot = np.eye(dk), np.zeros((dv, dk))
    for n, p in enumerate(parts):
        s, e = n * C, min(n * C + C, L)
        m = e - s
        assert np.allclose(np.triu(p["A"]), 0.0)
        pins._close((np.eye(m) + p["A"]) @ p["T"], np.eye(m), 1e-12, "T inverse")
        g = np.cumsum(la[s:e])
        pins._close((np.eye(m) + p["A"]) @ p["U"], be[s:e, None] * V[s:e],
                    1e-12, "U solve")
        pins._close((np.eye(m) + p["A"]) @ p["W"],
                    (be[s:e] * np.exp(g))[:, None] * K[s:e], 1e-12, "W solve")
        Mtot, Rtot = Mtot @ p["M"], Rtot @ p["M"] + p["R"]
    ref = pins.product_form_states(K, V, la, be, S0)[-1]
    pins._close(S0 @ Mtot + Rtot, ref, 1e-11, "composed affine maps")
    pins._close(S_end, ref, 1e-11, "chunk S_T vs product form")


def test_step_equals_forward():
    """T consecutive decode steps equal one forward over T tokens."""
    q, k, v, la, be, S0 = pins.rand_case(24, B=3, T=6, H=2, dk=5, dv=7)
    o_ref, s_ref = oracle.fwd(q, k, v, la, be, S0)
    S = S0
    for t in range(q.shape[1]):
        o_t, S = oracle.step(q[:, t], k[:, t], v[:, t], la[:, t], be[:, t], S)
        pins._close(o_t, o_ref[:, t], 1e-12, f"step {t} o")
    pins._close(S, s_ref, 1e-12, "steps S_T")


def test_oracle_threads_agree():
    """The OpenMP unit loop gives identical results at 1 and 4 threads."""
    q, k, v, la, be, S0 = pins.rand_case(25, B=4, T=33, H=3, dk=8, dv=8)
    o1, s1 = oracle.fwd(q, k, v, la, be, S0, threads=1)
    o4, s4 = oracle.fwd(q, k, v, la, be, S0, threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


def test_oracle_rejects_bad_cu_seqlens():
    q, k, v, la, be, _ = pins.rand_case(26, B=1, T=5, H=1)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, la, be, None, np.array([0, 3, 9], dtype=np.int32))
