"""Pins of the oracle's general DPLR recurrence (oracle.dplr_recurrent):

    S_t = (Diag(exp g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t

(zeroshot.it.com deep-dive, section 3.2 "DPLR Structure").  Checked against
exact rational arithmetic through explicit transition matrices, the KDA
special case (a = beta k, b = alpha * k, write beta k v^T: the pinned KDA
oracle), the gated-linear-attention closed form (a = 0), a hand-derived
two-token case, and packing; planted mistakes fail at least one pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _exact_pin(dplr):
    rng = np.random.default_rng(1)
    T, dk, dv = 5, 3, 2
    ints = lambda *s: rng.integers(-3, 4, s)
    q, k, a, b = (ints(T, dk) for _ in range(4))
    v = ints(T, dv)
    alpha = rng.integers(1, 5, (T, dk)) / 4.0         # exact in binary floating point
    S0 = ints(dk, dv)
    fr = lambda x: np.vectorize(lambda z: Fraction(z))(np.asarray(x, dtype=object))
    o_ex, S_ex = oracle.dplr_explicit(fr(q), fr(k), fr(v), fr(a), fr(b), fr(alpha), fr(S0))
    o, f = dplr(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None],
                np.log(alpha)[:, None], S0[None, None], None)
    np.testing.assert_allclose(o[:, 0], o_ex.astype(float), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f[0, 0], S_ex.astype(float), rtol=1e-12, atol=1e-12)


def _kda_pin(dplr):
    rng = np.random.default_rng(2)
    T, H, dk, dv = 17, 2, 5, 4
    q, k = (rng.standard_normal((T, H, dk)) for _ in range(2))
    v = rng.standard_normal((T, H, dv))
    g = -0.3 * rng.random((T, H, dk))
    beta = rng.random((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    bk = beta[:, :, None] * k
    o, f = dplr(q, bk, v, bk, np.exp(g) * k, g, S0, None)
    eo, ef = oracle.kda_recurrent(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o, eo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f, ef, rtol=1e-12, atol=1e-12)


def _gla_pin(dplr):
    # a = 0: S_t = Diag(gam_t) S0 + sum_{i<=t} Diag(gam_t / gam_i) k_i v_i^T
    rng = np.random.default_rng(3)
    T, dk, dv = 7, 3, 2
    q, k, b = (rng.standard_normal((T, 1, dk)) for _ in range(3))
    v = rng.standard_normal((T, 1, dv))
    g = -0.4 * rng.random((T, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, _ = dplr(q, k, v, np.zeros_like(k), b, g, S0, None)
    G = np.cumsum(g[:, 0], axis=0)
    for t in range(T):
        S = np.exp(G[t])[:, None] * S0[0, 0]
        for i in range(t + 1):
            S = S + np.exp(G[t] - G[i])[:, None] * np.outer(k[i, 0], v[i, 0])
        np.testing.assert_allclose(o[t, 0], S.T @ q[t, 0], rtol=1e-12, atol=1e-12)


def _two_token_pin(dplr):
    # g = 0, zero state: S_1 = k_1 v_1^T, S_2 = (I - a_2 b_2^T) S_1 + k_2 v_2^T, so
    # o_2 = v_1 ((k_1 . q_2) - (a_2 . q_2)(b_2 . k_1)) + v_2 (k_2 . q_2).
    rng = np.random.default_rng(4)
    q, k, a, b = (rng.standard_normal((2, 1, 3)) for _ in range(4))
    v = rng.standard_normal((2, 1, 2))
    o, _ = dplr(q, k, v, a, b, np.zeros((2, 1, 3)), None, None)
    k1, q2, a2, b2, k2 = k[0, 0], q[1, 0], a[1, 0], b[1, 0], k[1, 0]
    want = v[0, 0] * (k1 @ q2 - (a2 @ q2) * (b2 @ k1)) + v[1, 0] * (k2 @ q2)
    np.testing.assert_allclose(o[1, 0], want, rtol=1e-13)
    np.testing.assert_allclose(o[0, 0], v[0, 0] * (k[0, 0] @ q[0, 0]), rtol=1e-13)


def _packing_pin(dplr):
    rng = np.random.default_rng(5)
    lens = [3, 0, 6, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 3, 2
    q, k, a, b = (rng.standard_normal((T, H, dk)) for _ in range(4))
    v = rng.standard_normal((T, H, dv))
    g = -0.2 * rng.random((T, H, dk))
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, f = dplr(q, k, v, a, b, g, S0, cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, fn = dplr(q[sl], k[sl], v[sl], a[sl], b[sl], g[sl], S0[n:n + 1], None)
        np.testing.assert_allclose(o[sl], on, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(f[n], fn[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(f[1], S0[1])


PINS = [_exact_pin, _kda_pin, _gla_pin, _two_token_pin, _packing_pin]


def run_pins(dplr):
    for pin in PINS:
        pin(dplr)


def test_dplr_pins():
    run_pins(lambda q, k, v, a, b, g, S0, cu: oracle.dplr_recurrent(q, k, v, a, b, g, S0, cu))


def _copy(mut):
    def dplr(q, k, v, a, b, g, S0, cu):
        q, k, v, a, b, g = (np.asarray(x, float) for x in (q, k, v, a, b, g))
        T, H, dk = q.shape
        dv = v.shape[2]
        cu = np.array([0, T]) if cu is None else np.asarray(cu)
        N = len(cu) - 1
        S0 = np.zeros((N, H, dk, dv)) if S0 is None else np.asarray(S0, float)
        o = np.zeros((T, H, dv))
        fin = np.zeros((N, H, dk, dv))
        for n in range(N):
            for h in range(H):
                S = S0[n, h].copy()
                for t in range(int(cu[n]), int(cu[n + 1])):
                    al = np.exp(g[t, h])
                    if mut == "b_after_decay":
                        low = np.outer(a[t, h], b[t, h] @ (al[:, None] * S))
                    elif mut == "outer_transposed":
                        low = np.outer(b[t, h], a[t, h] @ S)
                    else:
                        low = np.outer(a[t, h], b[t, h] @ S)
                    sign = 1.0 if mut == "low_rank_sign" else -1.0
                    Sn = al[:, None] * S + sign * low + np.outer(k[t, h], v[t, h])
                    o[t, h] = (S if mut == "read_before_update" else Sn).T @ q[t, h]
                    S = Sn
                fin[n, h] = S
        return o, fin
    return dplr


MUTANTS = ["b_after_decay", "outer_transposed", "low_rank_sign", "read_before_update"]


def test_dplr_copy_is_faithful():
    run_pins(_copy(None))


@pytest.mark.parametrize("kind", MUTANTS)
def test_dplr_pins_catch_planted_mistakes(kind):
    with pytest.raises(AssertionError):
        run_pins(_copy(kind))
