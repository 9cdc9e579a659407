"""Pins of the oracle against facts that do not come from the oracle itself.

Each pin is checked on both oracle implementations of the recurrence (the C
one and the numpy twin); ``test_pins_catch_planted_mistakes`` shows that
every plausible slip in the recurrence (a dropped beta, the decay applied
after the correction, the output read before the update, a transposed state,
a flipped sign, decay on the wrong axis) fails at least one pin.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Implementations under test: one head, (q,k,v,g,beta,S0) -> (o, S_T).
# --------------------------------------------------------------------------

def impl_c(q, k, v, g, beta, S0=None):
    q, k, v, g = (np.asarray(a, dtype=np.float64)[:, None, :] for a in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)[:, None]
    s0 = None if S0 is None else np.asarray(S0, dtype=np.float64)[None, None]
    o, fin = oracle.kda_recurrent(q, k, v, g, beta, s0)
    return o[:, 0, :], fin[0, 0]


def impl_np(q, k, v, g, beta, S0=None):
    return oracle.kda_recurrent_np(q, k, v, g, beta, S0)


IMPLS = {"c": impl_c, "numpy": impl_np}


def _rand_head(rng, T, dk, dv, g_scale=0.3, s0=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, dk))) * g_scale
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


# --------------------------------------------------------------------------
# Pin checks.  Each returns normally on success and raises AssertionError on
# a mismatch, so the mutation test can count failures.
# --------------------------------------------------------------------------

def pin_two_channel_table(impl):
    """docsaid.org "Kimi Linear" notes, two-channel decay table (beta = 0)."""
    rows = np.loadtxt(os.path.join(GOLDEN, "p4_two_channel_decay.txt"))
    for s1, s2, a1, a2, e1, e2 in rows:
        S0 = np.array([[s1], [s2]])
        g = np.log(np.array([[a1, a2]]))
        # Any key, query and value: beta = 0 switches off correction and write.
        o, S = impl(np.array([[0.3, -0.2]]), np.array([[0.6, 0.8]]),
                    np.array([[1.7]]), g, np.array([0.0]), S0)
        np.testing.assert_allclose(S[:, 0], [e1, e2], rtol=1e-12, atol=1e-12)


def pin_single_token(impl):
    """One token from a zero state: o = beta (q.k) v, S = beta k v^T."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, _ = _rand_head(rng, 1, 5, 3)
    o, S = impl(q, k, v, g, beta, None)
    np.testing.assert_allclose(o[0], beta[0] * (q[0] @ k[0]) * v[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, beta[0] * np.outer(k[0], v[0]), rtol=1e-12, atol=1e-14)


def pin_beta_zero_no_decay(impl):
    """beta = 0 and g = 0: the state never changes and o_t = S0^T q_t."""
    rng = np.random.default_rng(12)
    q, k, v, _, _, S0 = _rand_head(rng, 6, 4, 3)
    o, S = impl(q, k, v, np.zeros((6, 4)), np.zeros(6), S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, q @ S0, rtol=1e-12, atol=1e-14)


def pin_beta_zero_pure_decay(impl):
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S0 and o_t = S0^T (q_t * exp(Gamma_t))."""
    rng = np.random.default_rng(13)
    q, k, v, g, _, S0 = _rand_head(rng, 7, 4, 3)
    o, S = impl(q, k, v, g, np.zeros(7), S0)
    Gam = np.cumsum(g, axis=0)
    np.testing.assert_allclose(S, np.exp(Gam[-1])[:, None] * S0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, (q * np.exp(Gam)) @ S0, rtol=1e-12, atol=1e-14)


def pin_reproduces_value(impl):
    """q_t = k_t, beta_t = 1, ||k_t|| = 1 exactly: the read-back equals v_t.

    The delta rule moves the memory so that S_t^T k_t = v_t (zeroshot.it.com
    deep-dive, section 2.2; greeksharifa summary, section 2.2).
    """
    rng = np.random.default_rng(14)
    T, dk, dv = 9, 4, 3
    k = 0.5 * rng.choice([-1.0, 1.0], size=(T, dk))          # norm exactly 1
    v = rng.standard_normal((T, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, dk))) * 0.5
    o, _ = impl(k, k, v, g, np.ones(T), rng.standard_normal((dk, dv)))
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def pin_one_hot_keys(impl):
    """Distinct one-hot keys from a zero state: no key ever reads an older write,
    so o_t = sum_{i<=t} beta_i (q_t . (k_i * exp(Gamma_t - Gamma_i))) v_i, i.e.
    linear attention (zeroshot.it.com section 2.1) with per-channel decay."""
    rng = np.random.default_rng(15)
    T, dk, dv = 5, 6, 3
    perm = rng.permutation(dk)[:T]
    k = np.eye(dk)[perm]
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, dk))) * 0.4
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    o, _ = impl(q, k, v, g, beta, None)
    Gam = np.cumsum(g, axis=0)
    exp_o = np.zeros((T, dv))
    for t in range(T):
        for i in range(t + 1):
            exp_o[t] += beta[i] * (q[t] @ (k[i] * np.exp(Gam[t] - Gam[i]))) * v[i]
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-13)


def pin_deltanet_gradient_step(impl):
    """alpha = 1: each step is one gradient-descent step of size beta_t on
    L_t(S) = 1/2 ||S^T k_t - v_t||^2 (zeroshot.it.com section 2.2).  The
    gradient is taken by automatic differentiation, not from a formula."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(16)
    T, dk, dv = 6, 4, 3
    q, k, v, _, beta, S0 = _rand_head(rng, T, dk, dv)
    o, S = impl(q, k, v, np.zeros((T, dk)), beta, S0)
    St = torch.tensor(S0, dtype=torch.float64)
    exp_o = []
    for t in range(T):
        Sv = St.clone().requires_grad_(True)
        loss = 0.5 * ((Sv.T @ torch.tensor(k[t]) - torch.tensor(v[t])) ** 2).sum()
        (grad,) = torch.autograd.grad(loss, Sv)
        St = (St - float(beta[t]) * grad).detach()
        exp_o.append((St.T @ torch.tensor(q[t])).numpy())
    np.testing.assert_allclose(o, np.array(exp_o), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, St.numpy(), rtol=1e-12, atol=1e-13)


def pin_scalar_gate_is_gdn(impl):
    """All channels sharing one gate gives Gated DeltaNet,
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
    (zeroshot.it.com section 2.3; docsaid.org notes, KDA section)."""
    rng = np.random.default_rng(17)
    T, dk, dv = 7, 4, 3
    q, k, v, _, beta, S0 = _rand_head(rng, T, dk, dv)
    a = np.exp(-np.logaddexp(0, rng.standard_normal(T)) * 0.5)
    o, S = impl(q, k, v, np.repeat(np.log(a)[:, None], dk, axis=1), beta, S0)
    St = S0.copy()
    exp_o = []
    for t in range(T):
        St = a[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ St + beta[t] * np.outer(k[t], v[t])
        exp_o.append(St.T @ q[t])
    np.testing.assert_allclose(o, np.array(exp_o), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, St, rtol=1e-12, atol=1e-13)


def pin_unrolled_fp64(impl):
    """Brute-force transition products vs the recurrence, random tiny cases."""
    rng = np.random.default_rng(18)
    for T, dk, dv in [(1, 2, 1), (3, 3, 2), (8, 4, 4), (6, 2, 3)]:
        q, k, v, g, beta, S0 = _rand_head(rng, T, dk, dv, g_scale=0.7)
        o, S = impl(q, k, v, g, beta, S0)
        eo, eS = oracle.kda_unrolled(q, k, v, np.exp(g), beta, S0)
        np.testing.assert_allclose(o, eo, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S, eS, rtol=1e-11, atol=1e-12)


def pin_unrolled_exact(impl):
    """Exact rational evaluation of the unrolled form vs the float64 recurrence.

    Inputs are dyadic rationals (exact in float64); alpha is one of a few
    dyadic values so the exact side needs no logarithm."""
    rng = np.random.default_rng(19)
    T, dk, dv = 5, 3, 2
    qi = rng.integers(-8, 9, (T, dk))
    ki = rng.integers(-8, 9, (T, dk))
    vi = rng.integers(-8, 9, (T, dv))
    si = rng.integers(-8, 9, (dk, dv))
    ai = rng.choice([4, 6, 7, 8], size=(T, dk))      # alpha = ai / 8
    bi = rng.integers(1, 9, T)                        # beta = bi / 8
    F = np.vectorize(lambda x, d: Fraction(int(x), d), otypes=[object])
    q, k, v, S0 = F(qi, 8), F(ki, 16), F(vi, 4), F(si, 4)
    alpha, beta = F(ai, 8), F(bi, 8)
    eo, eS = oracle.kda_unrolled(q, k, v, alpha, beta, S0)
    fl = lambda a: np.vectorize(float)(a)
    o, S = impl(fl(q), fl(k), fl(v), np.log(fl(alpha)), fl(beta), fl(S0))
    np.testing.assert_allclose(o, fl(eo), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, fl(eS), rtol=1e-12, atol=1e-12)


PINS = [pin_two_channel_table, pin_single_token, pin_beta_zero_no_decay,
        pin_beta_zero_pure_decay, pin_reproduces_value, pin_one_hot_keys,
        pin_deltanet_gradient_step, pin_scalar_gate_is_gdn, pin_unrolled_fp64,
        pin_unrolled_exact]


@pytest.mark.parametrize("impl", list(IMPLS), ids=list(IMPLS))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, impl):
    pin(IMPLS[impl])


# --------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# --------------------------------------------------------------------------

def _mutant(kind):
    def run(q, k, v, g, beta, S0=None):
        q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
        T, dk = q.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
        o = np.zeros((T, dv))
        for t in range(T):
            a = np.exp(g[t])
            if kind != "decay_after":
                S = a[:, None] * S if kind != "decay_cols" else S * a[None, :dv]
            b = 1.0 if kind == "no_beta" else beta[t]
            pred = S.T @ k[t]
            u = b * (v[t] + pred) if kind == "sign" else b * (v[t] - pred)
            if kind == "no_beta_write":
                u = v[t] - beta[t] * pred
            pre = S.T @ q[t]
            S = S + np.outer(k[t], u)
            if kind == "decay_after":
                S = a[:, None] * S
            if kind == "pre_update_read":
                o[t] = pre
            elif kind == "transposed_read":
                o[t] = (S @ q[t][:dv]) if dk == dv else S.T @ q[t] + 1e-3
            else:
                o[t] = S.T @ q[t]
        return o, S
    return run


MUTANTS = ["no_beta", "no_beta_write", "decay_after", "decay_cols", "sign",
           "pre_update_read", "transposed_read"]


def test_mutant_harness_is_faithful():
    # With no planted mistake the harness reproduces the oracle exactly.
    rng = np.random.default_rng(20)
    q, k, v, g, beta, S0 = _rand_head(rng, 5, 3, 3)
    o1, S1 = _mutant("none")(q, k, v, g, beta, S0)
    o2, S2 = impl_np(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-15)


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    mut = _mutant(kind)
    caught = []
    for pin in PINS + [pin_square_random_brute_force]:
        try:
            pin(mut)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {kind!r} passed every pin"


def pin_square_random_brute_force(impl):
    """Brute force with d_k = d_v (exposes transposed states)."""
    rng = np.random.default_rng(21)
    q, k, v, g, beta, S0 = _rand_head(rng, 5, 3, 3, g_scale=0.7)
    o, S = impl(q, k, v, g, beta, S0)
    eo, eS = oracle.kda_unrolled(q, k, v, np.exp(g), beta, S0)
    np.testing.assert_allclose(o, eo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, eS, rtol=1e-11, atol=1e-12)


def test_square_brute_force_on_oracles():
    for impl in IMPLS.values():
        pin_square_random_brute_force(impl)


# --------------------------------------------------------------------------
# Chunkwise algorithm: equal to the recurrence for every chunk size.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("C", [1, 2, 3, 5, 16, 37, 64])
def test_chunked_equals_recurrent(C):
    rng = np.random.default_rng(30 + C)
    q, k, v, g, beta, S0 = _rand_head(rng, 37, 8, 5, g_scale=0.3)
    o, S = oracle.kda_chunked(q, k, v, g, beta, C, S0)
    eo, eS = impl_c(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o, eo, rtol=0, atol=1e-12 * max(1, np.abs(eo).max()))
    np.testing.assert_allclose(S, eS, rtol=0, atol=1e-12 * max(1, np.abs(eS).max()))


def test_chunked_strong_decay():
    # g scaled x50: cumulative decays span e^-hundreds inside a chunk.
    rng = np.random.default_rng(40)
    q, k, v, g, beta, S0 = _rand_head(rng, 70, 8, 4, g_scale=5.0)
    o, S = oracle.kda_chunked(q, k, v, g, beta, 64, S0)
    eo, eS = impl_c(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o, eo, rtol=0, atol=1e-12 * max(1, np.abs(eo).max()))
    np.testing.assert_allclose(S, eS, rtol=0, atol=1e-12 * max(1, np.abs(eS).max()))


# --------------------------------------------------------------------------
# Boundary semantics of the C oracle: varlen packing, split/resume, linearity.
# --------------------------------------------------------------------------

def _multi(rng, T, H, dk, dv):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, H, dk))) * 0.1
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def test_c_matches_numpy_twin_multihead():
    rng = np.random.default_rng(50)
    q, k, v, g, beta = _multi(rng, 40, 3, 16, 20)
    s0 = rng.standard_normal((1, 3, 16, 20))
    o, fin = oracle.kda_recurrent(q, k, v, g, beta, s0)
    for h in range(3):
        eo, eS = impl_np(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], s0[0, h])
        np.testing.assert_allclose(o[:, h], eo, rtol=0, atol=1e-13)
        np.testing.assert_allclose(fin[0, h], eS, rtol=0, atol=1e-13)


def test_varlen_equals_per_sequence():
    rng = np.random.default_rng(51)
    lens = [7, 0, 13, 1, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _multi(rng, int(cu[-1]), 2, 8, 6)
    s0 = rng.standard_normal((len(lens), 2, 8, 6))
    o, fin = oracle.kda_recurrent(q, k, v, g, beta, s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        eo, ef = oracle.kda_recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0[n:n + 1])
        np.testing.assert_array_equal(o[a:b], eo)
        np.testing.assert_array_equal(fin[n], ef[0])
    # The empty sequence hands its initial state straight through.
    np.testing.assert_array_equal(fin[1], s0[1])


def test_split_resume():
    rng = np.random.default_rng(52)
    q, k, v, g, beta = _multi(rng, 50, 2, 8, 6)
    o, fin = oracle.kda_recurrent(q, k, v, g, beta)
    for t in (1, 17, 49):
        o1, f1 = oracle.kda_recurrent(q[:t], k[:t], v[:t], g[:t], beta[:t])
        o2, f2 = oracle.kda_recurrent(q[t:], k[t:], v[t:], g[t:], beta[t:], f1)
        np.testing.assert_array_equal(np.concatenate([o1, o2]), o)
        np.testing.assert_array_equal(f2, fin)


def test_linearity_in_values_and_state():
    # For fixed keys, gates and step sizes the map (V, S0) -> (O, S_T) is linear.
    rng = np.random.default_rng(53)
    q, k, v1, g, beta = _multi(rng, 30, 2, 8, 6)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, 2, 8, 6))
    s2 = rng.standard_normal((1, 2, 8, 6))
    a, b = 0.75, -1.5
    o1, f1 = oracle.kda_recurrent(q, k, v1, g, beta, s1)
    o2, f2 = oracle.kda_recurrent(q, k, v2, g, beta, s2)
    o3, f3 = oracle.kda_recurrent(q, k, a * v1 + b * v2, g, beta, a * s1 + b * s2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=0, atol=1e-12)


def test_decode_steps_equal_prefill():
    # Running single-token steps (a batch of sequences, one token each) equals
    # the prefill over the whole sequence.
    rng = np.random.default_rng(54)
    T, N, H, dk, dv = 12, 3, 2, 8, 6
    q, k, v, g, beta = _multi(rng, T * N, H, dk, dv)
    # token t of sequence n sits at row n*T + t
    cu = np.arange(N + 1) * T
    s0 = rng.standard_normal((N, H, dk, dv))
    o, fin = oracle.kda_recurrent(q, k, v, g, beta, s0, cu_seqlens=cu)
    state = s0.copy()
    for t in range(T):
        rows = np.arange(N) * T + t
        ot, state = oracle.kda_recurrent(q[rows], k[rows], v[rows], g[rows], beta[rows],
                                         state, cu_seqlens=np.arange(N + 1))
        np.testing.assert_array_equal(ot, o[rows])
    np.testing.assert_array_equal(state, fin)


def test_rejects_bad_cu_seqlens():
    rng = np.random.default_rng(55)
    q, k, v, g, beta = _multi(rng, 10, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.kda_recurrent(q, k, v, g, beta, cu_seqlens=np.array([0, 6, 4, 10]))
    with pytest.raises(ValueError):
        oracle.kda_recurrent(q, k, v, g, beta, cu_seqlens=np.array([0, 11]))
