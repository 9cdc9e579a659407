"""Pins of the oracle's backward pass (oracle.kda_backward).

The gradients of L = <dO, o> + <dS_N, S_N> are checked against
  * central finite differences of the forward oracle (every input element of
    a tiny packed problem with an initial state),
  * torch.autograd (float64, CPU) through the token recurrence,
  * closed forms: one token from a zero state, and beta = 0 (pure decay),
and planted mistakes in a copy of the backward each fail at least one pin.
"""
import numpy as np
import pytest

import oracle


def _problem(seed, lens=(4, 0, 3), H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N = int(cu[-1]), len(lens)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = -0.3 * np.abs(rng.standard_normal((T, H, dk)))
    b = rng.random((T, H))
    do = rng.standard_normal((T, H, dv))
    dF = rng.standard_normal((N, H, dk, dv))
    S0 = rng.standard_normal((N, H, dk, dv))
    return (q, k, v, g, b, S0), do, dF, cu


def _fd_pin(bwd):
    (q, k, v, g, b, S0), do, dF, cu = _problem(1)
    grads = bwd(q, k, v, g, b, do, dF, S0, cu)

    def loss(q, k, v, g, b, S0):
        o, f = oracle.kda_recurrent(q, k, v, g, b, S0, cu)
        return float((o * do).sum() + (f * dF).sum())

    base = [q, k, v, g, b, S0]
    eps = 1e-6
    for ai, a in enumerate(base):
        for idx in np.ndindex(a.shape):
            ap = [x.copy() for x in base]
            am = [x.copy() for x in base]
            ap[ai][idx] += eps
            am[ai][idx] -= eps
            fd = (loss(*ap) - loss(*am)) / (2 * eps)
            assert abs(fd - grads[ai][idx]) <= 1e-7 * (1 + abs(fd)), (ai, idx, fd, grads[ai][idx])


def _single_token_pin(bwd):
    # One token from a zero state: o = beta (q . k) v, so
    # dq = beta (do . v) k, dk = beta (do . v) q, dv = beta (q . k) do,
    # dbeta = (q . k)(do . v), dg = 0 (the decay acts on a zero state).
    rng = np.random.default_rng(2)
    q, k, g = (rng.standard_normal((1, 1, 4)) for _ in range(3))
    v = rng.standard_normal((1, 1, 3))
    b = np.array([[0.7]])
    do = rng.standard_normal((1, 1, 3))
    dq, dk, dv, dg, db, dS0 = bwd(q, k, v, g, b, do, None, None, None)
    qk, dov = float(q[0, 0] @ k[0, 0]), float(do[0, 0] @ v[0, 0])
    np.testing.assert_allclose(dq[0, 0], 0.7 * dov * k[0, 0], rtol=1e-13)
    np.testing.assert_allclose(dk[0, 0], 0.7 * dov * q[0, 0], rtol=1e-13)
    np.testing.assert_allclose(dv[0, 0], 0.7 * qk * do[0, 0], rtol=1e-13)
    np.testing.assert_allclose(db[0, 0], qk * dov, rtol=1e-13)
    np.testing.assert_array_equal(dg, 0.0)


def _pure_decay_pin(bwd):
    # beta = 0: S_t = Diag(a_t ... a_1) S0 and o_t = S_t^T q_t, so
    # dS0 = sum_t Diag(prod_{s<=t} a_s) q_t do_t^T and dk = dv = 0.
    rng = np.random.default_rng(3)
    T, dk, dv = 5, 3, 2
    q, k = (rng.standard_normal((T, 1, dk)) for _ in range(2))
    v = rng.standard_normal((T, 1, dv))
    g = -0.2 * np.abs(rng.standard_normal((T, 1, dk)))
    b = np.zeros((T, 1))
    do = rng.standard_normal((T, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    dq, dkk, dvv, dg, db, dS0 = bwd(q, k, v, g, b, do, None, S0, None)
    cum = np.exp(np.cumsum(g[:, 0], axis=0))                      # [T, dk]
    want = sum(cum[t][:, None] * np.outer(q[t, 0], do[t, 0]) for t in range(T))
    np.testing.assert_allclose(dS0[0, 0], want, rtol=1e-12)
    np.testing.assert_array_equal(dkk, 0.0)
    np.testing.assert_array_equal(dvv, 0.0)
    for t in range(T):  # dq_t = S_t do_t
        np.testing.assert_allclose(dq[t, 0], (cum[t][:, None] * S0[0, 0]) @ do[t, 0], rtol=1e-12)


def _autograd_pin(bwd):
    torch = pytest.importorskip("torch")
    (q, k, v, g, b, S0), do, dF, cu = _problem(4, lens=(9, 6), H=2, dk=5, dv=4)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, g, b, S0)]
    tq, tk, tv, tg, tb, tS0 = ts
    loss = 0.0
    for n in range(len(cu) - 1):
        S = tS0[n]
        for t in range(int(cu[n]), int(cu[n + 1])):
            Sp = torch.exp(tg[t])[:, :, None] * S
            r = torch.einsum("hij,hi->hj", Sp, tk[t])
            u = tb[t][:, None] * (tv[t] - r)
            S = Sp + tk[t][:, :, None] * u[:, None, :]
            loss = loss + (torch.einsum("hij,hi->hj", S, tq[t]) * torch.from_numpy(do[t])).sum()
        loss = loss + (S * torch.from_numpy(dF[n])).sum()
    loss.backward()
    grads = bwd(q, k, v, g, b, do, dF, S0, cu)
    for mine, t in zip(grads, ts):
        np.testing.assert_allclose(mine, t.grad.numpy(), rtol=1e-11, atol=1e-12)


PINS = [_single_token_pin, _pure_decay_pin, _fd_pin, _autograd_pin]


def run_pins(bwd):
    for pin in PINS:
        pin(bwd)


def _oracle(q, k, v, g, b, do, dF, S0, cu):
    return oracle.kda_backward(q, k, v, g, b, do, dF, S0, cu, block=2)


def test_backward_pins():
    run_pins(_oracle)


def test_backward_checkpoint_block_is_immaterial():
    (q, k, v, g, b, S0), do, dF, cu = _problem(5, lens=(11, 5))
    a = oracle.kda_backward(q, k, v, g, b, do, dF, S0, cu, block=1)
    c = oracle.kda_backward(q, k, v, g, b, do, dF, S0, cu, block=64)
    for x, y in zip(a, c):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# Planted mistakes in a copy of the backward (one token per step, one head).
# ---------------------------------------------------------------------------

def _bwd_copy(mut):
    def bwd(q, k, v, g, b, do, dF, S0, cu):
        q, k, v, g, b, do = (np.asarray(a, float) for a in (q, k, v, g, b, do))
        T, H, dk = q.shape
        dvv = v.shape[2]
        cu = np.array([0, T]) if cu is None else np.asarray(cu)
        N = len(cu) - 1
        S0 = np.zeros((N, H, dk, dvv)) if S0 is None else np.asarray(S0, float)
        dF = np.zeros((N, H, dk, dvv)) if dF is None else np.asarray(dF, float)
        out = [np.zeros_like(a) for a in (q, k, v, g, b)] + [np.zeros((N, H, dk, dvv))]
        for n in range(N):
            for h in range(H):
                bos, eos = int(cu[n]), int(cu[n + 1])
                Ss = [S0[n, h]]
                for t in range(bos, eos):
                    a = np.exp(g[t, h])
                    Sp = a[:, None] * Ss[-1]
                    u = b[t, h] * (v[t, h] - Sp.T @ k[t, h])
                    Ss.append(Sp + np.outer(k[t, h], u))
                dS = dF[n, h].copy()
                for t in range(eos - 1, bos - 1, -1):
                    S, Sn = Ss[t - bos], Ss[t - bos + 1]
                    a = np.exp(g[t, h])
                    Sp = a[:, None] * S
                    r = Sp.T @ k[t, h]
                    u = b[t, h] * (v[t, h] - r)
                    dS = dS + np.outer(q[t, h], do[t, h])
                    out[0][t, h] = (S if mut == "dq_from_old_state" else Sn) @ do[t, h]
                    du = dS.T @ k[t, h]
                    dkt = dS @ u
                    out[4][t, h] = du @ (v[t, h] - r) if mut != "dbeta_without_r" else du @ v[t, h]
                    out[2][t, h] = b[t, h] * du
                    dr = (1 if mut == "dr_sign" else -1) * b[t, h] * du
                    dSp = dS + np.outer(k[t, h], dr)
                    if mut != "drop_dk_through_r":
                        dkt += Sp @ dr
                    out[1][t, h] = dkt
                    Sd = Sn if mut == "dg_from_new_state" else S
                    out[3][t, h] = a * (dSp * Sd).sum(1)
                    dS = dSp if mut == "carry_without_decay" else a[:, None] * dSp
                out[5][n, h] = dS
        return tuple(out)
    return bwd


MUTANTS = ["dq_from_old_state", "dbeta_without_r", "dr_sign", "drop_dk_through_r",
           "dg_from_new_state", "carry_without_decay"]


def test_backward_copy_is_faithful():
    run_pins(_bwd_copy(None))


@pytest.mark.parametrize("kind", MUTANTS)
def test_backward_pins_catch_planted_mistakes(kind):
    with pytest.raises(AssertionError):
        run_pins(_bwd_copy(kind))
