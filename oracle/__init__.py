"""KDA oracle: plain, slow, float64 CPU evaluations of what KDA computes.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import or call anything here; the HIP
library never does, and this package never imports the HIP library.

Functions
---------
``kda_recurrent``      the definition, token by token, in C (float64).
``kda_recurrent_np``   the same definition as a numpy loop (tiny inputs).
``kda_unrolled``       the unrolled transition-product form, brute force;
                       works on float64 or on exact ``fractions.Fraction``.
``kda_chunked``        the chunkwise WY / UT-transform algorithm in float64.
``layer_prologue``     the per-head input transforms of a KDA layer: Swish and
                       L2 normalisation of q and k, Swish of v, sigmoid of beta.
``layer_epilogue``     head-wise RMSNorm of o times a sigmoid output gate.
``kda_layer``          prologue, recurrence, epilogue.
``short_conv``         causal depthwise convolution over the tokens of each
                       sequence, with a carried state of the last inputs.
``kda_layer_conv``     short convolution of q, k, v, then ``kda_layer``.
``dplr_recurrent``     the general diagonal-plus-low-rank recurrence
                       S_t = (Diag(exp g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T.
``dplr_explicit``      the same by explicit d_k x d_k transition matrices.
``kda_backward``       gradients of <dO, o> + <dS_N, S_N> with respect to q, k,
                       v, g, beta and the initial state: reverse-mode through
                       the token recurrence, written out by hand (float64).

Sources (pages this package follows):
  * Recurrence: "Kimi Linear" notes (docsaid.org), section "KDA: Splitting
    the Decay Across Channels"; greeksharifa.github.io summary, section 3
    "Kimi Delta Attention" (decay applied before the delta-rule correction,
    output o_t = S_t^T q_t).
  * Unrolled form: zeroshot.it.com deep-dive, section 3.3 "The Learned
    Position" (printed without beta_i and without the initial-state term;
    the complete form used here is derived from the recurrence).
  * Chunkwise algorithm: greeksharifa.github.io summary, section 3.1
    "Hardware-Efficient Chunkwise Algorithm" and Appendix B/C notes (WY
    representation, UT transform by forward substitution, output = state
    term + causally masked intra-chunk term).
  * Layer prologue and epilogue: "Kimi Linear" notes (docsaid.org), section
    "Other Components" (q, k: Swish then L2 normalisation; v: Swish; beta:
    sigmoid; output: per-head RMSNorm, then a data-dependent sigmoid gate);
    greeksharifa.github.io summary, section 4 (head-wise RMSNorm followed by
    a sigmoid gate; queries and keys normalised to unit length).
  * Short convolution: same docsaid.org section (q, k and v each pass through
    a short convolution after their projection, before Swish); the
    deepstudy.best introduction (short convolutions capture local token
    dependencies).  The pages give neither the width nor the padding; the
    reading taken is a causal, depthwise (per channel) convolution of width
    W <= 4 with no bias, restarted at every sequence start from a carried
    state (zeros when none is given).

  * General DPLR: zeroshot.it.com deep-dive, section 3.2 "DPLR Structure"
    (the update (D_t - a_t b_t^T) S_{t-1} + k_t v_t^T, with KDA the case
    a_t = beta_t k_t, b_t = k_t * alpha_t); greeksharifa.github.io summary,
    section 6.2 "Relation to DPLR".
  * Backward pass: the pages only say the chunkwise form also serves training
    (greeksharifa.github.io summary, sections 3.1 and 6.3; zeroshot.it.com
    deep-dive, section 4); the gradients here are the chain rule applied to
    the recurrence above, step by step in reverse token order.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, special cases, the two-channel decay table printed on the
docsaid.org page, exact rational arithmetic, and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (float64, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                           ctypes.POINTER(ctypes.c_int64),
                                           ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    return _load().kda_oracle_threads()


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def kda_recurrent(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                  nthreads: int = 0):
    """Token-by-token KDA in float64 (C).

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H] (any float dtype; the
    values are upcast exactly to float64).  ``cu_seqlens`` [N+1] packs N
    sequences; None means one sequence of length T.  ``initial_state``
    [N, H, dk, dv] or None (zeros).  Returns (o [T, H, dv], final [N, H, dk, dv]),
    both float64.
    """
    q, k, v, g, beta = (np.ascontiguousarray(a, dtype=np.float64)
                        for a in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    if cu[-1] > T:
        raise ValueError("cu_seqlens exceeds the token count")
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        if s0.shape != (N, H, dk, dv):
            raise ValueError(f"initial_state shape {s0.shape} != {(N, H, dk, dv)}")
    o = np.zeros((T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_prefill(
        _dptr(q), _dptr(k), _dptr(v), _dptr(g), _dptr(beta), _dptr(s0),
        _dptr(fin), _dptr(o), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill rejected its arguments")
    return o, fin


def kda_recurrent_np(q, k, v, g, beta, S0=None):
    """The same definition as ``kda_recurrent`` for ONE head, numpy loop.

    q, k, g: [T, dk]; v: [T, dv]; beta: [T]; S0: [dk, dv] or None.
    Returns (o [T, dv], S_T [dk, dv]).
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S = np.exp(g[t])[:, None] * S              # Diag(alpha_t) S
        u = beta[t] * (v[t] - S.T @ k[t])          # pseudo-value
        S = S + np.outer(k[t], u)                  # delta correction + write
        o[t] = S.T @ q[t]                          # read after the update
    return o, S


def kda_unrolled(q, k, v, alpha, beta, S0):
    """Brute-force unrolled KDA for ONE head (tiny inputs).

    With transition A_j = (I - beta_j k_j k_j^T) Diag(alpha_j) and
    Phi(t, i) = A_t A_{t-1} ... A_{i+1} (Phi(t, t) = I):

        o_t = (Phi(t, 0) S0)^T q_t + sum_{i<=t} beta_i (q_t^T Phi(t, i) k_i) v_i
        S_T = Phi(T, 0) S0 + sum_i beta_i Phi(T, i) k_i v_i^T

    Every Phi is formed as an explicit d_k x d_k matrix product, so this
    evaluates the position-dependent transition products directly rather
    than the recurrence.  Inputs may be float64 arrays or object arrays of
    ``fractions.Fraction`` (then the result is exact).  ``alpha`` is given
    directly ([T, dk]), not as a log-decay.
    """
    q, k, v, alpha = (np.asarray(a) for a in (q, k, v, alpha))
    beta = np.asarray(beta)
    S0 = np.asarray(S0)
    T, dk = q.shape
    dv = v.shape[1]
    exact = q.dtype == object
    one = Fraction(1) if exact else 1.0
    zero = Fraction(0) if exact else 0.0

    def eye():
        m = np.empty((dk, dk), dtype=object if exact else np.float64)
        for a in range(dk):
            for b in range(dk):
                m[a, b] = one if a == b else zero
        return m

    A = []
    for j in range(T):
        kk = np.outer(k[j], k[j])
        A.append((eye() - beta[j] * kk) @ np.diag(alpha[j]).astype(kk.dtype))

    def phi(t, i):  # A_t ... A_{i+1}, 1-based t, i
        m = eye()
        for j in range(i + 1, t + 1):
            m = A[j - 1] @ m
        return m

    o = np.empty((T, dv), dtype=object if exact else np.float64)
    for t in range(1, T + 1):
        acc = (phi(t, 0) @ S0).T @ q[t - 1]
        for i in range(1, t + 1):
            coef = beta[i - 1] * (q[t - 1] @ (phi(t, i) @ k[i - 1]))
            acc = acc + coef * v[i - 1]
        o[t - 1] = acc
    S = phi(T, 0) @ S0
    for i in range(1, T + 1):
        S = S + beta[i - 1] * np.outer(phi(T, i) @ k[i - 1], v[i - 1])
    return o, S


def _forward_substitution_inverse(L: np.ndarray) -> np.ndarray:
    """Inverse of a unit lower-triangular matrix, solved row by row."""
    n = L.shape[0]
    X = np.zeros_like(L)
    for r in range(n):
        X[r, r] = 1.0
        for i in range(r):
            # row r of L X = e_r  =>  X[r] = e_r - sum_{m<r} L[r, m] X[m]
            X[r] -= L[r, i] * X[i]
    return X


def kda_chunked(q, k, v, g, beta, C: int, S0=None):
    """Chunkwise KDA for ONE head in float64: WY representation + UT transform.

    Per chunk of n <= C rows (the last one may be shorter), entering state S:
      Gamma_r = sum_{s<=r} g_s (inclusive, per key channel);  gam_r = exp(Gamma_r)
      A[r, i] = beta_r * sum_c k_rc k_ic exp(Gamma_rc - Gamma_ic)   for i < r
      P[r, i] =          sum_c q_rc k_ic exp(Gamma_rc - Gamma_ic)   for i <= r
      T       = (I + A)^{-1} Diag(beta)      (forward substitution)
      W       = T (K * gam),  U0 = T V        (WY auxiliaries)
      U       = U0 - W S                      (delta-rule pseudo-values)
      O       = (Q * gam) S + P U             (state term + masked intra term)
      S_next  = Diag(gam_n) S + (K * exp(Gamma_n - Gamma))^T U
    The decay ratios are evaluated pairwise as exp of a difference, so no
    reciprocal of a cumulative decay is ever formed.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V, G, B = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C], g[c0:c0 + C], beta[c0:c0 + C]
        n = Q.shape[0]
        Gam = np.cumsum(G, axis=0)                       # [n, dk]
        E = np.exp(Gam[:, None, :] - Gam[None, :, :])    # E[r, i, c], used for i <= r
        KK = np.einsum("rc,ic,ric->ri", K, K, E)
        QK = np.einsum("rc,ic,ric->ri", Q, K, E)
        A = np.tril(B[:, None] * KK, -1)
        P = np.tril(QK, 0)
        Tm = _forward_substitution_inverse(np.eye(n) + A) * B[None, :]
        gam = np.exp(Gam)
        W = Tm @ (K * gam)
        U = Tm @ V - W @ S
        o[c0:c0 + n] = (Q * gam) @ S + P @ U
        Kbar = K * np.exp(Gam[-1][None, :] - Gam)
        S = gam[-1][:, None] * S + Kbar.T @ U
    return o, S


# ---------------------------------------------------------------------------
# Layer prologue / epilogue (docsaid.org notes, "Other Components")
# ---------------------------------------------------------------------------

L2_FLOOR = 1e-12  # norms below this are treated as this (zero vectors stay 0)


def swish(x):
    """Swish (SiLU): x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def l2_normalize(x, axis=-1):
    """x / ||x|| over ``axis`` (unit length), with the norm floored at
    L2_FLOOR."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt((x * x).sum(axis=axis, keepdims=True))
    return x / np.maximum(n, L2_FLOOR)


def layer_prologue(q_pre, k_pre, v_pre, beta_pre):
    """q = l2(swish(q_pre)), k = l2(swish(k_pre)) over d_k; v = swish(v_pre);
    beta = sigmoid(beta_pre).  Arrays are [T, H, D] / [T, H]."""
    return (l2_normalize(swish(q_pre)), l2_normalize(swish(k_pre)), swish(v_pre),
            sigmoid(beta_pre))


def layer_epilogue(o, gate, weight, eps):
    """Head-wise RMSNorm with a per-channel weight, times sigmoid(gate):
    y[t, h, c] = o[t, h, c] / sqrt(mean_c' o[t, h, c']^2 + eps) * weight[c]
                 * sigmoid(gate[t, h, c])."""
    o = np.asarray(o, dtype=np.float64)
    rms = np.sqrt((o * o).mean(axis=-1, keepdims=True) + eps)
    return o / rms * np.asarray(weight, dtype=np.float64) * sigmoid(gate)


def kda_layer(q_pre, k_pre, v_pre, g, beta_pre, gate=None, weight=None, eps=1e-6,
              initial_state=None, cu_seqlens=None):
    """Prologue, token-by-token recurrence (kda_recurrent), then the
    epilogue when ``gate`` is given.  Returns (y, final_state)."""
    q, k, v, beta = layer_prologue(q_pre, k_pre, v_pre, beta_pre)
    o, fin = kda_recurrent(q, k, v, g, beta, initial_state, cu_seqlens)
    if gate is not None:
        o = layer_epilogue(o, gate, weight, eps)
    return o, fin


def short_conv(x, weight, state=None, cu_seqlens=None):
    """Causal depthwise convolution over tokens, per sequence.

    x ``[T, H, D]``; weight ``[H, D, W]``; state ``[N, H, W-1, D]`` or None.
    For token t of sequence n (tokens bos..eos-1):
        y[t, h, c] = sum_{i=0}^{W-1} weight[h, c, i] * x(t - (W-1) + i)[h, c]
    where x(s) for s < bos is state[n, h, (W-1) + (s - bos)] (zero without a
    state): weight[..., W-1] multiplies the current token.  Returns y
    ``[T, H, D]`` and the final state, the last W-1 inputs of each sequence
    (state rows where the sequence is shorter than W-1), float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    T, H, D = x.shape
    W = w.shape[-1]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    st = (np.zeros((N, H, W - 1, D)) if state is None
          else np.asarray(state, dtype=np.float64).reshape(N, H, W - 1, D))
    y = np.zeros_like(x)
    fin = np.zeros((N, H, W - 1, D))
    for n in range(N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        # the sequence's inputs preceded by its state rows: position p of
        # ext holds x(bos - (W-1) + p)
        ext = np.concatenate([st[n].transpose(1, 0, 2), x[bos:eos]], axis=0)  # [W-1+len, H, D]
        for t in range(eos - bos):
            for i in range(W):
                y[bos + t] += w[:, :, i] * ext[t + i]
        fin[n] = ext[len(ext) - (W - 1):].transpose(1, 0, 2) if W > 1 else fin[n]
    return y, fin


def kda_layer_conv(q_pre, k_pre, v_pre, g, beta_pre, conv_weight, conv_state=None, gate=None,
                   weight=None, eps=1e-6, initial_state=None, cu_seqlens=None):
    """Short convolution of q_pre, k_pre, v_pre (``conv_weight`` = (w_q, w_k,
    w_v), ``conv_state`` = (s_q, s_k, s_v) or None), then :func:`kda_layer`.
    Returns (y, final_state, (conv state of q, k, v))."""
    states = (None, None, None) if conv_state is None else conv_state
    conv = [short_conv(x, w, s, cu_seqlens) for x, w, s in
            zip((q_pre, k_pre, v_pre), conv_weight, states)]
    y, fin = kda_layer(conv[0][0], conv[1][0], conv[2][0], g, beta_pre, gate, weight, eps,
                       initial_state, cu_seqlens)
    return y, fin, tuple(c[1] for c in conv)


def kda_backward(q, k, v, g, beta, do, dfinal=None, initial_state=None, cu_seqlens=None,
                 block: int = 64):
    """Gradients of  L = sum(do * o) + sum(dfinal * S_N)  for the token
    recurrence (kda_recurrent): per token t, with S the state before it,

        Sp = Diag(exp g_t) S;  r = Sp^T k_t;  u = beta_t (v_t - r)
        S' = Sp + k_t u^T;     o_t = S'^T q_t

    and in reverse order (dS the gradient of the state after token t):

        dS += q_t do_t^T;        dq_t = S' do_t
        du = dS^T k_t;           dk_t = dS u
        dbeta_t = du . (v_t - r);  dv_t = beta_t du;  dr = -beta_t du
        dSp = dS + k_t dr^T;     dk_t += Sp dr
        dg_t = exp(g_t) * rowsum(dSp * S);  dS <- Diag(exp g_t) dSp

    Shapes as in kda_recurrent; do [T, H, dv]; dfinal and initial_state
    [N, H, dk, dv] or None.  States are recomputed from checkpoints every
    ``block`` tokens.  Returns (dq, dk, dv, dg, dbeta, dS0), float64.
    """
    q, k, v, g, beta, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, do))
    T, H, dk = q.shape
    dvv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    S0 = (np.zeros((N, H, dk, dvv)) if initial_state is None
          else np.asarray(initial_state, dtype=np.float64))
    dF = (np.zeros((N, H, dk, dvv)) if dfinal is None
          else np.asarray(dfinal, dtype=np.float64))
    dq, dk_, dv_, dg = (np.zeros_like(a) for a in (q, k, v, g))
    db = np.zeros_like(beta)
    dS0 = np.zeros((N, H, dk, dvv))
    alpha = np.exp(g)

    def step(S, t):  # one token for all heads; returns (Sp, r, u, S')
        Sp = alpha[t][:, :, None] * S
        r = np.einsum("hij,hi->hj", Sp, k[t])
        u = beta[t][:, None] * (v[t] - r)
        return Sp, r, u, Sp + k[t][:, :, None] * u[:, None, :]

    for n in range(N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        # forward: checkpoints at block starts
        ck = {}
        S = S0[n].copy()
        for t in range(bos, eos):
            if (t - bos) % block == 0:
                ck[t] = S.copy()
            S = step(S, t)[3]
        dS = dF[n].copy()
        starts = sorted(ck)
        for b0 in reversed(starts):
            b1 = min(b0 + block, eos)
            states = [ck[b0]]  # state before each token of the block
            for t in range(b0, b1 - 1):
                states.append(step(states[-1], t)[3])
            for t in range(b1 - 1, b0 - 1, -1):
                Sprev = states[t - b0]
                Sp, r, u, Sn = step(Sprev, t)
                dS = dS + q[t][:, :, None] * do[t][:, None, :]
                dq[t] = np.einsum("hij,hj->hi", Sn, do[t])
                du = np.einsum("hij,hi->hj", dS, k[t])
                dkt = np.einsum("hij,hj->hi", dS, u)
                db[t] = np.einsum("hj,hj->h", du, v[t] - r)
                dv_[t] = beta[t][:, None] * du
                dr = -beta[t][:, None] * du
                dSp = dS + k[t][:, :, None] * dr[:, None, :]
                dkt += np.einsum("hij,hj->hi", Sp, dr)
                dk_[t] = dkt
                dg[t] = alpha[t] * np.einsum("hij,hij->hi", dSp, Sprev)
                dS = alpha[t][:, :, None] * dSp
        dS0[n] = dS
    return dq, dk_, dv_, dg, db, dS0


def dplr_recurrent(q, k, v, a, b, g, initial_state=None, cu_seqlens=None):
    """General DPLR recurrence, token by token, float64, all heads at once:

        S_t = Diag(exp g_t) S_{t-1} - a_t (b_t^T S_{t-1}) + k_t v_t^T,
        o_t = S_t^T q_t

    q, k, a, b, g: [T, H, dk]; v: [T, H, dv]; initial_state [N, H, dk, dv] or
    None.  Returns (o [T, H, dv], final [N, H, dk, dv])."""
    q, k, v, a, b, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b, g))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    S0 = (np.zeros((N, H, dk, dv)) if initial_state is None
          else np.asarray(initial_state, dtype=np.float64))
    o = np.zeros((T, H, dv))
    fin = np.zeros((N, H, dk, dv))
    for n in range(N):
        S = S0[n].copy()
        for t in range(int(cu[n]), int(cu[n + 1])):
            bS = np.einsum("hi,hij->hj", b[t], S)
            S = (np.exp(g[t])[:, :, None] * S - a[t][:, :, None] * bS[:, None, :]
                 + k[t][:, :, None] * v[t][:, None, :])
            o[t] = np.einsum("hij,hi->hj", S, q[t])
        fin[n] = S
    return o, fin


def dplr_explicit(q, k, v, a, b, g, S0):
    """The same for ONE head by explicit transition matrices
    A_t = Diag(alpha_t) - a_t b_t^T:  S_t = A_t S_{t-1} + k_t v_t^T,
    o_t = S_t^T q_t.  ``g`` is the log-decay for float input; for exact
    evaluation pass object arrays of fractions.Fraction and ``g`` holding
    alpha itself (exp of a rational is not rational)."""
    T, dk = q.shape
    dv = v.shape[1]
    exact = np.asarray(g).dtype == object
    S = np.array(S0, dtype=object if exact else np.float64)
    o = np.empty((T, dv), dtype=S.dtype)
    for t in range(T):
        alpha = g[t] if exact else np.exp(np.asarray(g[t], dtype=np.float64))
        A = np.empty((dk, dk), dtype=S.dtype)
        for i in range(dk):
            for j in range(dk):
                A[i, j] = (alpha[i] if i == j else 0) - a[t][i] * b[t][j]
        S = A.dot(S) + np.outer(k[t], v[t])
        o[t] = S.T.dot(q[t])
    return o, S
