"""Pins of the oracle's short convolution (oracle.short_conv, kda_layer_conv).

The convolution is causal and depthwise over the tokens of each sequence
("Kimi Linear" notes, docsaid.org, section "Other Components": q, k and v
pass through a short convolution after their projection).  It is pinned to
textbook routines (numpy.convolve, scipy.signal.lfilter), to a hand-worked
example, to its impulse response, and to state-carry and packing invariants;
planted mistakes (tap order, causality, an off-by-one shift, state rows
reversed, sequences leaking into each other, the state ignored or taken from
the wrong end) each fail at least one pin.
"""
import numpy as np
import pytest

import oracle



def _hand_example(conv):
    # W = 3, weights (1, 2, 3): the current token gets 3, the one before 2,
    # the one before that 1.  x = 1, 10, 100, 1000 from a zero state.
    w = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3)
    x = np.array([1.0, 10.0, 100.0, 1000.0]).reshape(4, 1, 1)
    y, fin = conv(x, w, None, None)
    np.testing.assert_array_equal(y[:, 0, 0], [3.0, 32.0, 321.0, 3210.0])
    np.testing.assert_array_equal(fin[0, 0, :, 0], [100.0, 1000.0])
    # With the state (5, 7) (7 the most recent): y0 = 3*1 + 2*7 + 1*5,
    # y1 = 3*10 + 2*1 + 1*7.
    y, fin = conv(x, w, np.array([5.0, 7.0]).reshape(1, 1, 2, 1), None)
    np.testing.assert_array_equal(y[:2, 0, 0], [22.0, 39.0])
    # A one-token sequence keeps the newer state row and appends its token.
    y, fin = conv(x[:1], w, np.array([5.0, 7.0]).reshape(1, 1, 2, 1), None)
    np.testing.assert_array_equal(fin[0, 0, :, 0], [7.0, 1.0])


def _textbook(conv):
    rng = np.random.default_rng(3)
    T, H, D, W = 23, 2, 3, 4
    x = rng.standard_normal((T, H, D))
    w = rng.standard_normal((H, D, W))
    y, _ = conv(x, w, None, None)
    from scipy.signal import lfilter
    for h in range(H):
        for c in range(D):
            np.testing.assert_allclose(y[:, h, c], np.convolve(x[:, h, c], w[h, c, ::-1])[:T],
                                       rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(y[:, h, c], lfilter(w[h, c, ::-1], [1.0], x[:, h, c]),
                                       rtol=1e-12, atol=1e-12)


def _impulse(conv):
    T, W = 12, 4
    w = np.array([0.5, -1.0, 2.0, 3.0]).reshape(1, 1, W)
    for t0 in (0, 5, 10):
        x = np.zeros((T, 1, 1))
        x[t0] = 1.0
        y, _ = conv(x, w, None, None)
        want = np.zeros(T)
        for m in range(W):
            if t0 + m < T:
                want[t0 + m] = w[0, 0, W - 1 - m]
        np.testing.assert_array_equal(y[:, 0, 0], want)


def _carry(conv):
    rng = np.random.default_rng(4)
    T, H, D, W = 17, 2, 5, 4
    x = rng.standard_normal((T, H, D))
    w = rng.standard_normal((H, D, W))
    s0 = rng.standard_normal((1, H, W - 1, D))
    y, fin = conv(x, w, s0, None)
    for a in (0, 1, 2, 3, 9, 16, 17):
        y1, f1 = conv(x[:a], w, s0, None)
        y2, f2 = conv(x[a:], w, f1, None)
        np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(f2, fin, rtol=0, atol=0)


def _packing(conv):
    rng = np.random.default_rng(5)
    lens = [4, 0, 1, 9, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, D, W = 2, 3, 4
    x = rng.standard_normal((cu[-1], H, D))
    w = rng.standard_normal((H, D, W))
    s0 = rng.standard_normal((len(lens), H, W - 1, D))
    y, fin = conv(x, w, s0, cu)
    for n in range(len(lens)):
        yn, fn = conv(x[cu[n]:cu[n + 1]], w, s0[n:n + 1], None)
        np.testing.assert_allclose(y[cu[n]:cu[n + 1]], yn, rtol=1e-14, atol=1e-14)
        np.testing.assert_array_equal(fin[n], fn[0])
    # an empty sequence hands its state on unchanged
    np.testing.assert_array_equal(fin[1], s0[1])


def _width_one(conv):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((7, 2, 3))
    w = rng.standard_normal((2, 3, 1))
    y, fin = conv(x, w, None, None)
    np.testing.assert_allclose(y, x * w[None, :, :, 0], rtol=1e-15)
    assert fin.shape == (1, 2, 0, 3)


PINS = [_hand_example, _textbook, _impulse, _carry, _packing, _width_one]


def run_pins(conv):
    for pin in PINS:
        pin(conv)


def test_short_conv_pins():
    run_pins(oracle.short_conv)


def test_kda_layer_conv_composes():
    """kda_layer_conv is the convolution followed by kda_layer; an identity
    kernel (1 on the current token) leaves kda_layer unchanged."""
    rng = np.random.default_rng(7)
    lens = [5, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, D, W = int(cu[-1]), 2, 4, 4
    qp, kp, vp = (rng.standard_normal((T, H, D)) for _ in range(3))
    g = -0.1 * rng.random((T, H, D))
    bp = rng.standard_normal((T, H))
    gate = rng.standard_normal((T, H, D))
    nw = 1 + 0.1 * rng.standard_normal(D)
    ws = tuple(rng.standard_normal((H, D, W)) for _ in range(3))
    ss = tuple(rng.standard_normal((2, H, W - 1, D)) for _ in range(3))
    y, fin, cs = oracle.kda_layer_conv(qp, kp, vp, g, bp, ws, ss, gate, nw, 1e-6, None, cu)
    conv = [oracle.short_conv(x, w, s, cu) for x, w, s in zip((qp, kp, vp), ws, ss)]
    y2, fin2 = oracle.kda_layer(conv[0][0], conv[1][0], conv[2][0], g, bp, gate, nw, 1e-6,
                                None, cu)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(fin, fin2)
    for a, b in zip(cs, conv):
        np.testing.assert_array_equal(a, b[1])
    ident = np.zeros((H, D, W))
    ident[:, :, W - 1] = 1.0
    y3, fin3, _ = oracle.kda_layer_conv(qp, kp, vp, g, bp, (ident,) * 3, None, gate, nw, 1e-6,
                                        None, cu)
    y4, fin4 = oracle.kda_layer(qp, kp, vp, g, bp, gate, nw, 1e-6, None, cu)
    np.testing.assert_allclose(y3, y4, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(fin3, fin4, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# ---------------------------------------------------------------------------

def _generic(x, w, state, cu, tap, fin_rows="last", restart=True, use_state=True):
    """A configurable causal convolution used to plant mistakes.  ``tap(t, i,
    W)`` gives the (relative) input position that weight i multiplies."""
    x = np.asarray(x, float)
    w = np.asarray(w, float)
    T, H, D = x.shape
    W = w.shape[-1]
    cu = np.array([0, T]) if cu is None else np.asarray(cu)
    N = len(cu) - 1
    st = np.zeros((N, H, W - 1, D)) if state is None else np.asarray(state, float)
    if not restart:
        cu = np.array([0, T])
        st = st[:1]
    y = np.zeros_like(x)
    fin = np.zeros((len(cu) - 1, H, W - 1, D))
    for n in range(len(cu) - 1):
        bos, eos = int(cu[n]), int(cu[n + 1])
        pre = st[n].transpose(1, 0, 2) if use_state else np.zeros((W - 1, H, D))
        ext = np.concatenate([pre, x[bos:eos]], axis=0)
        for t in range(eos - bos):
            for i in range(W):
                p = tap(t, i, W) + (W - 1)
                if 0 <= p < len(ext):
                    y[bos + t] += w[:, :, i] * ext[p]
        if W > 1:
            rows = ext[len(ext) - (W - 1):] if fin_rows == "last" else ext[:W - 1]
            fin[n] = rows.transpose(1, 0, 2)
    if not restart and N > 1:
        fin = np.repeat(fin, N, axis=0)
    return y, fin


def _mutants():
    right = lambda t, i, W: t - (W - 1) + i
    return {
        "taps_reversed": lambda x, w, s, cu: _generic(x, w, s, cu, lambda t, i, W: t - i),
        "anti_causal": lambda x, w, s, cu: _generic(x, w, s, cu, lambda t, i, W: t + i),
        "off_by_one": lambda x, w, s, cu: _generic(x, w, s, cu, lambda t, i, W: t - W + i),
        "state_rows_reversed": lambda x, w, s, cu: _generic(
            x, w, None if s is None else np.asarray(s)[:, :, ::-1], cu, right),
        "no_restart_between_sequences": lambda x, w, s, cu: _generic(x, w, s, cu, right,
                                                                     restart=False),
        "state_ignored": lambda x, w, s, cu: _generic(x, w, s, cu, right, use_state=False),
        "final_state_from_start": lambda x, w, s, cu: _generic(x, w, s, cu, right,
                                                               fin_rows="first"),
    }


def test_mutant_harness_is_faithful():
    """The unmutated generic form passes every pin, so a failing mutant fails
    because of its planted mistake."""
    run_pins(lambda x, w, s, cu: _generic(x, w, s, cu, lambda t, i, W: t - (W - 1) + i))


@pytest.mark.parametrize("kind", sorted(_mutants()))
def test_conv_pins_catch_planted_mistakes(kind):
    with pytest.raises(AssertionError):
        run_pins(_mutants()[kind])
