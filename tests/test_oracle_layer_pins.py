"""Pins of the oracle's layer prologue and epilogue (CPU only).

The prologue and epilogue follow the "Kimi Linear" notes (docsaid.org),
section "Other Components": q and k pass through Swish and are then L2
normalised, v through Swish, beta through a sigmoid; the output goes through
a per-head RMSNorm and is multiplied by a data-dependent sigmoid gate.  The
greeksharifa.github.io summary (section 4) says the same: queries and keys
are normalised to unit length; head-wise RMSNorm is followed by a sigmoid
gate.

Every value below is a constant worked out by hand (or a closed form), not
the oracle's formula typed again; the last test plants plausible mistakes in
copies of the functions and checks that each one fails a pin.
"""
import math

import numpy as np
import pytest

import oracle

SQRT125 = 3.5355339059327378      # sqrt(12.5)
SQRT13 = 3.605551275463989        # sqrt(13)


def pin_swish_values(sw):
    # x * sigmoid(x) at x = 0, 1, -1, 2 (sigmoid(1) = 0.7310585786300049,
    # sigmoid(2) = 0.8807970779778823), and its two asymptotes.
    np.testing.assert_allclose(sw(np.array([0.0, 1.0, -1.0, 2.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951,
                                1.7615941559557646], rtol=1e-15, atol=1e-16)
    assert abs(float(sw(np.array([30.0]))[0]) - 30.0) < 1e-10
    assert abs(float(sw(np.array([-40.0]))[0])) < 1e-15


def pin_sigmoid_values(sg):
    np.testing.assert_allclose(sg(np.array([0.0, math.log(3.0), -math.log(3.0)])),
                               [0.5, 0.75, 0.25], rtol=1e-15)


def pin_l2_rows(l2):
    # (3, 4) -> (0.6, 0.8); every (t, h) row independently; zero row stays 0.
    x = np.zeros((2, 3, 2))
    x[0, 0] = [3.0, 4.0]
    x[0, 1] = [-5.0, 12.0]
    x[1, 2] = [0.0, 2.0]
    y = l2(x)
    np.testing.assert_allclose(y[0, 0], [0.6, 0.8], rtol=1e-15)
    np.testing.assert_allclose(y[0, 1], [-5 / 13, 12 / 13], rtol=1e-15)
    np.testing.assert_allclose(y[1, 2], [0.0, 1.0], rtol=1e-15)
    assert np.all(y[0, 2] == 0) and np.all(y[1, 0] == 0)
    rng = np.random.default_rng(30)
    z = rng.standard_normal((5, 4, 16))
    n = np.sqrt((l2(z) ** 2).sum(-1))
    np.testing.assert_allclose(n, 1.0, rtol=1e-14)
    cos = (l2(z) * z).sum(-1) / np.sqrt((z * z).sum(-1))
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)


def pin_epilogue_worked_example(ep):
    # o = (3, 4): mean square 12.5.  weight (1, 2), gate (0, ln 3) -> sigmoid
    # (0.5, 0.75).  eps = 0: y = (3 / sqrt 12.5 * 0.5, 4 / sqrt 12.5 * 2 * 0.75);
    # eps = 0.5: the root becomes sqrt 13.
    o = np.array([[[3.0, 4.0]]])
    gate = np.array([[[0.0, math.log(3.0)]]])
    w = np.array([1.0, 2.0])
    np.testing.assert_allclose(ep(o, gate, w, 0.0)[0, 0],
                               [3 / SQRT125 * 0.5, 4 / SQRT125 * 1.5], rtol=1e-15)
    np.testing.assert_allclose(ep(o, gate, w, 0.5)[0, 0],
                               [3 / SQRT13 * 0.5, 4 / SQRT13 * 1.5], rtol=1e-15)


def pin_epilogue_invariants(ep):
    rng = np.random.default_rng(31)
    o = rng.standard_normal((4, 3, 16))
    open_gate = np.full_like(o, 60.0)               # sigmoid = 1 to fp64
    ones = np.ones(16)
    y = ep(o, open_gate, ones, 0.0)
    # unit root-mean-square per (token, head), scale invariance, half gate
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(ep(7.5 * o, open_gate, ones, 0.0), y, rtol=1e-14)
    np.testing.assert_allclose(ep(o, np.zeros_like(o), ones, 0.0), 0.5 * y, rtol=1e-14)
    # the weight scales channels one by one
    w = np.zeros(16)
    w[5] = 3.0
    yw = ep(o, open_gate, w, 0.0)
    np.testing.assert_allclose(yw[..., 5], 3.0 * y[..., 5], rtol=1e-14)
    assert np.all(np.delete(yw, 5, axis=-1) == 0)


def pin_prologue_composition(pro):
    # q_pre row (1, -1) -> swish (0.7310585786300049, -0.2689414213699951),
    # norm sqrt(0.5344466... + 0.0723295...) = 0.7789525...; v = swish;
    # beta = sigmoid.
    a, b = 0.7310585786300049, -0.2689414213699951
    n = math.sqrt(a * a + b * b)
    qp = np.array([[[1.0, -1.0]]])
    q, k, v, beta = pro(qp, 2 * qp, qp, np.array([[math.log(3.0)]]))
    np.testing.assert_allclose(q[0, 0], [a / n, b / n], rtol=1e-15)
    s2 = np.array([1.7615941559557646, -0.2384058440442351])  # swish(2), swish(-2)
    np.testing.assert_allclose(k[0, 0], s2 / np.sqrt((s2 * s2).sum()), rtol=1e-15)
    np.testing.assert_allclose(v[0, 0], [a, b], rtol=1e-15)
    np.testing.assert_allclose(beta, [[0.75]], rtol=1e-15)


IMPL = dict(sw=oracle.swish, sg=oracle.sigmoid, l2=oracle.l2_normalize,
            ep=oracle.layer_epilogue, pro=oracle.layer_prologue)


def run_pins(impl):
    pin_swish_values(impl["sw"])
    pin_sigmoid_values(impl["sg"])
    pin_l2_rows(impl["l2"])
    pin_epilogue_worked_example(impl["ep"])
    pin_epilogue_invariants(impl["ep"])
    pin_prologue_composition(impl["pro"])


def test_layer_pins():
    run_pins(IMPL)


def test_kda_layer_composes():
    """kda_layer = epilogue(recurrence(prologue(...))) on a small packed case,
    and without a gate it is the recurrence on the prologue's outputs."""
    rng = np.random.default_rng(32)
    T, H, D = 40, 2, 8
    qp, kp, vp = (rng.standard_normal((T, H, D)) for _ in range(3))
    bp = rng.standard_normal((T, H))
    g = -np.logaddexp(0, rng.standard_normal((T, H, D))) * 0.2
    gate = rng.standard_normal((T, H, D))
    w = rng.uniform(0.5, 1.5, D)
    cu = np.array([0, 15, 15, 40])
    s0 = rng.standard_normal((3, H, D, D)) * 0.1
    q, k, v, beta = oracle.layer_prologue(qp, kp, vp, bp)
    o, fin = oracle.kda_recurrent(q, k, v, g, beta, s0, cu)
    y, fin2 = oracle.kda_layer(qp, kp, vp, g, bp, gate, w, 1e-6, s0, cu)
    np.testing.assert_allclose(y, oracle.layer_epilogue(o, gate, w, 1e-6), rtol=1e-14)
    np.testing.assert_array_equal(fin, fin2)
    y0, _ = oracle.kda_layer(qp, kp, vp, g, bp, None, None, 1e-6, s0, cu)
    np.testing.assert_array_equal(y0, o)


def _mutants():
    sg = lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))
    base = dict(IMPL)
    out = {}
    m = dict(base); m["sw"] = sg; out["swish_is_sigmoid"] = m
    m = dict(base); m["sw"] = lambda x: np.asarray(x, float) * sg(-np.asarray(x, float)); out["swish_sign"] = m
    m = dict(base); m["l2"] = lambda x: np.asarray(x, float) / np.maximum(
        np.sqrt((np.asarray(x, float) ** 2).sum(axis=0, keepdims=True)), 1e-12); out["l2_axis"] = m
    m = dict(base); m["l2"] = lambda x: np.asarray(x, float) / np.maximum(
        (np.asarray(x, float) ** 2).sum(axis=-1, keepdims=True), 1e-12); out["l2_no_sqrt"] = m

    def ep_sum(o, gate, w, eps):
        o = np.asarray(o, float)
        return o / np.sqrt((o * o).sum(-1, keepdims=True) + eps) * w * sg(gate)
    m = dict(base); m["ep"] = ep_sum; out["rms_sum_not_mean"] = m

    def ep_eps_out(o, gate, w, eps):
        o = np.asarray(o, float)
        return o / (np.sqrt((o * o).mean(-1, keepdims=True)) + eps) * w * sg(gate)
    m = dict(base); m["ep"] = ep_eps_out; out["eps_outside_root"] = m

    def ep_heads(o, gate, w, eps):
        o = np.asarray(o, float)
        return o / np.sqrt((o * o).mean(-2, keepdims=True) + eps) * w * sg(gate)
    m = dict(base); m["ep"] = ep_heads; out["rms_over_heads"] = m

    def ep_gate_raw(o, gate, w, eps):
        o = np.asarray(o, float)
        return o / np.sqrt((o * o).mean(-1, keepdims=True) + eps) * w * np.asarray(gate, float)
    m = dict(base); m["ep"] = ep_gate_raw; out["gate_without_sigmoid"] = m

    def pro_no_swish(qp, kp, vp, bp):
        return (oracle.l2_normalize(qp), oracle.l2_normalize(kp), oracle.swish(vp), oracle.sigmoid(bp))
    m = dict(base); m["pro"] = pro_no_swish; out["prologue_skips_swish"] = m

    def pro_v_normalised(qp, kp, vp, bp):
        q, k, v, b = oracle.layer_prologue(qp, kp, vp, bp)
        return q, k, oracle.l2_normalize(v), b
    m = dict(base); m["pro"] = pro_v_normalised; out["prologue_normalises_v"] = m
    return out


@pytest.mark.parametrize("kind", sorted(_mutants()))
def test_layer_pins_catch_planted_mistakes(kind):
    with pytest.raises(AssertionError):
        run_pins(_mutants()[kind])
