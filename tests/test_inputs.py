"""The seeded input generator: determinism, recipe, bf16 rounding."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.3e38, -3.3e38, 1.00390625,
                                  1.01171875, np.inf, -np.inf], dtype=np.float32)])
    ours = inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    bits = inputs.bf16_bits(ours)
    np.testing.assert_array_equal(
        bits, torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_deterministic_and_recipe():
    w = inputs.WORKLOADS[1]
    a = inputs.workload_tokens(w, T=64)
    b = inputs.workload_tokens(w, T=64)
    for x, y in zip((a.q, a.k, a.v, a.g, a.beta), (b.q, b.k, b.v, b.g, b.beta)):
        np.testing.assert_array_equal(x, y)
    assert a.q.shape == (64, 32, 128) and a.beta.shape == (64, 32)
    # bf16-exact q/k/v; L2-normalised before rounding
    np.testing.assert_array_equal(inputs.bf16_round(a.q), a.q)
    n = np.linalg.norm(a.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all(a.g <= 0) and np.all(a.g > -2)
    assert np.all((a.beta > 0) & (a.beta < 1))
    assert a.g.dtype == np.float32 and a.beta.dtype == np.float32


def test_varlen_lengths():
    w = inputs.WORKLOADS[2]
    lens = inputs.varlen_lengths(w)
    assert len(lens) == 16 and lens.min() >= 512 and lens.max() <= 8192
    assert int(lens.sum()) == 68645
    cu = inputs.cu_seqlens_from_lengths(lens)
    assert cu[0] == 0 and cu[-1] == 68645 and cu.dtype == np.int32


def test_f32_workload():
    w = inputs.WORKLOADS[0]
    t = inputs.workload_tokens(w)
    assert t.q.shape == (256, 1, 64) and t.dtype == "f32"
    n = np.linalg.norm(t.q.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-6)


def test_decode_steps_differ():
    w = inputs.WORKLOADS[4]
    a = inputs.decode_step_inputs(w, 0)
    b = inputs.decode_step_inputs(w, 1)
    assert a.q.shape == (256, 32, 128)
    assert not np.array_equal(a.q, b.q)
