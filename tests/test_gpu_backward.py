"""Parity of the HIP backward pass (kda_backward, through the C ABI) with the
float64 oracle's kda_backward.

Error metric (per gradient tensor): max |x - y| / max |y|, with y the oracle.
Gates: 2e-3 for bf16 inputs, 1e-5 for fp32 inputs (the arithmetic is fp32
in both cases; bf16 inputs are bf16-exact values).
"""
import sys

import numpy as np
import pytest

import oracle
from gated_delta_rule_56_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import kda as k
    k.load()
    return k


def tdev(a, dtype=torch.float32):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).to(DEV) if dtype != torch.float32 else t.to(DEV)


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-30))


def host(t):
    return t.float().cpu().numpy()


def run_case(kda, x, C, s0=None, cu=None, with_dfin=True, seed=0):
    rng = np.random.default_rng([50, seed])
    T, H, D = x.q.shape
    N = 1 if cu is None else len(cu) - 1
    do = rng.standard_normal((T, H, x.v.shape[2])).astype(np.float32)
    dF = rng.standard_normal((N, H, D, x.v.shape[2])).astype(np.float32) if with_dfin else None
    ref = oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, do, dF, s0, cu)
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    cud = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(DEV)
    got = kda.backward(tdev(x.q, dt)[None], tdev(x.k, dt)[None], tdev(x.v, dt)[None],
                       tdev(x.g)[None], tdev(x.beta)[None], tdev(do)[None],
                       None if s0 is None else tdev(s0), None if dF is None else tdev(dF),
                       cud, cu_seqlens_host=None if cu is None else np.asarray(cu, np.int32),
                       chunk_size=C)
    torch.cuda.synchronize()
    errs = {}
    for name, a, r in zip(NAMES, got, ref):
        a = host(a)
        if name != "dS0":
            a = a[0]
        errs[name] = rel(a, r)
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    return errs


@pytest.mark.parametrize("dtype,D,C,T", [
    ("f32", 64, 16, 77), ("f32", 128, 64, 200), ("bf16", 128, 64, 300), ("bf16", 64, 32, 131),
    ("f32", 128, 32, 1), ("bf16", 128, 64, 64)])
def test_backward_matches_oracle(kda, dtype, D, C, T):
    say(f"backward dtype={dtype} D={D} C={C} T={T}")
    rng = np.random.default_rng([51, D, C, T])
    H = 2
    x = I.draw_tokens(rng, T, H, D, D, dtype)
    s0 = I.draw_states(rng, 1, H, D, D)
    errs = run_case(kda, x, C, s0=s0, seed=T)
    assert max(errs.values()) <= TOL[dtype], errs


def test_backward_varlen(kda):
    """Packed sequences, one empty and one a single token, no final-state
    gradient."""
    say("backward varlen")
    lens = [37, 0, 130, 1, 70]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(52)
    H, D = 2, 128
    x = I.draw_tokens(rng, int(cu[-1]), H, D, D, "f32")
    s0 = I.draw_states(rng, len(lens), H, D, D)
    errs = run_case(kda, x, 64, s0=s0, cu=cu, with_dfin=False, seed=1)
    assert max(errs.values()) <= TOL["f32"], errs


def test_backward_strong_decay(kda):
    """g scaled x50: chunk decays far past what a factored exp(-Gamma) could
    hold; the exact pairwise exponents keep the gradients right."""
    say("backward strong decay")
    rng = np.random.default_rng(53)
    x = I.draw_tokens(rng, 150, 2, 64, 64, "f32", g_scale=5.0)
    errs = run_case(kda, x, 64, seed=2)
    assert max(errs.values()) <= TOL["f32"], errs


def test_backward_full_size_sampled_heads(kda):
    """The headline shape (B=1, T=4096, H=32, d=128, bf16, chunk 64, initial
    state and final-state gradient), all heads on the GPU; the oracle
    replays two sampled heads over the whole sequence."""
    say("backward full size T=4096 H=32, sampled heads 0 and 19")
    T, H, D = 4096, 32, 128
    rng = np.random.default_rng(54)
    x = I.draw_tokens(rng, T, H, D, D, "bf16")
    s0 = I.draw_states(rng, 1, H, D, D)
    do = rng.standard_normal((T, H, D)).astype(np.float32)
    dF = rng.standard_normal((1, H, D, D)).astype(np.float32)
    got = kda.backward(tdev(x.q, torch.bfloat16)[None], tdev(x.k, torch.bfloat16)[None],
                       tdev(x.v, torch.bfloat16)[None], tdev(x.g)[None], tdev(x.beta)[None],
                       tdev(do)[None], tdev(s0), tdev(dF), chunk_size=64)
    torch.cuda.synchronize()
    hs = [0, 19]
    ref = oracle.kda_backward(x.q[:, hs], x.k[:, hs], x.v[:, hs], x.g[:, hs], x.beta[:, hs],
                              do[:, hs], dF[:, hs], s0[:, hs])
    errs = {}
    for name, a, r in zip(NAMES, got, ref):
        a = host(a)
        a = a[:, hs] if name == "dS0" else a[0][:, hs]
        errs[name] = rel(a, r)
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_no_tokens(kda):
    """T = 0: every token gradient is empty and dS0 equals dS_N."""
    say("backward T=0")
    H, D = 2, 64
    rng = np.random.default_rng(55)
    dF = rng.standard_normal((1, H, D, D)).astype(np.float32)
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device=DEV)
    got = kda.backward(z(1, 0, H, D), z(1, 0, H, D), z(1, 0, H, D), z(1, 0, H, D), z(1, 0, H),
                       z(1, 0, H, D), tdev(I.draw_states(rng, 1, H, D, D)), tdev(dF),
                       chunk_size=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got[5]), dF)
    assert got[0].numel() == 0


def run_case_opts(kda, x, C, options, s0=None, cu=None, seed=0):
    """run_case with kda_backward_ex options (forced segment lengths)."""
    rng = np.random.default_rng([56, seed])
    T, H, D = x.q.shape
    N = 1 if cu is None else len(cu) - 1
    do = rng.standard_normal((T, H, x.v.shape[2])).astype(np.float32)
    dF = rng.standard_normal((N, H, D, x.v.shape[2])).astype(np.float32)
    ref = oracle.kda_backward(x.q, x.k, x.v, x.g, x.beta, do, dF, s0, cu)
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    cud = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(DEV)
    got = kda.backward(tdev(x.q, dt)[None], tdev(x.k, dt)[None], tdev(x.v, dt)[None],
                       tdev(x.g)[None], tdev(x.beta)[None], tdev(do)[None],
                       None if s0 is None else tdev(s0), tdev(dF),
                       cud, cu_seqlens_host=None if cu is None else np.asarray(cu, np.int32),
                       chunk_size=C, options=options)
    torch.cuda.synchronize()
    errs = {}
    for name, a, r in zip(NAMES, got, ref):
        a = host(a)
        if name != "dS0":
            a = a[0]
        errs[name] = rel(a, r)
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    return errs


@pytest.mark.parametrize("dtype,D,C,T,L", [
    ("f32", 64, 16, 300, 1), ("f32", 128, 32, 300, 2), ("bf16", 128, 64, 700, 3),
    ("bf16", 64, 64, 200, 4)])
def test_backward_segments(kda, dtype, D, C, T, L):
    """Forced short segments: the forward sweep's states and the carried dS
    cross every segment boundary."""
    say(f"backward segments dtype={dtype} D={D} C={C} T={T} segment_chunks={L}")
    rng = np.random.default_rng([57, D, C, T])
    H = 2
    x = I.draw_tokens(rng, T, H, D, D, dtype)
    s0 = I.draw_states(rng, 1, H, D, D)
    errs = run_case_opts(kda, x, C, {"segment_chunks": L}, s0=s0, seed=L)
    assert max(errs.values()) <= TOL[dtype], errs


def test_backward_segments_varlen(kda):
    """Packed sequences of different chunk counts (one empty, one a single
    token) in 1-chunk and 2-chunk segments: sequences that end early hand
    their state and dS through the later segments unchanged."""
    lens = [37, 0, 130, 1, 70]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(58)
    H, D = 2, 128
    x = I.draw_tokens(rng, int(cu[-1]), H, D, D, "f32")
    s0 = I.draw_states(rng, len(lens), H, D, D)
    for C, L in ((16, 1), (32, 2)):
        say(f"backward varlen segments C={C} segment_chunks={L}")
        errs = run_case_opts(kda, x, C, {"segment_chunks": L}, s0=s0, cu=cu, seed=C)
        assert max(errs.values()) <= TOL["f32"], errs


def test_backward_long_sampled_heads(kda):
    """T = 65,536, H = 8, d = 128, bf16, chunk 64, initial state and final-state
    gradient: the automatic plan runs it in two segments (and a forced
    100-chunk segment length in eleven); the oracle replays two sampled heads
    over the whole sequence."""
    T, H, D = 65536, 8, 128
    rng = np.random.default_rng(59)
    x = I.draw_tokens(rng, T, H, D, D, "bf16")
    s0 = I.draw_states(rng, 1, H, D, D)
    do = rng.standard_normal((T, H, D)).astype(np.float32)
    dF = rng.standard_normal((1, H, D, D)).astype(np.float32)
    hs = [1, 6]
    say(f"backward long T={T} H={H}: oracle for heads {hs}")
    ref = oracle.kda_backward(x.q[:, hs], x.k[:, hs], x.v[:, hs], x.g[:, hs], x.beta[:, hs],
                              do[:, hs], dF[:, hs], s0[:, hs])
    args = (tdev(x.q, torch.bfloat16)[None], tdev(x.k, torch.bfloat16)[None],
            tdev(x.v, torch.bfloat16)[None], tdev(x.g)[None], tdev(x.beta)[None],
            tdev(do)[None], tdev(s0), tdev(dF))
    for options in (None, {"segment_chunks": 100}):
        nbytes = kda.backward_workspace_size(1, T, H, D, 1, 64, options=options)
        say(f"  options={options}: workspace {nbytes / 2**30:.2f} GiB")
        got = kda.backward(*args, chunk_size=64, options=options)
        torch.cuda.synchronize()
        errs = {}
        for name, a, r in zip(NAMES, got, ref):
            a = host(a)
            a = a[:, hs] if name == "dS0" else a[0][:, hs]
            errs[name] = rel(a, r)
        say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        assert max(errs.values()) <= TOL["bf16"], errs
        del got


@pytest.mark.parametrize("dtype,C,alpha", [("bf16", 64, 0.1), ("f32", 64, 0.1), ("f32", 32, 0.01),
                                           ("bf16", 16, 0.1), ("f32", 64, 1e-20)])
def test_backward_mixed_decay(kda, dtype, C, alpha):
    """Half the key channels at alpha per token: every chunk is past the
    chunk-wide span, so Bm, P and the pairwise gradient terms go through the
    tile-factored kernels (alpha = 0.01 and 1e-20: diagonal tiles past the
    tile span as well, summed with exact exponents)."""
    say(f"backward mixed decay dtype={dtype} C={C} alpha={alpha}")
    rng = np.random.default_rng([60, C, int(-np.log10(alpha))])
    T, H, D = 3 * C + 21, 2, 128
    x = I.draw_mixed_decay_tokens(rng, T, H, D, D, dtype, alpha=alpha)
    s0 = I.draw_states(rng, 1, H, D, D)
    errs = run_case(kda, x, C, s0=s0, seed=C)
    assert max(errs.values()) <= TOL[dtype], errs
