"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Error metric (per output tensor): max |x - y| / max |y|, with y the oracle.
Gates: 2e-3 for bf16 inputs, 1e-5 for fp32 inputs.
"""
import os
import sys

import numpy as np
import pytest

import oracle
from gated_delta_rule_56_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


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


DEV = "cuda:0"


def tdev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).to(DEV) if dtype != torch.float32 else t.to(DEV)


def tok_to_dev(x: I.TokenInputs, B=1):
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    shp = lambda a: a.reshape((B, a.shape[0] // B) + a.shape[1:])
    return (tdev(shp(x.q), dt), tdev(shp(x.k), dt), tdev(shp(x.v), dt),
            tdev(shp(x.g), torch.float32), tdev(shp(x.beta), torch.float32))


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-30))


def pair_rel(x, y, pair_axes):
    """Worst per-(sequence, head) error: max |x - y| / max |y| taken over the
    elements of each pair (the axes not in ``pair_axes``), then the maximum
    over pairs.  A pair whose outputs are small cannot hide behind a larger
    one, as it can in the per-tensor figure."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    red = tuple(a for a in range(x.ndim) if a not in pair_axes)
    num = np.abs(x - y).max(axis=red)
    den = np.maximum(np.abs(y).max(axis=red), 1e-30)
    return float((num / den).max())


def varlen_pair_rel(o, eo, cu):
    """Worst per-(sequence, head) error of packed outputs [tokens, H, D]."""
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            worst = max(worst, pair_rel(o[a:b], eo[a:b], (1,)))
    return worst


def host(t):
    return t.float().cpu().numpy()


def run_prefill(kda, x, C, s0=None, cu=None, out_dtype=None):
    q, k, v, g, b = tok_to_dev(x)
    s0d = None if s0 is None else torch.from_numpy(s0).to(DEV)
    cud = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(DEV)
    o, fin = kda.prefill(q, k, v, g, b, s0d, cud, cu_seqlens_host=cu, chunk_size=C,
                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(o)[0], host(fin)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_decode_steps_match_oracle(kda, dtype, D):
    say(f"decode dtype={dtype} D={D}")
    N, H, steps = 3, 2, 64
    rng = np.random.default_rng([7, D])
    x = I.draw_tokens(rng, N * steps, H, D, D, dtype)
    s0 = I.draw_states(rng, N, H, D, D)
    # token t of sequence n lives at row n*steps + t
    cu = np.arange(N + 1) * steps
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    state = torch.from_numpy(s0.copy()).to(DEV)
    worst = 0.0
    for t in range(steps):
        rows = np.arange(N) * steps + t
        o = kda.decode_step(tdev(x.q[rows], dt), tdev(x.k[rows], dt), tdev(x.v[rows], dt),
                            tdev(x.g[rows], torch.float32), tdev(x.beta[rows], torch.float32),
                            state)
        worst = max(worst, rel(host(o), eo[rows]))
    torch.cuda.synchronize()
    es = rel(host(state), ef)
    say(f"  o err {worst:.2e}  state err {es:.2e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]


def test_decode_bf16_output(kda):
    say("decode bf16 output")
    rng = np.random.default_rng(8)
    x = I.draw_tokens(rng, 5, 3, 128, 128, "bf16")
    s0 = I.draw_states(rng, 5, 3, 128, 128)
    eo, _ = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=np.arange(6))
    state = torch.from_numpy(s0).to(DEV)
    q, k, v, g, b = (a[0] for a in tok_to_dev(x))
    o = kda.decode_step(q, k, v, g, b, state, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    assert rel(host(o), eo) <= 8e-3   # one bf16 rounding of o


@pytest.mark.slow
def test_decode_workload4_full(kda):
    """256 sequences x 32 heads, d=128, bf16, state [256, 32, 128, 128] ~
    N(0, 0.1): all 1000 steps on the GPU.  The oracle replays every (sequence,
    head) pair over the same 1000 tokens; o is compared at steps 1, 10, 100
    and 1000 and the whole state after step 1000, per tensor and per pair."""
    from concurrent.futures import ThreadPoolExecutor
    w = I.WORKLOADS[4]
    N, H, D, steps = w.decode_N, w.H, w.Dk, w.decode_steps
    checks = (1, 10, 100, 1000)
    say(f"decode workload 4: {steps} steps, N={N}, H={H}")
    s0 = I.draw_states(np.random.default_rng([4, 2]), N, H, D, D)
    state = torch.from_numpy(s0).to(DEV)
    # host copies of every step's inputs for the oracle, [step, N, H, D]
    hq = np.empty((steps, N, H, D), np.float32)
    hk, hv, hg = np.empty_like(hq), np.empty_like(hq), np.empty_like(hq)
    hb = np.empty((steps, N, H), np.float32)
    o_chk = {}
    with ThreadPoolExecutor(8) as ex:
        futs = [ex.submit(I.decode_step_inputs, w, s) for s in range(min(16, steps))]
        for step in range(steps):
            x = futs[step].result()
            futs[step] = None
            if step + 16 < steps:
                futs.append(ex.submit(I.decode_step_inputs, w, step + 16))
            hq[step], hk[step], hv[step], hg[step], hb[step] = x.q, x.k, x.v, x.g, x.beta
            q, k, v, g, b = (a[0] for a in tok_to_dev(x))
            o = kda.decode_step(q, k, v, g, b, state)
            if step + 1 in checks:
                o_chk[step + 1] = host(o)
            if (step + 1) % 200 == 0:
                say(f"  step {step + 1}/{steps}")
    torch.cuda.synchronize()
    st = host(state)
    say("  oracle over every pair, 16 sequences at a time")
    cu = np.arange(17, dtype=np.int64) * steps
    worst_o_pair = worst_s_pair = 0.0
    seq_major = lambda a, n0: np.ascontiguousarray(
        a[:, n0:n0 + 16].swapaxes(0, 1).reshape((16 * steps,) + a.shape[2:]))
    max_o = {c: 0.0 for c in checks}
    err_o = {c: 0.0 for c in checks}
    max_s = err_s = 0.0
    for n0 in range(0, N, 16):
        eo, ef = oracle.kda_recurrent(seq_major(hq, n0), seq_major(hk, n0), seq_major(hv, n0),
                                      seq_major(hg, n0), seq_major(hb, n0), s0[n0:n0 + 16],
                                      cu_seqlens=cu)
        eo = eo.reshape(16, steps, H, D)
        for c in checks:
            x, y = o_chk[c][n0:n0 + 16], eo[:, c - 1]
            err_o[c] = max(err_o[c], float(np.abs(x - y).max()))
            max_o[c] = max(max_o[c], float(np.abs(y).max()))
            worst_o_pair = max(worst_o_pair, pair_rel(x, y, (0, 1)))
        x = st[n0:n0 + 16]
        err_s = max(err_s, float(np.abs(x - ef).max()))
        max_s = max(max_s, float(np.abs(ef).max()))
        worst_s_pair = max(worst_s_pair, pair_rel(x, ef, (0, 1)))
        if n0 % 64 == 0:
            say(f"  oracle sequences {n0}..{n0 + 15}")
    worst_o = max(err_o[c] / max_o[c] for c in checks)
    worst_s = err_s / max_s
    say("  o err " + " ".join(f"step{c} {err_o[c] / max_o[c]:.2e}" for c in checks) +
        f"  per pair {worst_o_pair:.2e}")
    say(f"  state err {worst_s:.2e}  per pair {worst_s_pair:.2e}")
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]
    assert worst_o_pair <= TOL["bf16"] and worst_s_pair <= TOL["bf16"]


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

@pytest.mark.parametrize("C", [16, 64])
def test_prefill_workload0(kda, C):
    """T=256, H=1, d=64, fp32 inputs, zero initial state, chunk 16 and 64."""
    say(f"prefill workload 0 C={C}")
    w = I.WORKLOADS[0]
    x = I.workload_tokens(w)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    o, fin = run_prefill(kda, x, C)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["f32"] and es_ <= TOL["f32"]


@pytest.mark.parametrize("dtype,D,C,T", [
    ("bf16", 128, 64, 300), ("bf16", 128, 32, 300), ("bf16", 128, 16, 77),
    ("bf16", 64, 64, 200), ("f32", 128, 64, 200), ("f32", 64, 32, 131),
    ("bf16", 128, 64, 1), ("bf16", 128, 64, 64), ("bf16", 128, 64, 65)])
def test_prefill_ragged_with_state(kda, dtype, D, C, T):
    say(f"prefill dtype={dtype} D={D} C={C} T={T}")
    rng = np.random.default_rng([9, D, C, T])
    H = 3
    x = I.draw_tokens(rng, T, H, D, D, dtype)
    s0 = I.draw_states(rng, 1, H, D, D)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0)
    o, fin = run_prefill(kda, x, C, s0=s0)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("vb", [16, 32])
def test_prefill_every_variant_multichunk(kda, dtype, D, C, vb):
    """Every built (dtype, head size, chunk) variant over several chunks with a
    ragged tail and an initial state, with 16 and with 32 value columns per
    carry-pass workgroup: exercises the inter-chunk pipeline (operands
    fetched one and two chunks ahead) for each instantiation."""
    T = 3 * C + 5
    say(f"prefill variant dtype={dtype} D={D} C={C} T={T} value_block={vb}")
    rng = np.random.default_rng([19, D, C])
    x = I.draw_tokens(rng, T, 2, D, D, dtype)
    s0 = I.draw_states(rng, 1, 2, D, D)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0)
    q, k, v, g, b = tok_to_dev(x)
    o, fin = kda.prefill(q, k, v, g, b, torch.from_numpy(s0).to(DEV), chunk_size=C,
                         options={"value_block": vb})
    torch.cuda.synchronize()
    o, fin = host(o)[0], host(fin)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]


@pytest.mark.parametrize("dtype,D,C", [(dt, D, C) for dt in ("bf16", "f32") for D in (64, 128)
                                       for C in (16, 32, 64)])
def test_prefill_many_pairs_automatic_block(kda, dtype, D, C):
    """Enough (sequence, head) pairs (80 packed sequences x 4 heads) for the
    automatic choice to take 32 value columns per carry-pass workgroup, for
    every (dtype, head size, chunk): ragged lengths, an empty sequence,
    initial states; per-(sequence, head) errors reported and gated."""
    rng = np.random.default_rng([25, D, C])
    lens = rng.integers(0, 3 * C + 9, 80)
    lens[7] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H = 4
    assert len(lens) * H * (D // 32) >= 512
    say(f"prefill many pairs dtype={dtype} D={D} C={C} tokens={int(cu[-1])}")
    x = I.draw_tokens(rng, int(cu[-1]), H, D, D, dtype)
    s0 = I.draw_states(rng, len(lens), H, D, D)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    o, fin = run_prefill(kda, x, C, s0=s0, cu=cu)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    po, ps = varlen_pair_rel(o, eo, cu), pair_rel(fin, ef, (0, 1))
    say(f"  o err {eo_:.2e} (per pair {po:.2e})  state err {es_:.2e} (per pair {ps:.2e})")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]
    assert po <= TOL[dtype] and ps <= TOL[dtype]
    np.testing.assert_array_equal(fin[7], s0[7])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_strong_decay(kda, dtype):
    """g scaled x50: chunk decay spans far past exp(-40), so the Grams take the
    exact pairwise path."""
    say(f"prefill strong decay {dtype}")
    rng = np.random.default_rng(10)
    x = I.draw_tokens(rng, 150, 2, 128, 128, dtype, g_scale=5.0)
    s0 = I.draw_states(rng, 1, 2, 128, 128)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0)
    o, fin = run_prefill(kda, x, 64, s0=s0)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]


@pytest.mark.parametrize("dtype,alpha,C", [("bf16", 0.1, 64), ("f32", 0.1, 64), ("bf16", 0.1, 16),
                                           ("bf16", 0.01, 64), ("f32", 0.01, 32),
                                           ("bf16", 1e-20, 64)])
def test_prefill_mixed_decay(kda, dtype, alpha, C):
    """Half the key channels decay at alpha near 0.1 per token (a 16-token
    tile spans about 37 in log-decay: products only), near 0.01 (about 74:
    the diagonal blocks of those tiles are evaluated pair by pair) or 1e-20
    (each token wipes those channels), the other half at the workload rate;
    packed sequences with initial states and ragged tails."""
    say(f"prefill mixed decay dtype={dtype} alpha={alpha} C={C}")
    lens = [3 * C + 9, 0, 2 * C, 37]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng([26, C, int(-np.log10(alpha))])
    H = 3
    x = I.draw_mixed_decay_tokens(rng, int(cu[-1]), H, 128, 128, dtype, alpha=alpha)
    s0 = I.draw_states(rng, len(lens), H, 128, 128)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    o, fin = run_prefill(kda, x, C, s0=s0, cu=cu)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    po, ps = varlen_pair_rel(o, eo, cu), pair_rel(fin, ef, (0, 1))
    say(f"  o err {eo_:.2e} (per pair {po:.2e})  state err {es_:.2e} (per pair {ps:.2e})")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]
    assert po <= TOL[dtype] and ps <= TOL[dtype]


def test_prefill_mixed_decay_full_size(kda):
    """The T=4096, H=32 workload with half the channels at alpha near 0.1."""
    say("prefill mixed decay T=4096 H=32")
    rng = np.random.default_rng(27)
    x = I.draw_mixed_decay_tokens(rng, 4096, 32, 128, 128, "bf16", alpha=0.1)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    o, fin = run_prefill(kda, x, 64)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    po, ps = pair_rel(o, eo, (1,)), pair_rel(fin, ef, (0, 1))
    say(f"  o err {eo_:.2e} (per head {po:.2e})  state err {es_:.2e} (per head {ps:.2e})")
    assert max(eo_, es_, po, ps) <= TOL["bf16"]


def test_prefill_weak_decay(kda):
    """g scaled x0.01: long memory, errors could accumulate across chunks."""
    say("prefill weak decay")
    rng = np.random.default_rng(11)
    x = I.draw_tokens(rng, 1024, 2, 128, 128, "bf16", g_scale=0.001)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    o, fin = run_prefill(kda, x, 64)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]


@pytest.mark.parametrize("C", [64, 16])
def test_prefill_varlen(kda, C):
    say(f"prefill varlen C={C}")
    lens = [1, 64, 0, 130, 200, 17, 65]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(12)
    H = 2
    x = I.draw_tokens(rng, int(cu[-1]), H, 128, 128, "bf16")
    s0 = I.draw_states(rng, len(lens), H, 128, 128)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    o, fin = run_prefill(kda, x, C, s0=s0, cu=cu)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]
    # the empty sequence hands its initial state through unchanged
    np.testing.assert_array_equal(fin[2], s0[2])


@pytest.mark.parametrize("dtype,C,seg", [("bf16", 16, 1), ("f32", 32, 2), ("bf16", 64, 3)])
def test_prefill_segments(kda, dtype, C, seg):
    """Short segments (1, 2 or 3 local chunks of every sequence per pass) make
    the prefill run as many intra/inter passes, each sequence's state carried
    between passes: packed sequences of different lengths finish in different
    segments, one is empty, and the final state is written over the initial
    state."""
    say(f"prefill segments dtype={dtype} C={C} segment={seg} chunks")
    lens = [37, 0, 130, 5, 200, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng([21, C])
    H = 2
    x = I.draw_tokens(rng, int(cu[-1]), H, 128, 128, dtype)
    s0 = I.draw_states(rng, len(lens), H, 128, 128)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    q, k, v, g, b = tok_to_dev(x)
    st = torch.from_numpy(s0.copy()).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    o, _ = kda.prefill(q, k, v, g, b, st, cud, cu_seqlens_host=cu, chunk_size=C, final_state=st,
                       options={"segment_chunks": seg})
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(st), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]
    np.testing.assert_array_equal(host(st)[1], s0[1])


def test_prefill_fixed_length_segments(kda):
    """B=3 equal sequences (no cu_seqlens) in segments of 2 chunks, fp32."""
    say("prefill fixed-length segments B=3")
    B, T, H = 3, 150, 2
    rng = np.random.default_rng(22)
    x = I.draw_tokens(rng, B * T, H, 64, 64, "f32")
    s0 = I.draw_states(rng, B, H, 64, 64)
    cu = np.arange(B + 1, dtype=np.int32) * T
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    q, k, v, g, b = tok_to_dev(x, B=B)
    o, fin = kda.prefill(q, k, v, g, b, torch.from_numpy(s0).to(DEV), chunk_size=32,
                         options={"segment_chunks": 2})
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o).reshape(B * T, H, 64), eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["f32"] and es_ <= TOL["f32"]


def test_prefill_workload1_full(kda):
    """B=1, H=32, T=4096, d=128, bf16, chunk 64: every output vs the oracle."""
    say("prefill workload 1 full")
    w = I.WORKLOADS[1]
    x = I.workload_tokens(w)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    o, fin = run_prefill(kda, x, 64)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]


def test_prefill_workload2_all_heads(kda):
    """16 packed sequences (68,645 tokens), H=32, initial states N(0, 0.1):
    every output and final state against the oracle, per tensor and per
    (sequence, head)."""
    say("prefill workload 2 (all heads)")
    w = I.WORKLOADS[2]
    cu = I.cu_seqlens_from_lengths(I.varlen_lengths(w))
    x = I.workload_tokens(w)
    s0 = I.workload_states(w, w.num_seqs)
    o, fin = run_prefill(kda, x, 64, s0=s0, cu=cu)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    po, ps = varlen_pair_rel(o, eo, cu), pair_rel(fin, ef, (0, 1))
    say(f"  o err {eo_:.2e} (per pair {po:.2e})  state err {es_:.2e} (per pair {ps:.2e})")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]
    assert po <= TOL["bf16"] and ps <= TOL["bf16"]


def test_prefill_workload1_per_pair(kda):
    """The T=4096, H=32 workload with a final state: the worst head."""
    say("prefill workload 1 per head")
    x = I.workload_tokens(I.WORKLOADS[1])
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    o, fin = run_prefill(kda, x, 64)
    po, ps = pair_rel(o, eo, (1,)), pair_rel(fin, ef, (0, 1))
    say(f"  per head: o {po:.2e}  state {ps:.2e}")
    assert po <= TOL["bf16"] and ps <= TOL["bf16"]


def test_prefill_bf16_output(kda):
    say("prefill bf16 output")
    rng = np.random.default_rng(13)
    x = I.draw_tokens(rng, 100, 2, 128, 128, "bf16")
    eo, _ = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    o, _ = run_prefill(kda, x, 64, out_dtype=torch.bfloat16)
    assert rel(o, eo) <= 8e-3


# --------------------------------------------------------------------------
# boundary semantics on the GPU
# --------------------------------------------------------------------------

def test_repeat_runs_bitwise_equal(kda):
    say("bitwise repeatability")
    rng = np.random.default_rng(14)
    x = I.draw_tokens(rng, 333, 4, 128, 128, "bf16")
    s0 = I.draw_states(rng, 1, 4, 128, 128)
    a = run_prefill(kda, x, 64, s0=s0)
    b = run_prefill(kda, x, 64, s0=s0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_split_resume_and_inplace_state(kda):
    say("split/resume")
    rng = np.random.default_rng(15)
    x = I.draw_tokens(rng, 300, 2, 128, 128, "bf16")
    o_full, f_full = run_prefill(kda, x, 64)
    o1, f1 = run_prefill(kda, x.slice(0, 100), 64)
    # resume with the state updated in place (final aliases initial)
    q, k, v, g, b = tok_to_dev(x.slice(100, 300))
    st = torch.from_numpy(f1).to(DEV)
    o2, f2 = kda.prefill(q, k, v, g, b, st, final_state=st, chunk_size=64)
    torch.cuda.synchronize()
    o_cat = np.concatenate([o1, host(o2)[0]])
    assert rel(o_cat, o_full) <= 1e-3 and rel(host(st), f_full) <= 1e-3


def test_decode_after_prefill_matches_oracle(kda):
    """Prefill a prompt, then generate with decode steps from its final state."""
    say("prefill then decode")
    rng = np.random.default_rng(16)
    x = I.draw_tokens(rng, 140, 2, 128, 128, "bf16")
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
    _, fin = run_prefill(kda, x.slice(0, 100), 64)
    st = torch.from_numpy(fin).to(DEV)
    worst = 0.0
    for t in range(100, 140):
        xs = x.slice(t, t + 1)
        q, k, v, g, b = (a[0] for a in tok_to_dev(xs))
        o = kda.decode_step(q, k, v, g, b, st)
        worst = max(worst, rel(host(o), eo[t:t + 1]))
    torch.cuda.synchronize()
    assert worst <= TOL["bf16"] and rel(host(st)[0], ef[0]) <= TOL["bf16"]


def test_empty_and_single_token(kda):
    say("T=0 and T=1")
    rng = np.random.default_rng(17)
    s0 = I.draw_states(rng, 1, 2, 64, 64)
    x = I.draw_tokens(rng, 1, 2, 64, 64, "f32")
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0)
    o, fin = run_prefill(kda, x, 16, s0=s0)
    assert rel(o, eo) <= 1e-5 and rel(fin, ef) <= 1e-5
    x0 = x.slice(0, 0)
    _, fin0 = run_prefill(kda, x0, 16, s0=s0)
    np.testing.assert_array_equal(fin0, s0)


# --------------------------------------------------------------------------
# Gated DeltaNet (scalar decay per token and head) through the same kernels
# --------------------------------------------------------------------------

def _scalar_gate(x, rng):
    """Replace the per-channel log-decay by one value per (token, head)."""
    T, H, Dk = x.g.shape
    gs = (-np.logaddexp(0.0, rng.standard_normal((T, H))) * 0.1).astype(np.float32)
    x.g = np.ascontiguousarray(np.repeat(gs[:, :, None], Dk, axis=2))
    return gs


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("f32", 16), ("bf16", 32)])
@pytest.mark.parametrize("vb", [16, 32])
def test_gdn_prefill_matches_oracle(kda, dtype, C, vb):
    """gdn_prefill (g [T, H]) equals the recurrence with g broadcast over the
    key channels: varlen packing, initial states, a ragged tail; 16 and 32
    value columns per carry-pass workgroup."""
    say(f"gdn prefill dtype={dtype} C={C} value_block={vb}")
    lens = [3 * C + 7, 0, 50, 2 * C]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng([23, C])
    H, D = 2, 128
    x = I.draw_tokens(rng, int(cu[-1]), H, D, D, dtype)
    gs = _scalar_gate(x, rng)
    s0 = I.draw_states(rng, len(lens), H, D, D)
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    q, k, v, _, b = tok_to_dev(x)
    g = torch.from_numpy(gs).to(DEV)[None]
    cud = torch.from_numpy(cu).to(DEV)
    o, fin = kda.prefill(q, k, v, g, b, torch.from_numpy(s0).to(DEV), cud, cu_seqlens_host=cu,
                         chunk_size=C, options={"value_block": vb})
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_gdn_decode_matches_oracle(kda, dtype, D):
    say(f"gdn decode dtype={dtype} D={D}")
    N, H, steps = 3, 2, 24
    rng = np.random.default_rng([24, D])
    x = I.draw_tokens(rng, N * steps, H, D, D, dtype)
    gs = _scalar_gate(x, rng)
    s0 = I.draw_states(rng, N, H, D, D)
    cu = np.arange(N + 1) * steps
    eo, ef = oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta, s0, cu_seqlens=cu)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    state = torch.from_numpy(s0.copy()).to(DEV)
    worst = 0.0
    for t in range(steps):
        rows = np.arange(N) * steps + t
        o = kda.decode_step(tdev(x.q[rows], dt), tdev(x.k[rows], dt), tdev(x.v[rows], dt),
                            tdev(gs[rows], torch.float32), tdev(x.beta[rows], torch.float32),
                            state)
        worst = max(worst, rel(host(o), eo[rows]))
    torch.cuda.synchronize()
    es = rel(host(state), ef)
    say(f"  o err {worst:.2e}  state err {es:.2e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]
