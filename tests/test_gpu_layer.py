"""Parity of the fused KDA layer entry points (kda_prefill_layer,
kda_decode_step_layer) with the float64 oracle's kda_layer: Swish + L2 norm of
q and k, Swish of v, sigmoid of beta, the recurrence, then the head-wise
RMSNorm times sigmoid(gate).

Error metric (per output tensor): max |x - y| / max |y|, with y the oracle.
Gates: 2e-3 for bf16 inputs, 1e-5 for fp32 inputs.
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
EPS = 1e-6


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


def tdev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).to(DEV) if dtype != torch.float32 else t.to(DEV)


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-30))


def host(t):
    return t.float().cpu().numpy()


def pair_rel(x, y, pair_axes):
    """Worst per-(sequence, head) error: max |x - y| / max |y| over the
    elements of each pair, then the maximum over pairs."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    red = tuple(a for a in range(x.ndim) if a not in pair_axes)
    num = np.abs(x - y).max(axis=red)
    den = np.maximum(np.abs(y).max(axis=red), 1e-30)
    return float((num / den).max())


def layer_to_dev(x: I.LayerInputs, lead=(1,)):
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    shp = lambda a: a.reshape(lead + a.shape[1:]) if len(lead) > 1 else a[None]
    f = lambda a, d: tdev(shp(a), d)
    return (f(x.q_pre, dt), f(x.k_pre, dt), f(x.v_pre, dt), f(x.g, torch.float32),
            f(x.beta_logit, torch.float32), f(x.gate, dt))


def oracle_layer(x, s0=None, cu=None, gate=True):
    return oracle.kda_layer(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit,
                            x.gate if gate else None, x.norm_weight, EPS,
                            initial_state=s0, cu_seqlens=cu)


@pytest.mark.parametrize("dtype,D,C,T,gate", [
    ("bf16", 128, 64, 300, True), ("f32", 64, 16, 131, True),
    ("bf16", 64, 32, 200, False), ("f32", 128, 64, 77, False),
    ("bf16", 128, 64, 1, True)])
def test_layer_prefill_matches_oracle(kda, dtype, D, C, T, gate):
    say(f"layer prefill dtype={dtype} D={D} C={C} T={T} gate={gate}")
    rng = np.random.default_rng([31, D, C, T])
    H = 3
    x = I.draw_layer_tokens(rng, T, H, D, D, dtype)
    s0 = I.draw_states(rng, 1, H, D, D)
    eo, ef = oracle_layer(x, s0, gate=gate)
    q, k, v, g, b, gt = layer_to_dev(x)
    o, fin = kda.layer_prefill(q, k, v, g, b, gt if gate else None,
                               tdev(x.norm_weight, torch.float32) if gate else None, EPS,
                               torch.from_numpy(s0).to(DEV), chunk_size=C)
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]


@pytest.mark.parametrize("seg", [None, 1])
def test_layer_prefill_varlen_segments(kda, seg):
    """Packed sequences (one empty) with the gated epilogue, in one pass or in
    segments of one local chunk each (the raw output buffer is reused by
    every segment)."""
    opts = None if seg is None else {"segment_chunks": seg}
    say(f"layer prefill varlen segments={seg}")
    lens = [37, 0, 130, 5, 200, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng([32, 0 if seg is None else seg])
    H, D = 2, 128
    x = I.draw_layer_tokens(rng, int(cu[-1]), H, D, D, "bf16")
    s0 = I.draw_states(rng, len(lens), H, D, D)
    eo, ef = oracle_layer(x, s0, cu=cu)
    q, k, v, g, b, gt = layer_to_dev(x)
    st = torch.from_numpy(s0.copy()).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    o, _ = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS, st, cud,
                             cu_seqlens_host=cu, chunk_size=64, final_state=st, options=opts)
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(st), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]
    np.testing.assert_array_equal(host(st)[1], s0[1])


def test_layer_prefill_strong_decay(kda):
    """Chunk decay far past exp(-40): the Grams take the pairwise path, which
    re-reads q and k and applies the prologue itself."""
    say("layer prefill strong decay")
    rng = np.random.default_rng(33)
    x = I.draw_layer_tokens(rng, 150, 2, 128, 128, "f32", g_scale=5.0)
    eo, ef = oracle_layer(x)
    q, k, v, g, b, gt = layer_to_dev(x)
    o, fin = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS,
                               chunk_size=64)
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["f32"] and es_ <= TOL["f32"]


@pytest.mark.parametrize("conv", [False, True])
def test_layer_prefill_bf16_output(kda, conv):
    """bf16 output against the oracle: one bf16 rounding of y can reach
    2^-9 of its magnitude, so the gate is 8e-3 (ungated mode)."""
    say(f"layer prefill bf16 output conv={conv}")
    rng = np.random.default_rng([34, int(conv)])
    T, H, D, W = 100, 2, 128, 4
    x = I.draw_layer_tokens(rng, T, H, D, D, "bf16")
    q, k, v, g, b, gt = layer_to_dev(x)
    w = tdev(x.norm_weight, torch.float32)
    if conv:
        ws, ss = I.draw_conv(rng, 1, H, D, W, "bf16")
        eo, _, _ = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                         x.gate, x.norm_weight, EPS)
        wd, sd = conv_to_dev(ws, ss, torch.bfloat16)
        o16, _, _ = kda.layer_prefill(q, k, v, g, b, gt, w, EPS, conv_weight=wd, conv_state=sd,
                                      chunk_size=64, out_dtype=torch.bfloat16)
    else:
        eo, _ = oracle_layer(x)
        o16, _ = kda.layer_prefill(q, k, v, g, b, gt, w, EPS, chunk_size=64,
                                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    e = rel(host(o16)[0], eo)
    say(f"  o err {e:.2e}")
    assert e <= 8e-3


def test_layer_prefill_full_size(kda):
    """The fused layer at B=1, H=32, T=4096, d=128, bf16, chunk 64, with the
    width-4 convolution from carried inputs, an initial state and the gated
    RMSNorm: every output, the final state and the carried inputs against the
    oracle, per tensor and per head."""
    say("layer prefill full size T=4096 H=32")
    rng = np.random.default_rng(40)
    T, H, D, W = 4096, 32, 128, 4
    x = I.draw_layer_tokens(rng, T, H, D, D, "bf16")
    s0 = I.draw_states(rng, 1, H, D, D)
    ws, ss = I.draw_conv(rng, 1, H, D, W, "bf16")
    eo, ef, ecs = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                        x.gate, x.norm_weight, EPS, s0)
    q, k, v, g, b, gt = layer_to_dev(x)
    wd, sd = conv_to_dev(ws, ss, torch.bfloat16)
    o, fin, cs = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS,
                                   torch.from_numpy(s0).to(DEV), conv_weight=wd, conv_state=sd,
                                   chunk_size=64)
    torch.cuda.synchronize()
    o, fin = host(o)[0], host(fin)
    eo_, es_ = rel(o, eo), rel(fin, ef)
    po, ps = pair_rel(o, eo, (1,)), pair_rel(fin, ef, (0, 1))
    say(f"  o err {eo_:.2e} (per head {po:.2e})  state err {es_:.2e} (per head {ps:.2e})")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]
    assert po <= TOL["bf16"] and ps <= TOL["bf16"]
    for a, e in zip(cs, ecs):
        np.testing.assert_array_equal(host(a), e.astype(np.float32))


@pytest.mark.parametrize("seg,out", [(1, "f32"), (2, "f32"), (2, "bf16"), (3, "bf16")])
def test_layer_prefill_segment_epilogues(kda, seg, out):
    """Fixed-length input (two sequences) in segments of 1-3 chunks with the
    convolution and the gated epilogue, whose raw output buffer every segment
    reuses.  Three calls in a row on a stream of the caller's own must give
    the same output each time, and every output and the final state match
    the oracle (bf16 output to its 8e-3 gate)."""
    say(f"layer prefill segment epilogues seg={seg} out={out}")
    rng = np.random.default_rng([42, seg])
    B, T, H, D, W = 2, 300, 3, 128, 4
    N = B
    cu = np.arange(B + 1, dtype=np.int32) * T
    x = I.draw_layer_tokens(rng, B * T, H, D, D, "bf16")
    s0 = I.draw_states(rng, N, H, D, D)
    ws, ss = I.draw_conv(rng, N, H, D, W, "bf16")
    eo, ef, _ = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                      x.gate, x.norm_weight, EPS, s0, cu)
    q, k, v, g, b, gt = layer_to_dev(x, lead=(B, T))
    wd, sd = conv_to_dev(ws, ss, torch.bfloat16)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    outs = []
    with torch.cuda.stream(side):
        for _ in range(3):
            o, fin, _ = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS,
                                          torch.from_numpy(s0).to(DEV), conv_weight=wd,
                                          conv_state=sd, chunk_size=64, out_dtype=odt,
                                          options={"segment_chunks": seg})
            outs.append((o.float().cpu().numpy(), fin.cpu().numpy()))
    side.synchronize()
    o0, f0 = outs[0]
    for o1, f1 in outs[1:]:
        np.testing.assert_array_equal(o1, o0)
        np.testing.assert_array_equal(f1, f0)
    eo_ = rel(o0.reshape(eo.shape), eo)
    es_ = rel(f0, ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= (8e-3 if out == "bf16" else TOL["bf16"]) and es_ <= TOL["bf16"]


@pytest.mark.parametrize("dtype,D,C", [(dt, D, C) for dt in ("bf16", "f32") for D in (64, 128)
                                       for C in (16, 32, 64)])
def test_layer_prefill_value_block_32(kda, dtype, D, C):
    """The layer path (raw output through the workspace, then the epilogue)
    with 32 value columns per carry-pass workgroup, for every (dtype, head
    size, chunk): packed sequences with a convolution and carried inputs."""
    say(f"layer prefill value_block=32 dtype={dtype} D={D} C={C}")
    lens = [2 * C + 3, 0, C, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, H, W = len(lens), 2, 4
    rng = np.random.default_rng([41, D, C])
    x = I.draw_layer_tokens(rng, int(cu[-1]), H, D, D, dtype)
    s0 = I.draw_states(rng, N, H, D, D)
    ws, ss = I.draw_conv(rng, N, H, D, W, dtype)
    eo, ef, _ = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                      x.gate, x.norm_weight, EPS, s0, cu)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, g, b, gt = layer_to_dev(x)
    wd, sd = conv_to_dev(ws, ss, dt)
    o, fin, _ = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS,
                                  torch.from_numpy(s0).to(DEV), torch.from_numpy(cu).to(DEV),
                                  conv_weight=wd, conv_state=sd, cu_seqlens_host=cu,
                                  chunk_size=C, options={"value_block": 32})
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]


@pytest.mark.parametrize("dtype,D,gate", [("bf16", 128, True), ("f32", 64, True),
                                          ("f32", 128, False), ("bf16", 64, False)])
def test_layer_decode_steps_match_oracle(kda, dtype, D, gate):
    say(f"layer decode dtype={dtype} D={D} gate={gate}")
    N, H, steps = 3, 2, 32
    rng = np.random.default_rng([35, D])
    x = I.draw_layer_tokens(rng, N * steps, H, D, D, dtype)
    s0 = I.draw_states(rng, N, H, D, D)
    cu = np.arange(N + 1) * steps
    eo, ef = oracle_layer(x, s0, cu=cu, gate=gate)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    state = torch.from_numpy(s0.copy()).to(DEV)
    w = tdev(x.norm_weight, torch.float32) if gate else None
    worst = 0.0
    for t in range(steps):
        rows = np.arange(N) * steps + t
        o = kda.layer_decode_step(tdev(x.q_pre[rows], dt), tdev(x.k_pre[rows], dt),
                                  tdev(x.v_pre[rows], dt), tdev(x.g[rows], torch.float32),
                                  tdev(x.beta_logit[rows], torch.float32), state,
                                  tdev(x.gate[rows], dt) if gate else None, w, EPS)
        worst = max(worst, rel(host(o), eo[rows]))
    torch.cuda.synchronize()
    es = rel(host(state), ef)
    say(f"  o err {worst:.2e}  state err {es:.2e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]


def test_layer_decode_continues_layer_prefill(kda):
    """A layer prefill's final state feeds layer decode steps; the outputs
    follow the oracle over the concatenated sequence.  (Slices are cloned:
    the C ABI wants 16-byte aligned tensors, and a one-token slice of beta
    is a contiguous view at an unaligned offset.)"""
    say("layer prefill then decode")
    rng = np.random.default_rng(36)
    T, H, D, steps = 130, 2, 128, 4
    x = I.draw_layer_tokens(rng, T + steps, H, D, D, "bf16")
    eo, ef = oracle_layer(x)
    q, k, v, g, b, gt = layer_to_dev(x)
    w = tdev(x.norm_weight, torch.float32)
    o, st = kda.layer_prefill(q[:, :T].clone(), k[:, :T].clone(),
                              v[:, :T].clone(), g[:, :T].clone(),
                              b[:, :T].clone(), gt[:, :T].clone(), w, EPS,
                              chunk_size=64)
    worst = rel(host(o)[0], eo[:T])
    for t in range(T, T + steps):
        od = kda.layer_decode_step(q[:, t].clone(), k[:, t].clone(),
                                   v[:, t].clone(), g[:, t].clone(),
                                   b[:, t].clone(), st, gt[:, t].clone(), w, EPS)
        worst = max(worst, rel(host(od)[0], eo[t]))
    torch.cuda.synchronize()
    es = rel(host(st), ef)
    say(f"  o err {worst:.2e}  state err {es:.2e}")
    assert worst <= TOL["bf16"] and es <= TOL["bf16"]


# --------------------------------------------------------------------------
# short convolution (causal, depthwise, carried inputs) in the prologue
# --------------------------------------------------------------------------

def conv_to_dev(ws, ss, dt):
    return (tuple(tdev(w, torch.float32) for w in ws),
            None if ss is None else tuple(tdev(s, dt) for s in ss))


@pytest.mark.parametrize("dtype,D,C,T,W,with_state", [
    ("bf16", 128, 64, 300, 4, True), ("f32", 64, 16, 131, 2, False),
    ("bf16", 64, 32, 70, 3, True), ("f32", 128, 64, 77, 1, False),
    ("bf16", 128, 64, 2, 4, True)])
def test_layer_prefill_conv_matches_oracle(kda, dtype, D, C, T, W, with_state):
    say(f"layer prefill conv dtype={dtype} D={D} C={C} T={T} W={W} state={with_state}")
    rng = np.random.default_rng([37, D, C, T, W])
    H = 3
    x = I.draw_layer_tokens(rng, T, H, D, D, dtype)
    s0 = I.draw_states(rng, 1, H, D, D)
    ws, ss = I.draw_conv(rng, 1, H, D, W, dtype)
    ss = ss if with_state else None
    eo, ef, ecs = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                        x.gate, x.norm_weight, EPS, s0)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, g, b, gt = layer_to_dev(x)
    wd, sd = conv_to_dev(ws, ss, dt)
    o, fin, cs = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS,
                                   torch.from_numpy(s0).to(DEV), conv_weight=wd, conv_state=sd,
                                   chunk_size=C)
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL[dtype] and es_ <= TOL[dtype]
    for a, e in zip(cs, ecs):  # carried inputs are copies: bit-exact
        np.testing.assert_array_equal(host(a), e.astype(np.float32))


@pytest.mark.parametrize("seg", [None, 1])
def test_layer_prefill_conv_varlen_in_place(kda, seg):
    """Packed sequences, some shorter than the convolution's reach (0, 1 and
    2 tokens), carried inputs and recurrent state updated in place, in one
    pass or in one-chunk segments."""
    opts = None if seg is None else {"segment_chunks": seg}
    say(f"layer prefill conv varlen in place segments={seg}")
    lens = [37, 0, 130, 1, 200, 2, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, H, D, W = len(lens), 2, 128, 4
    rng = np.random.default_rng([38, 0 if seg is None else seg])
    x = I.draw_layer_tokens(rng, int(cu[-1]), H, D, D, "bf16")
    s0 = I.draw_states(rng, N, H, D, D)
    ws, ss = I.draw_conv(rng, N, H, D, W, "bf16")
    eo, ef, ecs = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                        x.gate, x.norm_weight, EPS, s0, cu)
    q, k, v, g, b, gt = layer_to_dev(x)
    wd, sd = conv_to_dev(ws, ss, torch.bfloat16)
    st = torch.from_numpy(s0.copy()).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    o, _, cs = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS, st,
                                 cud, conv_weight=wd, conv_state=sd, conv_state_out=sd,
                                 cu_seqlens_host=cu, chunk_size=64, final_state=st, options=opts)
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(st), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["bf16"] and es_ <= TOL["bf16"]
    for a, e in zip(sd, ecs):
        np.testing.assert_array_equal(host(a), e.astype(np.float32))


def test_layer_prefill_conv_strong_decay(kda):
    """The pairwise Gram path convolves q and k itself."""
    say("layer prefill conv strong decay")
    rng = np.random.default_rng(39)
    T, H, D, W = 150, 2, 128, 4
    x = I.draw_layer_tokens(rng, T, H, D, D, "f32", g_scale=5.0)
    ws, ss = I.draw_conv(rng, 1, H, D, W, "f32")
    eo, ef, _ = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                      x.gate, x.norm_weight, EPS)
    q, k, v, g, b, gt = layer_to_dev(x)
    wd, sd = conv_to_dev(ws, ss, torch.float32)
    o, fin, _ = kda.layer_prefill(q, k, v, g, b, gt, tdev(x.norm_weight, torch.float32), EPS,
                                  conv_weight=wd, conv_state=sd, chunk_size=64)
    torch.cuda.synchronize()
    eo_, es_ = rel(host(o)[0], eo), rel(host(fin), ef)
    say(f"  o err {eo_:.2e}  state err {es_:.2e}")
    assert eo_ <= TOL["f32"] and es_ <= TOL["f32"]


@pytest.mark.parametrize("dtype,D,W", [("bf16", 128, 4), ("f32", 64, 3), ("bf16", 64, 1)])
def test_layer_decode_conv_matches_oracle(kda, dtype, D, W):
    """Decode steps with the convolution: its carried inputs and the state
    are updated in place, step after step."""
    say(f"layer decode conv dtype={dtype} D={D} W={W}")
    N, H, steps = 3, 2, 24
    rng = np.random.default_rng([40, D, W])
    x = I.draw_layer_tokens(rng, N * steps, H, D, D, dtype)
    s0 = I.draw_states(rng, N, H, D, D)
    ws, ss = I.draw_conv(rng, N, H, D, W, dtype)
    cu = np.arange(N + 1) * steps
    eo, ef, ecs = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, ss,
                                        x.gate, x.norm_weight, EPS, s0, cu)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    state = torch.from_numpy(s0.copy()).to(DEV)
    wd, sd = conv_to_dev(ws, ss, dt)
    w = tdev(x.norm_weight, torch.float32)
    worst = 0.0
    for t in range(steps):
        rows = np.arange(N) * steps + t
        o = kda.layer_decode_step(tdev(x.q_pre[rows], dt), tdev(x.k_pre[rows], dt),
                                  tdev(x.v_pre[rows], dt), tdev(x.g[rows], torch.float32),
                                  tdev(x.beta_logit[rows], torch.float32), state,
                                  tdev(x.gate[rows], dt), w, EPS, conv_weight=wd, conv_state=sd)
        worst = max(worst, rel(host(o), eo[rows]))
    torch.cuda.synchronize()
    es = rel(host(state), ef)
    say(f"  o err {worst:.2e}  state err {es:.2e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]
    for a, e in zip(sd, ecs):
        np.testing.assert_array_equal(host(a), e.astype(np.float32))


def test_layer_conv_decode_continues_prefill(kda):
    """Prefill with the convolution hands both states to decode steps."""
    say("layer conv prefill then decode")
    rng = np.random.default_rng(41)
    T, H, D, W, steps = 130, 2, 128, 4, 5
    x = I.draw_layer_tokens(rng, T + steps, H, D, D, "bf16")
    ws, _ = I.draw_conv(rng, 1, H, D, W, "bf16")
    eo, ef, ecs = oracle.kda_layer_conv(x.q_pre, x.k_pre, x.v_pre, x.g, x.beta_logit, ws, None,
                                        x.gate, x.norm_weight, EPS)
    q, k, v, g, b, gt = layer_to_dev(x)
    wd, _ = conv_to_dev(ws, None, torch.bfloat16)
    w = tdev(x.norm_weight, torch.float32)
    o, st, cs = kda.layer_prefill(q[:, :T].clone(), k[:, :T].clone(), v[:, :T].clone(),
                                  g[:, :T].clone(), b[:, :T].clone(), gt[:, :T].clone(), w, EPS,
                                  conv_weight=wd, chunk_size=64)
    worst = rel(host(o)[0], eo[:T])
    for t in range(T, T + steps):
        od = kda.layer_decode_step(q[:, t].clone(), k[:, t].clone(), v[:, t].clone(),
                                   g[:, t].clone(), b[:, t].clone(), st, gt[:, t].clone(), w, EPS,
                                   conv_weight=wd, conv_state=cs)
        worst = max(worst, rel(host(od)[0], eo[t]))
    torch.cuda.synchronize()
    es = rel(host(st), ef)
    say(f"  o err {worst:.2e}  state err {es:.2e}")
    assert worst <= TOL["bf16"] and es <= TOL["bf16"]
    for a, e in zip(cs, ecs):
        np.testing.assert_array_equal(host(a), e.astype(np.float32))
