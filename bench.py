"""KDA benchmark on one MI355X: chunked prefill tokens/s and decode-step GB/s.

One step = one pass of the whole hot path on synthetic resident inputs:
  * kda_prefill on B=1, H=32, T=4096, d_k=d_v=128, bf16 q/k/v, fp32 g/beta,
    chunk 64, fp32 output and final state (the prefill workload);
  * kda_decode_step on 256 sequences x 32 heads, d=128, fp32 state
    [256, 32, 128, 128] (the decode workload), one token per sequence.
Three prefill input sets and two decode input sets rotate so the 256 MB
Infinity Cache cannot hold a step's working set.

Prints ONE JSON line.  ``value`` is prefill tokens/s; the decode rate and the
per-call times are in ``decode`` / ``prefill``.  ``roofline`` describes the
unit that takes the most time per step (decided from the measured times): the
kda_prefill call (its intra- and inter-chunk launches) or the decode kernel;
``prefill_roofline`` gives the prefill call against HBM and bf16-MFMA peaks.
``copy`` is a 1 GiB device-to-device copy timed in the same process: a
measured bandwidth reference, and the kernel the HBM byte counters are
calibrated on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

# Workload sizes (see gated_delta_rule_56_amd/inputs.py WORKLOADS[1] and [4]).
P_T, P_H, P_D, P_C = 4096, 32, 128, 64
D_N, D_H, D_D = 256, 32, 128
COPY_BYTES, COPY_REPS = 1 << 30, 5


def prefill_algorithmic_bytes(T=P_T, H=P_H, d=P_D):
    # q, k, v bf16 + g fp32 + beta fp32 + o fp32 per token-head, + final state.
    return T * H * (3 * 2 * d + 4 * d + 4 + 4 * d) + H * d * d * 4


def prefill_flops(T=P_T, H=P_H, d=P_D, C=P_C):
    # Per-head chunked-KDA FLOPs, 6Td^2 + 3TCd + TC^2 (zeroshot.it.com
    # deep-dive, section 4; greeksharifa summary, section 6.3).
    return H * (6 * T * d * d + 3 * T * C * d + T * C * C)


def decode_algorithmic_bytes(N=D_N, H=D_H, d=D_D):
    # state read + write (fp32), q/k/v bf16, g fp32, beta fp32, o fp32.
    return N * H * (2 * d * d * 4 + 3 * 2 * d + 4 * d + 4 + 4 * d)


# HBM bytes per call measured with rocprofv3 FETCH_SIZE and WRITE_SIZE (one
# run each) on the command in profiles/hbm_traffic.md, each counter scaled by
# the ratio of known bytes to counted bytes for the 1 GiB copy in the same
# run.  A figure is reported only while the kernel sources still hash to the
# values it was measured on.
TRAFFIC = {
    "prefill": {"sources": "62e4a8e1274804fd", "bytes": 836423680},
    "decode": {"sources": "59534d0a63d13012", "bytes": 1089116640},
}


def sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_56_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# The files that define the measured kernels (launch arguments are plain
# structs declared elsewhere and do not change the kernels' memory traffic).
PREFILL_SOURCES = ("kda_prefill.hip", "kda_device.hpp")
DECODE_SOURCES = ("kda_decode.hip", "kda_device.hpp")


def measured_traffic(unit, names):
    t = TRAFFIC.get(unit)
    if t is None or t["sources"] != sources_digest(names):
        return None
    return t["bytes"]


def prefill_bytes_general(tokens, H, d, num_seqs, states_in, states_out):
    return tokens * H * (3 * 2 * d + 4 * d + 4 + 4 * d) + num_seqs * H * d * d * 4 * (
        int(states_in) + int(states_out))


def prefill_flops_general(tokens, H, d, C):
    return H * (6 * tokens * d * d + 3 * tokens * C * d + tokens * C * C)


def time_prefill(torch, kda, args, reps, **kw):
    """Mean time (s) of kda.prefill over ``reps`` calls after one warm-up,
    with the output, final state and workspace allocated once."""
    q = args[0]
    kda.prefill(*args, **kw)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        kda.prefill(*args, **kw)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps / 1e3


def other_workloads(torch, kda, I, dev):
    """Throughput on the other synthetic workloads (secondary to ``value``)."""
    out = {}
    # varlen: 16 packed sequences, lengths U[512, 8192], initial states
    w = I.WORKLOADS[2]
    cu = I.cu_seqlens_from_lengths(I.varlen_lengths(w))
    n_tok, N = int(cu[-1]), len(cu) - 1
    q, k, v, g, b = I.device_tokens(torch, n_tok, w.H, w.Dk, w.Dv, 2002, dev)
    s0 = torch.from_numpy(I.workload_states(w, N)).to(dev)
    cud = torch.from_numpy(cu).to(dev)
    fin = torch.empty_like(s0)
    o = torch.empty((1, n_tok, w.H, w.Dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(1, n_tok, w.H, w.Dk, N, 64, kda.KDA_BF16, cu),
                     dtype=torch.uint8, device=dev)
    t = time_prefill(torch, kda, (q, k, v, g, b, s0, cud), 3, cu_seqlens_host=cu, chunk_size=64,
                     o=o, final_state=fin, workspace=ws)
    by = prefill_bytes_general(n_tok, w.H, w.Dk, N, True, True)
    out["varlen"] = {"workload": f"kda_prefill 16 packed sequences ({n_tok} tokens), H=32, d=128, "
                                 "chunk 64, bf16 in / fp32 out, initial and final states",
                     "ms_per_call": round(t * 1e3, 3), "tokens_per_s": round(n_tok / t, 1),
                     "algorithmic_GBps": round(by / t / 1e9, 1),
                     "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_frac_bf16": round(prefill_flops_general(n_tok, w.H, w.Dk, 64) / t / 1e12
                                             / BF16_PEAK_TFLOPS, 4)}
    del q, k, v, g, b, o, ws, fin
    torch.cuda.empty_cache()
    # mixed decay: the T=4096, H=32 workload with half the key channels of
    # every head at alpha near 0.1 per token (and near 0.01, where the
    # diagonal Gram blocks of those tiles are evaluated pair by pair), timed
    # beside the workload itself
    mixed = {}
    for alpha in (0.1, 0.01):
        rng = np.random.default_rng([5, int(round(-np.log10(alpha)))])
        x = I.draw_mixed_decay_tokens(rng, P_T, P_H, P_D, P_D, "bf16", alpha=alpha)
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)[None]
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)[None]
        args = (bf(x.q), bf(x.k), bf(x.v), f32(x.g), f32(x.beta), None)
        t = time_prefill(torch, kda, args, 10, chunk_size=P_C)
        mixed[f"alpha_{alpha}_us_per_call"] = round(t * 1e6, 2)
    x = I.workload_tokens(I.WORKLOADS[1])
    args = (bf(x.q), bf(x.k), bf(x.v), f32(x.g), f32(x.beta), None)
    t0 = time_prefill(torch, kda, args, 10, chunk_size=P_C)
    mixed["workload_us_per_call"] = round(t0 * 1e6, 2)
    for alpha in (0.1, 0.01):
        mixed[f"alpha_{alpha}_over_workload"] = round(mixed[f"alpha_{alpha}_us_per_call"] / 1e6 / t0, 3)
    out["mixed_decay"] = {"workload": "kda_prefill B=1 H=32 T=4096 d=128 chunk 64 bf16, half of the "
                                      "key channels at alpha near 0.1 (or 0.01) per token", **mixed}
    # long context: one sequence of 1,048,576 tokens
    w = I.WORKLOADS[3]
    q, k, v, g, b = I.device_tokens(torch, w.T, w.H, w.Dk, w.Dv, 3003, dev)
    o = torch.empty((1, w.T, w.H, w.Dv), dtype=torch.float32, device=dev)
    fin = torch.empty((1, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(1, w.T, w.H, w.Dk, 1, 64, kda.KDA_BF16),
                     dtype=torch.uint8, device=dev)
    t = time_prefill(torch, kda, (q, k, v, g, b, None), 2, chunk_size=64, o=o, final_state=fin,
                     workspace=ws)
    by = prefill_bytes_general(w.T, w.H, w.Dk, 1, False, True)
    out["long_context"] = {"workload": "kda_prefill B=1 H=32 T=1,048,576 d=128 chunk 64, bf16 in / "
                                       "fp32 out, final state",
                           "ms_per_call": round(t * 1e3, 3), "tokens_per_s": round(w.T / t, 1),
                           "algorithmic_GBps": round(by / t / 1e9, 1),
                           "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                           "workspace_bytes": int(ws.numel())}
    del q, k, v, g, b, o, ws, fin
    torch.cuda.empty_cache()
    # tiny fp32 case (launch-bound; chunk 16 and 64)
    w = I.WORKLOADS[0]
    x = I.workload_tokens(w)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)[None]
    args = (f32(x.q), f32(x.k), f32(x.v), f32(x.g), f32(x.beta), None)
    tiny = {}
    for C in (16, 64):
        t = time_prefill(torch, kda, args, 20, chunk_size=C)
        tiny[f"chunk{C}_us_per_call"] = round(t * 1e6, 2)
        tiny[f"chunk{C}_tokens_per_s"] = round(w.T / t, 1)
    out["tiny_fp32"] = {"workload": "kda_prefill B=1 H=1 T=256 d=64 fp32", **tiny}
    out["layer"] = layer_workloads(torch, kda, I, dev)
    out["backward"] = backward_workload(torch, kda, I, dev)
    out["dplr"] = dplr_workloads(torch, kda, I, dev)
    return out


def dplr_workloads(torch, kda, I, dev):
    """General DPLR against KDA on the same KDA inputs (a = beta k,
    b = exp(g) k): dplr_prefill (four intra-chunk matrices), KDA through the
    same fp32 chunk pipeline (kda_prefill_chunk_fp32, two matrices) and the
    optimized kda_prefill.  B=1, 16 heads (the setting of the pages' kernel
    comparison) at 4K and 64K tokens, and the headline 32-head 4K shape."""
    res = []
    for T, H in ((4096, 16), (65536, 16), (4096, 32)):
        d = P_D
        q, k, v, g, b = I.device_tokens(torch, T, H, d, d, 6006 + T + H, dev)
        a = (b[..., None] * k.float()).to(torch.bfloat16)
        bb = (torch.exp(g) * k.float()).to(torch.bfloat16)
        o = torch.empty((1, T, H, d), dtype=torch.float32, device=dev)
        fin = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
        ws = torch.empty(kda.dplr_workspace_size(1, T, H, d, 1, P_C), dtype=torch.uint8,
                         device=dev)
        reps = 3 if T > 8192 else 10
        t_dplr = time_calls(torch, lambda: kda.dplr_prefill(q, a, v, a, bb, g, None, chunk_size=P_C,
                                                            o=o, final_state=fin, workspace=ws),
                            reps)
        t_tied = time_calls(torch, lambda: kda.prefill_chunk_fp32(q, k, v, g, b, None,
                                                                  chunk_size=P_C, o=o,
                                                                  final_state=fin, workspace=ws),
                            reps)
        del ws
        ws2 = torch.empty(kda.workspace_size(1, T, H, d, 1, P_C, kda.KDA_BF16), dtype=torch.uint8,
                          device=dev)
        t_kda = time_calls(torch, lambda: kda.prefill(q, k, v, g, b, None, chunk_size=P_C, o=o,
                                                      final_state=fin, workspace=ws2), reps)
        res.append({"T": T, "H": H, "d": d, "dplr_ms": round(t_dplr * 1e3, 3),
                    "kda_chunk_fp32_ms": round(t_tied * 1e3, 3),
                    "kda_prefill_ms": round(t_kda * 1e3, 3),
                    "dplr_over_kda_same_pipeline": round(t_dplr / t_tied, 2),
                    "dplr_over_kda_prefill": round(t_dplr / t_kda, 2)})
        del q, k, v, g, b, a, bb, o, fin, ws2
        torch.cuda.empty_cache()
    # one general DPLR decode step on the decode workload's shape
    N, H, d = D_N, D_H, D_D
    qd, kd, vd, ad, bd = (torch.randn((N, H, d), device=dev).to(torch.bfloat16) for _ in range(5))
    gd = -torch.nn.functional.softplus(torch.randn((N, H, d), device=dev)) * 0.1
    st = torch.randn((N, H, d, d), device=dev) * 0.1
    od = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    t = time_calls(torch, lambda: kda.dplr_decode_step(qd, kd, vd, ad, bd, gd, st, o=od), 20)
    by = N * H * (2 * d * d * 4 + 5 * 2 * d + 4 * d + 4 * d)
    dec = {"workload": f"dplr_decode_step N={N} H={H} d={d}, bf16 in / fp32 out",
           "us_per_step": round(t * 1e6, 2), "GBps": round(by / t / 1e9, 1),
           "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    return {"workload": "general DPLR vs KDA on the same inputs, bf16, chunk 64", "cases": res,
            "decode": dec}


def backward_workload(torch, kda, I, dev):
    """kda_backward on the headline prefill shape, initial state and
    final-state gradient included."""
    T, H, d = P_T, P_H, P_D
    q, k, v, g, b = I.device_tokens(torch, T, H, d, d, 5005, dev)
    do = torch.randn((1, T, H, d), device=dev)
    s0 = torch.randn((1, H, d, d), device=dev) * 0.1
    dF = torch.randn((1, H, d, d), device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = (torch.empty((1, T, H, d), **f32), torch.empty((1, T, H, d), **f32),
            torch.empty((1, T, H, d), **f32), torch.empty((1, T, H, d), **f32),
            torch.empty((1, T, H), **f32), torch.empty((1, H, d, d), **f32))
    ws = torch.empty(kda.backward_workspace_size(1, T, H, d, 1, P_C), dtype=torch.uint8,
                     device=dev)
    t = time_calls(torch, lambda: kda.backward(q, k, v, g, b, do, s0, dF, chunk_size=P_C,
                                               workspace=ws, out=outs), 5)
    # inputs q, k, v bf16, g, beta, d_o fp32; outputs dq, dk, dv, dg, dbeta
    # fp32; initial state, final-state gradient and its result
    by = T * H * (3 * 2 * d + 4 * d + 4 + 4 * d + 4 * 4 * d + 4) + 3 * H * d * d * 4
    # the same with half the key channels decaying at alpha near 0.1 per token
    rng = np.random.default_rng(5006)
    x = I.draw_mixed_decay_tokens(rng, T, H, d, d, "bf16", alpha=0.1)
    qm, km, vm = (torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)[None]
                  for a in (x.q, x.k, x.v))
    gm, bm = (torch.from_numpy(np.ascontiguousarray(a)).to(dev)[None] for a in (x.g, x.beta))
    tm = time_calls(torch, lambda: kda.backward(qm, km, vm, gm, bm, do, s0, dF, chunk_size=P_C,
                                                workspace=ws, out=outs), 3)
    return {"workload": f"kda_backward B=1 H={H} T={T} d={d} chunk {P_C}, bf16 q/k/v, fp32 "
                        "gradients, initial state and final-state gradient",
            "ms_per_call": round(t * 1e3, 3), "tokens_per_s": round(T / t, 1),
            "algorithmic_GBps": round(by / t / 1e9, 1),
            "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "workspace_bytes": int(ws.numel()),
            "mixed_decay_alpha_0.1_ms_per_call": round(tm * 1e3, 3),
            "mixed_decay_over_workload": round(tm / t, 3)}


def layer_workloads(torch, kda, I, dev):
    """The fused layer entry points on the headline shapes: prologue (short
    convolution of width 4, Swish, L2 norm, sigmoid) and gated RMSNorm
    epilogue in the kernels."""
    T, H, d, N = P_T, P_H, P_D, D_N
    # two input sets, alternated, so the inputs do not stay in the Infinity Cache
    sets = [I.device_layer_tokens(torch, T, H, d, d, 4004 + i, dev) for i in range(2)]
    w = sets[0][6]
    o = torch.empty((1, T, H, d), dtype=torch.float32, device=dev)
    fin = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(1, T, H, d, 1, P_C, kda.KDA_BF16, layer_gate=True),
                     dtype=torch.uint8, device=dev)
    calls = [0]
    W = 4
    cw = tuple(torch.randn((H, d, W), device=dev) / W ** 0.5 for _ in range(3))
    cs = tuple(torch.randn((1, H, W - 1, d), device=dev).to(torch.bfloat16) for _ in range(3))
    cs_out = tuple(torch.empty_like(c) for c in cs)

    def run():
        q, k, v, gate, g, b, _ = sets[calls[0] % 2]
        calls[0] += 1
        kda.layer_prefill(q, k, v, g, b, gate, w, 1e-6, chunk_size=P_C, o=o, final_state=fin,
                          workspace=ws, conv_weight=cw, conv_state=cs, conv_state_out=cs_out)

    t = time_calls(torch, run, 20)
    # q, k, v, gate bf16 + g fp32 + beta fp32 + o fp32 per token-head, + final state
    by = T * H * (4 * 2 * d + 4 * d + 4 + 4 * d) + H * d * d * 4 + d * 4
    res = {"prefill_workload": f"kda_prefill_layer B=1 H={H} T={T} d={d} chunk {P_C}, bf16 in / "
                               "fp32 out, short convolution W=4, gated RMSNorm epilogue, "
                               "final state",
           "prefill_us_per_call": round(t * 1e6, 2), "prefill_tokens_per_s": round(T / t, 1),
           "prefill_algorithmic_GBps": round(by / t / 1e9, 1)}
    del sets, o, fin, ws
    qd, kd, vd, gd, gtd, bd = (torch.randn((N, H, d), device=dev).to(torch.bfloat16)
                               for _ in range(6))
    gd = -torch.nn.functional.softplus(gd.float()) * 0.1
    bd = torch.randn((N, H), device=dev)
    st = torch.randn((N, H, d, d), device=dev) * 0.1
    od = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    csd = tuple(torch.randn((N, H, W - 1, d), device=dev).to(torch.bfloat16) for _ in range(3))
    t = time_calls(torch, lambda: kda.layer_decode_step(qd, kd, vd, gd, bd, st, gtd, w, 1e-6,
                                                         conv_weight=cw, conv_state=csd,
                                                         o=od), 20)
    by = N * H * (2 * d * d * 4 + 4 * 2 * d + 4 * d + 4 + 4 * d) + d * 4
    res.update({"decode_workload": f"kda_decode_step_layer N={N} H={H} d={d}, bf16 in / fp32 out, "
                                   "short convolution W=4, gated RMSNorm epilogue",
                "decode_us_per_step": round(t * 1e6, 2), "decode_GBps": round(by / t / 1e9, 1),
                "decode_hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)})
    return res


def time_calls(torch, fn, reps, warm_s=0.05):
    """Mean time (s) of ``fn()`` over ``reps`` calls, after warm-up calls
    for at least ``warm_s`` seconds (at least one): the GPU runs slower for
    a while after it has been idle, e.g. while the host drew the inputs."""
    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_s:
            break
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps / 1e3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(min_seconds=10.0, max_reps=200):
    """The float64 oracle on the host cores, on the whole prefill workload,
    repeated until about ``min_seconds`` of CPU work have been timed."""
    import oracle
    from gated_delta_rule_56_amd import inputs as I
    x = I.workload_tokens(I.WORKLOADS[1])
    reps, t = 0, 0.0
    while reps < max_reps and (t < min_seconds or reps == 0):
        t0 = time.perf_counter()
        oracle.kda_recurrent(x.q, x.k, x.v, x.g, x.beta)
        t += time.perf_counter() - t0
        reps += 1
    return {"value": reps * P_T / t, "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"whole prefill workload (B=1, H=32, T=4096, d=128), {reps} pass(es), "
                      f"float64 token-by-token recurrence, {t:.1f} s",
            "cpu": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # A fresh process runs the first few dozen steps slower (the prefill at
    # 256 us after 5 warm-up steps, 217 us after 100, 215 us after 300), so
    # the default warms up to the steady state before timing.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the secondary varlen / long-context / tiny measurements")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every configuration here fits one MI355X "
              "and this build has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_56_amd import inputs as I
    from gated_delta_rule_56_amd import kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load()

    # ---- resident inputs ----
    log("generating prefill inputs")
    wp = I.WORKLOADS[1]
    psets = []
    for s in range(3):
        rng = np.random.default_rng([wp.wid, 1, 1000 + s]) if s else None
        x = I.workload_tokens(wp) if s == 0 else I.draw_tokens(rng, P_T, P_H, P_D, P_D, "bf16")
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)[None]
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)[None]
        psets.append((bf(x.q), bf(x.k), bf(x.v), f32(x.g), f32(x.beta)))
    o = torch.empty((1, P_T, P_H, P_D), dtype=torch.float32, device=dev)
    fin = torch.empty((1, P_H, P_D, P_D), dtype=torch.float32, device=dev)
    ws_bytes = kda.workspace_size(1, P_T, P_H, P_D, 1, P_C, kda.KDA_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    log("generating decode inputs")
    wd = I.WORKLOADS[4]
    state = torch.from_numpy(I.draw_states(np.random.default_rng([4, 2]), D_N, D_H, D_D, D_D)).to(dev)
    dsets = []
    for s in range(2):
        x = I.decode_step_inputs(wd, s)
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        dsets.append((bf(x.q), bf(x.k), bf(x.v), f32(x.g), f32(x.beta)))
    od = torch.empty((D_N, D_H, D_D), dtype=torch.float32, device=dev)
    copy_src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    copy_dst = torch.empty_like(copy_src)
    torch.cuda.synchronize()

    def step(i, ev=None):
        q, k, v, g, b = psets[i % 3]
        if ev is not None:
            ev[0].record()
        kda.prefill(q, k, v, g, b, None, chunk_size=P_C, o=o, final_state=fin, workspace=ws)
        if ev is not None:
            ev[1].record()
        q, k, v, g, b = dsets[i % 2]
        kda.decode_step(q, k, v, g, b, state, o=od)
        if ev is not None:
            ev[2].record()

    log("warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    total_ms = start.elapsed_time(stop)
    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    # 1 GiB device copy: read + write bytes over the median time
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(COPY_REPS)]
    copy_dst.copy_(copy_src)
    for a, b in cev:
        a.record()
        copy_dst.copy_(copy_src)
        b.record()
    torch.cuda.synchronize()
    copy_s = float(np.median([a.elapsed_time(b) for a, b in cev])) / 1e3
    copy_gbs = 2 * COPY_BYTES / copy_s / 1e9

    pre_s = pre_ms.mean() / 1e3
    dec_s = dec_ms.mean() / 1e3
    p_bytes, p_flops = prefill_algorithmic_bytes(), prefill_flops()
    d_bytes = decode_algorithmic_bytes()
    prefill_tok_s = P_T / pre_s
    dec_gbs = d_bytes / dec_s / 1e9

    decode_roof = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic("decode", DECODE_SOURCES),
                   "kernel": "decode_step_kernel", "bytes_per_launch": d_bytes,
                   "frac_of_measured_copy": round(dec_gbs / copy_gbs, 4)}
    p_gbs = p_bytes / pre_s / 1e9
    p_tfl = p_flops / pre_s / 1e12
    prefill_roof = {"bound": "hbm", "achieved": round(p_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(p_gbs / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("prefill", PREFILL_SOURCES),
                    "kernels": "intra_chunk_kernel + inter_chunk_kernel per segment "
                               "(one kda_prefill call)",
                    "bytes_per_call": p_bytes, "flops_per_call": p_flops,
                    "mfma_tflops": round(p_tfl, 2),
                    "mfma_frac_bf16": round(p_tfl / BF16_PEAK_TFLOPS, 4),
                    "frac_of_measured_copy": round(p_gbs / copy_gbs, 4)}
    roof = decode_roof if dec_s >= pre_s else prefill_roof

    others = None
    if not args.no_other_workloads:
        log("timing the other workloads")
        others = other_workloads(torch, kda, I, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline()

    line = {
        "metric": "KDA prefill tokens/s (H=32, d=128) + decode-step HBM GB/s, 1 MI355X",
        "value": round(prefill_tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_prefill B=1 H=32 T=4096 d=128 chunk=64 bf16 in / fp32 out "
                               "+ kda_decode_step N=256 H=32 d=128 fp32 state",
                   "prefill": {"B": 1, "H": P_H, "T": P_T, "d": P_D, "chunk": P_C},
                   "decode": {"N": D_N, "H": D_H, "d": D_D}},
        "prefill": {"us_per_call": round(pre_s * 1e6, 2), "tokens_per_s": round(prefill_tok_s, 1),
                    "algorithmic_GBps": round(p_gbs, 1), "algorithmic_TFLOPs": round(p_tfl, 3)},
        "decode": {"us_per_step": round(dec_s * 1e6, 2), "GBps": round(dec_gbs, 1),
                   "tokens_per_s": round(D_N / dec_s, 1), "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4)},
        "copy": {"bytes_moved": 2 * COPY_BYTES, "us": round(copy_s * 1e6, 1),
                 "GBps": round(copy_gbs, 1)},
        "roofline": roof,
        "prefill_roofline": prefill_roof,
        "decode_roofline": decode_roof,
        "cpu_baseline": cpu,
        "other_workloads": others,
        "wall_s_timed_region": round(t_wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
