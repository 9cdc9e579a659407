"""Long-context prefill: B=1, H=32, T=1,048,576, d=128, bf16, chunk 64.

The sequence is drawn in 4096-token blocks (each with its own seed).  The GPU
runs the whole sequence in one call.  The oracle carries the state of eight
sampled heads (a quarter of them, spread over the head range) through all
1,048,576 tokens from a zero state, in 65,536-token pieces whose final state
starts the next piece (the same arithmetic as one call).  The GPU output is
compared on the first and last 4096-token windows, plus the final state of
those heads, per tensor and per head.  Eight heads keep the host copies at
2 GiB and the oracle's float64 pieces under 0.5 GiB.
"""
import os
import sys
import time

import numpy as np
import pytest

import oracle
from gated_delta_rule_56_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

HEADS = (0, 4, 9, 13, 18, 22, 27, 31)
PIECE = 65536


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def test_prefill_workload3_long_windows():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import kda
    kda.load()
    w = I.WORKLOADS[3]
    T, H, D, B = w.T, w.H, w.Dk, 4096
    nblk = T // B
    dev = "cuda:0"
    say(f"long prefill T={T}: allocating device inputs")
    q = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    g = torch.empty((1, T, H, D), dtype=torch.float32, device=dev)
    beta = torch.empty((1, T, H), dtype=torch.float32, device=dev)
    hs = list(HEADS)
    hq = np.empty((T, len(hs), D), np.float32)
    hk, hv, hg = np.empty_like(hq), np.empty_like(hq), np.empty_like(hq)
    hb = np.empty((T, len(hs)), np.float32)
    t0 = time.time()
    for b, x in I.long_blocks(w, range(nblk), B, workers=min(16, os.cpu_count() or 1)):
        sl = slice(b * B, (b + 1) * B)
        q[0, sl] = torch.from_numpy(x.q).to(torch.bfloat16).to(dev)
        k[0, sl] = torch.from_numpy(x.k).to(torch.bfloat16).to(dev)
        v[0, sl] = torch.from_numpy(x.v).to(torch.bfloat16).to(dev)
        g[0, sl] = torch.from_numpy(x.g).to(dev)
        beta[0, sl] = torch.from_numpy(x.beta).to(dev)
        hq[sl], hk[sl], hv[sl], hg[sl] = x.q[:, hs], x.k[:, hs], x.v[:, hs], x.g[:, hs]
        hb[sl] = x.beta[:, hs]
        if b % 64 == 0:
            say(f"  drew block {b}/{nblk} ({time.time() - t0:.0f} s)")
    say("running kda_prefill on 1M tokens")
    torch.cuda.synchronize()
    t2 = time.time()
    o, fin = kda.prefill(q, k, v, g, beta, None, chunk_size=64)
    torch.cuda.synchronize()
    say(f"  kda_prefill (workspace allocation included) {1e3 * (time.time() - t2):.1f} ms")
    del q, k, v, g, beta
    o_first = o[0, :B][:, hs].float().cpu().numpy()
    o_last = o[0, T - B:][:, hs].float().cpu().numpy()
    fin_h = fin[0, hs].cpu().numpy()
    del o
    say("oracle over the full sequence for the sampled heads")
    t1 = time.time()
    st = None
    eo_first = eo_last = None
    for p0 in range(0, T, PIECE):
        sl = slice(p0, p0 + PIECE)
        eo, st = oracle.kda_recurrent(hq[sl], hk[sl], hv[sl], hg[sl], hb[sl], st)
        if p0 == 0:
            eo_first = eo[:B].copy()
        if p0 + PIECE >= T:
            eo_last = eo[-B:].copy()
        if (p0 // PIECE) % 4 == 0:
            say(f"  oracle tokens {p0 + PIECE}/{T} ({time.time() - t1:.0f} s)")
    ef = st[0]
    rel = lambda x, y: float(np.abs(x - y).max() / np.abs(y).max())

    def per_head(x, y, axis):
        return max(rel(np.take(x, j, axis=axis), np.take(y, j, axis=axis))
                   for j in range(len(hs)))
    e_first = rel(o_first, eo_first)
    e_last = rel(o_last, eo_last)
    e_state = rel(fin_h, ef)
    p_first, p_last, p_state = (per_head(o_first, eo_first, 1), per_head(o_last, eo_last, 1),
                                per_head(fin_h, ef, 0))
    say(f"  first window {e_first:.2e} (per head {p_first:.2e})  last window {e_last:.2e} "
        f"(per head {p_last:.2e})  final state {e_state:.2e} (per head {p_state:.2e})")
    assert max(e_first, e_last, e_state) <= 2e-3
    assert max(p_first, p_last, p_state) <= 2e-3
