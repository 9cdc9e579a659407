"""Seeded synthetic inputs for the KDA prefill and decode workloads.

This module only draws random numbers and shapes them into the input
distributions of the workloads; it holds none of the KDA arithmetic, so the
oracle (under ``oracle/``) and the HIP path can both consume its output.

Input recipe (per token and head):
  * q, k ~ N(0, 1)^d_k, L2-normalised over d_k in float64 with no epsilon
    (q and k are L2-normalised in the model: "Kimi Linear" notes, section
    "Other Components").
  * v ~ N(0, 1)^d_v.
  * beta = sigmoid(N(0, 1))  (the step size is a sigmoid of a projection,
    same section).
  * g = -softplus(N(0, 1)) * 0.1, one value per key channel; alpha = exp(g).
  * q, k, v are then rounded to bfloat16 (round to nearest even) for the
    bf16 workloads, or kept as float32; g and beta stay float32.

Seeds: numpy PCG64 ``default_rng``.  A workload that is generated whole uses
``default_rng([workload_id, stream])``; streamed tensors (long sequences,
repeated decode steps) use ``default_rng([workload_id, stream, index])``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Stream ids inside one workload seed.
_STREAM_TOKENS = 1
_STREAM_STATE = 2
_STREAM_DECODE_STEP = 3


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    NaN stays NaN; values past the bf16 range become +-inf, as in hardware
    conversion.
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    r = u + np.uint32(0x7FFF)          # wraps only for NaN payloads, fixed below
    r += (u >> np.uint32(16)) & np.uint32(1)
    r &= np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of values that are already bf16-exact."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


@dataclasses.dataclass
class TokenInputs:
    """Per-token inputs, token-major ``[T, H, D]`` (float32 arrays).

    For ``dtype == "bf16"`` the q/k/v arrays hold bf16-exact float32 values.
    """
    q: np.ndarray       # [T, H, Dk]
    k: np.ndarray       # [T, H, Dk]
    v: np.ndarray       # [T, H, Dv]
    g: np.ndarray       # [T, H, Dk]  log-decay, <= 0
    beta: np.ndarray    # [T, H]
    dtype: str          # "bf16" or "f32"

    @property
    def T(self) -> int:
        return self.q.shape[0]

    def slice(self, t0: int, t1: int) -> "TokenInputs":
        return TokenInputs(self.q[t0:t1], self.k[t0:t1], self.v[t0:t1],
                           self.g[t0:t1], self.beta[t0:t1], self.dtype)


def draw_tokens(rng: np.random.Generator, T: int, H: int, Dk: int, Dv: int,
                dtype: str = "bf16", g_scale: float = 0.1) -> TokenInputs:
    """Draw T tokens for H heads with the recipe in the module docstring.

    ``g_scale`` multiplies the softplus term (0.1 in every workload; the
    stress tests pass other values to reach strong or weak decay).
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    q = _l2norm(rng.standard_normal((T, H, Dk)))
    k = _l2norm(rng.standard_normal((T, H, Dk)))
    v = rng.standard_normal((T, H, Dv))
    beta = _sigmoid(rng.standard_normal((T, H)))
    g = -_softplus(rng.standard_normal((T, H, Dk))) * g_scale
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    else:
        q, k, v = (a.astype(np.float32) for a in (q, k, v))
    return TokenInputs(q, k, v, g.astype(np.float32), beta.astype(np.float32), dtype)


def draw_mixed_decay_tokens(rng: np.random.Generator, T: int, H: int, Dk: int, Dv: int,
                            dtype: str = "bf16", alpha: float = 0.1,
                            frac: float = 0.5) -> TokenInputs:
    """Tokens as :func:`draw_tokens`, but on the last ``frac`` of the key
    channels of every head the decay is fast: g = log(alpha) (1 + 0.1 N(0, 1)),
    clipped to <= 0, i.e. alpha near ``alpha`` per token.  The other channels
    keep the workload recipe.  (Channel-wise forgetting at different rates is
    what the per-channel gate is for: the "Kimi Linear" notes, docsaid.org,
    section "KDA: Splitting the Decay Across Channels", illustrate it with a
    channel at alpha = 0.1.)"""
    x = draw_tokens(rng, T, H, Dk, Dv, dtype)
    c0 = Dk - int(round(frac * Dk))
    fast = np.log(alpha) * (1.0 + 0.1 * rng.standard_normal((T, H, Dk - c0)))
    x.g[:, :, c0:] = np.minimum(fast, 0.0).astype(np.float32)
    return x


@dataclasses.dataclass
class LayerInputs:
    """Inputs of the fused layer: the projections before their activations.

    q_pre, k_pre, v_pre, gate ~ N(0, 1) (bf16-exact for ``"bf16"``);
    beta_logit ~ N(0, 1) float32; g as in :func:`draw_tokens`; norm_weight
    ``[Dv]`` = 1 + 0.1 N(0, 1) float32.
    """
    q_pre: np.ndarray       # [T, H, Dk]
    k_pre: np.ndarray       # [T, H, Dk]
    v_pre: np.ndarray       # [T, H, Dv]
    g: np.ndarray           # [T, H, Dk]
    beta_logit: np.ndarray  # [T, H]
    gate: np.ndarray        # [T, H, Dv]
    norm_weight: np.ndarray  # [Dv]
    dtype: str


def draw_layer_tokens(rng: np.random.Generator, T: int, H: int, Dk: int, Dv: int,
                      dtype: str = "bf16", g_scale: float = 0.1) -> LayerInputs:
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    q = rng.standard_normal((T, H, Dk))
    k = rng.standard_normal((T, H, Dk))
    v = rng.standard_normal((T, H, Dv))
    gate = rng.standard_normal((T, H, Dv))
    beta = rng.standard_normal((T, H))
    g = -_softplus(rng.standard_normal((T, H, Dk))) * g_scale
    w = 1.0 + 0.1 * rng.standard_normal(Dv)
    rnd = bf16_round if dtype == "bf16" else (lambda a: a.astype(np.float32))
    return LayerInputs(rnd(q), rnd(k), rnd(v), g.astype(np.float32), beta.astype(np.float32),
                       rnd(gate), w.astype(np.float32), dtype)


def draw_states(rng: np.random.Generator, N: int, H: int, Dk: int, Dv: int,
                std: float = 0.1) -> np.ndarray:
    """Initial fast-weight states ``[N, H, Dk, Dv]`` ~ N(0, std^2), float32."""
    return (rng.standard_normal((N, H, Dk, Dv)) * std).astype(np.float32)


# --------------------------------------------------------------------------
# The workloads.  Ids 0..4 are fixed; their sizes are stated in each entry.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    H: int
    Dk: int
    Dv: int
    dtype: str
    chunk: int
    T: int = 0                      # tokens per sequence (fixed-length cases)
    B: int = 1
    num_seqs: int = 0               # varlen: number of packed sequences
    len_range: tuple = (0, 0)       # varlen: inclusive length range
    init_state_std: float = 0.0     # 0 => zero initial state
    decode_N: int = 0               # decode: concurrent sequences
    decode_steps: int = 0


WORKLOADS = {
    0: Workload(0, "tiny_f32_T256_H1_d64", H=1, Dk=64, Dv=64, dtype="f32",
                chunk=16, T=256),
    1: Workload(1, "prefill_bf16_T4096_H32_d128", H=32, Dk=128, Dv=128,
                dtype="bf16", chunk=64, T=4096),
    2: Workload(2, "varlen_bf16_16seq_512-8192_H32_d128", H=32, Dk=128, Dv=128,
                dtype="bf16", chunk=64, num_seqs=16, len_range=(512, 8192),
                init_state_std=0.1),
    3: Workload(3, "prefill_bf16_T1048576_H32_d128", H=32, Dk=128, Dv=128,
                dtype="bf16", chunk=64, T=1 << 20),
    4: Workload(4, "decode_bf16_N256_H32_d128_1000steps", H=32, Dk=128, Dv=128,
                dtype="bf16", chunk=0, decode_N=256, decode_steps=1000,
                init_state_std=0.1),
}


def varlen_lengths(w: Workload) -> np.ndarray:
    """Sequence lengths, uniform integers on the inclusive range."""
    lo, hi = w.len_range
    return np.random.default_rng(w.wid).integers(lo, hi + 1, w.num_seqs)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    return cu.astype(np.int32)


def workload_tokens(w: Workload, T: Optional[int] = None, workers: int = 8) -> TokenInputs:
    """All tokens of a whole-generated prefill workload (ids 0, 1, 2).

    Fixed-length workloads draw every token from one stream.  For the varlen
    workload each sequence n has its own stream ``[wid, 1, n]`` (so any subset
    can be drawn alone) and the sequences are packed back to back; ``workers``
    threads draw them concurrently.  ``T`` overrides the token count of a
    fixed-length workload (to draw a prefix).
    """
    if not w.num_seqs:
        rng = np.random.default_rng([w.wid, _STREAM_TOKENS])
        return draw_tokens(rng, w.T if T is None else T, w.H, w.Dk, w.Dv, w.dtype)
    lens = varlen_lengths(w)
    parts = [None] * len(lens)

    def one(n):
        rng = np.random.default_rng([w.wid, _STREAM_TOKENS, n])
        parts[n] = draw_tokens(rng, int(lens[n]), w.H, w.Dk, w.Dv, w.dtype)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(len(lens))))
    else:
        for n in range(len(lens)):
            one(n)
    cat = lambda name: np.concatenate([getattr(p, name) for p in parts])
    return TokenInputs(cat("q"), cat("k"), cat("v"), cat("g"), cat("beta"), w.dtype)


def workload_states(w: Workload, N: int) -> Optional[np.ndarray]:
    if w.init_state_std == 0.0:
        return None
    rng = np.random.default_rng([w.wid, _STREAM_STATE])
    return draw_states(rng, N, w.H, w.Dk, w.Dv, w.init_state_std)


def long_block(w: Workload, block: int, block_tokens: int = 4096) -> TokenInputs:
    """Block ``block`` of a streamed long sequence (``block_tokens`` tokens)."""
    rng = np.random.default_rng([w.wid, _STREAM_TOKENS, block])
    return draw_tokens(rng, block_tokens, w.H, w.Dk, w.Dv, w.dtype)


def decode_step_inputs(w: Workload, step: int) -> TokenInputs:
    """One new token for each of the ``decode_N`` sequences at ``step``.

    Returned with the sequence axis in the token position: arrays are
    ``[N, H, D]`` and ``beta`` is ``[N, H]``.
    """
    rng = np.random.default_rng([w.wid, _STREAM_DECODE_STEP, step])
    return draw_tokens(rng, w.decode_N, w.H, w.Dk, w.Dv, w.dtype)


def long_blocks(w: Workload, blocks, block_tokens: int = 4096, workers: int = 16):
    """Yield ``(block, TokenInputs)`` for the given block indices, in order,
    drawing up to ``workers`` blocks concurrently (each block has its own
    stream, so the result does not depend on the thread count)."""
    from concurrent.futures import ThreadPoolExecutor
    blocks = list(blocks)
    with ThreadPoolExecutor(max(1, workers)) as ex:
        futs = {}
        ahead = max(1, workers)
        for i, b in enumerate(blocks[:ahead]):
            futs[i] = ex.submit(long_block, w, b, block_tokens)
        for i, b in enumerate(blocks):
            x = futs.pop(i).result()
            j = i + ahead
            if j < len(blocks):
                futs[j] = ex.submit(long_block, w, blocks[j], block_tokens)
            yield b, x


def device_tokens(torch, T: int, H: int, Dk: int, Dv: int, seed: int, device,
                  dtype: str = "bf16", chunk_tokens: int = 65536):
    """The same input recipe drawn on the GPU with torch's seeded generator.

    For throughput measurements at sizes where drawing on the host would
    dominate (the million-token workload): the values follow the recipe above
    but come from torch's generator, so they differ from ``draw_tokens``.
    The L2 normalisation runs in float32 here.  Returns device tensors q, k, v
    ``[1, T, H, D]`` (bf16 or float32), g ``[1, T, H, Dk]`` and beta
    ``[1, T, H]`` (float32), filled ``chunk_tokens`` tokens at a time.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.empty((1, T, H, Dk), dtype=dt, device=device)
    k = torch.empty_like(q)
    v = torch.empty((1, T, H, Dv), dtype=dt, device=device)
    g = torch.empty((1, T, H, Dk), dtype=torch.float32, device=device)
    beta = torch.empty((1, T, H), dtype=torch.float32, device=device)
    for t0 in range(0, T, chunk_tokens):
        n = min(chunk_tokens, T - t0)
        sl = slice(t0, t0 + n)
        for dst, d in ((q, Dk), (k, Dk)):
            x = torch.randn((n, H, d), generator=gen, device=device)
            dst[0, sl] = (x / x.norm(dim=-1, keepdim=True)).to(dt)
        v[0, sl] = torch.randn((n, H, Dv), generator=gen, device=device).to(dt)
        g[0, sl] = -torch.nn.functional.softplus(
            torch.randn((n, H, Dk), generator=gen, device=device)) * 0.1
        beta[0, sl] = torch.sigmoid(torch.randn((n, H), generator=gen, device=device))
    return q, k, v, g, beta


def device_layer_tokens(torch, T: int, H: int, Dk: int, Dv: int, seed: int, device,
                        dtype: str = "bf16"):
    """The fused layer's inputs (recipe of :class:`LayerInputs`) drawn on the
    GPU with torch's seeded generator.  Returns q_pre, k_pre, v_pre, gate
    ``[1, T, H, D]`` (bf16 or float32), g ``[1, T, H, Dk]``, beta_logit
    ``[1, T, H]`` and norm_weight ``[Dv]`` (float32)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rn = lambda *s: torch.randn(s, generator=gen, device=device)
    q = rn(1, T, H, Dk).to(dt)
    k = rn(1, T, H, Dk).to(dt)
    v = rn(1, T, H, Dv).to(dt)
    gate = rn(1, T, H, Dv).to(dt)
    beta = rn(1, T, H)
    g = -torch.nn.functional.softplus(rn(1, T, H, Dk)) * 0.1
    w = 1.0 + 0.1 * rn(Dv)
    return q, k, v, gate, g, beta, w


def draw_conv(rng: np.random.Generator, N: int, H: int, D: int, W: int,
              dtype: str = "bf16"):
    """Short-convolution weights and carried inputs for the fused layer:
    three weights ``[H, D, W]`` ~ N(0, 1/W) float32 (q, k, v) and three
    states ``[N, H, W-1, D]`` ~ N(0, 1) (bf16-exact for ``"bf16"``)."""
    rnd = bf16_round if dtype == "bf16" else (lambda a: a.astype(np.float32))
    ws = tuple((rng.standard_normal((H, D, W)) / np.sqrt(W)).astype(np.float32)
               for _ in range(3))
    ss = tuple(rnd(rng.standard_normal((N, H, W - 1, D))) for _ in range(3))
    return ws, ss


def draw_dplr_tokens(rng: np.random.Generator, T: int, H: int, Dk: int, Dv: int,
                     dtype: str = "bf16", g_scale: float = 0.1):
    """Inputs of the general DPLR recurrence: q, k as in :func:`draw_tokens`;
    a = sigmoid(N(0, 1)) u and b = exp(g) * 0.5 w with u, w independent unit
    vectors (so the low-rank term has norm below 1/2); v ~ N(0, 1); g as in
    :func:`draw_tokens`.  Returns (q, k, v, a, b, g) float32 arrays
    (q, k, v, a, b bf16-exact for ``"bf16"``)."""
    q = _l2norm(rng.standard_normal((T, H, Dk)))
    k = _l2norm(rng.standard_normal((T, H, Dk)))
    v = rng.standard_normal((T, H, Dv))
    g = -_softplus(rng.standard_normal((T, H, Dk))) * g_scale
    a = _sigmoid(rng.standard_normal((T, H, 1))) * _l2norm(rng.standard_normal((T, H, Dk)))
    b = np.exp(g) * 0.5 * _l2norm(rng.standard_normal((T, H, Dk)))
    rnd = bf16_round if dtype == "bf16" else (lambda x: x.astype(np.float32))
    return rnd(q), rnd(k), rnd(v), rnd(a), rnd(b), g.astype(np.float32)
