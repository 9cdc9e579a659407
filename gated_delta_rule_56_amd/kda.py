"""Python binding of the KDA C ABI (include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libkda.so``.  PyTorch provides device memory and the stream.
The native library is required; if it is missing this module raises on first
use instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_BF16 = 0
KDA_F32 = 1

_lib = None


class KDAError(RuntimeError):
    pass


class LayerParams(ctypes.Structure):
    """``kda_layer_params`` of include/kda.h."""
    _fields_ = [("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("conv_width", ctypes.c_int),
                ("conv_weight", ctypes.c_void_p * 3), ("conv_state_in", ctypes.c_void_p * 3),
                ("conv_state_out", ctypes.c_void_p * 3)]


class PrefillOptions(ctypes.Structure):
    """``kda_prefill_options`` of include/kda.h (zero fields: automatic)."""
    _fields_ = [("segment_chunks", ctypes.c_int), ("segment_bytes", ctypes.c_size_t),
                ("value_block", ctypes.c_int)]


FORM_KDA, FORM_GDN, FORM_LAYER = 0, 1, 2


def _options(options) -> Optional[PrefillOptions]:
    """A dict with any of segment_chunks, segment_bytes, value_block (or
    None) as the C struct."""
    if options is None:
        return None
    unknown = set(options) - {"segment_chunks", "segment_bytes", "value_block"}
    if unknown:
        raise KDAError(f"unknown prefill options {sorted(unknown)}")
    return PrefillOptions(int(options.get("segment_chunks", 0)),
                          int(options.get("segment_bytes", 0)),
                          int(options.get("value_block", 0)))


def load() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by gated_delta_rule_56_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KDAError(f"{LIB_PATH} is missing: build it with "
                       "`python -m gated_delta_rule_56_amd.build` first")
    # torch's HIP runtime and the one libkda.so links share a soname, so the
    # first loaded serves the whole process.  Load torch's first: the device
    # pointers and streams handed to the library come from it.
    _torch()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.restype = i32
    lib.kda_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32, i32,
                                               ctypes.POINTER(sz)]
    lib.kda_prefill_workspace_size.restype = i32
    lib.kda_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                vp, sz, vp]
    lib.kda_prefill.restype = i32
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step.restype = i32
    lib.gdn_prefill.argtypes = lib.kda_prefill.argtypes
    lib.gdn_prefill.restype = i32
    lib.gdn_decode_step.argtypes = lib.kda_decode_step.argtypes
    lib.gdn_decode_step.restype = i32
    lp = ctypes.POINTER(LayerParams)
    lib.kda_prefill_layer_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32, i32,
                                                     lp, ctypes.POINTER(sz)]
    lib.kda_prefill_layer_workspace_size.restype = i32
    lib.kda_prefill_layer.argtypes = [vp, vp, vp, vp, vp, lp, vp, vp, vp, vp, vp,
                                      i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                      vp, sz, vp]
    lib.kda_prefill_layer.restype = i32
    lib.kda_decode_step_layer.argtypes = [vp, vp, vp, vp, vp, lp, vp, vp,
                                          i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step_layer.restype = i32
    lib.kda_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32,
                                                ctypes.POINTER(sz)]
    lib.kda_backward_workspace_size.restype = i32
    lib.kda_backward.argtypes = [vp] * 16 + [i32] * 8 + [vp, sz, vp]
    lib.kda_backward.restype = i32
    lib.dplr_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32,
                                                ctypes.POINTER(sz)]
    lib.dplr_prefill_workspace_size.restype = i32
    lib.dplr_prefill.argtypes = [vp] * 11 + [i32] * 8 + [vp, sz, vp]
    lib.dplr_prefill.restype = i32
    lib.kda_prefill_chunk_fp32.argtypes = [vp] * 10 + [i32] * 8 + [vp, sz, vp]
    lib.kda_prefill_chunk_fp32.restype = i32
    lib.dplr_decode_step.argtypes = [vp] * 8 + [i32] * 6 + [vp]
    lib.dplr_decode_step.restype = i32
    op = ctypes.POINTER(PrefillOptions)
    lib.kda_backward_workspace_size_ex.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32, op,
                                                   ctypes.POINTER(sz)]
    lib.kda_backward_workspace_size_ex.restype = i32
    lib.kda_backward_ex.argtypes = [vp] * 16 + [i32] * 8 + [op, vp, sz, vp]
    lib.kda_backward_ex.restype = i32
    lib.kda_prefill_workspace_size_ex.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, i32, i32,
                                                  vp, op, ctypes.POINTER(sz)]
    lib.kda_prefill_workspace_size_ex.restype = i32
    lib.kda_prefill_ex.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, i32, i32, i32, op, vp, sz, vp]
    lib.kda_prefill_ex.restype = i32
    lib.kda_prefill_noalloc.argtypes = [vp] * 10 + [i32] * 9 + [vp]
    lib.kda_prefill_noalloc.restype = i32
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().kda_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise KDAError(f"{what}: {status_string(code)}")


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise KDAError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_device(dev, named):
    """Every tensor handed to the C ABI must live on q's GPU: the kernels
    dereference the raw pointers on that device."""
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda or t.device != dev:
            raise KDAError(f"{name} must be a GPU tensor on the device of q ({dev}), "
                           f"got {t.device}")


def _out_dtype(o, out_dtype):
    """The dtype written to o: o's own when o is given (out_dtype, if also
    given, must agree), else out_dtype, else float32.  A given o must be
    contiguous: the kernels write it densely."""
    torch = _torch()
    if o is not None:
        if out_dtype is not None and out_dtype != o.dtype:
            raise KDAError(f"o has dtype {o.dtype} but out_dtype is {out_dtype}")
        if not o.is_contiguous():
            raise KDAError("o must be contiguous")
        _dtype_code(o.dtype)
        return o.dtype
    return out_dtype or torch.float32


def _workspace(ws, nbytes, dev):
    """A caller's workspace when it is a large enough contiguous byte buffer
    on the device, else a new one."""
    torch = _torch()
    if ws is not None:
        if ws.dtype != torch.uint8 or not ws.is_contiguous():
            raise KDAError("workspace must be a contiguous uint8 tensor")
        _on_device(dev, [("workspace", ws)])
        if ws.numel() >= nbytes:
            return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _host_cu(cu_seqlens, cu_seqlens_host) -> np.ndarray:
    if cu_seqlens_host is not None:
        return np.ascontiguousarray(np.asarray(cu_seqlens_host), dtype=np.int32)
    return np.ascontiguousarray(cu_seqlens.detach().cpu().numpy(), dtype=np.int32)


def workspace_size(B: int, T: int, H: int, D: int, num_seqs: int, chunk_size: int,
                   in_dtype: int, cu_seqlens_host: Optional[np.ndarray] = None,
                   layer_gate: Optional[bool] = None, options=None, form=None) -> int:
    """Workspace bytes of kda_prefill (``layer_gate`` None) or of
    kda_prefill_layer with (True) or without (False) the gated epilogue;
    with ``options`` (see :func:`prefill`) those of kda_prefill_ex."""
    out = ctypes.c_size_t(0)
    cu_p = None if cu_seqlens_host is None else cu_seqlens_host.ctypes.data
    if options is not None:
        if form is None:
            form = FORM_KDA if layer_gate is None else FORM_LAYER
        lp = LayerParams()
        lp.gate = 1 << 20 if layer_gate else None  # only its presence is read
        opts = _options(options)
        _check(load().kda_prefill_workspace_size_ex(form, B, T, H, D, D, num_seqs, cu_p,
                                                    chunk_size, in_dtype, ctypes.addressof(lp),
                                                    ctypes.byref(opts), ctypes.byref(out)),
               "kda_prefill_workspace_size_ex")
    elif layer_gate is None:
        _check(load().kda_prefill_workspace_size(B, T, H, D, D, num_seqs, cu_p, chunk_size,
                                                 in_dtype, ctypes.byref(out)),
               "kda_prefill_workspace_size")
    else:
        lp = LayerParams()
        lp.gate = 1 << 20 if layer_gate else None  # only its presence is read
        _check(load().kda_prefill_layer_workspace_size(B, T, H, D, D, num_seqs, cu_p,
                                                       chunk_size, in_dtype, ctypes.byref(lp),
                                                       ctypes.byref(out)),
               "kda_prefill_layer_workspace_size")
    return out.value


def _expect(name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise KDAError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *,
            cu_seqlens_host: Optional[Union[Sequence[int], np.ndarray]] = None,
            chunk_size: int = 64, out_dtype=None, output_final_state: bool = True,
            final_state=None, o=None, workspace=None, options=None):
    """Chunked KDA forward (``kda_prefill``).

    Shapes: q, k, g ``[B, T, H, Dk]``; v ``[B, T, H, Dv]``; beta ``[B, T, H]``.
    A g of shape ``[B, T, H]`` (one log-decay per token and head) selects the
    scalar-decay Gated DeltaNet form (``gdn_prefill``).  With ``cu_seqlens``
    (int32 device tensor ``[N+1]``), B must be 1 and the N packed sequences
    share the T axis.  ``initial_state`` ``[N, H, Dk, Dv]`` float32 or None.
    Returns ``(o, final_state)`` (final_state None unless requested).
    ``final_state`` may be passed (it may alias initial_state).  A given
    ``o`` sets the output dtype.  ``options`` (a dict of
    ``kda_prefill_options`` fields: segment_chunks, segment_bytes,
    value_block) calls ``kda_prefill_ex`` with them.
    """
    return _prefill(q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, chunk_size,
                    out_dtype, output_final_state, final_state, o, workspace, None, options)


def prefill_noalloc(q, k, v, g, beta, o, initial_state=None, final_state=None, cu_seqlens=None,
                    *, cu_seqlens_host=None, chunk_size: int = 64):
    """``kda_prefill_noalloc``: :func:`prefill` without a workspace, for
    callers that cannot allocate.  The caller passes every output (``o``,
    and ``final_state`` or None); with ``cu_seqlens`` the host copy
    ``cu_seqlens_host`` is required too.  Nothing is allocated here or in the
    library (its intermediates live in a static device array), and calls that
    overlap on one GPU race.  Returns ``(o, final_state)``."""
    torch = _torch()
    if q.dim() != 4:
        raise KDAError("q must be [B, T, H, D]")
    B, T, H, D = q.shape
    Dv = v.shape[-1]
    _expect("k", k, (B, T, H, D))
    _expect("v", v, (B, T, H, Dv))
    _expect("g", g, (B, T, H, D))
    _expect("beta", beta, (B, T, H))
    _expect("o", o, (B, T, H, Dv))
    in_code = _dtype_code(q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise KDAError(f"{name} must have the dtype of q")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise KDAError("g and beta must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous")
    out_code = _dtype_code(_out_dtype(o, None))
    if cu_seqlens is not None:
        if cu_seqlens_host is None:
            raise KDAError("cu_seqlens_host is required with cu_seqlens")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
            raise KDAError("cu_seqlens must be contiguous int32")
        cu_h = np.ascontiguousarray(np.asarray(cu_seqlens_host), dtype=np.int32)
        N = len(cu_h) - 1
    else:
        cu_h = None
        N = B
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        _expect(name, t, (N, H, D, Dv))
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise KDAError(f"{name} must be contiguous float32")
    _on_device(q.device, [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o),
                          ("initial_state", initial_state), ("final_state", final_state),
                          ("cu_seqlens", cu_seqlens)])
    cu_hp = None if cu_h is None else cu_h.ctypes.data
    _check(load().kda_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o), _ptr(initial_state),
        _ptr(final_state), _ptr(cu_seqlens), cu_hp, B, T, H, D, Dv, N, chunk_size, in_code,
        out_code, _stream_ptr(q.device)), "kda_prefill_noalloc")
    return o, final_state


def layer_prefill(q_pre, k_pre, v_pre, g, beta_logit, gate=None, norm_weight=None,
                  norm_eps: float = 1e-6, initial_state=None, cu_seqlens=None, *,
                  conv_weight=None, conv_state=None, conv_state_out=None,
                  cu_seqlens_host: Optional[Union[Sequence[int], np.ndarray]] = None,
                  chunk_size: int = 64, out_dtype=None, output_final_state: bool = True,
                  final_state=None, o=None, workspace=None, options=None):
    """KDA layer forward with the fused prologue and epilogue
    (``kda_prefill_layer``): the short convolution of q, k, v when
    ``conv_weight`` = (w_q, w_k, w_v) ``[H, D, W]`` float32 is given (carried
    inputs ``conv_state`` = three ``[N, H, W-1, D]`` tensors of q's dtype, or
    None), Swish + L2 norm of q and k, Swish of v, sigmoid of beta, the
    recurrence, then with ``gate`` ``[B, T, H, Dv]`` (dtype of q) the
    head-wise RMSNorm times ``norm_weight`` ``[Dv]`` float32 times
    sigmoid(gate).  Shapes and the rest as in :func:`prefill` (KDA decay g
    ``[B, T, H, Dk]`` only).  Returns ``(o, final_state)``, and with the
    convolution ``(o, final_state, conv_state_out)`` (three tensors, written
    over ``conv_state_out`` when given; it may be ``conv_state``)."""
    layer = _Layer(gate, norm_weight, norm_eps, conv_weight, conv_state, conv_state_out)
    o, fin = _prefill(q_pre, k_pre, v_pre, g, beta_logit, initial_state, cu_seqlens,
                      cu_seqlens_host, chunk_size, out_dtype, output_final_state, final_state, o,
                      workspace, layer, options)
    return (o, fin) if conv_weight is None else (o, fin, layer.conv_state_out)


class _Layer:
    def __init__(self, gate, weight, eps, conv_weight, conv_state, conv_state_out):
        self.gate, self.weight, self.eps = gate, weight, float(eps)
        self.conv_weight, self.conv_state, self.conv_state_out = (conv_weight, conv_state,
                                                                  conv_state_out)

    def check(self, q, out_shape, N, H, D):
        """Validate shapes and dtypes; allocate missing conv outputs."""
        torch = _torch()
        if self.gate is not None:
            _expect("gate", self.gate, out_shape)
            if self.gate.dtype != q.dtype or not self.gate.is_contiguous():
                raise KDAError("gate must be contiguous with the dtype of q")
            if self.weight is None:
                raise KDAError("norm_weight is required with gate")
            _expect("norm_weight", self.weight, (out_shape[-1],))
            if self.weight.dtype != torch.float32 or not self.weight.is_contiguous():
                raise KDAError("norm_weight must be contiguous float32")
            _on_device(q.device, [("gate", self.gate), ("norm_weight", self.weight)])
        if self.conv_weight is None:
            return
        if len(self.conv_weight) != 3:
            raise KDAError("conv_weight must hold the q, k and v weights")
        W = self.conv_weight[0].shape[-1]
        if not 1 <= W <= 4:
            raise KDAError("convolution width must be 1..4")
        for t in self.conv_weight:
            _expect("conv_weight", t, (H, D, W))
            if t.dtype != torch.float32 or not t.is_contiguous():
                raise KDAError("conv_weight must be contiguous float32")
        for name in ("conv_state", "conv_state_out"):
            st = getattr(self, name)
            if st is None:
                continue
            if len(st) != 3:
                raise KDAError(f"{name} must hold three tensors (q, k, v)")
            for t in st:
                _expect(name, t, (N, H, W - 1, D))
                if t.dtype != q.dtype or not t.is_contiguous():
                    raise KDAError(f"{name} must be contiguous with the dtype of q")
        _on_device(q.device, [("conv_weight", t) for t in self.conv_weight] +
                   [("conv_state", t) for t in (self.conv_state or ())] +
                   [("conv_state_out", t) for t in (self.conv_state_out or ())])
        if self.conv_state_out is None:
            self.conv_state_out = tuple(torch.empty((N, H, W - 1, D), dtype=q.dtype,
                                                    device=q.device) for _ in range(3))

    def params(self) -> LayerParams:
        lp = LayerParams()
        lp.gate = _ptr(self.gate)
        lp.norm_weight = _ptr(self.weight) if self.gate is not None else None
        lp.norm_eps = self.eps
        if self.conv_weight is not None:
            lp.conv_width = self.conv_weight[0].shape[-1]
            for x in range(3):
                lp.conv_weight[x] = _ptr(self.conv_weight[x])
                lp.conv_state_in[x] = None if self.conv_state is None else _ptr(
                    self.conv_state[x])
                lp.conv_state_out[x] = _ptr(self.conv_state_out[x])
        return lp


def _prefill(q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, chunk_size,
             out_dtype, output_final_state, final_state, o, workspace, layer, options=None):
    torch = _torch()
    if q.dim() != 4:
        raise KDAError("q must be [B, T, H, D]")
    B, T, H, D = q.shape
    Dv = v.shape[-1]
    scalar_g = g.dim() == 3
    if layer is not None and scalar_g:
        raise KDAError("the fused layer takes the per-channel decay g [B, T, H, Dk]")
    _expect("k", k, (B, T, H, D))
    _expect("v", v, (B, T, H, Dv))
    _expect("g", g, (B, T, H) if scalar_g else (B, T, H, D))
    _expect("beta", beta, (B, T, H))
    in_code = _dtype_code(q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise KDAError(f"{name} must have the dtype of q")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise KDAError("g and beta must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
            raise KDAError("cu_seqlens must be contiguous int32")
        _on_device(q.device, [("q", q), ("cu_seqlens", cu_seqlens)])
        cu_h = _host_cu(cu_seqlens, cu_seqlens_host)
        N = len(cu_h) - 1
    else:
        cu_h = None
        N = B
    out_dtype = _out_dtype(o, out_dtype)
    out_code = _dtype_code(out_dtype)
    _expect("o", o, (B, T, H, Dv))
    if not output_final_state:
        final_state = None
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        _expect(name, t, (N, H, D, Dv))
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise KDAError(f"{name} must be contiguous float32")
    if layer is not None:
        layer.check(q, (B, T, H, Dv), N, H, D)
    _on_device(q.device, [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o),
                          ("initial_state", initial_state), ("final_state", final_state)])
    opts = _options(options)
    gate = None if layer is None else layer.gate is not None
    ws_bytes = workspace_size(B, T, H, D, N, chunk_size, in_code, cu_h, gate, options,
                              FORM_LAYER if layer is not None else
                              FORM_GDN if scalar_g else FORM_KDA)
    workspace = _workspace(workspace, ws_bytes, q.device)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, D, Dv), dtype=torch.float32, device=q.device)
    cu_hp = None if cu_h is None else cu_h.ctypes.data
    lp = layer.params() if layer is not None else None
    if opts is not None:
        form = FORM_LAYER if layer is not None else FORM_GDN if scalar_g else FORM_KDA
        _check(load().kda_prefill_ex(
            form, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            None if lp is None else ctypes.addressof(lp), _ptr(o), _ptr(initial_state),
            _ptr(final_state), _ptr(cu_seqlens), cu_hp, B, T, H, D, Dv, N, chunk_size, in_code,
            out_code, ctypes.byref(opts), _ptr(workspace), workspace.numel(),
            _stream_ptr(q.device)), "kda_prefill_ex")
        return o, final_state
    if layer is not None:
        _check(load().kda_prefill_layer(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), ctypes.byref(lp),
            _ptr(o), _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), cu_hp,
            B, T, H, D, Dv, N, chunk_size, in_code, out_code,
            _ptr(workspace), workspace.numel(), _stream_ptr(q.device)),
            "kda_prefill_layer")
        return o, final_state
    fn = load().gdn_prefill if scalar_g else load().kda_prefill
    _check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
        _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), cu_hp,
        B, T, H, D, Dv, N, chunk_size, in_code, out_code,
        _ptr(workspace), workspace.numel(), _stream_ptr(q.device)),
        "gdn_prefill" if scalar_g else "kda_prefill")
    return o, final_state


def decode_step(q, k, v, g, beta, state, *, out_dtype=None, o=None):
    """One recurrent KDA step (``kda_decode_step``); ``state`` updated in place.

    Shapes: q, k, g ``[N, H, Dk]``; v ``[N, H, Dv]``; beta ``[N, H]``;
    state ``[N, H, Dk, Dv]`` float32.  A g of shape ``[N, H]`` selects the
    scalar-decay Gated DeltaNet form (``gdn_decode_step``).  Returns o
    ``[N, H, Dv]``.
    """
    return _decode(q, k, v, g, beta, state, out_dtype, o, None)


def layer_decode_step(q_pre, k_pre, v_pre, g, beta_logit, state, gate=None, norm_weight=None,
                      norm_eps: float = 1e-6, *, conv_weight=None, conv_state=None,
                      out_dtype=None, o=None):
    """One KDA layer step with the fused prologue and epilogue
    (``kda_decode_step_layer``); see :func:`layer_prefill`.  gate
    ``[N, H, Dv]``; ``state`` and ``conv_state`` (three ``[N, H, W-1, D]``
    tensors, required with ``conv_weight`` unless W = 1) are updated in
    place."""
    if conv_weight is not None and conv_state is None and conv_weight[0].shape[-1] > 1:
        raise KDAError("conv_state is required with conv_weight in a decode step")
    layer = _Layer(gate, norm_weight, norm_eps, conv_weight, conv_state, conv_state)
    return _decode(q_pre, k_pre, v_pre, g, beta_logit, state, out_dtype, o, layer)


def _decode(q, k, v, g, beta, state, out_dtype, o, layer):
    torch = _torch()
    if q.dim() != 3:
        raise KDAError("q must be [N, H, D]")
    N, H, D = q.shape
    Dv = v.shape[-1]
    scalar_g = g.dim() == 2
    if layer is not None and scalar_g:
        raise KDAError("the fused layer takes the per-channel decay g [N, H, Dk]")
    _expect("k", k, (N, H, D))
    _expect("v", v, (N, H, Dv))
    _expect("g", g, (N, H) if scalar_g else (N, H, D))
    _expect("beta", beta, (N, H))
    _expect("state", state, (N, H, D, Dv))
    _expect("o", o, (N, H, Dv))
    in_code = _dtype_code(q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise KDAError(f"{name} must have the dtype of q")
    out_dtype = _out_dtype(o, out_dtype)
    out_code = _dtype_code(out_dtype)
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)):
        if not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous")
    if state.dtype != torch.float32 or g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise KDAError("state, g and beta must be float32")
    if layer is not None:
        layer.check(q, (N, H, Dv), N, H, D)
    _on_device(q.device, [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                          ("state", state), ("o", o)])
    if o is None:
        o = torch.empty((N, H, Dv), dtype=out_dtype, device=q.device)
    if layer is not None:
        lp = layer.params()
        _check(load().kda_decode_step_layer(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), ctypes.byref(lp),
            _ptr(state), _ptr(o), N, H, D, Dv, in_code, out_code, _stream_ptr(q.device)),
            "kda_decode_step_layer")
        return o
    fn = load().gdn_decode_step if scalar_g else load().kda_decode_step
    _check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
        N, H, D, Dv, in_code, out_code, _stream_ptr(q.device)),
        "gdn_decode_step" if scalar_g else "kda_decode_step")
    return o


def backward_workspace_size(B: int, T: int, H: int, D: int, num_seqs: int, chunk_size: int,
                            cu_seqlens_host: Optional[np.ndarray] = None, options=None) -> int:
    """Bytes of ``kda_backward``'s workspace; ``options`` (segment_chunks,
    segment_bytes) as for :func:`backward`."""
    out = ctypes.c_size_t(0)
    cu_p = None if cu_seqlens_host is None else cu_seqlens_host.ctypes.data
    if options is None:
        _check(load().kda_backward_workspace_size(B, T, H, D, D, num_seqs, cu_p, chunk_size,
                                                  ctypes.byref(out)), "kda_backward_workspace_size")
    else:
        o = _options(options)
        _check(load().kda_backward_workspace_size_ex(B, T, H, D, D, num_seqs, cu_p, chunk_size,
                                                     ctypes.byref(o), ctypes.byref(out)),
               "kda_backward_workspace_size_ex")
    return out.value


def backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, cu_seqlens=None, *,
             cu_seqlens_host: Optional[Union[Sequence[int], np.ndarray]] = None,
             chunk_size: int = 64, output_d_initial_state: bool = True, workspace=None,
             out=None, options=None):
    """Backward of :func:`prefill` (``kda_backward``): gradients of
    ``sum(d_o * o) + sum(d_final_state * final_state)`` with respect to q, k,
    v, g, beta and the initial state.  Shapes as in :func:`prefill`; d_o
    ``[B, T, H, Dv]`` float32.  Returns ``(dq, dk, dv, dg, dbeta, d_initial_state)``
    (float32; the last is None unless requested).  ``out`` may pass the six
    output tensors to write."""
    torch = _torch()
    if q.dim() != 4:
        raise KDAError("q must be [B, T, H, D]")
    B, T, H, D = q.shape
    Dv = v.shape[-1]
    _expect("k", k, (B, T, H, D))
    _expect("v", v, (B, T, H, Dv))
    _expect("g", g, (B, T, H, D))
    _expect("beta", beta, (B, T, H))
    _expect("d_o", d_o, (B, T, H, Dv))
    in_code = _dtype_code(q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise KDAError(f"{name} must have the dtype of q")
    for name, t in (("g", g), ("beta", beta), ("d_o", d_o)):
        if t.dtype != torch.float32:
            raise KDAError(f"{name} must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("d_o", d_o)):
        if not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous")
    if cu_seqlens is not None:
        cu_h = _host_cu(cu_seqlens, cu_seqlens_host)
        N = len(cu_h) - 1
        if cu_seqlens.dtype != torch.int32:
            raise KDAError("cu_seqlens must be int32")
    else:
        cu_h = None
        N = B
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        _expect(name, t, (N, H, D, Dv))
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise KDAError(f"{name} must be contiguous float32")
    if out is not None:
        for name, t in zip(("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"), out):
            _on_device(q.device, [(name, t)])
    _on_device(q.device, [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("d_o", d_o),
                          ("initial_state", initial_state), ("d_final_state", d_final_state),
                          ("cu_seqlens", cu_seqlens)])
    if out is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        out = (torch.empty((B, T, H, D), **f32), torch.empty((B, T, H, D), **f32),
               torch.empty((B, T, H, Dv), **f32), torch.empty((B, T, H, D), **f32),
               torch.empty((B, T, H), **f32),
               torch.empty((N, H, D, Dv), **f32) if output_d_initial_state else None)
    dq, dk, dv, dg, db, ds0 = out
    for name, t, shp in (("dq", dq, (B, T, H, D)), ("dk", dk, (B, T, H, D)),
                         ("dv", dv, (B, T, H, Dv)), ("dg", dg, (B, T, H, D)),
                         ("dbeta", db, (B, T, H)), ("d_initial_state", ds0, (N, H, D, Dv))):
        _expect(name, t, shp)
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise KDAError(f"{name} must be contiguous float32")
    ws_bytes = backward_workspace_size(B, T, H, D, N, chunk_size, cu_h, options)
    workspace = _workspace(workspace, ws_bytes, q.device)
    cu_hp = None if cu_h is None else cu_h.ctypes.data
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(d_o),
            _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(ds0),
            _ptr(cu_seqlens), cu_hp, B, T, H, D, Dv, N, chunk_size, in_code)
    tail = (_ptr(workspace), workspace.numel(), _stream_ptr(q.device))
    if options is None:
        _check(load().kda_backward(*args, *tail), "kda_backward")
    else:
        o = _options(options)
        _check(load().kda_backward_ex(*args, ctypes.byref(o), *tail), "kda_backward_ex")
    return dq, dk, dv, dg, db, ds0


def dplr_workspace_size(B: int, T: int, H: int, D: int, num_seqs: int, chunk_size: int,
                        cu_seqlens_host: Optional[np.ndarray] = None) -> int:
    out = ctypes.c_size_t(0)
    cu_p = None if cu_seqlens_host is None else cu_seqlens_host.ctypes.data
    _check(load().dplr_prefill_workspace_size(B, T, H, D, D, num_seqs, cu_p, chunk_size,
                                              ctypes.byref(out)), "dplr_prefill_workspace_size")
    return out.value


def _dplr_call(tied, q, k, v, a, b, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
               chunk_size, output_final_state, final_state, o, workspace):
    torch = _torch()
    if q.dim() != 4:
        raise KDAError("q must be [B, T, H, D]")
    B, T, H, D = q.shape
    Dv = v.shape[-1]
    _expect("k", k, (B, T, H, D))
    _expect("v", v, (B, T, H, Dv))
    _expect("g", g, (B, T, H, D))
    in_code = _dtype_code(q.dtype)
    named = [("q", q), ("k", k), ("v", v)]
    if tied:
        _expect("beta", beta, (B, T, H))
        f32s = [("g", g), ("beta", beta)]
    else:
        _expect("a", a, (B, T, H, D))
        _expect("b", b, (B, T, H, D))
        named += [("a", a), ("b", b)]
        f32s = [("g", g)]
    for name, t in named:
        if t.dtype != q.dtype or not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous with the dtype of q")
    for name, t in f32s:
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous float32")
    if cu_seqlens is not None:
        cu_h = _host_cu(cu_seqlens, cu_seqlens_host)
        N = len(cu_h) - 1
    else:
        cu_h = None
        N = B
    if not output_final_state:
        final_state = None
    for name, t in (("o", o), ("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise KDAError(f"{name} must be contiguous float32")
    _expect("o", o, (B, T, H, Dv))
    _expect("initial_state", initial_state, (N, H, D, Dv))
    _expect("final_state", final_state, (N, H, D, Dv))
    _on_device(q.device, named + f32s + [("o", o), ("initial_state", initial_state),
                                         ("final_state", final_state), ("cu_seqlens", cu_seqlens)])
    ws_bytes = dplr_workspace_size(B, T, H, D, N, chunk_size, cu_h)
    workspace = _workspace(workspace, ws_bytes, q.device)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, D, Dv), dtype=torch.float32, device=q.device)
    cu_hp = None if cu_h is None else cu_h.ctypes.data
    if tied:
        code = load().kda_prefill_chunk_fp32(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o), _ptr(initial_state),
            _ptr(final_state), _ptr(cu_seqlens), cu_hp, B, T, H, D, Dv, N, chunk_size, in_code,
            _ptr(workspace), workspace.numel(), _stream_ptr(q.device))
    else:
        code = load().dplr_prefill(
            _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(g), _ptr(o), _ptr(initial_state),
            _ptr(final_state), _ptr(cu_seqlens), cu_hp, B, T, H, D, Dv, N, chunk_size, in_code,
            _ptr(workspace), workspace.numel(), _stream_ptr(q.device))
    _check(code, "kda_prefill_chunk_fp32" if tied else "dplr_prefill")
    return o, final_state


def dplr_prefill(q, k, v, a, b, g, initial_state=None, cu_seqlens=None, *,
                 cu_seqlens_host: Optional[Union[Sequence[int], np.ndarray]] = None,
                 chunk_size: int = 64, output_final_state: bool = True, final_state=None,
                 o=None, workspace=None):
    """General DPLR forward (``dplr_prefill``):
    S_t = (Diag(exp g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.
    q, k, a, b, g ``[B, T, H, Dk]``; v ``[B, T, H, Dv]``.  Returns (o float32,
    final_state)."""
    return _dplr_call(False, q, k, v, a, b, g, None, initial_state, cu_seqlens,
                      cu_seqlens_host, chunk_size, output_final_state, final_state, o, workspace)


def prefill_chunk_fp32(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *,
                       cu_seqlens_host: Optional[Union[Sequence[int], np.ndarray]] = None,
                       chunk_size: int = 64, output_final_state: bool = True, final_state=None,
                       o=None, workspace=None):
    """KDA through the DPLR pipeline's fp32 chunk planes (``kda_prefill_chunk_fp32``);
    arguments as :func:`prefill`, o float32."""
    return _dplr_call(True, q, k, v, None, None, g, beta, initial_state, cu_seqlens,
                      cu_seqlens_host, chunk_size, output_final_state, final_state, o, workspace)


def dplr_decode_step(q, k, v, a, b, g, state, *, out_dtype=None, o=None):
    """One general DPLR step (``dplr_decode_step``); ``state`` updated in place.
    q, k, a, b, g ``[N, H, Dk]`` (g float32); v ``[N, H, Dv]``; state
    ``[N, H, Dk, Dv]`` float32.  Returns o ``[N, H, Dv]``."""
    torch = _torch()
    N, H, D = q.shape
    Dv = v.shape[-1]
    for name, t in (("k", k), ("a", a), ("b", b)):
        _expect(name, t, (N, H, D))
        if t.dtype != q.dtype or not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous with the dtype of q")
    _expect("v", v, (N, H, Dv))
    _expect("g", g, (N, H, D))
    _expect("state", state, (N, H, D, Dv))
    if v.dtype != q.dtype or not v.is_contiguous() or not q.is_contiguous():
        raise KDAError("q and v must be contiguous with one dtype")
    for name, t in (("g", g), ("state", state)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise KDAError(f"{name} must be contiguous float32")
    _expect("o", o, (N, H, Dv))
    out_dtype = _out_dtype(o, out_dtype)
    _on_device(q.device, [("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("g", g),
                          ("state", state), ("o", o)])
    if o is None:
        o = torch.empty((N, H, Dv), dtype=out_dtype, device=q.device)
    _check(load().dplr_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(g), _ptr(state), _ptr(o),
        N, H, D, Dv, _dtype_code(q.dtype), _dtype_code(out_dtype), _stream_ptr(q.device)),
        "dplr_decode_step")
    return o
