"""The C ABI on the host: every declared symbol is exported, and argument
validation returns the documented status codes before anything reaches a GPU
(no call here passes validation, so nothing is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_delta_rule_56_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x100000  # 16-byte aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:kda|gdn|dplr)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kda_prefill", "kda_decode_step", "kda_prefill_workspace_size",
            "kda_status_string", "kda_version", "gdn_prefill", "gdn_decode_step",
            "kda_prefill_layer", "kda_decode_step_layer", "kda_backward", "dplr_prefill",
            "kda_prefill_chunk_fp32"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in kda.h but not exported"


def test_status_strings(lib):
    for code in range(5):
        s = kda.status_string(code)
        assert s.startswith("KDA_")
    assert "UNKNOWN" in kda.status_string(99)
    assert lib.kda_version() >= 100


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, s0=None, s1=None,
             cu=None, cu_host=None, B=1, T=128, H=2, Dk=128, Dv=128, N=1, C=64,
             ind=0, outd=1, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"], a["s0"], a["s1"],
                           a["cu"], a["cu_host"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"],
                           a["N"], a["C"], a["ind"], a["outd"], a["ws"], a["wsb"], a["stream"])


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == INVALID
    assert _prefill(lib, H=0) == INVALID
    assert _prefill(lib, Dk=96, Dv=96) == UNSUPPORTED
    assert _prefill(lib, Dk=128, Dv=64) == UNSUPPORTED
    assert _prefill(lib, C=48) == UNSUPPORTED
    assert _prefill(lib, ind=7) == INVALID
    assert _prefill(lib, g=FAKE + 4) == INVALID            # misaligned
    assert _prefill(lib, N=2) == INVALID                    # N must equal B without cu_seqlens
    assert _prefill(lib, ws=None) == WORKSPACE
    assert _prefill(lib, wsb=1024) == WORKSPACE
    assert _prefill(lib, ws=FAKE + 16) == INVALID           # workspace not 256-aligned
    assert _prefill(lib, T=-1) == INVALID


def test_prefill_varlen_validation(lib):
    good = np.array([0, 50, 50, 128], dtype=np.int32)
    bad_order = np.array([0, 60, 50, 128], dtype=np.int32)
    bad_end = np.array([0, 50, 60, 127], dtype=np.int32)
    bad_start = np.array([4, 50, 60, 128], dtype=np.int32)
    hp = lambda a: a.ctypes.data
    # host copy required with a device copy, and B must be 1
    assert _prefill(lib, cu=FAKE, cu_host=None, N=3) == INVALID
    assert _prefill(lib, cu=FAKE, cu_host=hp(good), N=3, B=2) == INVALID
    assert _prefill(lib, cu=FAKE, cu_host=hp(bad_order), N=3) == INVALID
    assert _prefill(lib, cu=FAKE, cu_host=hp(bad_end), N=3) == INVALID
    assert _prefill(lib, cu=FAKE, cu_host=hp(bad_start), N=3) == INVALID
    # a valid table with a too-small workspace fails only on the workspace
    assert _prefill(lib, cu=FAKE, cu_host=hp(good), N=3, wsb=16) == WORKSPACE


def test_workspace_size(lib):
    # B=1, T=4096, H=32, D=128, C=64, bf16: 64 chunks of 32 heads x 147968 B
    # (Q*gam 32 KB, W 32 KB, K-bar 32 KB, P 16 KB as bf16 hi + lo; U0 = T V
    # 32 KB fp32; gam_n 512 B).  The workspace holds one segment of chunks
    # (a 160 MiB budget: at most 35 chunks, so 2 equal segments of 32) and the
    # fp32 state carried between segments (32 x 128 x 128 x 4 B); fixed-length
    # input needs no slot table.
    if "KDA_PREFILL_SEGMENT_KB" in os.environ:
        pytest.skip("segment budget overridden")
    n = kda.workspace_size(1, 4096, 32, 128, 1, 64, kda.KDA_BF16)
    assert n == 32 * 32 * 147968 + 32 * 128 * 128 * 4
    # one segment: no carry buffer
    n1 = kda.workspace_size(1, 2048, 32, 128, 1, 64, kda.KDA_BF16)
    assert n1 == 32 * 32 * 147968
    # varlen, fp32, D=64, C=16, H=4: lengths 100, 0, 200 -> 7, 0, 13 chunks,
    # one segment of 13 local chunks holding 7 + 13 slots of 4 x 22784 B
    # (Q*gam 4 KB, W 4 KB, K-bar 8 KB, P 2 KB, U0 4 KB, gam_n 256 B, a
    # multiple of 256 B), plus the 256-byte slot table.
    cu = np.array([0, 100, 100, 300], dtype=np.int32)
    m = kda.workspace_size(1, 300, 4, 64, 3, 16, kda.KDA_F32, cu)
    assert m == 20 * 4 * 22784 + 256
    with pytest.raises(kda.KDAError):
        kda.workspace_size(1, 300, 4, 80, 3, 16, kda.KDA_F32, cu)


def test_workspace_segments(monkeypatch):
    # Segments hold at least 16 local chunks: with a 1000 KB budget (less
    # than 16 chunks of one head, 2.37 MB), T=4096 (64 chunks) runs as 4
    # segments of 16, plus the carried state.
    monkeypatch.setenv("KDA_PREFILL_SEGMENT_KB", "1000")
    n = kda.workspace_size(1, 4096, 1, 128, 1, 64, kda.KDA_BF16)
    assert n == 16 * 147968 + 128 * 128 * 4
    # 4000 KB fits 27 chunks: 3 segments, evened out to 22 chunks each.
    monkeypatch.setenv("KDA_PREFILL_SEGMENT_KB", "4000")
    n = kda.workspace_size(1, 4096, 1, 128, 1, 64, kda.KDA_BF16)
    assert n == 22 * 147968 + 128 * 128 * 4


def test_decode_validation(lib):
    d = lambda **kw: lib.kda_decode_step(
        *[kw.get(n, FAKE) for n in ("q", "k", "v", "g", "beta", "state", "o")],
        kw.get("N", 4), kw.get("H", 2), kw.get("Dk", 64), kw.get("Dv", 64),
        kw.get("ind", 1), kw.get("outd", 1), None)
    assert d(state=None) == INVALID
    assert d(N=-1) == INVALID
    assert d(H=0) == INVALID
    assert d(Dk=32, Dv=32) == UNSUPPORTED
    assert d(o=FAKE + 8) == INVALID
    assert d(outd=5) == INVALID


def test_layer_workspace_size(lib):
    # Without the gate the layer call needs exactly the plain workspace; with
    # it, one segment's raw fp32 output as well: 32 slots x 32 heads x 64 x
    # 128 x 4 B at T=4096 (two segments of 32 chunks).
    if "KDA_PREFILL_SEGMENT_KB" in os.environ or "KDA_PREFILL_SEGMENT_CHUNKS" in os.environ:
        pytest.skip("segment plan overridden")
    plain = kda.workspace_size(1, 4096, 32, 128, 1, 64, kda.KDA_BF16)
    assert kda.workspace_size(1, 4096, 32, 128, 1, 64, kda.KDA_BF16, layer_gate=False) == plain
    gated = kda.workspace_size(1, 4096, 32, 128, 1, 64, kda.KDA_BF16, layer_gate=True)
    assert gated == plain + 32 * 32 * 64 * 128 * 4


def _params(gate=FAKE, w=FAKE, eps=1e-6, cw=0, cwt=(FAKE, FAKE, FAKE), csin=(None,) * 3,
            csout=(None,) * 3):
    lp = kda.LayerParams()
    lp.gate, lp.norm_weight, lp.norm_eps, lp.conv_width = gate, w, eps, cw
    for x in range(3):
        lp.conv_weight[x], lp.conv_state_in[x], lp.conv_state_out[x] = cwt[x], csin[x], csout[x]
    return lp


def _layer_prefill(lib, layer=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE,
             s0=None, s1=None, cu=None, cu_host=None, B=1, T=128, H=2, Dk=128, Dv=128, N=1,
             C=64, ind=0, outd=1, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    lp = _params() if layer is None else layer
    return lib.kda_prefill_layer(a["q"], a["k"], a["v"], a["g"], a["beta"], ctypes.byref(lp),
                                 a["o"], a["s0"], a["s1"], a["cu"], a["cu_host"],
                                 a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["C"],
                                 a["ind"], a["outd"], a["ws"], a["wsb"], a["stream"])


def test_layer_validation(lib):
    # Every call fails validation; the first check that fails decides.
    assert _layer_prefill(lib, _params(w=None), ws=None) == INVALID      # gate without weight
    assert _layer_prefill(lib, _params(eps=-1.0), ws=None) == INVALID
    assert _layer_prefill(lib, _params(eps=float("inf")), ws=None) == INVALID
    assert _layer_prefill(lib, _params(eps=float("nan")), ws=None) == INVALID
    assert _layer_prefill(lib, _params(gate=FAKE + 2), ws=None) == INVALID  # misaligned gate
    assert _layer_prefill(lib, _params(cw=5), ws=None) == INVALID         # width beyond 4
    assert _layer_prefill(lib, _params(cw=-1), ws=None) == INVALID
    assert _layer_prefill(lib, _params(cw=4, cwt=(FAKE, None, FAKE)), ws=None) == INVALID
    assert _layer_prefill(lib, _params(cw=4, csin=(FAKE + 8, None, None)), ws=None) == INVALID
    assert _layer_prefill(lib, _params(), ws=None) == WORKSPACE
    assert _layer_prefill(lib, _params(cw=4), ws=None) == WORKSPACE
    assert _layer_prefill(lib, _params(gate=None, w=None), ws=None) == WORKSPACE
    assert _layer_prefill(lib, _params(), Dk=96, Dv=96) == UNSUPPORTED
    d = lambda lp, **kw: lib.kda_decode_step_layer(
        *[kw.get(n, FAKE) for n in ("q", "k", "v", "g", "beta")], ctypes.byref(lp),
        kw.get("state", FAKE), kw.get("o", FAKE), kw.get("N", 4), kw.get("H", 2),
        kw.get("Dk", 64), kw.get("Dv", 64), kw.get("ind", 1), kw.get("outd", 1), None)
    assert d(_params(w=None)) == INVALID
    assert d(_params(eps=-0.5)) == INVALID
    assert d(_params(cw=7)) == INVALID
    assert d(_params(), state=None) == INVALID
    assert d(_params(), Dk=32, Dv=32) == UNSUPPORTED
