"""Host-side checks of libswattn.so that need no GPU: the library loads, exports
every symbol include/swattn.h declares, its integer helpers (layer windows,
visible-pair count, band tile enumeration) agree bit-exactly with the oracle,
and every invalid argument is rejected before any HIP call."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from oracle import attention as A
import sliding_window_causal_qk_amd as sw
from sliding_window_causal_qk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swattn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(_lib.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name
    assert L.attn_version() >= 100


def test_status_strings():
    for s, name in ((0, "ATTN_OK"), (1, "ATTN_ERR_INVALID_ARG"), (2, "ATTN_ERR_UNSUPPORTED"),
                    (3, "ATTN_ERR_WORKSPACE"), (4, "ATTN_ERR_HIP")):
        assert sw.status_string(s) == name
    assert sw.status_string(99) == "ATTN_UNKNOWN_STATUS"


@pytest.mark.parametrize("pattern", ["SSSL", "L", "S", "SL", "SLLL", "SSSS", "sssl", "LS"])
@pytest.mark.parametrize("n_layer", [1, 2, 4, 7, 8, 12])
@pytest.mark.parametrize("T", [1, 2, 513, 2048, 8192])
def test_layer_windows_match_oracle(pattern, n_layer, T):
    assert sw.layer_windows(pattern, n_layer, T) == oracle.layer_windows(pattern, n_layer, T)


def test_layer_windows_golden(golden_dir):
    import json
    g = json.load(open(os.path.join(golden_dir, "window_schedule.json")))
    for c in g["cases"]:
        assert sw.layer_windows(c["pattern"], c["n_layer"], c["seq_len"]) == c["windows"]


@pytest.mark.parametrize("bad", [("", 4, 2048), ("SXL", 4, 2048), ("SSSL", 0, 2048), ("SSSL", 4, 0)])
def test_layer_windows_rejects(bad):
    with pytest.raises(sw.SwattnError):
        sw.layer_windows(*bad)


def test_visible_pairs_match_oracle():
    for T in (0, 1, 2, 3, 17, 64, 127, 128, 129, 1000):
        for W in (-1, 0, 1, 5, T // 2, T - 1, T, T + 3):
            if W < -1:
                continue
            assert sw.visible_pairs(T, W) == (oracle.n_visible(T, W) if T > 0 else 0), (T, W)
    for T, W, n in ((128, 64, 6240), (2048, 1024, 1574400), (2048, 2048, 2098176),
                    (8192, 4096, 25171968), (8192, 8192, 33558528)):
        assert sw.visible_pairs(T, W) == n == oracle.n_visible(T, W)
    with pytest.raises(sw.SwattnError):
        sw.visible_pairs(10, -2)


def _brute_tiles(T, W, rows, cols, by_key):
    m = A.visible_mask(T, W)   # [query, key]
    if by_key:
        m = m.T
    nr, nc = math.ceil(T / rows), math.ceil(T / cols)
    out = []
    for r in range(nr):
        blocks = []
        for cb in range(nc):
            blk = np.zeros((rows, cols), dtype=bool)
            sub = m[r * rows:(r + 1) * rows, cb * cols:(cb + 1) * cols]
            blk[:sub.shape[0], :sub.shape[1]] = sub
            blocks.append((blk.any(), blk.all()))
        vis = [i for i, (a, _) in enumerate(blocks) if a]
        if not vis:
            out.append((0, -1, 0, 0))
            continue
        first, last = vis[0], vis[-1]
        assert vis == list(range(first, last + 1))   # the band is contiguous
        npart = sum(1 for i in range(first, last + 1) if not blocks[i][1])
        out.append((first, last, npart, 0))
    return out


@pytest.mark.parametrize("T,W", [(1, 0), (100, 0), (100, 7), (128, 64), (130, 64), (200, -1),
                                 (257, 128), (300, 299), (333, 31), (512, 256)])
@pytest.mark.parametrize("rows,cols,by_key", [(128, 64, False), (64, 128, True), (32, 64, False),
                                              (16, 16, False), (64, 64, True)])
def test_band_tiles_match_mask(T, W, rows, cols, by_key):
    assert sw.band_tiles(T, W, rows, cols, by_key) == _brute_tiles(T, W, rows, cols, by_key)


# ------------------------------------------------------ argument validation
# Fake device addresses: validation must reject these calls before any HIP
# call, so they are never dereferenced.
P = 0x10000
ALIGNED = [P + i * 0x1000000 for i in range(12)]


def _fwd(**kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], o=ALIGNED[3], lse=ALIGNED[4],
             ws=ALIGNED[5], wsb=1 << 40, B=2, T=64, H=2, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["wsb"],
                               a["B"], a["T"], a["H"], a["D"], a["window"], a["causal"],
                               a["eps"], None)


def _bwd(**kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], o=ALIGNED[3], lse=ALIGNED[4],
             do=ALIGNED[5], dq=ALIGNED[6], dk=ALIGNED[7], dv=ALIGNED[8], ws=ALIGNED[9],
             wsb=1 << 40, B=2, T=64, H=2, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                               a["dk"], a["dv"], a["ws"], a["wsb"], a["B"], a["T"], a["H"],
                               a["D"], a["window"], a["causal"], a["eps"], None)


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(lse=None),
    dict(q=P + 2), dict(v=P + 8),
    dict(B=-1), dict(T=-5), dict(H=-1), dict(D=0), dict(D=-64),
    dict(eps=0.0), dict(eps=-1e-6), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(window=-2), dict(causal=2), dict(causal=-1),
]


@pytest.mark.parametrize("kw", INVALID, ids=[str(k) for k in INVALID])
def test_fwd_invalid(kw):
    assert _fwd(**kw) == _lib.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", INVALID + [dict(do=None), dict(dq=None), dict(dk=P + 4)],
                         ids=[str(k) for k in INVALID + [dict(do=None), dict(dq=None), dict(dk=P + 4)]])
def test_bwd_invalid(kw):
    assert _bwd(**kw) == _lib.ATTN_ERR_INVALID_ARG


def test_aliasing_rejected():
    assert _fwd(o=ALIGNED[0]) == _lib.ATTN_ERR_INVALID_ARG
    assert _bwd(dq=ALIGNED[1]) == _lib.ATTN_ERR_INVALID_ARG
    assert _bwd(dv=ALIGNED[6]) == _lib.ATTN_ERR_INVALID_ARG


QB = 2 * 64 * 2 * 64 * 2       # bytes of q (and of o, dq, ...) at the default B=2, T=64, H=2, D=64


def test_partial_overlap_rejected():
    """Outputs may share no byte with an input, another output or the
    workspace, and the workspace none with an input or output: ranges that
    overlap by a single 16-byte chunk are rejected, not only equal pointers."""
    inv, wsc = _lib.ATTN_ERR_INVALID_ARG, _lib.ATTN_ERR_WORKSPACE
    assert _fwd(o=ALIGNED[0] + QB - 16) == inv          # o starts in q's last chunk
    assert _fwd(o=ALIGNED[2] - QB + 16) == inv          # o ends in v's first chunk
    assert _fwd(lse=ALIGNED[3] + QB - 16) == inv        # lse inside o
    assert _fwd(o=ALIGNED[4] - QB + 16) == inv          # o over lse's first bytes
    assert _fwd(ws=ALIGNED[1] + QB - 256) == wsc        # workspace over k's tail
    assert _fwd(ws=ALIGNED[3] - 256) == wsc             # workspace runs into o
    assert _bwd(dq=ALIGNED[5] + QB - 16) == inv         # dq starts in dout's last chunk
    assert _bwd(dv=ALIGNED[7] + QB - 16) == inv         # dv overlaps dk
    assert _bwd(dk=ALIGNED[4] + 2 * 2 * 64 * 4 - 16) == inv   # dk over lse's last chunk
    assert _bwd(ws=ALIGNED[8] + 256) == wsc             # workspace inside dv
    assert _bwd(ws=ALIGNED[0] + 256) == wsc             # workspace inside q


@pytest.mark.parametrize("kind", ["gqa", "rope", "ve"])
def test_reuse_partial_overlap_rejected(kind):
    ws = ALIGNED[9] if kind != "ve" else P + 15 * 0x1000000
    dv = ALIGNED[8] if kind != "ve" else ALIGNED[11]
    assert _bwd_reuse(kind, fws=dv + 256) == _lib.ATTN_ERR_INVALID_ARG     # forward workspace inside dv
    assert _bwd_reuse(kind, fws=ws + 256) == _lib.ATTN_ERR_WORKSPACE       # inside this call's workspace
    if kind == "rope":   # an output over the tail of the sin table (T rows of D/2 bf16)
        assert _bwd_reuse(kind, dq=ALIGNED[11] + 64 * 32 * 2 - 16) == _lib.ATTN_ERR_INVALID_ARG
    if kind == "ve":     # dx over the gate input's last token (32 channels read at stride 512)
        assert _bwd_reuse(kind, dx=ALIGNED[4] + (2 * 64 - 1) * 512 * 2) == _lib.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=96), dict(D=512), dict(D=32), dict(causal=0),
                                dict(B=1 << 12, T=1 << 12, H=8, D=128),
                                dict(B=1, T=1 << 24, H=1, D=128),     # 2^31 elements: one past the largest
                                dict(B=1, T=1 << 23, H=1, D=256)])
def test_unsupported(kw):
    assert _fwd(**kw) == _lib.ATTN_ERR_UNSUPPORTED
    assert _bwd(**kw) == _lib.ATTN_ERR_UNSUPPORTED


def test_workspace_checks():
    need_f = sw.fwd_workspace_bytes(2, 64, 2, 64)
    need_b = sw.bwd_workspace_bytes(2, 64, 2, 64)
    assert need_f >= 2 * 2 * 64 * 4                     # fp32 key scales
    assert need_b >= 2 * 64 * 2 * 64 * 2 + 3 * 2 * 2 * 64 * 4
    assert _fwd(ws=None) == _lib.ATTN_ERR_WORKSPACE
    assert _fwd(wsb=need_f - 1) == _lib.ATTN_ERR_WORKSPACE
    assert _fwd(ws=P + 16) == _lib.ATTN_ERR_WORKSPACE
    assert _bwd(ws=None) == _lib.ATTN_ERR_WORKSPACE
    assert _bwd(wsb=need_b - 1) == _lib.ATTN_ERR_WORKSPACE


def _fwd_gqa(H_kv, wsb=1 << 40, **kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], o=ALIGNED[3], lse=ALIGNED[4],
             ws=ALIGNED[5], B=2, T=64, H=4, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], wsb,
                                   a["B"], a["T"], a["H"], H_kv, a["D"], a["window"], a["causal"],
                                   a["eps"], None)


def _bwd_gqa(H_kv, wsb=1 << 40, **kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], o=ALIGNED[3], lse=ALIGNED[4],
             do=ALIGNED[5], dq=ALIGNED[6], dk=ALIGNED[7], dv=ALIGNED[8], ws=ALIGNED[9],
             B=2, T=64, H=4, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_bwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                   a["dk"], a["dv"], a["ws"], wsb, a["B"], a["T"], a["H"], H_kv,
                                   a["D"], a["window"], a["causal"], a["eps"], None)


@pytest.mark.parametrize("H,H_kv", [(4, 0), (4, -1), (4, 3), (4, 8), (6, 4), (0, -1)])
def test_gqa_invalid_head_counts(H, H_kv):
    assert _fwd_gqa(H_kv, H=H) == _lib.ATTN_ERR_INVALID_ARG
    assert _bwd_gqa(H_kv, H=H) == _lib.ATTN_ERR_INVALID_ARG


def test_gqa_validation_and_workspace():
    for H_kv in (1, 2, 4):
        need_f = sw.fwd_workspace_bytes(2, 64, 4, 64, H_kv)
        need_b = sw.bwd_workspace_bytes(2, 64, 4, 64, H_kv)
        # the key scales cover the H_kv key/value heads only
        assert need_f >= 2 * H_kv * 64 * 4
        assert need_b >= 2 * 64 * 4 * 64 * 2 + 3 * 2 * 4 * 64 * 4
        assert _fwd_gqa(H_kv, wsb=need_f - 1) == _lib.ATTN_ERR_WORKSPACE
        assert _bwd_gqa(H_kv, wsb=need_b - 1) == _lib.ATTN_ERR_WORKSPACE
        assert _fwd_gqa(H_kv, q=None) == _lib.ATTN_ERR_INVALID_ARG
        assert _bwd_gqa(H_kv, dk=P + 4) == _lib.ATTN_ERR_INVALID_ARG
        assert _bwd_gqa(H_kv, dv=ALIGNED[6]) == _lib.ATTN_ERR_INVALID_ARG
        assert _fwd_gqa(H_kv, D=96) == _lib.ATTN_ERR_UNSUPPORTED
    assert sw.fwd_workspace_bytes(2, 64, 4, 64, 1) < sw.fwd_workspace_bytes(2, 64, 4, 64, 4)
    assert sw.fwd_workspace_bytes(2, 64, 4, 64, 4) == sw.fwd_workspace_bytes(2, 64, 4, 64)
    assert sw.bwd_workspace_bytes(2, 64, 4, 64, 4) == sw.bwd_workspace_bytes(2, 64, 4, 64)
    nulls = dict(q=None, k=None, v=None, o=None, lse=None, ws=None)
    assert _fwd_gqa(0, wsb=0, H=0, **nulls) == _lib.ATTN_OK


def _fwd_rope(wsb=1 << 40, **kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], c=ALIGNED[10], s=ALIGNED[11], o=ALIGNED[3],
             lse=ALIGNED[4], ws=ALIGNED[5], B=2, T=64, H=4, H_kv=2, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_fwd_rope(a["q"], a["k"], a["v"], a["c"], a["s"], a["o"], a["lse"], a["ws"],
                                    wsb, a["B"], a["T"], a["H"], a["H_kv"], a["D"], a["window"],
                                    a["causal"], a["eps"], None)


def _bwd_rope(wsb=1 << 40, **kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], c=ALIGNED[10], s=ALIGNED[11], o=ALIGNED[3],
             lse=ALIGNED[4], do=ALIGNED[5], dq=ALIGNED[6], dk=ALIGNED[7], dv=ALIGNED[8], ws=ALIGNED[9],
             B=2, T=64, H=4, H_kv=2, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_bwd_rope(a["q"], a["k"], a["v"], a["c"], a["s"], a["o"], a["lse"], a["do"],
                                    a["dq"], a["dk"], a["dv"], a["ws"], wsb, a["B"], a["T"], a["H"],
                                    a["H_kv"], a["D"], a["window"], a["causal"], a["eps"], None)


ROPE_INVALID = [dict(c=None), dict(s=None), dict(c=P + 8), dict(s=P + 2), dict(H_kv=3), dict(H_kv=0),
                dict(window=-2), dict(eps=0.0), dict(q=None)]


@pytest.mark.parametrize("kw", ROPE_INVALID, ids=[str(k) for k in ROPE_INVALID])
def test_rope_invalid(kw):
    assert _fwd_rope(**kw) == _lib.ATTN_ERR_INVALID_ARG
    assert _bwd_rope(**kw) == _lib.ATTN_ERR_INVALID_ARG


def test_rope_aliasing_workspace_unsupported():
    assert _fwd_rope(o=ALIGNED[10]) == _lib.ATTN_ERR_INVALID_ARG       # output over the cos table
    assert _bwd_rope(dk=ALIGNED[11]) == _lib.ATTN_ERR_INVALID_ARG      # output over the sin table
    assert _fwd_rope(D=96) == _lib.ATTN_ERR_UNSUPPORTED
    assert _bwd_rope(causal=0) == _lib.ATTN_ERR_UNSUPPORTED
    need_f = sw.fwd_rope_workspace_bytes(2, 64, 4, 64, 2)
    need_b = sw.bwd_rope_workspace_bytes(2, 64, 4, 64, 2)
    # the rotated keys, bf16 [B, T, H_kv, D], come on top of the plain workspaces
    assert need_f >= sw.fwd_workspace_bytes(2, 64, 4, 64, 2) + 2 * 64 * 2 * 64 * 2
    assert need_b >= sw.bwd_workspace_bytes(2, 64, 4, 64, 2) + 2 * 64 * 2 * 64 * 2
    assert _fwd_rope(wsb=need_f - 1) == _lib.ATTN_ERR_WORKSPACE
    assert _bwd_rope(wsb=need_b - 1) == _lib.ATTN_ERR_WORKSPACE
    assert _fwd_rope(ws=P + 16) == _lib.ATTN_ERR_WORKSPACE
    nulls = dict(q=None, k=None, v=None, c=None, s=None, o=None, lse=None, ws=None)
    assert _fwd_rope(wsb=0, T=0, **nulls) == _lib.ATTN_OK


def _fwd_ve(wsb=1 << 40, **kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], ve=ALIGNED[3], x=ALIGNED[4], xs=512, gw=ALIGNED[5],
             c=None, s=None, o=ALIGNED[6], lse=ALIGNED[7], ws=ALIGNED[8], B=2, T=64, H=4, H_kv=2, D=64,
             window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_fwd_ve(a["q"], a["k"], a["v"], a["ve"], a["x"], a["xs"], a["gw"], a["c"], a["s"],
                                  a["o"], a["lse"], a["ws"], wsb, a["B"], a["T"], a["H"], a["H_kv"], a["D"],
                                  a["window"], a["causal"], a["eps"], None)


def _bwd_ve(wsb=1 << 40, **kw):
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], ve=ALIGNED[3], x=ALIGNED[4], xs=512, gw=ALIGNED[5],
             c=None, s=None, o=ALIGNED[6], lse=ALIGNED[7], do=ALIGNED[8], dq=ALIGNED[9], dk=ALIGNED[10],
             dv=ALIGNED[11], dve=P + 12 * 0x1000000, dx=P + 13 * 0x1000000, dgw=P + 14 * 0x1000000,
             ws=P + 15 * 0x1000000, B=2, T=64, H=4, H_kv=2, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return _lib.lib().attn_bwd_ve(a["q"], a["k"], a["v"], a["ve"], a["x"], a["xs"], a["gw"], a["c"], a["s"],
                                  a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["dve"], a["dx"],
                                  a["dgw"], a["ws"], wsb, a["B"], a["T"], a["H"], a["H_kv"], a["D"],
                                  a["window"], a["causal"], a["eps"], None)


VE_INVALID = [dict(ve=None), dict(x=None), dict(gw=None), dict(ve=P + 8), dict(x=P + 4), dict(xs=16),
              dict(xs=36), dict(c=ALIGNED[10]), dict(s=ALIGNED[11]), dict(H_kv=3), dict(eps=-1.0)]


@pytest.mark.parametrize("kw", VE_INVALID, ids=[str(k) for k in VE_INVALID])
def test_ve_invalid(kw):
    assert _fwd_ve(**kw) == _lib.ATTN_ERR_INVALID_ARG
    assert _bwd_ve(**kw) == _lib.ATTN_ERR_INVALID_ARG


def test_ve_outputs_workspace_unsupported():
    for kw in (dict(dve=None), dict(dx=None), dict(dgw=P + 4), dict(dve=ALIGNED[3]), dict(dx=ALIGNED[4]),
               dict(dgw=ALIGNED[9]), dict(dve=ALIGNED[10])):
        assert _bwd_ve(**kw) == _lib.ATTN_ERR_INVALID_ARG, kw
    assert _fwd_ve(o=ALIGNED[3]) == _lib.ATTN_ERR_INVALID_ARG      # output over ve
    assert _fwd_ve(H=32, H_kv=32) == _lib.ATTN_ERR_UNSUPPORTED      # more key/value heads than the gate kernels take
    need_f = sw.fwd_ve_workspace_bytes(2, 64, 4, 64, 2)
    need_b = sw.bwd_ve_workspace_bytes(2, 64, 4, 64, 2)
    # the gated values on top of the rope workspace
    assert need_f >= sw.fwd_rope_workspace_bytes(2, 64, 4, 64, 2) + 2 * 64 * 2 * 64 * 2
    # gated values, the gate, dz and the partial sums of dgate_w on top of the rope workspace
    assert need_b >= sw.bwd_rope_workspace_bytes(2, 64, 4, 64, 2) + 2 * 64 * 2 * 64 * 2 + 2 * 2 * 2 * 64 * 4
    assert _fwd_ve(wsb=need_f - 1) == _lib.ATTN_ERR_WORKSPACE
    assert _bwd_ve(wsb=need_b - 1) == _lib.ATTN_ERR_WORKSPACE
    nulls = dict(q=None, k=None, v=None, ve=None, x=None, gw=None, o=None, lse=None, ws=None)
    assert _fwd_ve(wsb=0, B=0, **nulls) == _lib.ATTN_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(H=0)])
def test_empty_problem_is_ok_and_touches_nothing(kw):
    nulls = dict(q=None, k=None, v=None, o=None, lse=None, ws=None, wsb=0)
    assert _fwd(**kw, **nulls) == _lib.ATTN_OK
    assert _bwd(**kw, **nulls, do=None, dq=None, dk=None, dv=None) == _lib.ATTN_OK


# ---- backward entry points that reuse the forward's key pre-pass

FWS = P + 20 * 0x1000000   # a distinct, 256-byte aligned fake forward workspace


def _bwd_reuse(kind, fws=FWS, fwsb=1 << 40, wsb=1 << 40, **kw):
    L = _lib.lib()
    if kind == "gqa":
        a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], o=ALIGNED[3], lse=ALIGNED[4], do=ALIGNED[5],
                 dq=ALIGNED[6], dk=ALIGNED[7], dv=ALIGNED[8], ws=ALIGNED[9], B=2, T=64, H=4, H_kv=2, D=64,
                 window=8, causal=1, eps=1e-6)
        a.update(kw)
        return L.attn_bwd_gqa_reuse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                    a["dv"], fws, fwsb, a["ws"], wsb, a["B"], a["T"], a["H"],
                                    a["H_kv"], a["D"], a["window"], a["causal"], a["eps"], None)
    if kind == "rope":
        a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], c=ALIGNED[10], s=ALIGNED[11], o=ALIGNED[3],
                 lse=ALIGNED[4], do=ALIGNED[5], dq=ALIGNED[6], dk=ALIGNED[7], dv=ALIGNED[8], ws=ALIGNED[9],
                 B=2, T=64, H=4, H_kv=2, D=64, window=8, causal=1, eps=1e-6)
        a.update(kw)
        return L.attn_bwd_rope_reuse(a["q"], a["k"], a["v"], a["c"], a["s"], a["o"], a["lse"], a["do"],
                                     a["dq"], a["dk"], a["dv"], fws, fwsb, a["ws"], wsb, a["B"], a["T"],
                                     a["H"], a["H_kv"], a["D"], a["window"], a["causal"], a["eps"], None)
    a = dict(q=ALIGNED[0], k=ALIGNED[1], v=ALIGNED[2], ve=ALIGNED[3], x=ALIGNED[4], xs=512, gw=ALIGNED[5],
             c=None, s=None, o=ALIGNED[6], lse=ALIGNED[7], do=ALIGNED[8], dq=ALIGNED[9], dk=ALIGNED[10],
             dv=ALIGNED[11], dve=P + 12 * 0x1000000, dx=P + 13 * 0x1000000, dgw=P + 14 * 0x1000000,
             ws=P + 15 * 0x1000000, B=2, T=64, H=4, H_kv=2, D=64, window=8, causal=1, eps=1e-6)
    a.update(kw)
    return L.attn_bwd_ve_reuse(a["q"], a["k"], a["v"], a["ve"], a["x"], a["xs"], a["gw"], a["c"], a["s"],
                               a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["dve"], a["dx"],
                               a["dgw"], fws, fwsb, a["ws"], wsb, a["B"], a["T"], a["H"], a["H_kv"],
                               a["D"], a["window"], a["causal"], a["eps"], None)


@pytest.mark.parametrize("kind", ["gqa", "rope", "ve"])
def test_reuse_rejects_bad_forward_workspace(kind):
    fwd_bytes = {"gqa": sw.fwd_workspace_bytes(2, 64, 4, 64, 2),
                 "rope": sw.fwd_rope_workspace_bytes(2, 64, 4, 64, 2),
                 "ve": sw.fwd_ve_workspace_bytes(2, 64, 4, 64, 2)}[kind]
    ws = ALIGNED[9] if kind != "ve" else P + 15 * 0x1000000
    dq = ALIGNED[6] if kind != "ve" else ALIGNED[9]
    assert _bwd_reuse(kind, fws=None) == _lib.ATTN_ERR_WORKSPACE
    assert _bwd_reuse(kind, fwsb=fwd_bytes - 1) == _lib.ATTN_ERR_WORKSPACE
    assert _bwd_reuse(kind, fws=FWS + 16) == _lib.ATTN_ERR_WORKSPACE      # not 256-byte aligned
    assert _bwd_reuse(kind, fws=ws) == _lib.ATTN_ERR_WORKSPACE            # the backward's own workspace
    assert _bwd_reuse(kind, fws=dq) == _lib.ATTN_ERR_INVALID_ARG          # an output
    # the other rules are those of the plain backward
    assert _bwd_reuse(kind, eps=0.0) == _lib.ATTN_ERR_INVALID_ARG
    assert _bwd_reuse(kind, wsb=0) == _lib.ATTN_ERR_WORKSPACE
    # an empty problem needs no memory at all
    assert _bwd_reuse(kind, fws=None, fwsb=0, wsb=0, B=0) == _lib.ATTN_OK


def test_forward_ve_workspace_keeps_the_gate():
    # the gate (fp32 [B, H_kv, T]) follows the gated values in the forward workspace
    assert (sw.fwd_ve_workspace_bytes(2, 64, 4, 64, 2)
            >= sw.fwd_rope_workspace_bytes(2, 64, 4, 64, 2) + 2 * 64 * 2 * 64 * 2 + 2 * 2 * 64 * 4)
