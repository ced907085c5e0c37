"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance for every bf16 output and the fp32 lse: an element passes iff
|gpu - oracle| <= 2e-2 + 1e-2 * |oracle| (max-abs 2e-2, max-rel 1e-2).
Small shapes are compared element by element over every output; the
full-size workloads (in the launch configuration bench.py times) on sampled
rows and keys the oracle computes one by one.
"""
import sys

import numpy as np
import pytest

import oracle
from tests import rounding_model
from workloads import (make_layer_inputs, make_gate_inputs, WORKLOADS, workload, bf16_bits_to_f32,
                       rope_tables_bf16)

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2
EPS = 1e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _to_dev(torch, bits):
    t = torch.from_numpy(bits.view(np.int16).copy())
    return t.view(torch.bfloat16).cuda()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close(name, got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - want)
    bad = err > ATOL + RTOL * np.abs(want)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {bad.sum()} / {bad.size} elements out of tolerance; "
                             f"first at {tuple(idx)}: got {got[tuple(idx)]}, want {want[tuple(idx)]}; "
                             f"max abs err {err.max():.3g}")
    return float(err.max())


def _close_named(name, got, want, model, allowed):
    """The check of a (case, tensor) that tests/precision_exceptions.py names:
    got within the stated tolerance of the model of the kernels' stated
    rounding at every element; within the stated tolerance of the oracle,
    widened at each element by the model's own distance from the oracle; and
    outside the plain bound on at most `allowed` elements (-1: any number),
    each of them one where the model is outside it too."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    model = np.asarray(model, dtype=np.float64)
    _close(f"{name} vs the rounding model", got, model)
    err = np.abs(got - want)
    dev = np.abs(model - want)
    bound = ATOL + RTOL * np.abs(want)
    wide = err > bound + dev
    assert not wide.any(), (f"{name}: {wide.sum()} elements beyond the bound plus the model's deviation; "
                            f"max err {err.max():.3g}")
    out = err > bound
    assert allowed < 0 or out.sum() <= allowed, f"{name}: {out.sum()} elements outside the bound, {allowed} named"
    assert not (out & ~(dev > bound)).any(), f"{name}: outside the bound where the rounding model is not"
    return int(out.sum())


def _check(case_id, name, got, want, model=None):
    """Plain element-wise bound, or the named check of precision_exceptions."""
    from tests.precision_exceptions import allowed
    a = allowed(case_id, name)
    if a is None:
        _close(name, got, want)
        if model is not None:
            _close(f"{name} vs the rounding model", got, model)
    else:
        assert model is not None, f"{case_id} {name}: the named check needs the rounding model"
        _close_named(name, got, want, model, a)


def _fwd_ws(torch, nbytes, reuse):
    """A forward workspace kept for the backward (reuse), else None (the
    library call allocates its own and the backward runs its own pre-pass)."""
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda") if reuse else None


def _run(torch, inp, window, eps=EPS, reuse=False):
    import sliding_window_causal_qk_amd as sw
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    B, T, H, D = q.shape
    fws = _fwd_ws(torch, sw.fwd_workspace_bytes(B, T, H, D, k.shape[2]), reuse)
    o, lse = sw.attn_fwd(q, k, v, window, True, eps, workspace=fws)
    dq, dk, dv = sw.attn_bwd(q, k, v, o, lse, do, window, True, eps, fwd_workspace=fws)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


SMALL = [
    # (B, T, H, D, W, seed)
    (1, 128, 2, 64, 64, 0),      # the tiny workload
    (1, 1, 1, 64, 0, 1),
    (1, 5, 2, 128, 2, 2),
    (2, 100, 3, 128, 0, 3),
    (2, 100, 3, 64, 1, 4),
    (1, 129, 2, 128, 64, 5),
    (2, 257, 2, 64, -1, 6),
    (1, 255, 1, 128, 127, 7),
    (2, 333, 3, 128, 100, 8),
    (1, 384, 2, 128, 383, 9),
    (1, 300, 2, 64, 1000, 10),
    (1, 512, 4, 128, 256, 11),
    (1, 448, 2, 128, 63, 12),
    (1, 448, 2, 128, 65, 13),
    # head size 256 (the tutorial's tuning table, §10.1.1, goes up to 256)
    (1, 300, 2, 256, 100, 14),
    (2, 257, 2, 256, -1, 15),
    (1, 129, 1, 256, 64, 16),
    (1, 20, 2, 256, 3, 17),
]


@pytest.mark.parametrize("B,T,H,D,W,seed", SMALL, ids=[f"B{c[0]}T{c[1]}H{c[2]}D{c[3]}W{c[4]}" for c in SMALL])
def test_small_full_parity(torch_dev, B, T, H, D, W, seed):
    _say(f"[parity] small B={B} T={T} H={H} D={D} W={W} seed={seed}")
    inp = make_layer_inputs(B, T, H, D, seed)
    qf, kf, vf, dof = inp.as_f32()
    o, lse, dq, dk, dv = _run(torch_dev, inp, W)
    ro, rl = oracle.attention_fwd(qf, kf, vf, W, True, EPS)
    rq, rk, rv = oracle.attention_bwd(qf, kf, vf, dof, W, True, EPS)
    _close("o", _np(o), ro)
    _close("lse", _np(lse), rl)
    _close("dq", _np(dq), rq)
    _close("dk", _np(dk), rk)
    _close("dv", _np(dv), rv)


GQA_SMALL = [
    # (B, T, H, H_kv, D, W, seed): grouped key/value heads
    (1, 128, 4, 2, 64, 64, 40),
    (1, 20, 4, 2, 128, 5, 41),     # one query block per key tile: every step changes query head
    (2, 257, 4, 1, 128, 100, 42),
    (1, 300, 6, 3, 128, -1, 43),
    (2, 333, 4, 2, 64, 0, 44),
    (1, 448, 8, 2, 128, 65, 45),
    (1, 129, 2, 1, 64, 2000, 46),
    (1, 200, 4, 2, 256, 70, 47),
]


@pytest.mark.parametrize("B,T,H,H_kv,D,W,seed", GQA_SMALL,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}Hkv{c[3]}D{c[4]}W{c[5]}" for c in GQA_SMALL])
def test_gqa_small_full_parity(torch_dev, B, T, H, H_kv, D, W, seed):
    _say(f"[parity] gqa B={B} T={T} H={H} H_kv={H_kv} D={D} W={W} seed={seed}")
    inp = make_layer_inputs(B, T, H, D, seed, H_kv=H_kv)
    qf, kf, vf, dof = inp.as_f32()
    o, lse, dq, dk, dv = _run(torch_dev, inp, W)
    assert tuple(dk.shape) == (B, T, H_kv, D) and tuple(dv.shape) == (B, T, H_kv, D)
    ro, rl = oracle.attention_fwd(qf, kf, vf, W, True, EPS)
    rq, rk, rv = oracle.attention_bwd(qf, kf, vf, dof, W, True, EPS)
    _close("o", _np(o), ro)
    _close("lse", _np(lse), rl)
    _close("dq", _np(dq), rq)
    _close("dk", _np(dk), rk)
    _close("dv", _np(dv), rv)


def test_gqa_entry_with_equal_heads_is_the_plain_entry(torch_dev):
    """attn_fwd_gqa / attn_bwd_gqa with H_kv = H give bit-identical results to
    attn_fwd / attn_bwd."""
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    B, T, H, D, W = 1, 200, 2, 128, 60
    _say(f"[parity] gqa entry with H_kv = H, T={T}")
    inp = make_layer_inputs(B, T, H, D, 47)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    L = sw.lib()
    s = torch.cuda.current_stream().cuda_stream
    outs = []
    for gqa in (False, True):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        wf = torch.empty(sw.fwd_workspace_bytes(B, T, H, D, H), dtype=torch.uint8, device="cuda")
        wb = torch.empty(sw.bwd_workspace_bytes(B, T, H, D, H), dtype=torch.uint8, device="cuda")
        head = (H, H) if gqa else (H,)
        f = L.attn_fwd_gqa if gqa else L.attn_fwd
        bw = L.attn_bwd_gqa if gqa else L.attn_bwd
        sw.check(f(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), wf.data_ptr(),
                   wf.numel(), B, T, *head, D, W, 1, EPS, s), "fwd")
        sw.check(bw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), wb.data_ptr(), wb.numel(), B, T, *head, D,
                    W, 1, EPS, s), "bwd")
        torch.cuda.synchronize()
        outs.append((o, lse, dq, dk, dv))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_gqa_autograd(torch_dev):
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    _say("[parity] gqa autograd wrapper")
    inp = make_layer_inputs(1, 200, 4, 128, 48, H_kv=2)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    ref = _run(torch, inp, 50)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = sw.attention(qq, kk, vv, 50)
    o.backward(do)
    assert torch.equal(o.detach(), ref[0])
    assert torch.equal(qq.grad, ref[2]) and torch.equal(kk.grad, ref[3]) and torch.equal(vv.grad, ref[4])


# The persistent dK/dV kernel runs one workgroup per compute unit (256 on
# MI355X; two per unit at D = 64) over B * H_kv * ceil(T / BNK) key tiles
# (BNK = 128 keys, 64 at D = 256).  These cases have more tiles than
# workgroups, so some workgroups run two or more tiles in a row: the stream of
# query blocks that carries on across tiles and the prefetch of the next
# tile's K and V rows are compared element by element.
MULTI_TILE = [
    # (B, T, H, H_kv, D, W, rope, gate C or 0, reuse, seed)
    (16, 768, 8, 8, 64, 300, False, 0, True, 7001),
    (8, 1024, 8, 8, 128, 300, False, 0, True, 7002),
    (8, 1024, 8, 8, 256, 400, False, 0, True, 7003),
    (9, 1000, 8, 4, 128, 333, False, 0, True, 7004),     # grouped heads, ragged T
    (9, 1000, 8, 4, 128, -1, True, 0, True, 7005),       # rotary embedding, full causal
    (9, 1000, 8, 4, 128, 200, False, 64, True, 7006),    # value-embedding gate
    (3, 1100, 11, 11, 128, 129, False, 0, False, 7007),  # tile count not a multiple of 8
    (16, 768, 8, 8, 64, 0, False, 0, False, 7008),
    (24, 768, 8, 4, 64, 200, False, 0, True, 7009),      # D = 64 (two workgroups per CU), grouped heads
    (28, 640, 4, 4, 64, 150, True, 64, True, 7010),      # D = 64, rotary embedding and gate
]
N_CU = 256


@pytest.mark.parametrize("B,T,H,H_kv,D,W,rope,C,reuse,seed", MULTI_TILE,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}Hkv{c[3]}D{c[4]}W{c[5]}{'rope' if c[6] else ''}C{c[7]}"
                              for c in MULTI_TILE])
def test_multi_tile_full_parity(torch_dev, B, T, H, H_kv, D, W, rope, C, reuse, seed):
    torch = torch_dev
    bnk, grid = (64 if D == 256 else 128), N_CU * (2 if D <= 64 else 1)
    assert B * H_kv * -(-T // bnk) > grid, "the case must give some workgroup a second key tile"
    assert torch.cuda.get_device_properties(0).multi_processor_count <= N_CU
    _say(f"[parity] multi-tile B={B} T={T} H={H} H_kv={H_kv} D={D} W={W} rope={rope} C={C} seed={seed}")
    inp = make_layer_inputs(B, T, H, D, seed, H_kv=H_kv)
    qf, kf, vf, dof = inp.as_f32()
    tables = rope_tables_bf16(T, D) if rope else None
    c, sn = (bf16_bits_to_f32(t) for t in tables) if rope else (None, None)
    cid = f"B{B}T{T}H{H}Hkv{H_kv}D{D}W{W}{'rope' if rope else ''}C{C}"
    gk = {}
    if C:
        gi = make_gate_inputs(B, T, H_kv, D, C, seed + 100)
        vef, xf = bf16_bits_to_f32(gi.ve), bf16_bits_to_f32(gi.x)
        gk = dict(ve=vef, xg=xf, gate_w=gi.gate_w)
        got = _run_ve(torch, inp, gi, W, tables, reuse=reuse)
        want = oracle.attention_fwd_ve(qf, kf, vf, vef, xf, gi.gate_w, W, True, EPS, c, sn) + \
            oracle.attention_bwd_ve(qf, kf, vf, dof, vef, xf, gi.gate_w, W, True, EPS, c, sn)
        names = ("o", "lse", "dq", "dk", "dv", "dve", "dx32", "dgate_w")
    elif rope:
        got = _run_rope(torch, inp, tables, W, reuse=reuse)
        want = oracle.attention_fwd_rope(qf, kf, vf, c, sn, W, True, EPS) + \
            oracle.attention_bwd_rope(qf, kf, vf, dof, c, sn, W, True, EPS)
        names = ("o", "lse", "dq", "dk", "dv")
    else:
        got = _run(torch, inp, W, reuse=reuse)
        want = oracle.attention_fwd(qf, kf, vf, W, True, EPS) + oracle.attention_bwd(qf, kf, vf, dof, W, True, EPS)
        names = ("o", "lse", "dq", "dk", "dv")
    from tests.precision_exceptions import allowed
    model = [None] * len(names)
    if any(allowed(cid, n) is not None for n in names):   # the rounding model only where a check names it
        mo, ml = rounding_model.forward(qf, kf, vf, W, EPS, c, sn, **gk)
        model = (mo, ml) + rounding_model.backward(qf, kf, vf, mo, ml, dof, W, EPS, c, sn, **gk)
    for name, g, w, m in zip(names, got, want, model):
        _check(cid, name, _np(g), w, m)


ROPE_SMALL = [
    # (B, T, H, H_kv, D, W, seed): rotary embedding ahead of the norm
    (1, 128, 2, 2, 64, 64, 50),
    (2, 257, 4, 2, 128, 100, 51),
    (1, 300, 2, 1, 128, -1, 52),
    (1, 20, 4, 2, 128, 5, 53),
    (2, 333, 2, 2, 64, 0, 54),
    (1, 448, 2, 2, 128, 65, 55),
    (1, 1, 1, 1, 64, 0, 56),
    (1, 160, 2, 1, 256, 40, 57),
]


def _run_rope(torch, inp, tables, window, eps=EPS, reuse=False):
    import sliding_window_causal_qk_amd as sw
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    rope = tuple(_to_dev(torch, t) for t in tables)
    B, T, H, D = q.shape
    fws = _fwd_ws(torch, sw.fwd_rope_workspace_bytes(B, T, H, D, k.shape[2]), reuse)
    o, lse = sw.attn_fwd(q, k, v, window, True, eps, rope=rope, workspace=fws)
    dq, dk, dv = sw.attn_bwd(q, k, v, o, lse, do, window, True, eps, rope=rope, fwd_workspace=fws)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("B,T,H,H_kv,D,W,seed", ROPE_SMALL,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}Hkv{c[3]}D{c[4]}W{c[5]}" for c in ROPE_SMALL])
def test_rope_small_full_parity(torch_dev, B, T, H, H_kv, D, W, seed):
    _say(f"[parity] rope B={B} T={T} H={H} H_kv={H_kv} D={D} W={W} seed={seed}")
    inp = make_layer_inputs(B, T, H, D, seed, H_kv=H_kv)
    tables = rope_tables_bf16(T, D)
    c, sn = (bf16_bits_to_f32(t) for t in tables)
    qf, kf, vf, dof = inp.as_f32()
    o, lse, dq, dk, dv = _run_rope(torch_dev, inp, tables, W)
    ro, rl = oracle.attention_fwd_rope(qf, kf, vf, c, sn, W, True, EPS)
    rq, rk, rv = oracle.attention_bwd_rope(qf, kf, vf, dof, c, sn, W, True, EPS)
    _close("o", _np(o), ro)
    _close("lse", _np(lse), rl)
    _close("dq", _np(dq), rq)
    _close("dk", _np(dk), rk)
    _close("dv", _np(dv), rv)


def test_rope_with_identity_tables_is_the_plain_path(torch_dev):
    """cos = 1, sin = 0 rotates nothing: bit-identical to the plain entry points
    (the rotated keys are the keys, the norm sees the same values)."""
    torch = torch_dev
    B, T, H, D, W = 1, 200, 2, 128, 60
    _say("[parity] rope with identity tables")
    inp = make_layer_inputs(B, T, H, D, 57)
    ones = np.full((T, D // 2), 0x3F80, dtype=np.uint16)    # bf16 1.0
    zeros = np.zeros((T, D // 2), dtype=np.uint16)
    a = _run(torch, inp, W)
    b = _run_rope(torch, inp, (ones, zeros), W)
    for name, x, y in zip(("o", "lse", "dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), name


def test_rope_autograd(torch_dev):
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    _say("[parity] rope autograd wrapper")
    inp = make_layer_inputs(1, 200, 4, 128, 58, H_kv=2)
    tables = rope_tables_bf16(200, 128)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    rope = tuple(_to_dev(torch, t) for t in tables)
    ref = _run_rope(torch, inp, tables, 50)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = sw.attention(qq, kk, vv, 50, rope=rope)
    o.backward(do)
    assert torch.equal(o.detach(), ref[0])
    assert torch.equal(qq.grad, ref[2]) and torch.equal(kk.grad, ref[3]) and torch.equal(vv.grad, ref[4])


VE_SMALL = [
    # (B, T, H, H_kv, D, W, C, rope, seed): value-embedding gate (C: block input width)
    (1, 128, 2, 2, 64, 64, 64, False, 60),
    (2, 257, 4, 2, 128, 100, 512, False, 61),
    (1, 300, 2, 1, 128, -1, 40, True, 62),
    (1, 20, 4, 2, 128, 5, 64, True, 63),
    (2, 333, 2, 2, 64, 0, 32, False, 64),
    (1, 1, 1, 1, 64, 0, 32, False, 65),
    (1, 150, 2, 2, 256, 30, 64, True, 67),
]


def _gate_dev(torch, gi):
    ve, x = (_to_dev(torch, t) for t in (gi.ve, gi.x))
    return ve, x, torch.from_numpy(gi.gate_w.copy()).cuda()


def _run_ve(torch, inp, gi, window, tables=None, eps=EPS, reuse=False):
    import sliding_window_causal_qk_amd as sw
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    gate = _gate_dev(torch, gi)
    rope = None if tables is None else tuple(_to_dev(torch, t) for t in tables)
    B, T, H, D = q.shape
    fws = _fwd_ws(torch, sw.fwd_ve_workspace_bytes(B, T, H, D, k.shape[2]), reuse)
    o, lse = sw.attn_fwd(q, k, v, window, True, eps, rope=rope, gate=gate, workspace=fws)
    grads = sw.attn_bwd(q, k, v, o, lse, do, window, True, eps, rope=rope, gate=gate, fwd_workspace=fws)
    torch.cuda.synchronize()
    return (o, lse) + tuple(grads)


@pytest.mark.parametrize("B,T,H,H_kv,D,W,C,rope,seed", VE_SMALL,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}Hkv{c[3]}D{c[4]}W{c[5]}C{c[6]}{'rope' if c[7] else ''}"
                              for c in VE_SMALL])
def test_ve_small_full_parity(torch_dev, B, T, H, H_kv, D, W, C, rope, seed):
    _say(f"[parity] ve gate B={B} T={T} H={H} H_kv={H_kv} D={D} W={W} C={C} rope={rope} seed={seed}")
    inp = make_layer_inputs(B, T, H, D, seed, H_kv=H_kv)
    gi = make_gate_inputs(B, T, H_kv, D, C, seed + 100)
    tables = rope_tables_bf16(T, D) if rope else None
    c, sn = (bf16_bits_to_f32(t) for t in tables) if rope else (None, None)
    qf, kf, vf, dof = inp.as_f32()
    vef, xf = bf16_bits_to_f32(gi.ve), bf16_bits_to_f32(gi.x)
    got = _run_ve(torch_dev, inp, gi, W, tables)
    ro, rl = oracle.attention_fwd_ve(qf, kf, vf, vef, xf, gi.gate_w, W, True, EPS, c, sn)
    ref = oracle.attention_bwd_ve(qf, kf, vf, dof, vef, xf, gi.gate_w, W, True, EPS, c, sn)
    mo, ml = rounding_model.forward(qf, kf, vf, W, EPS, c, sn, ve=vef, xg=xf, gate_w=gi.gate_w)
    mod = (mo, ml) + rounding_model.backward(qf, kf, vf, mo, ml, dof, W, EPS, c, sn, ve=vef, xg=xf,
                                             gate_w=gi.gate_w)
    cid = f"B{B}T{T}H{H}Hkv{H_kv}D{D}W{W}C{C}{'rope' if rope else ''}"
    for name, g, want, m in zip(("o", "lse", "dq", "dk", "dv", "dve", "dx32", "dgate_w"), got, (ro, rl) + ref,
                                mod):
        _check(cid, name, _np(g), want, m)


def test_ve_autograd(torch_dev):
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    _say("[parity] ve gate autograd wrapper")
    B, T, H, H_kv, D, C = 1, 200, 4, 2, 128, 48
    inp = make_layer_inputs(B, T, H, D, 66, H_kv=H_kv)
    gi = make_gate_inputs(B, T, H_kv, D, C, 166)
    ref = _run_ve(torch, inp, gi, 50)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    ve, x, gw = (t.clone().requires_grad_(True) for t in _gate_dev(torch, gi))
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = sw.attention(qq, kk, vv, 50, gate=(ve, x, gw))
    o.backward(do)
    assert torch.equal(o.detach(), ref[0])
    for g, r in ((qq.grad, ref[2]), (kk.grad, ref[3]), (vv.grad, ref[4]), (ve.grad, ref[5]),
                 (x.grad[..., :32], ref[6]), (gw.grad, ref[7])):
        assert torch.equal(g, r)
    assert float(x.grad[..., 32:].abs().max()) == 0.0


def _sample_rows(T, W, rng, n=6):
    fixed = [0, 1, 63, 64, 127, 128, T // 2, T - 2, T - 1]
    if W >= 0:
        fixed += [W - 1, W, W + 1, W + 64]
    rows = sorted({r for r in fixed if 0 <= r < T} | set(rng.integers(0, T, n).tolist()))
    return rows


def _sample_keys(T, W, rng):
    """One key in every 128-key tile (the unit of the persistent dK/dV kernel),
    plus the sequence ends and the keys at the window's edge."""
    ks = {min(T - 1, 128 * t + int(rng.integers(0, 128))) for t in range((T + 127) // 128)}
    ks |= {0, 1, 127, 128, T - 129, T - 128, T - 2, T - 1}
    if 0 <= W < T:
        ks |= {T - 2 - W, T - 1 - W, T - W}
    return sorted(k for k in ks if 0 <= k < T)


def _sampled_check(torch, wl, layer, window, slices, whole=()):
    """Sampled rows and keys of `slices`; every row and key of the (b, h)
    slices in `whole`."""
    # full-size runs take the path bench.py times: the backward reuses the
    # forward's key pre-pass
    inp = make_layer_inputs(wl.B, wl.T, wl.H, wl.D, wl.seed(layer), wl.sigma_qkv, wl.sigma_do,
                            H_kv=wl.H_kv)
    qf, kf, vf, dof = inp.as_f32()
    if wl.ve_gate:
        # the gated values are v' = v + gate ve: the oracle runs on v' (fp64)
        gi = make_gate_inputs(wl.B, wl.T, wl.kv_heads, wl.D, wl.H * wl.D, wl.seed(layer) + 100)
        o, lse, dq, dk, dv, dve, dx32, _ = _run_ve(torch, inp, gi, window, None, wl.eps, reuse=True)
        gate = oracle.ve_gate(bf16_bits_to_f32(np.ascontiguousarray(gi.x[..., :32])), gi.gate_w)
        vef = bf16_bits_to_f32(gi.ve)
        vf = vf + gate[..., None] * vef
    elif wl.rope:
        tables = rope_tables_bf16(wl.T, wl.D)
        c, sn = (bf16_bits_to_f32(t) for t in tables)
        o, lse, dq, dk, dv = _run_rope(torch, inp, tables, window, wl.eps, reuse=True)
    else:
        o, lse, dq, dk, dv = _run(torch, inp, window, wl.eps, reuse=True)
    rng = np.random.default_rng(1234 + layer)
    for (b, h) in list(slices) + list(whole):
        if (b, h) in whole:
            rows = keys = list(range(wl.T))
        else:
            rows = _sample_rows(wl.T, window, rng)
            keys = _sample_keys(wl.T, window, rng)
        _say(f"    slice ({b}, {h}): {len(rows)} rows, {len(keys)} keys")
        if wl.rope:
            # the oracle on batch b's rotated q and k; gradients rotated back per row
            qb, kb = oracle.rope(qf[b:b + 1], c, sn), oracle.rope(kf[b:b + 1], c, sn)
            ro, rl = oracle.fwd_rows(qb, kb, vf[b:b + 1], 0, h, rows, window, True, wl.eps)
            sq, sk, sv = oracle.bwd_rows(qb, kb, vf[b:b + 1], dof[b:b + 1], 0, h, rows, keys, window,
                                         True, wl.eps)
            sq = oracle.rope_bwd(sq, c[rows], sn[rows])
            sk = oracle.rope_bwd(sk, c[keys], sn[keys])
        else:
            ro, rl = oracle.fwd_rows(qf, kf, vf, b, h, rows, window, True, wl.eps)
            sq, sk, sv = oracle.bwd_rows(qf, kf, vf, dof, b, h, rows, keys, window, True, wl.eps)
        _close(f"o[{b},{h}]", _np(o[b, rows, h]), ro)
        _close(f"lse[{b},{h}]", _np(lse[b, h, rows]), rl)
        hk = oracle.kv_head(h, wl.H, wl.kv_heads)   # dk, dv: the key/value head h reads
        _close(f"dq[{b},{h}]", _np(dq[b, rows, h]), sq)
        _close(f"dk[{b},{hk}]", _np(dk[b, keys, hk]), sk)
        _close(f"dv[{b},{hk}]", _np(dv[b, keys, hk]), sv)
        if wl.ve_gate:
            _close(f"dve[{b},{hk}]", _np(dve[b, keys, hk]), gate[b, keys, hk][:, None] * sv)
    if wl.ve_gate:
        # dx of sampled tokens: dz over every key/value head of each token
        b = slices[0][0]
        keys = _sample_keys(wl.T, window, rng)[:5]
        G = wl.H // wl.kv_heads
        dz = np.zeros((len(keys), wl.kv_heads))
        for hk in range(wl.kv_heads):
            _, _, sv = oracle.bwd_rows(qf, kf, vf, dof, b, hk * G, keys[:1], keys, window, True, wl.eps)
            g = gate[b, keys, hk]
            dz[:, hk] = np.sum(sv * vef[b, keys, hk], axis=1) * g * (1 - g / 2)
        _close(f"dx32[{b}]", _np(dx32[b, keys]), dz @ gi.gate_w.astype(np.float64))
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} has non-finite values"


@pytest.mark.parametrize("name", ["s_layer", "l_layer"])
def test_single_layer_workloads(torch_dev, name):
    """The pages' S and L layers at full size (B=8, T=2048, H=4, D=128), in the
    launch configuration bench.py times: every element of o, lse, dq, dk and
    dv of two whole (batch, head) slices, sampled rows and keys of a third."""
    wl = workload(name)
    _say(f"[parity] workload {name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} W={wl.explicit_window}")
    _sampled_check(torch_dev, wl, 0, wl.explicit_window, [(3, 2)], whole=[(0, 0), (wl.B - 1, wl.H - 1)])


@pytest.mark.parametrize("name,layer", [("sssl_stack", 0), ("sssl_stack", 3), ("long", 0), ("long", 3),
                                        ("gqa_sssl_stack", 0), ("gqa_sssl_stack", 3),
                                        ("rope_sssl_stack", 0), ("rope_sssl_stack", 3),
                                        ("ve_sssl_stack", 0), ("ve_sssl_stack", 3),
                                        ("d256_sssl_stack", 0), ("d256_sssl_stack", 3),
                                        ("t512_sssl_stack", 0), ("t512_sssl_stack", 7),
                                        ("t1024_sssl_stack", 0), ("slll_stack", 0), ("l_stack", 0),
                                        ("sl_stack", 1), ("ssss_stack", 0), ("ssss_stack", 7),
                                        ("d64_sssl_stack", 0), ("d64_sssl_stack", 3)])
def test_stack_and_long_workloads_sampled(torch_dev, name, layer):
    import sliding_window_causal_qk_amd as sw
    wl = workload(name)
    window = sw.layer_windows(wl.pattern, wl.n_layer, wl.T)[layer]
    _say(f"[parity] workload {name} layer {layer} B={wl.B} T={wl.T} H={wl.H} D={wl.D} W={window}")
    slices = [(0, 0), (wl.B - 1, wl.H - 1)]
    _sampled_check(torch_dev, wl, layer, window, slices)



def test_partial_schedule_rounds(torch_dev):
    """37 query tiles and 37 key tiles per (batch, head), 8 heads: 296 of each,
    so the forward and dQ grids fit the CUs at once with a last, partial round
    of 5 workgroups per XCD whose order is reversed, and the persistent dK/dV
    kernel runs two rounds, the second mirrored and partial (5 of 32 tiles per
    XCD).  Every element of one (batch, head) slice; sampled rows and keys
    (one key in every key tile) of two more."""
    from workloads import Workload
    wl = Workload("partial_rounds", B=1, T=37 * 128, H=8, D=128, pattern="W", n_layer=1, seed0=777,
                  explicit_window=300)
    _say(f"[parity] B={wl.B} T={wl.T} H={wl.H} D={wl.D} W=300: partial schedule rounds")
    _sampled_check(torch_dev, wl, 0, 300, [(0, 0), (0, 7)], whole=[(0, 3)])

# ------------------------------------------------------------ structured probes

def test_probe_one_hot_value_marks_window_edge(torch_dev):
    """v_{j*} = e_0, other values 0: o_{i,0} > 0 exactly where (i, j*) is visible."""
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    B, T, H, D, W = 1, 300, 1, 128, 100
    _say(f"[parity] probe one-hot V T={T} W={W}")
    inp = make_layer_inputs(B, T, H, D, 21)
    q, k = _to_dev(torch, inp.q), _to_dev(torch, inp.k)
    from oracle.attention import visible_mask
    mask = visible_mask(T, W)
    for jstar in (0, 99, 100, 101, 199, 299):
        v = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
        v[0, jstar, 0, 0] = 1.0
        o, _ = sw.attn_fwd(q, k, v, W)
        col = _np(o[0, :, 0, 0])
        assert np.array_equal(col > 0, mask[:, jstar]), jstar
        assert float(o[0, :, 0, 1:].abs().max()) == 0.0


def test_probe_identical_keys(torch_dev):
    """All keys equal: lse_i = s_i + ln(#visible) pins the key count per row."""
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    B, T, H, D, W = 1, 260, 2, 128, 70
    _say(f"[parity] probe identical keys T={T} W={W}")
    inp = make_layer_inputs(B, T, H, D, 22)
    kb = np.broadcast_to(inp.k[:, :1], inp.k.shape).copy()
    qf, _, vf, dof = inp.as_f32()
    kf = bf16_bits_to_f32(kb)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, kb, inp.v, inp.do))
    o, lse = sw.attn_fwd(q, k, v, W)
    dq, dk, dv = sw.attn_bwd(q, k, v, o, lse, do, W)
    ro, rl = oracle.attention_fwd(qf, kf, vf, W, True, EPS)
    rq, rk, rv = oracle.attention_bwd(qf, kf, vf, dof, W, True, EPS)
    _close("o", _np(o), ro)
    _close("lse", _np(lse), rl)
    _close("dq", _np(dq), rq)   # ~0: the rows of dS sum to zero
    _close("dk", _np(dk), rk)
    _close("dv", _np(dv), rv)
    assert float(dq.abs().max()) < 2e-2


def test_deterministic(torch_dev):
    torch = torch_dev
    inp = make_layer_inputs(2, 333, 2, 128, 30)
    _say("[parity] determinism")
    a = _run(torch, inp, 100)
    b = _run(torch, inp, 100)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function_matches_abi(torch_dev):
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    _say("[parity] autograd wrapper")
    inp = make_layer_inputs(1, 200, 2, 128, 31)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    ref = _run(torch, inp, 50)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = sw.attention(qq, kk, vv, 50)
    o.backward(do)
    assert torch.equal(o.detach(), ref[0])
    assert torch.equal(qq.grad, ref[2]) and torch.equal(kk.grad, ref[3]) and torch.equal(vv.grad, ref[4])


def test_empty_and_errors_on_device(torch_dev):
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    z = torch.empty((0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = sw.attn_fwd(z, z, z, 4)
    assert o.shape == z.shape and lse.shape == (0, 2, 16)
    x = torch.zeros((1, 16, 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sw.SwattnError):
        sw.attn_fwd(x, x, x, 4)


REUSE_CASES = [
    # (B, T, H, H_kv, D, W, rope, gate C or 0, seed)
    (2, 300, 2, 2, 128, 100, False, 0, 80),
    (1, 257, 4, 2, 64, -1, False, 0, 81),
    (1, 200, 4, 2, 128, 60, True, 0, 82),
    (2, 150, 2, 1, 128, 40, False, 64, 83),
    (1, 130, 2, 2, 256, 30, True, 40, 84),
]


@pytest.mark.parametrize("B,T,H,H_kv,D,W,rope,C,seed", REUSE_CASES,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}Hkv{c[3]}D{c[4]}W{c[5]}{'rope' if c[6] else ''}C{c[7]}"
                              for c in REUSE_CASES])
def test_backward_reusing_the_forward_workspace_is_bit_identical(torch_dev, B, T, H, H_kv, D, W, rope, C, seed):
    """The *_reuse entry points read the forward's key pre-pass instead of
    running it again; every output must equal the plain backward's bit for bit."""
    import sliding_window_causal_qk_amd as sw
    torch = torch_dev
    _say(f"[parity] reuse B={B} T={T} H={H} H_kv={H_kv} D={D} W={W} rope={rope} C={C} seed={seed}")
    inp = make_layer_inputs(B, T, H, D, seed, H_kv=H_kv)
    q, k, v, do = (_to_dev(torch, t) for t in (inp.q, inp.k, inp.v, inp.do))
    tables = tuple(_to_dev(torch, t) for t in rope_tables_bf16(T, D)) if rope else None
    gate = _gate_dev(torch, make_gate_inputs(B, T, H_kv, D, C, seed + 100)) if C else None
    nb = (sw.fwd_ve_workspace_bytes if gate is not None else
          sw.fwd_rope_workspace_bytes if rope else sw.fwd_workspace_bytes)(B, T, H, D, H_kv)
    fws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o, lse = sw.attn_fwd(q, k, v, W, True, EPS, rope=tables, gate=gate, workspace=fws)
    plain = sw.attn_bwd(q, k, v, o, lse, do, W, True, EPS, rope=tables, gate=gate)
    reuse = sw.attn_bwd(q, k, v, o, lse, do, W, True, EPS, rope=tables, gate=gate, fwd_workspace=fws)
    torch.cuda.synchronize()
    assert len(plain) == len(reuse)
    for i, (a, b) in enumerate(zip(plain, reuse)):
        assert torch.equal(a, b), f"output {i} differs"
