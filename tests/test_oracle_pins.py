"""Pins of the fp64 oracle to things other than itself.

Each check compares the oracle with something it does not compute the same
way: a pure-Python brute force on tiny inputs, torch's own RMSNorm and
scaled-dot-product attention (fp64, CPU) with autograd, central finite
differences, closed forms of special inputs, invariants of softmax, and values
printed on the pages (tests/golden/).  tests/test_oracle_mutants.py checks that
plausible mistakes planted in the oracle fail at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import schedule as S

EPS = 1e-6


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force

def brute_force_fwd(q, k, v, window, causal, eps):
    """Triple loop over (b, h, i) with explicit per-key visibility tests."""
    B, T, H, D = q.shape
    o = np.zeros((B, T, H, v.shape[3]))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            def normed(x):
                ms = sum(float(t) * float(t) for t in x) / len(x)
                return [float(t) / math.sqrt(ms + eps) for t in x]
            qn = [normed(q[b, t, h]) for t in range(T)]
            kn = [normed(k[b, t, h]) for t in range(T)]
            for i in range(T):
                keys = []
                for j in range(T):
                    if causal:
                        ok = j <= i and (window < 0 or i - j <= window)
                    else:
                        ok = window < 0 or abs(i - j) <= window
                    if ok:
                        keys.append(j)
                s = [sum(a * c for a, c in zip(qn[i], kn[j])) / math.sqrt(D) for j in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                lse[b, h, i] = m + math.log(z)
                for jj, j in enumerate(keys):
                    o[b, i, h] += (e[jj] / z) * v[b, j, h]
    return o, lse


@pytest.mark.parametrize("T,D,W,causal", [
    (1, 4, 0, True), (7, 4, 0, True), (9, 8, 3, True), (12, 4, 1, True),
    (11, 8, 10, True), (11, 8, 11, True), (10, 4, -1, True), (13, 8, 5, False),
    (8, 4, -1, False),
])
def test_fwd_matches_brute_force(T, D, W, causal):
    q, k, v = (_rand((2, T, 2, D), s) for s in (1, 2, 3))
    o, lse = oracle.attention_fwd(q, k, v, W, causal, EPS)
    ob, lb = brute_force_fwd(q, k, v, W, causal, EPS)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def test_n_visible_brute_force_and_closed_form():
    for T in (1, 2, 5, 16, 33):
        for W in (-1, 0, 1, 3, T - 2, T - 1, T, T + 5):
            if W < -1:
                continue
            brute = sum(1 for i in range(T) for j in range(T)
                        if j <= i and (W < 0 or i - j <= W))
            closed = sum((i if W < 0 else min(i, W)) + 1 for i in range(T))
            assert oracle.n_visible(T, W) == brute == closed
            brute_nc = sum(1 for i in range(T) for j in range(T) if W < 0 or abs(i - j) <= W)
            assert oracle.n_visible(T, W, causal=False) == brute_nc


def test_n_visible_workload_sizes():
    # closed form sum_i (min(i, W) + 1) at the five workloads' shapes
    assert oracle.n_visible(128, 64) == 6240
    assert oracle.n_visible(2048, 1024) == 1574400
    assert oracle.n_visible(2048, 2048) == 2098176 == 2048 * 2049 // 2
    assert oracle.n_visible(8192, 4096) == 25171968
    assert oracle.n_visible(8192, 8192) == 33558528 == 8192 * 8193 // 2


# ---------------------------------------------------------- library routines

def test_rms_norm_matches_torch():
    torch = pytest.importorskip("torch")
    x = _rand((5, 7, 3, 16), 4, 3.0)
    for eps in (1e-6, 1e-2, 0.5):
        xh, r = oracle.rms_norm(x, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (16,), eps=eps).numpy()
        np.testing.assert_allclose(xh, ref, rtol=1e-14, atol=1e-14)
        ms = np.mean(x * x, axis=-1)
        np.testing.assert_allclose(np.mean(xh * xh, axis=-1), ms / (ms + eps), rtol=1e-13)


def _torch_reference(q, k, v, do, window, causal, eps):
    """RMSNorm + scaled_dot_product_attention with a boolean band mask, fp64 CPU."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, T, H, D = q.shape
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    qn = F.rms_norm(qt, (D,), eps=eps).transpose(1, 2)
    kn = F.rms_norm(kt, (D,), eps=eps).transpose(1, 2)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    if causal:
        mask = (j <= i) & ((i - j <= window) if window >= 0 else torch.ones(T, T, dtype=torch.bool))
    else:
        mask = (abs(i - j) <= window) if window >= 0 else torch.ones(T, T, dtype=torch.bool)
    o = F.scaled_dot_product_attention(qn, kn, vt.transpose(1, 2), attn_mask=mask,
                                       enable_gqa=k.shape[2] != H)
    o = o.transpose(1, 2)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("T,D,W,causal", [
    (40, 16, 7, True), (40, 16, 0, True), (40, 16, -1, True), (33, 8, 39, True),
    (24, 16, 5, False), (64, 32, 31, True),
])
def test_fwd_bwd_match_torch_sdpa(T, D, W, causal):
    q, k, v, do = (_rand((2, T, 3, D), s) for s in (5, 6, 7, 8))
    o_ref, dq_ref, dk_ref, dv_ref = _torch_reference(q, k, v, do, W, causal, EPS)
    o, _ = oracle.attention_fwd(q, k, v, W, causal, EPS)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, causal, EPS)
    for a, b in ((o, o_ref), (dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


# ------------------------------------------------- grouped key/value heads

@pytest.mark.parametrize("H,H_kv,T,D,W", [
    (4, 2, 40, 16, 7), (4, 1, 33, 8, -1), (6, 3, 24, 16, 0), (6, 2, 48, 8, 13),
])
def test_gqa_matches_torch_sdpa(H, H_kv, T, D, W):
    """torch's SDPA with enable_gqa (query head h reads key/value head
    h // (H / H_kv)), autograd for the gradients of the shared heads."""
    q, do = (_rand((2, T, H, D), s) for s in (41, 42))
    k, v = (_rand((2, T, H_kv, D), s) for s in (43, 44))
    o_ref, dq_ref, dk_ref, dv_ref = _torch_reference(q, k, v, do, W, True, EPS)
    o, _ = oracle.attention_fwd(q, k, v, W, True, EPS)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, True, EPS)
    assert dk.shape == k.shape and dv.shape == v.shape
    for a, b in ((o, o_ref), (dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_gqa_equals_repeated_heads():
    """Grouped heads are the plain case with every key/value head repeated for
    its G query heads; the shared head's gradient is the sum over the group."""
    B, T, H, H_kv, D, W = 1, 30, 6, 2, 8, 5
    G = H // H_kv
    q, do = (_rand((B, T, H, D), s) for s in (45, 46))
    k, v = (_rand((B, T, H_kv, D), s) for s in (47, 48))
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o, lse = oracle.attention_fwd(q, k, v, W, True, EPS)
    o_r, lse_r = oracle.attention_fwd(q, kr, vr, W, True, EPS)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_r, rtol=0, atol=1e-14)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, True, EPS)
    dq_r, dk_r, dv_r = oracle.attention_bwd(q, kr, vr, do, W, True, EPS)
    np.testing.assert_allclose(dq, dq_r, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk_r.reshape(B, T, H_kv, G, D).sum(axis=3), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv_r.reshape(B, T, H_kv, G, D).sum(axis=3), rtol=0, atol=1e-13)


def test_gqa_rejects_uneven_groups():
    q = _rand((1, 4, 3, 4), 1)
    k = _rand((1, 4, 2, 4), 2)
    with pytest.raises(ValueError):
        oracle.attention_fwd(q, k, k, 2, True, EPS)


# ------------------------------------------------------- rotary embedding

def rope_tables(T, D, base=10000.0, offset=0):
    """Exact fp64 cos/sin tables: position t, pair i has angle t / base^(2i/D)."""
    inv = 1.0 / base ** (np.arange(0, D, 2) / D)
    ang = np.outer(np.arange(offset, offset + T), inv)
    return np.cos(ang), np.sin(ang)


def bf16_round(x):
    """Round to bfloat16 (nearest even) and back to float64, via torch."""
    torch = pytest.importorskip("torch")
    return torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()


def test_rope_matches_complex_rotation():
    """Each pair (x_i, x_{i+D/2}) as the complex number x_i + j x_{i+D/2},
    multiplied by e^{-j theta}: the real part is the first half, the imaginary
    part the second."""
    T, H, D = 9, 2, 16
    x = _rand((2, T, H, D), 60)
    c, s = (bf16_round(t) for t in rope_tables(T, D))
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * (c - 1j * s)[None, :, None, :]
    y = oracle.rope(x, c, s)
    np.testing.assert_allclose(y[..., :D // 2], z.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[..., D // 2:], z.imag, rtol=0, atol=1e-14)
    e = np.zeros((1, T, 1, D))
    e[..., 3] = 1.0
    y = oracle.rope(e, c, s)
    np.testing.assert_array_equal(y[0, :, 0, 3], c[:, 3])
    np.testing.assert_array_equal(y[0, :, 0, 3 + D // 2], -s[:, 3])


def test_rope_exact_tables_are_rotations():
    T, D = 12, 8
    x = _rand((1, T, 3, D), 61)
    c, s = rope_tables(T, D)
    y = oracle.rope(x, c, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    np.testing.assert_allclose(oracle.rope_bwd(y, c, s), x, rtol=0, atol=1e-14)   # R^T R = I


def test_rope_attention_depends_on_relative_position():
    """With exact tables, shifting every position by the same amount leaves
    the attention output unchanged: scores see only i - j."""
    T, D, W = 24, 16, 7
    q, k, v = (_rand((1, T, 2, D), s) for s in (62, 63, 64))
    c0, s0 = rope_tables(T, D)
    c1, s1 = rope_tables(T, D, offset=37)
    o0, l0 = oracle.attention_fwd_rope(q, k, v, c0, s0, W, True, EPS)
    o1, l1 = oracle.attention_fwd_rope(q, k, v, c1, s1, W, True, EPS)
    np.testing.assert_allclose(o0, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l0, l1, rtol=0, atol=1e-12)
    o2, _ = oracle.attention_fwd(q, k, v, W, True, EPS)
    assert np.max(np.abs(o0 - o2)) > 1e-3      # the rotation does change the result


def _torch_rope_reference(q, k, v, do, c, s, window, eps):
    """torch autograd through a complex-multiplication rotary embedding,
    rms_norm and SDPA with a band mask (fp64, CPU)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, T, H, D = q.shape
    h = D // 2
    rot = torch.complex(torch.tensor(c), -torch.tensor(s))[None, :, None, :]
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))

    def rotate(x):
        z = torch.complex(x[..., :h], x[..., h:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)
    qn = F.rms_norm(rotate(qt), (D,), eps=eps).transpose(1, 2)
    kn = F.rms_norm(rotate(kt), (D,), eps=eps).transpose(1, 2)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & ((i - j <= window) if window >= 0 else torch.ones(T, T, dtype=torch.bool))
    o = F.scaled_dot_product_attention(qn, kn, vt.transpose(1, 2), attn_mask=mask,
                                       enable_gqa=k.shape[2] != H).transpose(1, 2)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("H,H_kv,T,D,W", [(2, 2, 30, 16, 6), (4, 2, 33, 8, -1), (2, 1, 20, 16, 0)])
def test_rope_fwd_bwd_match_torch(H, H_kv, T, D, W):
    q, do = (_rand((2, T, H, D), s) for s in (65, 66))
    k, v = (_rand((2, T, H_kv, D), s) for s in (67, 68))
    c, s = (bf16_round(t) for t in rope_tables(T, D))
    ref = _torch_rope_reference(q, k, v, do, c, s, W, EPS)
    o, _ = oracle.attention_fwd_rope(q, k, v, c, s, W, True, EPS)
    got = (o,) + tuple(oracle.attention_bwd_rope(q, k, v, do, c, s, W, True, EPS))
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_rope_bwd_matches_finite_differences():
    T, D, W = 10, 8, 4
    q, k, v, do = (_rand((1, T, 1, D), s) for s in (69, 70, 71, 72))
    c, s = (bf16_round(t) for t in rope_tables(T, D))
    dq, dk, dv = oracle.attention_bwd_rope(q, k, v, do, c, s, W, True, EPS)

    def loss(qq, kk, vv):
        return float(np.sum(oracle.attention_fwd_rope(qq, kk, vv, c, s, W, True, EPS)[0] * do))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(num - grad)) / np.max(np.abs(grad))
        assert err < 1e-7, (which, err)


# ------------------------------------------------- value-embedding gate

def _torch_ve_reference(q, k, v, do, ve, xg, gw, window, eps, c=None, s=None):
    """torch autograd through F.linear + sigmoid (the gate), the mix into v,
    optionally a complex-multiplication rotation, rms_norm and SDPA (fp64)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, T, H, D = q.shape
    ts = [torch.tensor(x, requires_grad=True) for x in (q, k, v, ve, xg, gw)]
    qt, kt, vt, vet, xt, wt = ts
    gate = 2.0 * torch.sigmoid(F.linear(xt[..., :32], wt))
    vg = vt + gate[..., None] * vet
    if c is not None:
        rot = torch.complex(torch.tensor(c), -torch.tensor(s))[None, :, None, :]

        def rotate(x):
            z = torch.complex(x[..., :D // 2], x[..., D // 2:]) * rot
            return torch.cat([z.real, z.imag], dim=-1)
        qr, kr = rotate(qt), rotate(kt)
    else:
        qr, kr = qt, kt
    qn = F.rms_norm(qr, (D,), eps=eps).transpose(1, 2)
    kn = F.rms_norm(kr, (D,), eps=eps).transpose(1, 2)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & ((i - j <= window) if window >= 0 else torch.ones(T, T, dtype=torch.bool))
    o = F.scaled_dot_product_attention(qn, kn, vg.transpose(1, 2), attn_mask=mask,
                                       enable_gqa=k.shape[2] != H).transpose(1, 2)
    o.backward(torch.tensor(do))
    return (o.detach().numpy(),) + tuple(t.grad.numpy() for t in ts)


@pytest.mark.parametrize("H,H_kv,T,D,W,rope", [(2, 2, 24, 16, 5, False), (4, 2, 30, 8, -1, False),
                                               (2, 1, 20, 16, 3, True)])
def test_ve_fwd_bwd_match_torch(H, H_kv, T, D, W, rope):
    q, do = (_rand((2, T, H, D), s) for s in (73, 74))
    k, v, ve = (_rand((2, T, H_kv, D), s) for s in (75, 76, 77))
    xg = _rand((2, T, 40), 78)          # a wider block input: only channels 0..31 feed the gate
    gw = _rand((H_kv, 32), 79, 0.2)
    c, sn = (bf16_round(t) for t in rope_tables(T, D)) if rope else (None, None)
    ref = _torch_ve_reference(q, k, v, do, ve, xg, gw, W, EPS, c, sn)
    o, _ = oracle.attention_fwd_ve(q, k, v, ve, xg, gw, W, True, EPS, c, sn)
    dq, dk, dv, dve, dx, dW = oracle.attention_bwd_ve(q, k, v, do, ve, xg, gw, W, True, EPS, c, sn)
    np.testing.assert_allclose(o, ref[0], rtol=1e-10, atol=1e-12)
    for a, b in ((dq, ref[1]), (dk, ref[2]), (dv, ref[3]), (dve, ref[4]), (dW, ref[6])):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dx, ref[5][..., :32], rtol=1e-10, atol=1e-11)
    assert np.all(ref[5][..., 32:] == 0)


def test_ve_gate_closed_forms():
    """W_g = 0 gives gate = 1 exactly (v' = v + ve); ve = 0 leaves attention
    unchanged and gives no gate gradient."""
    T, D, W = 20, 8, 6
    q, k, v, ve, do = (_rand((1, T, 2, D), s) for s in (80, 81, 82, 83, 84))
    xg = _rand((1, T, 32), 85)
    zero_w = np.zeros((2, 32))
    assert np.all(oracle.ve_gate(xg, zero_w) == 1.0)
    o, lse = oracle.attention_fwd_ve(q, k, v, ve, xg, zero_w, W, True, EPS)
    o2, lse2 = oracle.attention_fwd(q, k, v + ve, W, True, EPS)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14)
    gw = _rand((2, 32), 86, 0.3)
    dq, dk, dv, dve, dx, dW = oracle.attention_bwd_ve(q, k, v, do, np.zeros_like(ve), xg, gw, W, True, EPS)
    assert np.all(dx == 0) and np.all(dW == 0)
    np.testing.assert_allclose(dve, oracle.ve_gate(xg, gw)[..., None] * dv, rtol=0, atol=0)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, W, True, EPS)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_ve_bwd_matches_finite_differences():
    T, D, W = 8, 4, 3
    q, do = (_rand((1, T, 2, D), s) for s in (87, 88))
    k, v, ve = (_rand((1, T, 1, D), s) for s in (89, 90, 91))
    xg = _rand((1, T, 32), 92, 0.5)
    gw = _rand((1, 32), 93, 0.3)
    grads = oracle.attention_bwd_ve(q, k, v, do, ve, xg, gw, W, True, EPS)
    args = [q, k, v, ve, xg, gw]
    which_of = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4, 5: 5}   # grads: dq, dk, dv, dve, dx, dW

    def loss(a):
        return float(np.sum(oracle.attention_fwd_ve(*a[:6], W, True, EPS)[0] * do))

    h = 1e-6
    for gi, ai in which_of.items():
        grad = grads[gi]
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[ai][idx] += h
            am[ai][idx] -= h
            num[idx] = (loss(ap) - loss(am)) / (2 * h)
        err = np.max(np.abs(num - grad)) / np.max(np.abs(grad))
        assert err < 1e-7, (gi, err)


# -------------------------------------------------------- finite differences

@pytest.mark.parametrize("W,causal", [(5, True), (-1, True), (3, False)])
def test_bwd_matches_finite_differences(W, causal):
    T, D = 16, 8
    q, k, v, do = (_rand((1, T, 1, D), s) for s in (9, 10, 11, 12))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, causal, EPS)

    def loss(qq, kk, vv):
        o, _ = oracle.attention_fwd(qq, kk, vv, W, causal, EPS)
        return float(np.sum(o * do))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(num - grad)) / np.max(np.abs(grad))
        assert err < 1e-7, (which, err)


def test_gqa_bwd_matches_finite_differences():
    T, D, W = 10, 4, 3
    q, do = (_rand((1, T, 4, D), s) for s in (49, 50))
    k, v = (_rand((1, T, 2, D), s) for s in (51, 52))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, True, EPS)

    def loss(qq, kk, vv):
        return float(np.sum(oracle.attention_fwd(qq, kk, vv, W, True, EPS)[0] * do))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(num - grad)) / np.max(np.abs(grad))
        assert err < 1e-7, (which, err)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("W", [0, 1, 4, 17, -1])
def test_identical_keys_closed_form(W):
    """All keys equal: P is uniform over the visible keys, so o_i is the mean of
    the visible values, lse_i = s_i + ln(#visible keys) and dq = 0."""
    T, D = 24, 16
    q, v, do = (_rand((1, T, 2, D), s) for s in (13, 14, 15))
    k = np.broadcast_to(_rand((1, 1, 2, D), 16), (1, T, 2, D)).copy()
    o, lse = oracle.attention_fwd(q, k, v, W, True, EPS)
    dq, _, _ = oracle.attention_bwd(q, k, v, do, W, True, EPS)
    qh, _ = oracle.rms_norm(q, EPS)
    kh, _ = oracle.rms_norm(k[:, :1], EPS)
    for h in range(2):
        for i in range(T):
            n = (i if W < 0 else min(i, W)) + 1
            s_i = float(qh[0, i, h] @ kh[0, 0, h]) / math.sqrt(D)
            assert abs(lse[0, h, i] - (s_i + math.log(n))) < 1e-12
            np.testing.assert_allclose(o[0, i, h], v[0, i - n + 1:i + 1, h].mean(axis=0),
                                       rtol=0, atol=1e-13)
    assert np.max(np.abs(dq)) < 1e-12


def test_window_zero_is_identity():
    """W = 0: each query sees only itself, so o = v, lse_i = s_ii, dv = dO, dq = dk = 0."""
    T, D = 20, 16
    q, k, v, do = (_rand((2, T, 2, D), s) for s in (17, 18, 19, 20))
    o, lse = oracle.attention_fwd(q, k, v, 0, True, EPS)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0, True, EPS)
    assert np.array_equal(o, v)
    qh, _ = oracle.rms_norm(q, EPS)
    kh, _ = oracle.rms_norm(k, EPS)
    diag = np.einsum("bthd,bthd->bht", qh, kh) / math.sqrt(D)
    np.testing.assert_allclose(lse, diag, rtol=0, atol=1e-14)
    assert np.array_equal(dv, do)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


@pytest.mark.parametrize("W,causal", [(6, True), (-1, True), (4, False)])
def test_one_hot_value_marks_visibility(W, causal):
    """v_{j*} = e_0 and all other values 0: o_{i,0} = P_{i,j*}, positive iff visible."""
    T, D = 30, 8
    q, k = _rand((1, T, 1, D), 21), _rand((1, T, 1, D), 22)
    mask = A.visible_mask(T, W, causal)
    for jstar in (0, 5, 17, T - 1):
        v = np.zeros((1, T, 1, D))
        v[0, jstar, 0, 0] = 1.0
        o, _ = oracle.attention_fwd(q, k, v, W, causal, EPS)
        assert np.array_equal(o[0, :, 0, 0] > 0, mask[:, jstar])
        assert np.all(o[0, :, 0, 1:] == 0)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("W,causal", [(0, True), (5, True), (-1, True), (3, False)])
def test_softmax_rows_and_exact_zeros(W, causal):
    T, D = 50, 16
    q, k = _rand((1, T, 1, D), 23, 4.0), _rand((1, T, 1, D), 24, 4.0)
    p, lse = oracle.probabilities(q, k, 0, 0, W, causal, EPS)
    mask = A.visible_mask(T, W, causal)
    assert np.all(p[~mask] == 0.0)
    assert np.all(p[mask] > 0) and np.all(p[mask] <= 1.0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14
    s = oracle.scores(q, k, 0, 0, W, causal, EPS)
    np.testing.assert_allclose(lse, np.log(np.sum(np.exp(np.where(mask, s, -np.inf)), axis=1)),
                               rtol=0, atol=1e-12)


def test_logit_bound():
    """QK-norm bounds every scaled logit by sqrt(D), whatever the input scale."""
    for D, scale in ((8, 1e-3), (64, 1.0), (128, 300.0)):
        q, k = _rand((1, 64, 1, D), 25, scale), _rand((1, 64, 1, D), 26, scale)
        k[0, 10] = q[0, 40] * 7.0   # an aligned pair reaches close to the bound
        s = oracle.scores(q, k, 0, 0, -1, True, EPS)
        fin = s[np.isfinite(s)]
        assert np.all(np.abs(fin) < math.sqrt(D))
        # parallel q and k: s = sqrt(D) * sqrt(ms_q/(ms_q+eps)) * sqrt(ms_k/(ms_k+eps))
        mq = np.mean(q[0, 40, 0] ** 2)
        mk = np.mean(k[0, 10, 0] ** 2)
        want = math.sqrt(D) * math.sqrt(mq / (mq + EPS)) * math.sqrt(mk / (mk + EPS))
        assert abs(s[40, 10] - want) < 1e-12


def test_large_window_equals_full_causal():
    T, D = 37, 8
    q, k, v, do = (_rand((1, T, 2, D), s) for s in (27, 28, 29, 30))
    ref = oracle.attention_fwd(q, k, v, -1, True, EPS)
    refb = oracle.attention_bwd(q, k, v, do, -1, True, EPS)
    for W in (T - 1, T, 4 * T):
        o, lse = oracle.attention_fwd(q, k, v, W, True, EPS)
        assert np.array_equal(o, ref[0]) and np.array_equal(lse, ref[1])
        for a, b in zip(oracle.attention_bwd(q, k, v, do, W, True, EPS), refb):
            assert np.array_equal(a, b)


def test_sampled_rows_match_full():
    T, D, W = 70, 16, 9
    q, k, v, do = (_rand((2, T, 2, D), s) for s in (31, 32, 33, 34))
    o, lse = oracle.attention_fwd(q, k, v, W, True, EPS)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, True, EPS)
    rows = [0, 3, 9, 10, 45, T - 1]
    for b, h in ((0, 0), (1, 1)):
        orow, lrow = oracle.fwd_rows(q, k, v, b, h, rows, W, True, EPS)
        np.testing.assert_allclose(orow, o[b, rows, h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lrow, lse[b, h, rows], rtol=0, atol=1e-14)
        sq, sk, sv = oracle.bwd_rows(q, k, v, do, b, h, rows, rows, W, True, EPS)
        np.testing.assert_allclose(sq, dq[b, rows, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sk, dk[b, rows, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sv, dv[b, rows, h], rtol=0, atol=1e-12)


def test_sampled_rows_match_full_gqa():
    T, D, W, H, H_kv = 50, 8, 11, 4, 2
    q, do = (_rand((1, T, H, D), s) for s in (53, 54))
    k, v = (_rand((1, T, H_kv, D), s) for s in (55, 56))
    o, lse = oracle.attention_fwd(q, k, v, W, True, EPS)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, True, EPS)
    rows = [0, 7, 11, 12, 30, T - 1]
    for h in range(H):
        orow, lrow = oracle.fwd_rows(q, k, v, 0, h, rows, W, True, EPS)
        np.testing.assert_allclose(orow, o[0, rows, h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lrow, lse[0, h, rows], rtol=0, atol=1e-14)
        sq, sk, sv = oracle.bwd_rows(q, k, v, do, 0, h, rows, rows, W, True, EPS)
        hk = oracle.kv_head(h, H, H_kv)
        np.testing.assert_allclose(sq, dq[0, rows, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sk, dk[0, rows, hk], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sv, dv[0, rows, hk], rtol=0, atol=1e-12)


def test_invalid_window_rejected():
    with pytest.raises(ValueError):
        A.visible_mask(8, -2)


# ------------------------------------------------------- values on the pages

def test_window_schedule_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "window_schedule.json")))
    for c in g["cases"]:
        w = S.layer_windows(c["pattern"], c["n_layer"], c["seq_len"])
        assert w == c["windows"]
        assert [i for i, x in enumerate(w) if x == c["seq_len"]] == c["global_layers"]


def test_window_schedule_rules():
    assert S.layer_windows("SSSS", 4, 2048) == [1024, 1024, 1024, 2048]   # last forced L
    assert S.layer_windows("L", 3, 512) == [512, 512, 512]
    assert S.layer_windows("sl", 5, 1000) == [500, 1000, 500, 1000, 1000]
    assert S.layer_windows("SSSL", 4, 8192) == [4096, 4096, 4096, 8192]
    with pytest.raises(ValueError):
        S.layer_windows("SXL", 4, 2048)


def test_flops_per_token_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "flops_per_token.json")))
    pc = g["param_counts"]
    assert sum(v for k, v in pc.items() if k != "total") == pc["total"]
    windows = S.layer_windows(g["pattern"], g["n_layer"], g["seq_len"])
    f = S.flops_per_token(pc["transformer_matrices"], pc["lm_head"], g["n_head"],
                          g["head_dim"], windows, g["seq_len"])
    assert f == g["flops_per_token"]
