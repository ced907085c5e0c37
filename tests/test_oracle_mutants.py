"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.

Each mutant is a copy of oracle/attention.py with one textual change, loaded as
a separate module.  The pins used here are the independent ones of
test_oracle_pins.py: brute force, torch fp64 SDPA + autograd, closed forms of
identical keys and W = 0, and finite differences.
"""
import math
import os
import types

import numpy as np
import pytest

from tests.test_oracle_pins import (_rand, _torch_reference, _torch_rope_reference, _torch_ve_reference,
                                    bf16_round, brute_force_fwd, rope_tables)

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")
EPS = 1e-6

MUTANTS = [
    # (name, original text, planted mistake)
    ("window_off_by_one", "m &= d <= window", "m &= d < window"),
    ("window_wrong_side", "m = d >= 0", "m = d <= 0"),
    ("no_eps", "np.mean(x * x, axis=-1) + eps", "np.mean(x * x, axis=-1)"),
    ("sum_not_mean", "np.mean(x * x, axis=-1) + eps", "np.sum(x * x, axis=-1) + eps"),
    ("no_scale", "s = (qh @ kh.T) / np.sqrt(D)", "s = (qh @ kh.T)"),
    ("k_not_normed", "kh, _ = rms_norm(ks, eps)\n    s =", "kh = ks\n    s ="),
    ("lse_log2", "return e / z[:, None], m + np.log(z)", "return e / z[:, None], m + np.log2(z)"),
    ("lse_no_max", "return e / z[:, None], m + np.log(z)", "return e / z[:, None], np.log(z)"),
    ("dropped_delta", "ds = p * (dp - delta[:, None])\n        dq_hat[rows]",
     "ds = p * dp\n        dq_hat[rows]"),
    ("delta_sign", "ds = p * (dp - delta[:, None])\n        dq_hat[rows]",
     "ds = p * (dp + delta[:, None])\n        dq_hat[rows]"),
    ("dq_uses_q", "dq_hat[rows] = ds @ kh / np.sqrt(D)", "dq_hat[rows] = ds @ qh[rows] / np.sqrt(D)"),
    ("dk_transposed", "dk_hat += ds.T @ qh[rows] / np.sqrt(D)",
     "dk_hat += ds.T @ kh[rows] / np.sqrt(D)"),
    ("dk_no_scale", "dk_hat += ds.T @ qh[rows] / np.sqrt(D)", "dk_hat += ds.T @ qh[rows]"),
    ("dv_uses_do_of_wrong_side", "dv += p.T @ dos[rows]", "dv += p.T @ vs[rows]"),
    ("dp_transposed", "dp = dos[rows] @ vs.T\n        delta = np.sum(dos[rows] * o, axis=1)\n        ds = p * (dp - delta[:, None])\n        dq_hat",
     "dp = vs[rows] @ dos.T\n        delta = np.sum(dos[rows] * o, axis=1)\n        ds = p * (dp - delta[:, None])\n        dq_hat"),
    ("norm_bwd_no_projection", "return r[..., None] * (dx_hat - x_hat * proj)",
     "return r[..., None] * dx_hat"),
    ("norm_bwd_projection_sign", "return r[..., None] * (dx_hat - x_hat * proj)",
     "return r[..., None] * (dx_hat + x_hat * proj)"),
    ("norm_bwd_no_r", "return r[..., None] * (dx_hat - x_hat * proj)",
     "return (dx_hat - x_hat * proj)"),
    ("gqa_heads_interleaved", "return h // (H // H_kv)", "return h % H_kv"),
    ("gqa_dk_last_head_only", "dk_hat[b, :, hk] += dkh", "dk_hat[b, :, hk] = dkh"),
    ("gqa_dv_last_head_only", "dv[b, :, hk] += dvh", "dv[b, :, hk] = dvh"),
    ("rope_sign", "[x1 * c + x2 * s, x2 * c - x1 * s]", "[x1 * c - x2 * s, x2 * c + x1 * s]"),
    ("rope_interleaved_pairs", "x1, x2 = x[..., :h], x[..., h:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    ("rope_bwd_sign", "[g1 * c - g2 * s, g1 * s + g2 * c]", "[g1 * c + g2 * s, g2 * c - g1 * s]"),
    ("rope_bwd_missing", "return rope_bwd(dq, cos, sin), rope_bwd(dk, cos, sin), dv",
     "return dq, dk, dv"),
    ("ve_gate_no_factor_2", "return 2.0 / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    ("ve_sigmoid_derivative", "gate * (1.0 - gate / 2.0)", "gate * (1.0 - gate)"),
    ("ve_dve_without_gate", "dve = gate[..., None] * dvg", "dve = dvg"),
    ("ve_dx_transposed_map", "dx = dz @ _f64(gate_w)", "dx = np.sum(dz, axis=-1, keepdims=True) * np.sum(_f64(gate_w), axis=0)"),
]


def _load(src: str) -> types.ModuleType:
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(A) -> bool:
    """True iff the (possibly mutated) oracle passes every pin used here."""
    try:
        # brute force, forward
        for (T, D, W, causal) in ((9, 8, 3, True), (8, 4, 2, False)):
            q, k, v = (_rand((1, T, 2, D), s) for s in (1, 2, 3))
            o, lse = A.attention_fwd(q, k, v, W, causal, EPS)
            ob, lb = brute_force_fwd(q, k, v, W, causal, EPS)
            if not (np.allclose(o, ob, rtol=0, atol=1e-12) and np.allclose(lse, lb, rtol=0, atol=1e-12)):
                return False
        # library: fp64 SDPA + autograd
        for (T, D, W) in ((24, 16, 5), (20, 8, -1)):
            q, k, v, do = (_rand((1, T, 2, D), s) for s in (5, 6, 7, 8))
            ref = _torch_reference(q, k, v, do, W, True, EPS)
            got = (A.attention_fwd(q, k, v, W, True, EPS)[0],) + tuple(A.attention_bwd(q, k, v, do, W, True, EPS))
            if not all(np.allclose(a, b, rtol=1e-9, atol=1e-11) for a, b in zip(got, ref)):
                return False
        # library: fp64 SDPA with grouped key/value heads
        T, D, W = 20, 8, 6
        q, do = (_rand((1, T, 4, D), s) for s in (21, 22))
        k, v = (_rand((1, T, 2, D), s) for s in (23, 24))
        ref = _torch_reference(q, k, v, do, W, True, EPS)
        got = (A.attention_fwd(q, k, v, W, True, EPS)[0],) + tuple(A.attention_bwd(q, k, v, do, W, True, EPS))
        if not all(a.shape == b.shape and np.allclose(a, b, rtol=1e-9, atol=1e-11) for a, b in zip(got, ref)):
            return False
        # library: complex-multiplication rotary embedding + fp64 SDPA, autograd
        T, D, W = 14, 8, 5
        q, k, v, do = (_rand((1, T, 2, D), s) for s in (25, 26, 27, 28))
        c, s = (bf16_round(t) for t in rope_tables(T, D))
        ref = _torch_rope_reference(q, k, v, do, c, s, W, EPS)
        got = ((A.attention_fwd_rope(q, k, v, c, s, W, True, EPS)[0],)
               + tuple(A.attention_bwd_rope(q, k, v, do, c, s, W, True, EPS)))
        if not all(a.shape == b.shape and np.allclose(a, b, rtol=1e-9, atol=1e-11) for a, b in zip(got, ref)):
            return False
        # library: F.linear + sigmoid gate, autograd
        T, D, W = 12, 8, 4
        q, k, v, ve, do = (_rand((1, T, 2, D), s) for s in (29, 30, 31, 32, 33))
        xg = _rand((1, T, 32), 34)
        gw = _rand((2, 32), 35, 0.3)
        ref = _torch_ve_reference(q, k, v, do, ve, xg, gw, W, EPS)
        got = ((A.attention_fwd_ve(q, k, v, ve, xg, gw, W, True, EPS)[0],)
               + tuple(A.attention_bwd_ve(q, k, v, do, ve, xg, gw, W, True, EPS)))
        want = ref[:5] + (ref[5][..., :32], ref[6])
        if not all(a.shape == b.shape and np.allclose(a, b, rtol=1e-9, atol=1e-11) for a, b in zip(got, want)):
            return False
        # closed form: identical keys
        T, D = 16, 8
        q, v, do = (_rand((1, T, 1, D), s) for s in (13, 14, 15))
        k = np.broadcast_to(_rand((1, 1, 1, D), 16), (1, T, 1, D)).copy()
        o, lse = A.attention_fwd(q, k, v, 4, True, EPS)
        for i in range(T):
            n = min(i, 4) + 1
            if not np.allclose(o[0, i, 0], v[0, i - n + 1:i + 1, 0].mean(axis=0), atol=1e-12):
                return False
        # closed form: W = 0
        q, k, v, do = (_rand((1, T, 1, D), s) for s in (17, 18, 19, 20))
        o, _ = A.attention_fwd(q, k, v, 0, True, EPS)
        dq, dk, dv = A.attention_bwd(q, k, v, do, 0, True, EPS)
        if not (np.allclose(o, v, atol=1e-13) and np.allclose(dv, do, atol=1e-13)
                and np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12):
            return False
        # finite differences on dq, dk, dv
        T, D, W = 8, 4, 3
        q, k, v, do = (_rand((1, T, 1, D), s) for s in (9, 10, 11, 12))
        grads = A.attention_bwd(q, k, v, do, W, True, EPS)

        def loss(qq, kk, vv):
            return float(np.sum(A.attention_fwd(qq, kk, vv, W, True, EPS)[0] * do))
        h = 1e-6
        for which, g in enumerate(grads):
            for idx in ((0, 0, 0, 0), (0, 5, 0, 2), (0, 7, 0, 3)):
                ap = [q.copy(), k.copy(), v.copy()]
                am = [q.copy(), k.copy(), v.copy()]
                ap[which][idx] += h
                am[which][idx] -= h
                num = (loss(*ap) - loss(*am)) / (2 * h)
                if abs(num - g[idx]) > 1e-6 * max(1.0, abs(num)):
                    return False
    except (ValueError, FloatingPointError, IndexError):
        return False
    return True


def test_unmutated_oracle_passes():
    pytest.importorskip("torch")
    assert _pins_pass(_load(open(SRC).read()))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    pytest.importorskip("torch")
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutant = _load(src.replace(old, new, 1))
    with np.errstate(all="ignore"):
        assert not _pins_pass(mutant), f"planted mistake {name} passed every pin"
