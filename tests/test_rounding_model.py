"""CPU checks of tests/rounding_model.py, the model of the kernels' stated
mixed precision, and of the exceptions it backs (no GPU).

  * The model is a faithful model of the method: on ordinary problems it meets
    the stated tolerance against the fp64 oracle on every output.
  * Every (case, tensor) that tests/precision_exceptions.py names is one where
    the model itself -- bf16 operands, fp32 accumulation, no kernel involved --
    lands outside the stated tolerance, on at least one and at most the named
    number of elements, by an excess close to the one measured on the GPU.
  * dW_g, a sum over every token, misses the plain bound in the stated
    precision (so it takes the named check everywhere), while the model's
    value still meets the bound applied to each of its terms.
"""
import numpy as np
import pytest

import oracle
from tests import rounding_model as rm
from tests.precision_exceptions import ELEMENTWISE_EXCEPTIONS
from tests.test_gpu_parity import MULTI_TILE
from tests.test_gpu_random_shapes import CASES, IDS
from workloads import bf16_bits_to_f32, make_gate_inputs, make_layer_inputs, rope_tables_bf16

EPS = 1e-6
ATOL, RTOL = 2e-2, 1e-2


def _case_params():
    out = dict(zip(IDS, CASES))
    for c in MULTI_TILE:
        B, T, H, H_kv, D, W, rope, C, reuse, seed = c
        out[f"B{B}T{T}H{H}Hkv{H_kv}D{D}W{W}{'rope' if rope else ''}C{C}"] = c
    return out


def _run_case(B, T, H, H_kv, D, W, rope, C, reuse, seed):
    """(names, oracle outputs, model outputs) of one case."""
    inp = make_layer_inputs(B, T, H, D, seed, H_kv=H_kv)
    qf, kf, vf, dof = inp.as_f32()
    c, sn = (bf16_bits_to_f32(t) for t in rope_tables_bf16(T, D)) if rope else (None, None)
    gk = {}
    if C:
        gi = make_gate_inputs(B, T, H_kv, D, C, seed + 100)
        vef, xf = bf16_bits_to_f32(gi.ve), bf16_bits_to_f32(gi.x)
        gk = dict(ve=vef, xg=xf, gate_w=gi.gate_w)
        want = oracle.attention_fwd_ve(qf, kf, vf, vef, xf, gi.gate_w, W, True, EPS, c, sn) + \
            oracle.attention_bwd_ve(qf, kf, vf, dof, vef, xf, gi.gate_w, W, True, EPS, c, sn)
        names = ("o", "lse", "dq", "dk", "dv", "dve", "dx32", "dgate_w")
    elif rope:
        want = oracle.attention_fwd_rope(qf, kf, vf, c, sn, W, True, EPS) + \
            oracle.attention_bwd_rope(qf, kf, vf, dof, c, sn, W, True, EPS)
        names = ("o", "lse", "dq", "dk", "dv")
    else:
        want = oracle.attention_fwd(qf, kf, vf, W, True, EPS) + oracle.attention_bwd(qf, kf, vf, dof, W, True, EPS)
        names = ("o", "lse", "dq", "dk", "dv")
    mo, ml = rm.forward(qf, kf, vf, W, EPS, c, sn, **gk)
    model = (mo, ml) + rm.backward(qf, kf, vf, mo, ml, dof, W, EPS, c, sn, **gk)
    return names, want, model, (qf, kf, vf, dof, gk)


def _excess(got, want):
    err = np.abs(np.asarray(got, np.float64) - want) - (ATOL + RTOL * np.abs(want))
    return int((err > 0).sum()), float(err.max())


@pytest.mark.parametrize("key", sorted(ELEMENTWISE_EXCEPTIONS), ids=[f"{k[0]}-{k[1]}" for k in
                                                                     sorted(ELEMENTWISE_EXCEPTIONS)])
def test_named_exception_is_the_stated_precision(key):
    cid, tensor = key
    count, gpu_excess = ELEMENTWISE_EXCEPTIONS[key]
    names, want, model, _ = _run_case(*_case_params()[cid])
    i = names.index(tensor)
    n, ex = _excess(model[i], want[i])
    assert 1 <= n <= count, (cid, tensor, n, count)
    assert 0.5 * gpu_excess <= ex <= 1.5 * gpu_excess, (cid, tensor, ex, gpu_excess)
    # every other output of the case meets the plain bound in the model too,
    # unless it is named as well
    for j, name in enumerate(names):
        if j != i and name != "dgate_w" and (cid, name) not in ELEMENTWISE_EXCEPTIONS:
            assert _excess(model[j], want[j])[0] == 0, (cid, name)


FAITHFUL = [
    # (B, T, H, H_kv, D, W, rope, C, reuse, seed): ordinary problems
    (1, 128, 2, 2, 64, 64, False, 0, False, 0),       # the tiny workload
    (2, 257, 4, 2, 128, 100, False, 0, False, 42),
    (1, 300, 2, 1, 128, -1, True, 0, False, 52),
    (1, 200, 2, 2, 256, 70, False, 0, False, 47),
    (2, 150, 4, 2, 128, 30, False, 64, False, 61),
]


@pytest.mark.parametrize("case", FAITHFUL, ids=[f"T{c[1]}D{c[4]}W{c[5]}{'rope' if c[6] else ''}C{c[7]}"
                                                for c in FAITHFUL])
def test_model_meets_the_tolerance_on_ordinary_problems(case):
    names, want, model, _ = _run_case(*case)
    for name, w, m in zip(names, want, model):
        if name == "dgate_w":
            continue
        assert _excess(m, w)[0] == 0, name


def test_model_window_zero_closed_forms():
    """W = 0: each query sees only itself, so o = v (bf16 values) and dv = dO,
    dq = dk = 0 up to the rounding of P = p / bf16(p) near 1."""
    inp = make_layer_inputs(1, 50, 2, 64, 3)
    qf, kf, vf, dof = inp.as_f32()
    o, lse = rm.forward(qf, kf, vf, 0, EPS)
    assert np.max(np.abs(o - vf)) <= np.max(np.abs(vf)) * 2.0 ** -8
    dq, dk, dv = rm.backward(qf, kf, vf, o, lse, dof, 0, EPS)
    assert np.max(np.abs(dv - dof)) <= np.max(np.abs(dof)) * 2.0 ** -7
    assert np.max(np.abs(dq)) < 1e-3 and np.max(np.abs(dk)) < 1e-3


GATE_CASES = [cid for cid, c in zip(IDS, CASES) if c[7]]


def test_gate_weight_gradient_is_a_reduction():
    """dW_g in the stated precision, over the sweep's gate cases: outside the
    plain bound somewhere (so it takes the named check everywhere), and always
    within the bound applied per term, 2e-2 + 1e-2 sum_t |dz x|."""
    misses = 0
    for cid in GATE_CASES:
        names, want, model, (qf, kf, vf, dof, gk) = _run_case(*_case_params()[cid])
        i = names.index("dgate_w")
        gate = oracle.ve_gate(gk["xg"], gk["gate_w"])
        dz = np.sum(want[4] * gk["ve"], axis=-1) * gate * (1 - gate / 2)
        scale = np.einsum("bth,btc->hc", np.abs(dz), np.abs(np.asarray(gk["xg"], np.float64)[..., :32]))
        err = np.abs(np.asarray(model[i], np.float64) - want[i])
        assert np.all(err <= ATOL + RTOL * scale), cid
        misses += _excess(model[i], want[i])[0]
    assert misses > 0
