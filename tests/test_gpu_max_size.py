"""GPU parity at the largest problems the library accepts.

The boundary takes B·T·H·D < 2^31 elements per tensor (beyond that
ATTN_ERR_UNSUPPORTED, `tests/test_abi.py`).  With B = H = 1 one (batch, head)
slice is the whole tensor, so the kernels' per-slice byte counts and row
offsets reach their largest values: just under 2^32 bytes of K or dO rows
behind a slice's first row.  The window is short (W = 64) so the work stays
small while every row, key tile and block of the band is visited.

Inputs are drawn on the GPU from a seed (`workloads.make_layer_inputs_device`);
for each sampled row or key the test copies the input rows that row depends on
(its window for o, lse and dq; keys j - W .. j + W for dk, dv) back to the
host, and the fp64 oracle computes it on that sub-sequence: query i sees keys
max(0, i - W) .. i, and key j is seen by queries j .. j + W, whose windows lie
inside j - W .. j + W.  Tolerance: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import make_layer_inputs_device

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2
EPS = 1e-6
W = 64


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close(name, got, want):
    err = np.abs(got - want)
    bad = err > ATOL + RTOL * np.abs(want)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert not bad.any(), f"{name}: {int(bad.sum())} elements off, max err {err.max():.4g}"


@pytest.mark.parametrize("T,D", [((1 << 24) - 1, 128), ((1 << 23) - 1, 256)])
def test_largest_accepted_problem(torch_dev, T, D):
    torch = torch_dev
    import sliding_window_causal_qk_amd as sw
    L = sw.lib()
    B, H = 1, 1
    assert B * T * H * D < (1 << 31) and B * (T + 1) * H * D >= (1 << 31)
    print(f"[max_size] B={B} T={T} H={H} D={D} W={W}", flush=True)
    sys.stdout.flush()
    q, k, v, do = make_layer_inputs_device(B, T, H, D, 4242, device="cuda")
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    fws = torch.empty(sw.fwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    bws = torch.empty(L.attn_bwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    sw.check(L.attn_fwd(p(q), p(k), p(v), p(o), p(lse), p(fws), fws.numel(), B, T, H, D, W, 1, EPS, s),
             "attn_fwd")
    sw.check(L.attn_bwd(p(q), p(k), p(v), p(o), p(lse), p(do), p(dq), p(dk), p(dv), p(bws), bws.numel(),
                        B, T, H, D, W, 1, EPS, s), "attn_bwd")
    torch.cuda.synchronize()
    print("[max_size] kernels done", flush=True)

    def window(lo, hi):   # input rows lo .. hi (inclusive) as a [1, n, 1, D] problem
        return tuple(_host(t[:, lo:hi + 1]) for t in (q, k, v, do))

    for i in (0, 1, W, W + 1, T // 2, T - 129, T - 2, T - 1):
        lo = max(0, i - W)
        qs, ks, vs, dos = window(lo, i)
        ro, rl = oracle.fwd_rows(qs, ks, vs, 0, 0, [i - lo], W, True, EPS)
        rq, _, _ = oracle.bwd_rows(qs, ks, vs, dos, 0, 0, [i - lo], [i - lo], W, True, EPS)
        _close(f"o[{i}]", _host(o[0, i:i + 1, 0]), ro)
        _close(f"lse[{i}]", lse[0, 0, i:i + 1].cpu().numpy().astype(np.float64), rl)
        _close(f"dq[{i}]", _host(dq[0, i:i + 1, 0]), rq)
    for j in (0, 1, 127, 128, T // 2, T - W - 1, T - 129, T - 1):
        lo, hi = max(0, j - W), min(T - 1, j + W)
        qs, ks, vs, dos = window(lo, hi)
        _, rk, rv = oracle.bwd_rows(qs, ks, vs, dos, 0, 0, [j - lo], [j - lo], W, True, EPS)
        _close(f"dk[{j}]", _host(dk[0, j:j + 1, 0]), rk)
        _close(f"dv[{j}]", _host(dv[0, j:j + 1, 0]), rv)
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} has non-finite values"
    del q, k, v, do, o, dq, dk, dv, lse, fws, bws
    torch.cuda.empty_cache()
