"""attn_fwd_noalloc, the forward for callers that cannot allocate: through the
C ABI on the GPU, its outputs must equal attn_fwd's (the same kernels on the
same inputs, the key scales in the library's device array instead of a
workspace) bit for bit, on two calls in a row, the second one smaller, so
that the second call runs over the first call's leftover scratch."""
import ctypes

import numpy as np
import pytest

import oracle
from workloads import make_layer_inputs

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dev(torch, bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _both(torch, B, T, H, D, W, seed):
    import sliding_window_causal_qk_amd as sw
    L = sw.lib()
    inp = make_layer_inputs(B, T, H, D, seed)
    q, k, v = (_dev(torch, t) for t in (inp.q, inp.k, inp.v))
    s = torch.cuda.current_stream().cuda_stream
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    ws = torch.empty(sw.fwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    sw.check(L.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(),
                        ws.data_ptr(), ws.numel(), B, T, H, D, W, 1, EPS, s), "attn_fwd")
    sw.check(L.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                                B, T, H, D, W, 1, EPS, s), "attn_fwd_noalloc")
    torch.cuda.synchronize()
    return inp, (o1, l1), (o2, l2)


def test_noalloc_forward_matches_the_allocating_entry_point(torch_dev):
    torch = torch_dev
    # a large call first, then a smaller one over its leftover scratch
    for (B, T, H, D, W, seed) in ((4, 1000, 4, 128, 300, 91), (1, 257, 2, 64, 64, 92)):
        print(f"[no_alloc] B={B} T={T} H={H} D={D} W={W}", flush=True)
        inp, (o1, l1), (o2, l2) = _both(torch, B, T, H, D, W, seed)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        # and to the stated tolerance of the fp64 oracle on one slice
        qf, kf, vf, _ = inp.as_f32()
        ro, rl = oracle.fwd_rows(qf, kf, vf, B - 1, H - 1, range(T), W, True, EPS)
        got = o2[B - 1, :, H - 1].float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ro) <= 2e-2 + 1e-2 * np.abs(ro))
        gl = l2[B - 1, H - 1].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(gl - rl) <= 2e-2 + 1e-2 * np.abs(rl))


def test_noalloc_rejects_problems_beyond_its_scratch(torch_dev):
    import sliding_window_causal_qk_amd as sw
    L = sw.lib()
    cap = L.attn_fwd_noalloc_max_bytes()
    assert cap == 8 << 20
    # B H T = 2^21 + 1 rows of key scales: one more than fits; nothing is launched
    # (distinct, non-overlapping placeholder addresses: the call returns before any HIP call)
    st = L.attn_fwd_noalloc(1 << 32, 2 << 32, 3 << 32, 4 << 32, 5 << 32, 1, (1 << 21) + 1, 1, 64, 8, 1, EPS,
                            None)
    assert st == sw.ATTN_ERR_WORKSPACE
