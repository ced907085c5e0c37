"""MI355X (gfx950) causal sliding-window attention with RMSNorm on Q and K.

Thin binding over libswattn.so (include/swattn.h): argument marshalling only.
Every step of the attention runs in the HIP kernels; PyTorch provides device
memory and the current stream.

    from sliding_window_causal_qk_amd import attention, layer_windows
    windows = layer_windows("SSSL", n_layer=8, seq_len=2048)   # [1024, ..., 2048]
    o = attention(q, k, v, window=windows[l])                    # autograd-aware

q: bf16 CUDA tensor [B, T, H, D] (contiguous), D in {64, 128, 256}; k, v: bf16
[B, T, H_kv, D] with H_kv dividing H (grouped key/value heads: query head h
reads key/value head h // (H // H_kv); H_kv = H is plain multi-head attention).
rope=(cos, sin): bf16 [T, D/2] tables; q and k are then the projections before
the rotary embedding, which the kernels apply ahead of the norm.
gate=(ve, x, gate_w): the value-embedding gate, attention on
v + 2 sigmoid(x[..., :32] gate_w^T) ve; ve bf16 [B, T, H_kv, D], x bf16
[B, T, C >= 32] (the block input), gate_w fp32 [H_kv, 32].
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Tuple

from ._lib import (  # noqa: F401
    ATTN_ERR_HIP, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_OK,
    EXPORTS, LIB_PATH, SwattnError, check, lib, status_string,
)

__all__ = [
    "attention", "attn_fwd", "attn_bwd", "layer_windows", "visible_pairs", "band_tiles",
    "fwd_workspace_bytes", "bwd_workspace_bytes", "fwd_rope_workspace_bytes",
    "bwd_rope_workspace_bytes", "fwd_ve_workspace_bytes", "bwd_ve_workspace_bytes", "SwattnError",
]


def layer_windows(pattern: str, n_layer: int, seq_len: int) -> List[int]:
    out = (ctypes.c_int * max(n_layer, 1))()
    check(lib().attn_layer_windows(pattern.encode(), n_layer, seq_len, out), "attn_layer_windows")
    return list(out[:n_layer])


def visible_pairs(T: int, window: int) -> int:
    n = lib().attn_visible_pairs(T, window)
    if n < 0:
        raise SwattnError(ATTN_ERR_INVALID_ARG, "attn_visible_pairs")
    return int(n)


def band_tiles(T: int, window: int, rows: int, cols: int, by_key: bool = False):
    """Per row block: (first, last, n_partial, n_empty) column blocks visited."""
    n = max((T + rows - 1) // rows, 1) if rows > 0 else 1
    arrs = [(ctypes.c_int * n)() for _ in range(4)]
    check(lib().attn_band_tiles(T, window, rows, cols, int(by_key), *arrs), "attn_band_tiles")
    return [tuple(a[i] for a in arrs) for i in range((T + rows - 1) // rows)]


def fwd_workspace_bytes(B: int, T: int, H: int, D: int, H_kv: Optional[int] = None) -> int:
    if H_kv is None:
        return int(lib().attn_fwd_workspace_bytes(B, T, H, D))
    return int(lib().attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D))


def bwd_workspace_bytes(B: int, T: int, H: int, D: int, H_kv: Optional[int] = None) -> int:
    if H_kv is None:
        return int(lib().attn_bwd_workspace_bytes(B, T, H, D))
    return int(lib().attn_bwd_gqa_workspace_bytes(B, T, H, H_kv, D))


def fwd_rope_workspace_bytes(B: int, T: int, H: int, D: int, H_kv: Optional[int] = None) -> int:
    return int(lib().attn_fwd_rope_workspace_bytes(B, T, H, H if H_kv is None else H_kv, D))


def bwd_rope_workspace_bytes(B: int, T: int, H: int, D: int, H_kv: Optional[int] = None) -> int:
    return int(lib().attn_bwd_rope_workspace_bytes(B, T, H, H if H_kv is None else H_kv, D))


def fwd_ve_workspace_bytes(B: int, T: int, H: int, D: int, H_kv: Optional[int] = None) -> int:
    return int(lib().attn_fwd_ve_workspace_bytes(B, T, H, H if H_kv is None else H_kv, D))


def bwd_ve_workspace_bytes(B: int, T: int, H: int, D: int, H_kv: Optional[int] = None) -> int:
    return int(lib().attn_bwd_ve_workspace_bytes(B, T, H, H if H_kv is None else H_kv, D))


def _check_gate(gate, B, T, H_kv, D):
    torch = _torch()
    if not (isinstance(gate, (tuple, list)) and len(gate) == 3):
        raise ValueError("gate must be a (ve, x, gate_w) triple of tensors")
    ve, x, gw = gate
    _check_tensor(ve, "ve", (B, T, H_kv, D), torch.bfloat16)
    _check_tensor(x, "x", None, torch.bfloat16)
    if x.dim() != 3 or tuple(x.shape[:2]) != (B, T) or x.shape[2] < 32 or x.shape[2] % 8:
        raise ValueError(f"x must be [B, T, C] with C >= 32 a multiple of 8, got {tuple(x.shape)}")
    _check_tensor(gw, "gate_w", (H_kv, 32), torch.float32)
    return ve, x, gw


def _check_rope(rope, T, D):
    torch = _torch()
    if not (isinstance(rope, (tuple, list)) and len(rope) == 2):
        raise ValueError("rope must be a (cos, sin) pair of tensors")
    for n, t in zip(("rope cos", "rope sin"), rope):
        _check_tensor(t, n, (T, D // 2), torch.bfloat16)
    return rope


def _torch():
    import torch
    return torch


def _check_tensor(t, name, shape=None, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the HIP kernels are the only path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t) -> Optional[int]:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def attn_fwd(q, k, v, window: int, causal: bool = True, eps: float = 1e-6, *,
             out=None, lse=None, workspace=None, stream=None, rope=None,
             gate=None) -> Tuple["object", "object"]:
    """Forward through the C ABI.  Returns (o bf16 [B,T,H,D], lse fp32 [B,H,T])."""
    torch = _torch()
    B, T, H, D = q.shape
    H_kv = k.shape[2] if k.dim() == 4 else -1
    _check_tensor(q, "q", (B, T, H, D), torch.bfloat16)
    for n, t in (("k", k), ("v", v)):
        _check_tensor(t, n, (B, T, H_kv, D), torch.bfloat16)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(o, "out", (B, T, H, D), torch.bfloat16)
    _check_tensor(l, "lse", (B, H, T), torch.float32)
    if gate is not None:
        ve, x, gw = _check_gate(gate, B, T, H_kv, D)
        rc, rs = _check_rope(rope, T, D) if rope is not None else (None, None)
        nbytes = fwd_ve_workspace_bytes(B, T, H, D, H_kv)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
        st = lib().attn_fwd_ve(_ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(x), x.shape[2], _ptr(gw),
                               _ptr(rc), _ptr(rs), _ptr(o), _ptr(l), ws.data_ptr(), ws.numel(),
                               B, T, H, H_kv, D, int(window), int(bool(causal)), float(eps),
                               _stream(stream))
        check(st, "attn_fwd_ve")
        return o, l
    if rope is not None:
        rc, rs = _check_rope(rope, T, D)
        nbytes = fwd_rope_workspace_bytes(B, T, H, D, H_kv)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
        st = lib().attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(rc), _ptr(rs), _ptr(o), _ptr(l),
                                 ws.data_ptr(), ws.numel(), B, T, H, H_kv, D, int(window),
                                 int(bool(causal)), float(eps), _stream(stream))
        check(st, "attn_fwd_rope")
        return o, l
    nbytes = fwd_workspace_bytes(B, T, H, D, H_kv)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
    if H_kv == H:
        st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), ws.data_ptr(), ws.numel(),
                            B, T, H, D, int(window), int(bool(causal)), float(eps), _stream(stream))
    else:
        st = lib().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), ws.data_ptr(),
                                ws.numel(), B, T, H, H_kv, D, int(window), int(bool(causal)),
                                float(eps), _stream(stream))
    check(st, "attn_fwd")
    return o, l


def attn_bwd(q, k, v, o, lse, dout, window: int, causal: bool = True, eps: float = 1e-6, *,
             dq=None, dk=None, dv=None, workspace=None, stream=None, rope=None, gate=None,
             fwd_workspace=None):
    """Backward through the C ABI.  Returns (dq, dk, dv): bf16, dq [B,T,H,D],
    dk and dv shaped like k and v; with gate=(ve, x, gate_w) also dve (bf16,
    like ve), dx32 (bf16 [B, T, 32], the gradient of x's first 32 channels)
    and dgate_w (fp32 [H_kv, 32]).  fwd_workspace: the workspace of the
    attn_fwd call that produced o and lse (same options), left unchanged; the
    backward then reuses its key pre-pass (the *_reuse entry points)."""
    torch = _torch()
    B, T, H, D = q.shape
    H_kv = k.shape[2] if k.dim() == 4 else -1
    for n, t in (("q", q), ("o", o), ("dout", dout)):
        _check_tensor(t, n, (B, T, H, D), torch.bfloat16)
    for n, t in (("k", k), ("v", v)):
        _check_tensor(t, n, (B, T, H_kv, D), torch.bfloat16)
    _check_tensor(lse, "lse", (B, H, T), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor(dq, "dq", (B, T, H, D), torch.bfloat16)
    for n, t in (("dk", dk), ("dv", dv)):
        _check_tensor(t, n, (B, T, H_kv, D), torch.bfloat16)
    if gate is not None:
        ve, x, gw = _check_gate(gate, B, T, H_kv, D)
        rc, rs = _check_rope(rope, T, D) if rope is not None else (None, None)
        dve = torch.empty_like(ve)
        dx32 = torch.empty((B, T, 32), dtype=torch.bfloat16, device=q.device)
        dgw = torch.empty((H_kv, 32), dtype=torch.float32, device=q.device)
        nbytes = bwd_ve_workspace_bytes(B, T, H, D, H_kv)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
        head = (_ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(x), x.shape[2], _ptr(gw), _ptr(rc), _ptr(rs),
                _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dve), _ptr(dx32), _ptr(dgw))
        tail = (ws.data_ptr(), ws.numel(), B, T, H, H_kv, D, int(window), int(bool(causal)), float(eps),
                _stream(stream))
        if fwd_workspace is None:
            st = lib().attn_bwd_ve(*head, *tail)
        else:
            st = lib().attn_bwd_ve_reuse(*head, fwd_workspace.data_ptr(), fwd_workspace.numel(), *tail)
        check(st, "attn_bwd_ve")
        return dq, dk, dv, dve, dx32, dgw
    if rope is not None:
        rc, rs = _check_rope(rope, T, D)
        nbytes = bwd_rope_workspace_bytes(B, T, H, D, H_kv)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
        head = (_ptr(q), _ptr(k), _ptr(v), _ptr(rc), _ptr(rs), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                _ptr(dk), _ptr(dv))
        tail = (ws.data_ptr(), ws.numel(), B, T, H, H_kv, D, int(window), int(bool(causal)), float(eps),
                _stream(stream))
        if fwd_workspace is None:
            st = lib().attn_bwd_rope(*head, *tail)
        else:
            st = lib().attn_bwd_rope_reuse(*head, fwd_workspace.data_ptr(), fwd_workspace.numel(), *tail)
        check(st, "attn_bwd_rope")
        return dq, dk, dv
    nbytes = bwd_workspace_bytes(B, T, H, D, H_kv)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
    if fwd_workspace is not None:
        st = lib().attn_bwd_gqa_reuse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                      _ptr(dq), _ptr(dk), _ptr(dv), fwd_workspace.data_ptr(),
                                      fwd_workspace.numel(), ws.data_ptr(), ws.numel(), B, T, H, H_kv, D,
                                      int(window), int(bool(causal)), float(eps), _stream(stream))
    elif H_kv == H:
        st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dk), _ptr(dv), ws.data_ptr(), ws.numel(),
                            B, T, H, D, int(window), int(bool(causal)), float(eps), _stream(stream))
    else:
        st = lib().attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                _ptr(dq), _ptr(dk), _ptr(dv), ws.data_ptr(), ws.numel(),
                                B, T, H, H_kv, D, int(window), int(bool(causal)), float(eps),
                                _stream(stream))
    check(st, "attn_bwd")
    return dq, dk, dv


def _make_function():
    torch = _torch()

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, window, causal, eps, rope_cos, rope_sin, ve, x, gate_w):
            rope = None if rope_cos is None else (rope_cos, rope_sin)
            gate = None if ve is None else (ve, x, gate_w)
            B, T, H, D = q.shape
            H_kv = k.shape[2] if k.dim() == 4 else H   # a malformed k is rejected by attn_fwd
            nb = (fwd_ve_workspace_bytes if gate is not None else
                  fwd_rope_workspace_bytes if rope is not None else fwd_workspace_bytes)(B, T, H, D, H_kv)
            fws = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
            o, lse = attn_fwd(q, k, v, window, causal, eps, rope=rope, gate=gate, workspace=fws)
            ctx.save_for_backward(q, k, v, o, lse)
            # the forward's key pre-pass (key scales, rotated keys, gated values)
            # serves the backward too
            ctx.cfg = (window, causal, eps, rope, gate, fws)
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            window, causal, eps, rope, gate, fws = ctx.cfg
            g = attn_bwd(q, k, v, o, lse, do.contiguous(), window, causal, eps, rope=rope, gate=gate,
                         fwd_workspace=fws)
            if gate is None:
                return g[0], g[1], g[2], None, None, None, None, None, None, None, None
            dq, dk, dv, dve, dx32, dgw = g
            x = gate[1]
            dx = torch.zeros_like(x)
            dx[..., :32] = dx32
            return dq, dk, dv, None, None, None, None, None, dve, dx, dgw

    return _Attention


_fn = None


def attention(q, k, v, window: int, causal: bool = True, eps: float = 1e-6, rope=None, gate=None):
    """Autograd-aware QK-RMSNorm causal sliding-window attention (HIP kernels).
    rope=(cos, sin) applies the rotary embedding to q and k before the norm;
    the tables get no gradient.  gate=(ve, x, gate_w) mixes the value
    embedding into v; ve, x (its first 32 channels) and gate_w get gradients."""
    global _fn
    if _fn is None:
        _fn = _make_function()
    rc, rs = (None, None) if rope is None else rope
    ve, x, gw = (None, None, None) if gate is None else gate
    return _fn.apply(q, k, v, window, causal, eps, rc, rs, ve, x, gw)
