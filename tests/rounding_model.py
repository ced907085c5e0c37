"""CPU model of the kernels' stated mixed precision (test infrastructure).

The fp64 oracle (`oracle/`) is the reference for parity.  This module is a
second, independent description of the same attention in the precision the
HIP kernels state they compute in, written in plain numpy float32.  The tests
use it for one purpose: to show that where a GPU result misses the stated
tolerance against the fp64 oracle, the stated arithmetic alone (bf16 operands
of the matrix products, fp32 accumulation, bf16 outputs) already misses it at
the same elements, by a comparable amount -- so the miss is the precision,
not a fault.  It shares no code with the HIP path or with the oracle.

The operation is the one the oracle follows ("Autoresearch 深度教程" §7.3: RMSNorm
with no weight on q and k; §5.2.2: the (W, 0) window; §7.4: the rotary
embedding; §5.2.3: the value-embedding gate; the scale 1/sqrt(D)).  The
rounding points are the kernels' documented ones:

  forward:   q_hat = bf16(q r_q) (r_q in fp32);  K enters the product raw (bf16)
             and every logit is scaled by kscale = log2(e) r_k / sqrt(D);
             p = exp2(s kscale - sqrt(D) log2(e)) is rounded to bf16, the row
             sum adds the rounded p, o = bf16((sum_j bf16(p) v_j) / l),
             lse = sqrt(D) + ln l  (QK-norm bounds |s| < sqrt(D), so the fixed
             shift replaces a running maximum)
  backward:  Delta = dO . o (o the bf16 output), P = exp2(s kscale - lse log2 e)
             in fp32; dV += bf16(P)^T dO; dS = P (dP - Delta) rounded to bf16
             for dK_hat += dS^T q_hat; dQ takes bf16(P (dP - Delta) kscale) times
             the raw K; the RMSNorm backward of q and k runs in fp32 on the
             fp32 accumulators and is rounded to bf16 once; for q its x_hat is
             the bf16 q_hat of the products, for k the raw K times r_k
  rotary:    the rotated keys are stored in bf16 (the K of the products); the
             rotated queries go to the norm unrounded; the gradients are
             rotated back in fp32
  gate:      gate = 2 sigmoid(W_g x[:32]) in fp32; V of the products is
             bf16(v + gate ve); dve = bf16(gate dV) and
             dz = (dV . ve) gate (1 - gate / 2) come from the fp32 dV
             accumulator; dx = bf16(dz W_g), dW_g = sum dz x in fp32

Only the order of the fp32 sums differs from the kernels, which moves results
by fp32 rounding, far below bf16's.
"""
from __future__ import annotations

import numpy as np

LOG2E = np.float32(1.4426950408889634)
F32 = np.float32


def bf16(x) -> np.ndarray:
    """Round fp32 to the nearest bf16 value (ties to even); returned as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def _recip_rms(x, eps) -> np.ndarray:
    """1 / sqrt(mean x^2 + eps) over the last axis, in fp32."""
    D = x.shape[-1]
    ss = np.sum(x * x, axis=-1, dtype=np.float32)
    return (F32(1.0) / np.sqrt(ss * F32(1.0 / D) + F32(eps))).astype(np.float32)


def _rotate(x, c, s) -> np.ndarray:
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1).astype(np.float32)


def _rotate_back(g, c, s) -> np.ndarray:
    h = g.shape[-1] // 2
    g1, g2 = g[..., :h], g[..., h:]
    return np.concatenate([g1 * c - g2 * s, g1 * s + g2 * c], axis=-1).astype(np.float32)


def _mask(T: int, W: int) -> np.ndarray:
    d = np.arange(T)[:, None] - np.arange(T)[None, :]
    m = d >= 0
    if 0 <= W < T:
        m &= d <= W
    return m


def _kernel_kv(k, v, eps, cos, sin, ve, xg, gate_w):
    """Per key row: the K and V the products read, kscale, and the gate."""
    B, T, Hkv, D = k.shape
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    if cos is not None:
        kk = bf16(_rotate(k, cos[None, :, None, :], sin[None, :, None, :]))
    else:
        kk = k
    ksc = _recip_rms(kk, eps) * (LOG2E / F32(np.sqrt(D)))          # [B, T, Hkv]
    gate = None
    vv = v
    if ve is not None:
        z = np.asarray(xg, np.float32)[..., :32] @ np.asarray(gate_w, np.float32).T   # [B, T, Hkv]
        gate = (F32(2.0) / (F32(1.0) + np.exp2(-z * LOG2E))).astype(np.float32)
        vv = bf16(v + gate[..., None] * np.asarray(ve, np.float32))
    return kk, vv, ksc, gate


def _queries(q, eps, cos, sin):
    """The norm's input (rotated or not, fp32), r_q and q_hat (bf16)."""
    q = np.asarray(q, np.float32)
    qx = _rotate(q, cos[None, :, None, :], sin[None, :, None, :]) if cos is not None else q
    r = _recip_rms(qx, eps)
    return qx, r, bf16(qx * r[..., None])


def forward(q, k, v, window: int, eps: float = 1e-6, cos=None, sin=None, ve=None, xg=None,
            gate_w=None):
    """o (bf16 values, fp32 array) [B, T, H, D] and lse (fp32) [B, H, T]."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    cos = None if cos is None else np.asarray(cos, np.float32)
    sin = None if sin is None else np.asarray(sin, np.float32)
    kk, vv, ksc, _ = _kernel_kv(k, v, eps, cos, sin, ve, xg, gate_w)
    _, _, qh = _queries(q, eps, cos, sin)
    m = _mask(T, window)
    shift = F32(np.sqrt(D)) * LOG2E
    o = np.empty((B, T, H, D), np.float32)
    lse = np.empty((B, H, T), np.float32)
    for b in range(B):
        for h in range(H):
            hk = h // G
            s = qh[b, :, h] @ kk[b, :, hk].T
            p = np.where(m, np.exp2(s * ksc[b, :, hk][None, :] - shift), F32(0))
            pb = bf16(p)
            lsum = np.sum(pb, axis=1, dtype=np.float32)
            o[b, :, h] = bf16((pb @ vv[b, :, hk]) * (F32(1.0) / lsum)[:, None])
            lse[b, h] = F32(np.sqrt(D)) + np.log(lsum)
    return o, lse


def backward(q, k, v, o, lse, do, window: int, eps: float = 1e-6, cos=None, sin=None, ve=None,
             xg=None, gate_w=None):
    """dq [B, T, H, D], dk, dv [B, T, Hkv, D] (bf16 values), and with the gate
    also dve (bf16 values), dx [B, T, 32] (bf16 values) and dW_g [Hkv, 32]."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    cos = None if cos is None else np.asarray(cos, np.float32)
    sin = None if sin is None else np.asarray(sin, np.float32)
    kk, vv, ksc, gate = _kernel_kv(k, v, eps, cos, sin, ve, xg, gate_w)
    qx, rq, qh = _queries(q, eps, cos, sin)
    o = np.asarray(o, np.float32)
    do = np.asarray(do, np.float32)
    m = _mask(T, window)
    inv_sqrt_d = F32(1.0 / np.sqrt(D))
    dq = np.empty((B, T, H, D), np.float32)
    acc_dk = np.zeros((B, T, Hkv, D), np.float32)
    acc_dv = np.zeros((B, T, Hkv, D), np.float32)
    for b in range(B):
        for h in range(H):
            hk = h // G
            lq = np.asarray(lse[b, h], np.float32) * LOG2E
            delta = np.sum(do[b, :, h] * o[b, :, h], axis=1, dtype=np.float32)
            s = qh[b, :, h] @ kk[b, :, hk].T
            p = np.where(m, np.exp2(s * ksc[b, :, hk][None, :] - lq[:, None]), F32(0))
            dp = do[b, :, h] @ vv[b, :, hk].T
            dpd = dp - delta[:, None]
            acc_dv[b, :, hk] += bf16(p).T @ do[b, :, h]
            acc_dk[b, :, hk] += bf16(p * dpd).T @ qh[b, :, h]
            dqh = (bf16(p * dpd * ksc[b, :, hk][None, :]) @ kk[b, :, hk]) * (F32(1.0) / LOG2E)
            xh = qh[b, :, h]   # the bf16 q_hat of the products is the norm's output
            mean = np.sum(dqh * xh, axis=1, dtype=np.float32) * F32(1.0 / D)
            y = rq[b, :, h][:, None] * (dqh - xh * mean[:, None])
            if cos is not None:
                y = _rotate_back(y, cos, sin)
            dq[b, :, h] = bf16(y)
    rk = ksc * (F32(np.sqrt(D)) / LOG2E)
    khat = kk * rk[..., None]
    a = acc_dk * inv_sqrt_d
    mean = np.sum(a * khat, axis=-1, dtype=np.float32) * F32(1.0 / D)
    y = rk[..., None] * (a - khat * mean[..., None])
    if cos is not None:
        y = _rotate_back(y, cos[None, :, None, :], sin[None, :, None, :])
    dk = bf16(y)
    dv = bf16(acc_dv)
    if ve is None:
        return dq, dk, dv
    ve = np.asarray(ve, np.float32)
    dve = bf16(gate[..., None] * acc_dv)
    dz = np.sum(acc_dv * ve, axis=-1, dtype=np.float32) * gate * (F32(1.0) - F32(0.5) * gate)
    x32 = np.asarray(xg, np.float32)[..., :32]
    dx = bf16(dz @ np.asarray(gate_w, np.float32))
    dw = np.einsum("bth,btc->hc", dz, x32).astype(np.float32)
    return dq, dk, dv, dve, dx, dw
