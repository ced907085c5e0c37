"""fp64 reference for causal sliding-window attention with RMSNorm on Q and K.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy in float64,
one (batch, head) slice at a time, with no tiling, fusion or reordering beyond
what the definitions below state.

What is computed (per batch b and head h; x[t] is the D-vector at position t):

  RMSNorm  ("Autoresearch 深度教程" §7.3, the `norm` helper, and the okx.com
  line-by-line review, paragraph on QK-norm: queries and keys are RMS-normalised
  right before the attention product, with no learned weight):
      r(x) = 1 / sqrt(mean_d x_d^2 + eps),   x_hat = x * r(x)

  Mask  ("Autoresearch 深度教程" §5.2.2: each layer gets a (W, 0) window, i.e. W
  keys to the left and none to the right, as FlashAttention's window tuple;
  §5.2.1 loads FA3 with that tuple):
      causal:      key j is visible to query i  iff  0 <= i - j <= W
      non-causal:  |i - j| <= W
      W = -1 means no bound (full causal, resp. full bidirectional).

  Scores / softmax / output (the attention product itself; the pages leave the
  scale unstated, so FlashAttention's default 1/sqrt(D) is used):
      s_ij = (q_hat_i . k_hat_j) / sqrt(D) on visible pairs, -inf elsewhere
      P_ij = exp(s_ij - m_i) / sum_visible exp(s_ij - m_i),  m_i = max_visible s_ij
      o_i  = sum_j P_ij v_j
      lse_i = m_i + ln sum_visible exp(s_ij - m_i)      (natural log, scaled logits)

  Grouped key/value heads ("Autoresearch 深度教程" §7.3: the attention module
  has n_kv_head key/value heads, allowed to be fewer than n_head; the K and V
  projections are n_kv_head heads wide).  The pages do not spell out which
  query heads share a key/value head; FlashAttention's grouping is taken:
  with G = H / H_kv, query head h reads key/value head floor(h / G).  K and V
  are then [B, T, H_kv, D]; a shared head's gradient is the sum over the G
  query heads that read it.

  Rotary position embedding, optionally applied to q and k before the norm
  ("Autoresearch 深度教程" §7.4: each head's D channels are split into the
  halves x1 = x[:D/2], x2 = x[D/2:]; position t rotates every pair (x1_i, x2_i)
  by the angle whose cosine and sine are cos[t, i], sin[t, i], tables held in
  bf16; §7.3's attention module rotates q and k, then normalises them):
      y1 = x1 * cos + x2 * sin,   y2 = x2 * cos - x1 * sin
  The backward maps a gradient g of y back through the transpose:
      dx1 = g1 * cos - g2 * sin,  dx2 = g1 * sin + g2 * cos

  Value-embedding gate, optionally applied to v ("Autoresearch 深度教程"
  §5.2.3: a layer with a value embedding ve [B, T, H_kv, D] mixes it into v
  through a per-token, per-head gate computed from the first 32 channels of
  the block input x by a bias-free linear map W_g [H_kv, 32]):
      z[b, t, h] = sum_c W_g[h, c] x[b, t, c],   gate = 2 sigmoid(z)
      v' = v + gate * ve          (attention then uses v')
  The backward, given dv' (the gradient attention hands to v'):
      dv = dv',  dve = gate * dv',  dgate = sum_d dv' * ve,
      dz = dgate * gate * (1 - gate / 2),
      dW_g[h, c] = sum_{b,t} dz[b, t, h] x[b, t, c],  dx[b, t, c] = sum_h dz[b, t, h] W_g[h, c]

  Backward, given dO (chain rule through the three steps above):
      dV = P^T dO
      dP = dO V^T
      Delta_i = dO_i . o_i
      dS = P * (dP - Delta)
      dq_hat = dS k_hat / sqrt(D),   dk_hat = dS^T q_hat / sqrt(D)
      dx = r * (dx_hat - x_hat * mean_d(dx_hat * x_hat))   for x in {q, k}
"""
from __future__ import annotations

from typing import Iterable, Sequence, Tuple

import numpy as np

_ROW_BLOCK = 512


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """RMSNorm over the last axis with unit gain; returns (x_hat, r)."""
    x = _f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * r[..., None], r


def visible_mask(T: int, window: int, causal: bool = True,
                 rows: Sequence[int] | None = None) -> np.ndarray:
    """Boolean mask [len(rows), T]: True where key j is visible to query i."""
    if window < -1:
        raise ValueError("window must be >= -1")
    i = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(T)
    d = i[:, None] - j[None, :]
    if causal:
        m = d >= 0
        if window >= 0:
            m &= d <= window
    else:
        m = np.ones_like(d, dtype=bool) if window < 0 else (np.abs(d) <= window)
    return m


def n_visible(T: int, window: int, causal: bool = True) -> int:
    """Number of visible (i, j) pairs of one (batch, head) slice."""
    total = 0
    for i0 in range(0, T, _ROW_BLOCK):
        rows = range(i0, min(T, i0 + _ROW_BLOCK))
        total += int(visible_mask(T, window, causal, rows).sum())
    return total


def _slice(x: np.ndarray, b: int, h: int) -> np.ndarray:
    return _f64(x[b, :, h, :])


def rope(x, cos, sin) -> np.ndarray:
    """Rotary embedding of x [..., T, H, D] (or [T, D]) with tables cos, sin
    [T, D/2]: position t rotates the pair (x[..., i], x[..., i + D/2]) by the
    angle of (cos[t, i], sin[t, i])."""
    x = _f64(x)
    c, s = _f64(cos), _f64(sin)
    if x.ndim == 4:
        c, s = c[None, :, None, :], s[None, :, None, :]
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def rope_bwd(g, cos, sin) -> np.ndarray:
    """Gradient w.r.t. the input of rope, given the gradient g of its output."""
    g = _f64(g)
    c, s = _f64(cos), _f64(sin)
    if g.ndim == 4:
        c, s = c[None, :, None, :], s[None, :, None, :]
    h = g.shape[-1] // 2
    g1, g2 = g[..., :h], g[..., h:]
    return np.concatenate([g1 * c - g2 * s, g1 * s + g2 * c], axis=-1)


def ve_gate(xg, gate_w) -> np.ndarray:
    """gate [B, T, H_kv] = 2 sigmoid(x[..., :32] W_g^T), xg [B, T, >= 32],
    gate_w [H_kv, 32]."""
    z = _f64(xg)[..., :32] @ _f64(gate_w).T
    return 2.0 / (1.0 + np.exp(-z))


def attention_fwd_ve(q, k, v, ve, xg, gate_w, window: int, causal: bool = True,
                     eps: float = 1e-6, cos=None, sin=None):
    """Forward with the value-embedding gate on v (and, given tables, the
    rotary embedding of q and k)."""
    vg = _f64(v) + ve_gate(xg, gate_w)[..., None] * _f64(ve)
    if cos is not None:
        return attention_fwd_rope(q, k, vg, cos, sin, window, causal, eps)
    return attention_fwd(q, k, vg, window, causal, eps)


def attention_bwd_ve(q, k, v, do, ve, xg, gate_w, window: int, causal: bool = True,
                     eps: float = 1e-6, cos=None, sin=None):
    """dq, dk, dv, dve, dxg [B, T, 32], dgate_w [H_kv, 32] of attention_fwd_ve."""
    gate = ve_gate(xg, gate_w)
    vg = _f64(v) + gate[..., None] * _f64(ve)
    if cos is not None:
        dq, dk, dvg = attention_bwd_rope(q, k, vg, do, cos, sin, window, causal, eps)
    else:
        dq, dk, dvg = attention_bwd(q, k, vg, do, window, causal, eps)
    dve = gate[..., None] * dvg
    dz = np.sum(dvg * _f64(ve), axis=-1) * gate * (1.0 - gate / 2.0)
    x32 = _f64(xg)[..., :32]
    dW = np.einsum("bth,btc->hc", dz, x32)
    dx = dz @ _f64(gate_w)
    return dq, dk, dvg, dve, dx, dW


def attention_fwd_rope(q, k, v, cos, sin, window: int, causal: bool = True,
                       eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray]:
    """Forward with rotary embedding of q and k before the norm."""
    return attention_fwd(rope(q, cos, sin), rope(k, cos, sin), v, window, causal, eps)


def attention_bwd_rope(q, k, v, do, cos, sin, window: int, causal: bool = True,
                       eps: float = 1e-6):
    """dq, dk (w.r.t. the q, k before rotation), dv of attention_fwd_rope."""
    dq, dk, dv = attention_bwd(rope(q, cos, sin), rope(k, cos, sin), v, do, window, causal, eps)
    return rope_bwd(dq, cos, sin), rope_bwd(dk, cos, sin), dv


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h (G = H / H_kv consecutive query
    heads share one)."""
    if H_kv < 1 or H % H_kv:
        raise ValueError("the number of query heads must be a multiple of H_kv")
    return h // (H // H_kv)


def _kv(q, k, h: int) -> int:
    return kv_head(h, np.shape(q)[2], np.shape(k)[2])


def scores(q, k, b: int, h: int, window: int, causal: bool, eps: float,
           rows: Sequence[int] | None = None) -> np.ndarray:
    """Masked scaled scores s [len(rows), T] of slice (b, h); -inf where masked."""
    qs, ks = _slice(q, b, h), _slice(k, b, _kv(q, k, h))
    T, D = ks.shape
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    qh, _ = rms_norm(qs[rows], eps)
    kh, _ = rms_norm(ks, eps)
    s = (qh @ kh.T) / np.sqrt(D)
    return np.where(visible_mask(T, window, causal, rows), s, -np.inf)


def probabilities(q, k, b: int, h: int, window: int, causal: bool, eps: float,
                  rows: Sequence[int] | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax rows P [len(rows), T] (masked entries exactly 0) and lse [len(rows)]."""
    s = scores(q, k, b, h, window, causal, eps, rows)
    m = np.max(s, axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(s - m[:, None])          # exp(-inf) = 0 exactly on masked entries
    z = np.sum(e, axis=1)
    return e / z[:, None], m + np.log(z)


def fwd_rows(q, k, v, b: int, h: int, rows: Sequence[int], window: int,
             causal: bool = True, eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray]:
    """Output rows o[rows] [n, D] and lse[rows] [n] of slice (b, h)."""
    rows = np.asarray(rows, dtype=np.int64)
    vs = _slice(v, b, _kv(q, v, h))
    o = np.empty((len(rows), vs.shape[1]))
    lse = np.empty(len(rows))
    for s0 in range(0, len(rows), _ROW_BLOCK):
        r = rows[s0:s0 + _ROW_BLOCK]
        p, l = probabilities(q, k, b, h, window, causal, eps, r)
        o[s0:s0 + len(r)] = p @ vs
        lse[s0:s0 + len(r)] = l
    return o, lse


def attention_fwd(q, k, v, window: int, causal: bool = True,
                  eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray]:
    """Full forward: o [B, T, H, D] and lse [B, H, T], both float64 (k, v may
    have fewer heads than q: grouped key/value heads)."""
    B, T, H, D = np.shape(q)
    o = np.empty((B, T, H, np.shape(v)[3]))
    lse = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            o[b, :, h, :], lse[b, h, :] = fwd_rows(q, k, v, b, h, range(T), window, causal, eps)
    return o, lse


def _rms_norm_bwd(x: np.ndarray, dx_hat: np.ndarray, eps: float) -> np.ndarray:
    """Gradient w.r.t. the pre-norm rows x, given the gradient w.r.t. x_hat."""
    x_hat, r = rms_norm(x, eps)
    proj = np.mean(dx_hat * x_hat, axis=-1, keepdims=True)
    return r[..., None] * (dx_hat - x_hat * proj)


def _bwd_slice(q, k, v, do, b, h, window, causal, eps):
    """Of query head h: dq [T, D], and its contributions dk_hat, dv [T, D] to
    the gradients of the key/value head it reads."""
    hk = _kv(q, k, h)
    qs, dos = _slice(q, b, h), _slice(do, b, h)
    ks, vs = _slice(k, b, hk), _slice(v, b, hk)
    T, D = qs.shape
    qh, _ = rms_norm(qs, eps)
    kh, _ = rms_norm(ks, eps)
    dq_hat = np.zeros_like(qs)
    dk_hat = np.zeros_like(ks)
    dv = np.zeros_like(vs)
    for i0 in range(0, T, _ROW_BLOCK):
        rows = np.arange(i0, min(T, i0 + _ROW_BLOCK))
        p, _ = probabilities(q, k, b, h, window, causal, eps, rows)
        o = p @ vs
        dv += p.T @ dos[rows]
        dp = dos[rows] @ vs.T
        delta = np.sum(dos[rows] * o, axis=1)
        ds = p * (dp - delta[:, None])
        dq_hat[rows] = ds @ kh / np.sqrt(D)
        dk_hat += ds.T @ qh[rows] / np.sqrt(D)
    return _rms_norm_bwd(qs, dq_hat, eps), dk_hat, dv


def attention_bwd(q, k, v, do, window: int, causal: bool = True,
                  eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full backward: dq [B, T, H, D], dk and dv [B, T, H_kv, D], float64
    (w.r.t. the pre-norm q, k)."""
    B, T, H, D = np.shape(q)
    H_kv = np.shape(k)[2]
    dq = np.empty((B, T, H, D))
    dk_hat = np.zeros((B, T, H_kv, D))
    dv = np.zeros((B, T, H_kv, np.shape(v)[3]))
    for b in range(B):
        for h in range(H):
            hk = _kv(q, k, h)
            dq[b, :, h], dkh, dvh = _bwd_slice(q, k, v, do, b, h, window, causal, eps)
            dk_hat[b, :, hk] += dkh
            dv[b, :, hk] += dvh
    dk = np.empty((B, T, H_kv, D))
    for b in range(B):
        for hk in range(H_kv):
            dk[b, :, hk] = _rms_norm_bwd(_slice(k, b, hk), dk_hat[b, :, hk], eps)
    return dq, dk, dv


def _rows_seeing(keys: Iterable[int], T: int, window: int, causal: bool) -> np.ndarray:
    """All query rows i that see at least one of the given keys."""
    keys = np.asarray(list(keys), dtype=np.int64)
    if len(keys) == 0:
        return keys
    need = np.zeros(T, dtype=bool)
    for i0 in range(0, T, _ROW_BLOCK):
        rows = np.arange(i0, min(T, i0 + _ROW_BLOCK))
        need[rows] = visible_mask(T, window, causal, rows)[:, keys].any(axis=1)
    return np.nonzero(need)[0]


def bwd_rows(q, k, v, do, b: int, h: int, q_rows: Sequence[int], k_rows: Sequence[int],
             window: int, causal: bool = True, eps: float = 1e-6):
    """Sampled gradients: dq[q_rows] of query head h; dk[k_rows], dv[k_rows] of
    the key/value head that h reads, summed over every query head reading it.

    dq_i needs only row i of P and dP.  dk_j and dv_j need column j of P and dS,
    hence every row that sees key j (each with its own lse and Delta), in every
    query head of the group."""
    H, H_kv = np.shape(q)[2], np.shape(k)[2]
    hk = kv_head(h, H, H_kv)
    qs, dos = _slice(q, b, h), _slice(do, b, h)
    ks, vs = _slice(k, b, hk), _slice(v, b, hk)
    T, D = qs.shape
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    kh, _ = rms_norm(ks, eps)

    dq = np.empty((len(q_rows), D))
    for s0 in range(0, len(q_rows), _ROW_BLOCK):
        rows = q_rows[s0:s0 + _ROW_BLOCK]
        p, _ = probabilities(q, k, b, h, window, causal, eps, rows)
        o = p @ vs
        dp = dos[rows] @ vs.T
        delta = np.sum(dos[rows] * o, axis=1)
        ds = p * (dp - delta[:, None])
        dq[s0:s0 + len(rows)] = _rms_norm_bwd(qs[rows], ds @ kh / np.sqrt(D), eps)

    dk_hat = np.zeros((len(k_rows), D))
    dv = np.zeros((len(k_rows), vs.shape[1]))
    need = _rows_seeing(k_rows, T, window, causal)
    G = H // H_kv
    for hq in range(hk * G, hk * G + G):
        qs_g, dos_g = _slice(q, b, hq), _slice(do, b, hq)
        for s0 in range(0, len(need), _ROW_BLOCK):
            rows = need[s0:s0 + _ROW_BLOCK]
            p, _ = probabilities(q, k, b, hq, window, causal, eps, rows)
            o = p @ vs
            dp = dos_g[rows] @ vs.T
            delta = np.sum(dos_g[rows] * o, axis=1)
            ds = p * (dp - delta[:, None])
            qh, _ = rms_norm(qs_g[rows], eps)
            dv += p[:, k_rows].T @ dos_g[rows]
            dk_hat += ds[:, k_rows].T @ qh / np.sqrt(D)
    dk = _rms_norm_bwd(ks[k_rows], dk_hat, eps)
    return dq, dk, dv
