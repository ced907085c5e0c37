"""Seeded synthetic workloads: shapes, seeds and value distributions only.

This module is shared by the oracle side and the HIP side of the tests and the
bench. It holds no attention arithmetic: it draws Gaussian tensors from a seed,
rounds them to bf16 and names the five workloads. Each side turns a layer
pattern into windows with its own code.

The shapes are those of the pages' training run: the model config line of
"自主AI研究员Autoresearch彻夜炼丹" (watermelonwater.tech) gives sequence_len 2048,
n_head = n_kv_head = 4, n_embd 512 (so head_dim 128) and window_pattern SSSL; the
tutorial "Autoresearch 深度教程" (gitee brotherddc/autoresearch) §10.1 gives the
device batch 128 and the per-layer window rule.  The pages train on real text
activations, which are not available; seeded N(0, sigma^2) bf16 tensors of the
same shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

EPS = 1e-6


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian_bf16(shape: Tuple[int, ...], rng: np.random.Generator, sigma: float = 1.0) -> np.ndarray:
    """Draw N(0, sigma^2) in fp32 and round to bf16; returns the uint16 bit patterns."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return round_to_bf16_bits(x)


def rope_tables_bf16(T: int, D: int, base: float = 10000.0) -> Tuple[np.ndarray, np.ndarray]:
    """Rotary tables as the tutorial's model precomputes them ("Autoresearch
    深度教程" §7.4): inverse frequencies base^(-c / D) for c = 0, 2, .., D - 2,
    angles t * inv_freq for positions t < T, cos and sin in fp32, rounded to
    bf16.  Returns the (cos, sin) bit patterns, [T, D/2] uint16."""
    channel = np.arange(0, D, 2, dtype=np.float32)
    inv_freq = (1.0 / (np.float32(base) ** (channel / np.float32(D)))).astype(np.float32)
    ang = np.outer(np.arange(T, dtype=np.float32), inv_freq).astype(np.float32)
    return round_to_bf16_bits(np.cos(ang)), round_to_bf16_bits(np.sin(ang))


@dataclass
class LayerInputs:
    """bf16 bit patterns (uint16) in the [B, T, H, D] layout."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray

    def as_f32(self):
        return tuple(bf16_bits_to_f32(t) for t in (self.q, self.k, self.v, self.do))


def make_layer_inputs(B: int, T: int, H: int, D: int, seed: int,
                      sigma_qkv: float = 1.0, sigma_do: float = 1.0,
                      H_kv: int | None = None) -> LayerInputs:
    """Q, K, V then dO, drawn in that order from one default_rng(seed) stream.
    Q and dO have H heads, K and V H_kv (default H)."""
    rng = np.random.default_rng(seed)
    shape = (B, T, H, D)
    kv_shape = (B, T, H if H_kv is None else H_kv, D)
    q = gaussian_bf16(shape, rng, sigma_qkv)
    k = gaussian_bf16(kv_shape, rng, sigma_qkv)
    v = gaussian_bf16(kv_shape, rng, sigma_qkv)
    do = gaussian_bf16(shape, rng, sigma_do)
    return LayerInputs(q, k, v, do)


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    D: int
    pattern: str              # per-layer pattern, e.g. "SSSL"; "W<n>" rows use an explicit window
    n_layer: int
    seed0: int
    sigma_qkv: float = 1.0
    sigma_do: float = 1.0
    explicit_window: int | None = None   # for the single-layer configs
    eps: float = EPS
    notes: str = ""
    H_kv: int | None = None   # key/value heads (None: H, plain multi-head attention)
    rope: bool = False        # q, k are given before the rotary embedding (base 10000)
    ve_gate: bool = False     # value-embedding gate on v (block input width n_embd = H D)

    def seed(self, layer: int) -> int:
        return self.seed0 + layer

    @property
    def kv_heads(self) -> int:
        return self.H if self.H_kv is None else self.H_kv


WORKLOADS: List[Workload] = [
    Workload("tiny", B=1, T=128, H=2, D=64, pattern="S", n_layer=1, seed0=0,
             explicit_window=64,
             notes="parity case the oracle finishes in seconds; window 64 = T/2"),
    Workload("s_layer", B=8, T=2048, H=4, D=128, pattern="S", n_layer=1, seed0=1,
             explicit_window=1024, notes="one sliding-window layer, window T/2"),
    Workload("l_layer", B=8, T=2048, H=4, D=128, pattern="L", n_layer=1, seed0=2,
             explicit_window=2048, notes="one full-causal layer, window T"),
    Workload("sssl_stack", B=64, T=2048, H=4, D=128, pattern="SSSL", n_layer=8, seed0=1000,
             notes="depth-8 SSSL stack: 8 independent layers, throughput summed"),
    Workload("long", B=4, T=8192, H=8, D=128, pattern="SSSL", n_layer=4, seed0=2000,
             sigma_qkv=2.0 ** 0.5,
             notes="one SSSL period at T=8192; Q/K/V variance 2, dO variance 1"),
    Workload("gqa_sssl_stack", B=64, T=2048, H=4, D=128, pattern="SSSL", n_layer=8, seed0=3000,
             H_kv=2,
             notes="the SSSL stack with grouped key/value heads, n_kv_head = n_head / 2"),
    Workload("rope_sssl_stack", B=64, T=2048, H=4, D=128, pattern="SSSL", n_layer=8, seed0=4000,
             rope=True,
             notes="the SSSL stack with the rotary embedding fused ahead of the QK norm"),
    Workload("d256_sssl_stack", B=64, T=2048, H=2, D=256, pattern="SSSL", n_layer=8, seed0=6000,
             notes="the SSSL stack at head size 256 (same n_embd = 512: 2 heads)"),
    Workload("ve_sssl_stack", B=64, T=2048, H=4, D=128, pattern="SSSL", n_layer=8, seed0=5000,
             ve_gate=True,
             notes="the SSSL stack with the value-embedding gate fused into the V load"),
    # the tutorial's tuning space (§10.1.1): shorter sequences and the other
    # window patterns, at the stack's 131072 tokens per step
    Workload("t512_sssl_stack", B=256, T=512, H=4, D=128, pattern="SSSL", n_layer=8, seed0=7000,
             notes="the SSSL stack at sequence length 512 (windows 256 / 512), same tokens per step"),
    Workload("t1024_sssl_stack", B=128, T=1024, H=4, D=128, pattern="SSSL", n_layer=8, seed0=7100,
             notes="the SSSL stack at sequence length 1024 (windows 512 / 1024), same tokens per step"),
    Workload("l_stack", B=64, T=2048, H=4, D=128, pattern="L", n_layer=8, seed0=7200,
             notes="pattern L: every layer full causal"),
    Workload("slll_stack", B=64, T=2048, H=4, D=128, pattern="SLLL", n_layer=8, seed0=7300,
             notes="pattern SLLL: one sliding-window layer in four"),
    Workload("sl_stack", B=64, T=2048, H=4, D=128, pattern="SL", n_layer=8, seed0=7400,
             notes="pattern SL: sliding-window and full-causal layers alternate"),
    Workload("ssss_stack", B=64, T=2048, H=4, D=128, pattern="SSSS", n_layer=8, seed0=7500,
             notes="pattern SSSS: sliding window everywhere but the last layer, which is full"),
    Workload("d64_sssl_stack", B=64, T=2048, H=8, D=64, pattern="SSSL", n_layer=8, seed0=7600,
             notes="the SSSL stack at head size 64 (same n_embd = 512: 8 heads)"),
]


@dataclass
class GateInputs:
    """Value-embedding gate inputs: ve bf16 bits [B, T, H_kv, D], the block
    input x bf16 bits [B, T, C] (its first 32 channels feed the gate) and the
    gate map fp32 [H_kv, 32]."""
    ve: np.ndarray
    x: np.ndarray
    gate_w: np.ndarray


def make_gate_inputs(B: int, T: int, H_kv: int, D: int, C: int, seed: int,
                     w_sigma: float = 0.2) -> GateInputs:
    """ve ~ N(0, 1) and x ~ N(0, 1) rounded to bf16, gate_w ~ N(0, w_sigma^2) in
    fp32, drawn in that order from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    ve = gaussian_bf16((B, T, H_kv, D), rng)
    x = gaussian_bf16((B, T, C), rng)
    gw = (rng.standard_normal((H_kv, 32), dtype=np.float32) * np.float32(w_sigma)).astype(np.float32)
    return GateInputs(ve, x, gw)


def workload(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_layer_inputs_device(B: int, T: int, H: int, D: int, seed: int,
                             sigma_qkv: float = 1.0, sigma_do: float = 1.0, device="cuda",
                             H_kv: int | None = None):
    """Same recipe drawn on the GPU (torch's Philox stream, not numpy's): N(0, sigma^2)
    in fp32, rounded to bf16 (round to nearest even), Q, K, V then dO from one
    generator seeded with `seed`.  For timing runs, where only the distribution
    matters, and for problems too large to draw on the host; the other parity
    tests use make_layer_inputs, which the oracle also reads."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (B, T, H, D)
    kv_shape = (B, T, H if H_kv is None else H_kv, D)
    out = []
    for sigma, shp in ((sigma_qkv, shape), (sigma_qkv, kv_shape), (sigma_qkv, kv_shape), (sigma_do, shape)):
        x = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)
