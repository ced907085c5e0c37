"""Per-layer window schedule and the pages' FLOPs-per-token estimate.

TEST INFRASTRUCTURE ONLY (see the package docstring).

layer_windows follows "Autoresearch 深度教程" §5.2.2 (sliding-window attention):
the pattern character of layer l is pattern[l % len(pattern)]; "L" gives a
window of the full sequence length, "S" half of it; the last layer is always
"L".  The okx.com line-by-line review states the same mapping for depth 8 with
SSSL: layers 0, 1, 2 local, 3 global, 4, 5, 6 local, 7 global.

flops_per_token is this module's reading of the "Estimated FLOPs per token"
figure printed on "让 AI 在你的显卡上自主做研究——autoresearch" (xyutech.top,
full run): 6 FLOPs per parameter of the matrices that see every token (the
transformer matrices and lm_head; the embedding tables and scalars are
lookups), plus, per layer, 12 * n_head * head_dim * w, where w is the number of
keys a query attends to in that layer, min(window, T).  With the printed
parameter counts and the SSSL schedule at T = 2048 this reproduces the printed
2.390784e+08 exactly; a wrong schedule would not.
"""
from __future__ import annotations

from typing import List


def layer_windows(pattern: str, n_layer: int, seq_len: int) -> List[int]:
    """Window W (keys to the left, the (W, 0) tuple's first entry) of every layer."""
    pattern = pattern.upper()
    if not pattern or any(c not in "SL" for c in pattern):
        raise ValueError(f"pattern must be a non-empty string over 'S'/'L': {pattern!r}")
    if n_layer < 1 or seq_len < 1:
        raise ValueError("n_layer and seq_len must be positive")
    long_w = seq_len
    short_w = seq_len // 2
    out = [long_w if pattern[l % len(pattern)] == "L" else short_w for l in range(n_layer)]
    out[-1] = long_w
    return out


def flops_per_token(matrix_params: int, lm_head_params: int, n_head: int, head_dim: int,
                    windows: List[int], seq_len: int) -> int:
    """The pages' per-token training FLOP estimate (see module docstring)."""
    attn = sum(12 * n_head * head_dim * min(w, seq_len) for w in windows)
    return 6 * (matrix_params + lm_head_params) + attn
