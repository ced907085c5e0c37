"""Plain fp64 CPU oracle for QK-RMSNorm causal sliding-window attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the graft entry
point and the cpu_baseline leg of bench.py may import this package.  The
product path (the HIP library and its Python binding) never calls it, and it
shares no code with that path: the only thing both sides use is the seeded
input generator in `workloads`, which holds none of the method's arithmetic.

Sources (the pages this follows):
  * "Autoresearch 深度教程：AI 自主训练研究指南" (gitee brotherddc/autoresearch
    README): §5.2.2 (sliding-window sizes per layer), §7.3 (the `norm` helper,
    an RMSNorm with no weight), §5.2.1 (FlashAttention-3 with a (W, 0) window).
  * Line-by-line review of karpathy/autoresearch (web3.okx.com discover post,
    Russian): the paragraph on RMSNorm of queries and keys right before the
    attention product, and the paragraph on the SSSL pattern.
  * "让 AI 在你的显卡上自主做研究——autoresearch" (xyutech.top): the parameter
    counts and "Estimated FLOPs per token" lines of the full run.

Every function is pinned by tests under tests/ (brute force, closed forms,
library routines, finite differences, values printed on the pages); none is
"parity unpinned".
"""
from .attention import (  # noqa: F401
    rms_norm,
    kv_head,
    visible_mask,
    n_visible,
    scores,
    probabilities,
    attention_fwd,
    attention_bwd,
    fwd_rows,
    bwd_rows,
    rope,
    rope_bwd,
    attention_fwd_rope,
    attention_bwd_rope,
    ve_gate,
    attention_fwd_ve,
    attention_bwd_ve,
)
from .schedule import layer_windows, flops_per_token  # noqa: F401
