#!/usr/bin/env python3
"""Throughput of QK-RMSNorm causal sliding-window attention, forward + backward,
on one MI355X, through the C ABI of libswattn.

A step is one pass of the whole hot path over one batch: the forward of every
layer of the workload, then the backward of every layer in reverse order (each
backward reuses its forward's key pre-pass, as a training step would).  The
default workload is the depth-8 SSSL stack (8 independent layers, windows
1024 x3, 2048, 1024 x3, 2048; B=64, T=2048, H=4, D=128, bf16), the shape of the
pages' 5-minute training run.  Inputs are synthetic, seeded and already in HBM
when the timed region starts.

Effective FLOPs (F14): 14 * D * N_vis per (batch, head) and layer, N_vis the
number of visible (query, key) pairs: 4 D for the forward (QK^T, PV) and 10 D
for the backward with recomputation (QK^T, dP, dV, dQ, dK).  Masked pairs,
extra recomputation and the RMSNorm arithmetic are not credited.  value_f12
is the same step on the pages' 12 * D * N_vis count; value_executed_mfma is
the MFMA work the matrix cores executed (rocprofv3 counters of the same
workload and kernel sources, profiles/mfma.json; null when those are stale).

Per-kernel durations come from HIP events on the launch stream.  The events
around a launch cost the stream a few microseconds, so the timed region
records only the dominant kernel (the roofline's); the other kernels are
recorded over a few untimed steps just before it.

    python bench.py [--steps K] [--warmup W] [--workload sssl_stack]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (AMD's published figure)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "attn fwd+bwd effective TFLOP/s & % bf16 MFMA peak, T=2048 H=4 D=128 SSSL"

# algorithmic work credited to each kernel, per visible pair (FLOPs = c * D * N_vis)
# or per launch bytes for the memory-bound passes
KERNELS = {
    0: ("fwd_prep", "hbm"),
    1: ("attn_fwd", "mfma"),
    2: ("bwd_kscale", "hbm"),
    3: ("bwd_dkdv", "mfma"),
    4: ("bwd_dq", "mfma"),
    5: ("bwd_gate", "hbm"),
}
FWD_KERNELS = ("fwd_prep", "attn_fwd")
FLOPS_PER_PAIR_D = {1: 4, 3: 8, 4: 2}


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sliding_window_causal_qk_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_units(kid, B, T, H, D, n_vis, H_kv=None, rope=False, gate=False):
    """(amount, unit) of algorithmic work of one launch of kernel `kid`
    (H query heads, H_kv key/value heads; rope: the pre-passes also read the
    two bf16 [T, D/2] tables and write the rotated keys; gate: they read ve and
    the 32 gate channels of x, and the backward one also reads v and writes the
    gated values and the gate)."""
    H_kv = H if H_kv is None else H_kv
    E_kv = B * T * H_kv * D
    if kid in FLOPS_PER_PAIR_D:
        return FLOPS_PER_PAIR_D[kid] * D * n_vis * B * H, "flop"
    extra = (2 * E_kv + 2 * T * D) if rope else 0
    if kid == 5:   # read dz and x's 32 gate channels, write dx (bf16) and the partial sums
        return 4 * B * T * H_kv + 64 * B * T + 64 * B * T, "byte"
    # the key pre-pass (kid 0 in the forward, 2 in the backward): read K, write
    # the key scales; with the gate also read v, ve and x's 32 gate channels and
    # write the gated values (the backward also keeps the gate)
    if gate:
        extra += 6 * E_kv + 64 * B * T + (4 * B * H_kv * T if kid == 2 else 0)
    return 2 * E_kv + 4 * B * H_kv * T + extra, "byte"


def cpu_baseline(wl, windows, budget_s):
    """Time the fp64 oracle (as it stands) on (batch, head) slices of the
    workload's layers, cycling through the layer windows, for about budget_s."""
    import numpy as np
    import oracle
    from workloads import make_layer_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    flops = 0.0
    n = 0
    dt = 0.0
    layer = 0
    while dt < budget_s:
        W = windows[layer % len(windows)]
        inp = make_layer_inputs(1, wl.T, 1, wl.D, wl.seed(layer), wl.sigma_qkv, wl.sigma_do)
        q, k, v, do = inp.as_f32()
        ts = time.perf_counter()
        oracle.attention_fwd(q, k, v, W, True, wl.eps)
        oracle.attention_bwd(q, k, v, do, W, True, wl.eps)
        dt += time.perf_counter() - ts
        flops += 14 * wl.D * oracle.n_visible(wl.T, W)
        n += 1
        layer += 1
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n} (batch, head) slices of T={wl.T}, D={wl.D} cycling through the layer "
                   f"windows {sorted(set(windows))}, fp64 numpy forward + backward, {dt:.1f} s "
                   f"of oracle time; F14 credited per slice"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sample-steps", type=int, default=2,
                    help="untimed steps before the timed region that record every kernel's launches")
    ap.add_argument("--workload", default="sssl_stack")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain elementwise copy (torch.neg, fp32) over this many MiB, "
                         "the reference point for scaling HBM counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this attention path has no multi-GPU mode: every (batch, head) is independent, so a "
              "data-parallel run is N independent copies of the one-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_window_causal_qk_amd as sw
    from workloads import make_layer_inputs_device, rope_tables_bf16, workload

    wl = workload(args.workload)
    B, T, H, D, H_kv = wl.B, wl.T, wl.H, wl.D, wl.kv_heads
    if wl.explicit_window is not None:
        windows = [wl.explicit_window] * wl.n_layer
    else:
        windows = sw.layer_windows(wl.pattern, wl.n_layer, T)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: B={B} T={T} H={H} H_kv={H_kv} D={D} windows={windows}",
          file=sys.stderr, flush=True)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18          # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)              # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] copy calibration: 2 launches of {args.copy_calibration_mib} MiB read + "
              f"{args.copy_calibration_mib} MiB written", file=sys.stderr, flush=True)

    rope = None
    if wl.rope:
        rope = tuple(torch.from_numpy(t.view("int16")).view(torch.bfloat16).to(dev)
                     for t in rope_tables_bf16(T, D))
    fws = (sw.fwd_ve_workspace_bytes if wl.ve_gate else
           sw.fwd_rope_workspace_bytes if wl.rope else sw.fwd_workspace_bytes)
    bws = (sw.bwd_ve_workspace_bytes if wl.ve_gate else
           sw.bwd_rope_workspace_bytes if wl.rope else sw.bwd_workspace_bytes)
    layers = []
    for l, W in enumerate(windows):
        q, k, v, do = make_layer_inputs_device(B, T, H, D, wl.seed(l), wl.sigma_qkv, wl.sigma_do, dev,
                                               H_kv=H_kv)
        layers.append(dict(
            W=W, q=q, k=k, v=v, do=do,
            o=torch.empty_like(q), lse=torch.empty((B, H, T), dtype=torch.float32, device=dev),
            dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
            wsf=torch.empty(fws(B, T, H, D, H_kv), dtype=torch.uint8, device=dev),
            wsb=torch.empty(bws(B, T, H, D, H_kv), dtype=torch.uint8, device=dev),
            n_vis=sw.visible_pairs(T, W),
        ))
        if wl.ve_gate:   # value embedding, block input (n_embd = H D channels) and gate map
            g = torch.Generator(device=dev)
            g.manual_seed(wl.seed(l) + 100)
            layers[-1]["gate"] = (
                torch.randn((B, T, H_kv, D), generator=g, device=dev).to(torch.bfloat16),
                torch.randn((B, T, H * D), generator=g, device=dev).to(torch.bfloat16),
                torch.randn((H_kv, 32), generator=g, device=dev) * 0.2)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step():
        for L in layers:
            sw.attn_fwd(L["q"], L["k"], L["v"], L["W"], True, wl.eps,
                        out=L["o"], lse=L["lse"], workspace=L["wsf"], stream=stream, rope=rope,
                        gate=L.get("gate"))
        for L in reversed(layers):
            sw.attn_bwd(L["q"], L["k"], L["v"], L["o"], L["lse"], L["do"], L["W"], True, wl.eps,
                        dq=L["dq"], dk=L["dk"], dv=L["dv"], workspace=L["wsb"], stream=stream, rope=rope,
                        gate=L.get("gate"), fwd_workspace=L["wsf"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    import ctypes
    lib = sw.lib()

    def read_kernels(kids, nsteps):
        """Per-kernel averages of the recorded launches of kernels `kids` over nsteps steps."""
        res = {}
        for kid in kids:
            name, bound = KERNELS[kid]
            tot = ctypes.c_double()
            cnt = ctypes.c_longlong()
            sw.check(lib.attn_profile_read(kid, ctypes.byref(tot), ctypes.byref(cnt)), "attn_profile_read")
            if cnt.value == 0:
                continue
            work = 0.0
            unit = None
            for L in layers:
                amt, unit = algorithmic_units(kid, B, T, H, D, L["n_vis"], H_kv, wl.rope, wl.ve_gate)
                work += amt * nsteps
            secs = tot.value * 1e-3
            if unit == "flop":
                achieved, u, peak = work / secs / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS
            else:
                achieved, u, peak = work / secs / 1e9, "GB/s", PEAK_HBM_GBS
            res[name] = dict(kid=kid, avg_us=tot.value * 1e3 / cnt.value, launches=cnt.value,
                             total_ms_per_step=tot.value / nsteps, bound=bound,
                             achieved=achieved, unit=u, peak=peak, frac=achieved / peak,
                             work_per_launch=work / cnt.value, work_unit=unit)
        return res

    # Every kernel's launches in a short untimed sample; the events around
    # each launch cost the stream a few microseconds, so the timed region
    # below records only the dominant kernel, whose figures feed the roofline.
    sw.check(lib.attn_profile_enable(1), "attn_profile_enable")
    for _ in range(args.sample_steps):
        step()
    torch.cuda.synchronize()
    per_kernel = read_kernels(list(KERNELS), args.sample_steps)
    dom_name = max(per_kernel, key=lambda n: per_kernel[n]["total_ms_per_step"])
    dom_kid = per_kernel[dom_name]["kid"]

    sw.check(lib.attn_profile_enable_mask(1 << dom_kid), "attn_profile_enable_mask")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / args.steps * 1e3
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    per_kernel.update(read_kernels([dom_kid], args.steps))   # the timed region's own figures
    sw.check(lib.attn_profile_enable(0), "attn_profile_enable")
    for v in per_kernel.values():
        v.pop("kid")

    flops_step = sum(14 * D * L["n_vis"] * B * H for L in layers)
    flops12_step = sum(12 * D * L["n_vis"] * B * H for L in layers)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    dom = per_kernel[dom_name]
    traffic = None
    tf = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if os.path.exists(tf):
        try:
            rec = json.load(open(tf))
            if (rec.get("sources_sha") == kernel_sources_sha() and rec.get("workload") == wl.name
                    and dom_name in rec.get("kernels", {})):
                traffic = rec["kernels"][dom_name].get("bytes_per_launch")
        except Exception:
            traffic = None
    # third figure: the MFMA FLOPs the matrix cores executed (rocprofv3
    # counters of the same workload and sources, profiles/mfma.json), masked
    # blocks and recomputation included
    value_executed = None
    mf = os.path.join(ROOT, "profiles", "mfma.json")
    if os.path.exists(mf):
        try:
            rec = json.load(open(mf))
            if rec.get("sources_sha") == kernel_sources_sha() and rec.get("workload") == wl.name:
                ex = 0.0
                for name, v in per_kernel.items():
                    k = rec["kernels"].get(name)
                    if k:
                        v["executed_flops_per_launch"] = k["executed_flops_per_launch"]
                        v["mfma_busy"] = k["mfma_busy"]
                        ex += k["executed_flops_per_launch"] * len(windows)
                value_executed = ex / (ms_per_step * 1e-3) / 1e12
        except Exception:
            value_executed = None
    roofline = {"kernel": dom_name, "bound": dom["bound"], "achieved": round(dom["achieved"], 3),
                "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4),
                "traffic": traffic,
                "work_per_launch": dom["work_per_launch"], "work_unit": dom["work_unit"],
                "avg_launch_us": round(dom["avg_us"], 2)}

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, windows, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "H_kv": H_kv, "D": D, "rope": wl.rope,
                   "ve_gate": wl.ve_gate,
                   "pattern": wl.pattern,
                   "n_layer": len(windows), "windows": windows, "eps": wl.eps,
                   "flop_convention": "F14 = 14*D*N_vis per (batch, head, layer)",
                   "flops_per_step": flops_step, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "value_f12": round(flops12_step / (ms_per_step * 1e-3) / 1e12, 3),
        "value_executed_mfma": None if value_executed is None else round(value_executed, 3),
        # kernel time per step of each pass, from the per-kernel event sums
        "fwd_kernel_ms_per_step": round(sum(v["total_ms_per_step"] for k, v in per_kernel.items()
                                            if k in FWD_KERNELS), 4),
        "bwd_kernel_ms_per_step": round(sum(v["total_ms_per_step"] for k, v in per_kernel.items()
                                            if k not in FWD_KERNELS), 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in per_kernel.items()},
        "kernels_timing": (f"HIP events on the launch stream: {dom_name} over the timed region, the "
                           f"other kernels over {args.sample_steps} untimed steps just before it"),
        "kernel_sources_sha": kernel_sources_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
