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

Timing: `value` and `ms_per_step` come from the wall clock over exactly K
steps between two device synchronisations.  Every timed step also records HIP
events on the launch stream at its start, after its forwards and at its end;
their medians give the forward, backward and whole-step times.  Per-kernel
durations come from HIP events around each launch; they cost the stream a few
microseconds each, so the timed region brackets only the dominant kernel (the
roofline's) and the other kernels are recorded over a few untimed steps just
before it.

After the headline workload the same run measures the other single-GPU
workloads of the method's configuration list (the S layer, the L layer and the
long-context SSSL period: keys s_layer, l_layer, long) and the shorter
sequences and other window patterns of the pages' tuning space (SSSL at
T = 512 and 1024 with the same tokens per step, patterns L and SLLL: keys
t512_sssl_stack, t1024_sssl_stack, l_stack, slll_stack), with the same step
definition.  The CPU baseline (the fp64 oracle) runs first, before anything
touches the GPU, over a process pool with one BLAS thread per process.

    python bench.py [--steps K] [--warmup W] [--workload sssl_stack]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (AMD's published figure)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
BF16_FLOP_PER_CLK_CU = 4096   # gfx950 dense bf16 MFMA FLOP per clock per compute unit
METRIC = "attn fwd+bwd effective TFLOP/s & % bf16 MFMA peak, T=2048 H=4 D=128 SSSL"
# the method's other single-GPU configurations, then the shorter sequences and
# other window patterns of the pages' tuning space
EXTRA_WORKLOADS = ("s_layer", "l_layer", "long", "t512_sssl_stack", "t1024_sssl_stack", "l_stack",
                   "slll_stack", "sl_stack", "ssss_stack", "d256_sssl_stack", "d64_sssl_stack", "gqa_sssl_stack",
                   "rope_sssl_stack", "ve_sssl_stack")
MAX_POOL = 16                 # host worker processes at most (one GPU's share of the host)

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


# ------------------------------------------------------------------ CPU baseline

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_slice(task):
    """One (batch, head) slice through the fp64 oracle, forward then backward,
    on one BLAS thread.  Returns (seconds, F14 FLOPs credited)."""
    T, D, W, seed, sigma_qkv, sigma_do, eps = task
    from threadpoolctl import threadpool_limits
    import oracle
    from workloads import make_layer_inputs
    with threadpool_limits(limits=1):
        inp = make_layer_inputs(1, T, 1, D, seed, sigma_qkv, sigma_do)
        q, k, v, do = inp.as_f32()
        t0 = time.perf_counter()
        oracle.attention_fwd(q, k, v, W, True, eps)
        oracle.attention_bwd(q, k, v, do, W, True, eps)
        dt = time.perf_counter() - t0
    return dt, 14 * D * oracle.n_visible(T, W)


def cpu_baseline(wl, windows, budget_s):
    """Time the fp64 oracle (as it stands) on (batch, head) slices of the
    workload's layers, cycling through the layer windows, over a pool of
    worker processes with one BLAS thread each, for about budget_s of wall
    time.  Runs before the GPU is touched, so the workers start from a clean
    interpreter."""
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    n = max(1, min(affinity, MAX_POOL))
    tasks = [(wl.T, wl.D, windows[i % len(windows)], wl.seed(i % len(windows)) + 7919 * (i // len(windows)),
              wl.sigma_qkv, wl.sigma_do, wl.eps) for i in range(100000)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(n) as pool:
        pool.map(_oracle_slice, tasks[:n])                       # warm the workers (imports)
        t0 = time.perf_counter()
        first = pool.map(_oracle_slice, tasks[n:2 * n])          # one round to size the sample
        t1 = time.perf_counter() - t0
        rounds = max(1, int(budget_s / max(t1, 1e-3)) - 1)
        rest = pool.map(_oracle_slice, tasks[2 * n:2 * n + rounds * n])
        wall = time.perf_counter() - t0
    done = first + rest
    flops = sum(f for _, f in done)
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": n,
        "kind": "oracle",
        "sample": (f"{len(done)} (batch, head) slices of T={wl.T}, D={wl.D} cycling through the layer "
                   f"windows {sorted(set(windows))}, fp64 numpy forward + backward, one slice per task on "
                   f"{n} worker processes with one BLAS thread each, {wall:.1f} s wall; F14 credited per "
                   f"slice"),
        "affinity_cores": affinity,
        "cpu_count": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "busy_s": round(sum(t for t, _ in done), 2),
    }


# ------------------------------------------------------------------ GPU side

def _setup(wl, sw, torch, dev):
    """Inputs, outputs and workspaces of every layer of the workload."""
    from workloads import make_layer_inputs_device, rope_tables_bf16
    B, T, H, D, H_kv = wl.B, wl.T, wl.H, wl.D, wl.kv_heads
    if wl.explicit_window is not None:
        windows = [wl.explicit_window] * wl.n_layer
    else:
        windows = sw.layer_windows(wl.pattern, wl.n_layer, T)
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
    return layers, windows, rope


def measure(wl, args, sw, torch, dev, want_traffic=True):
    """Times the workload's step; returns a dict of figures."""
    import ctypes
    B, T, H, D, H_kv = wl.B, wl.T, wl.H, wl.D, wl.kv_heads
    layers, windows, rope = _setup(wl, sw, torch, dev)
    print(f"[bench] workload {wl.name}: B={B} T={T} H={H} H_kv={H_kv} D={D} windows={windows}",
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def fwd_all():
        for L in layers:
            sw.attn_fwd(L["q"], L["k"], L["v"], L["W"], True, wl.eps,
                        out=L["o"], lse=L["lse"], workspace=L["wsf"], stream=stream, rope=rope,
                        gate=L.get("gate"))

    def bwd_all():
        for L in reversed(layers):
            sw.attn_bwd(L["q"], L["k"], L["v"], L["o"], L["lse"], L["do"], L["W"], True, wl.eps,
                        dq=L["dq"], dk=L["dk"], dv=L["dv"], workspace=L["wsb"], stream=stream, rope=rope,
                        gate=L.get("gate"), fwd_workspace=L["wsf"])

    steps = args.steps if wl.name == args.workload else max(args.steps, args.extra_steps)
    for _ in range(args.warmup):
        fwd_all()
        bwd_all()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

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

    # every kernel's launches over a short untimed sample
    sw.check(lib.attn_profile_enable(1), "attn_profile_enable")
    for _ in range(args.sample_steps):
        fwd_all()
        bwd_all()
    torch.cuda.synchronize()
    per_kernel = read_kernels(list(KERNELS), args.sample_steps)
    dom_name = max(per_kernel, key=lambda n: per_kernel[n]["total_ms_per_step"])
    dom_kid = per_kernel[dom_name]["kid"]

    # the timed region: K steps between two synchronisations; per-step events on
    # the launch stream, and events around the dominant kernel's launches only
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    sw.check(lib.attn_profile_enable_mask(1 << dom_kid), "attn_profile_enable_mask")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        fwd_all()
        ev[s][1].record(stream)
        bwd_all()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / steps * 1e3
    per_kernel.update(read_kernels([dom_kid], steps))   # the timed region's own figures
    sw.check(lib.attn_profile_enable(0), "attn_profile_enable")
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    print(f"[bench] {wl.name}: timed {steps} steps: {ms_per_step:.3f} ms/step (wall), "
          f"{statistics.median(step_ms):.3f} ms median (events)", file=sys.stderr, flush=True)
    for v in per_kernel.values():
        v.pop("kid")

    flops_step = sum(14 * D * L["n_vis"] * B * H for L in layers)
    flops12_step = sum(12 * D * L["n_vis"] * B * H for L in layers)
    dom = per_kernel[dom_name]
    traffic = None
    if want_traffic:
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
    res = dict(
        wl=wl, windows=windows, steps=steps, ms_per_step=ms_per_step,
        step_ms_median=statistics.median(step_ms), fwd_ms_median=statistics.median(fwd_ms),
        bwd_ms_median=statistics.median(bwd_ms), flops_step=flops_step, flops12_step=flops12_step,
        value=flops_step / (ms_per_step * 1e-3) / 1e12, per_kernel=per_kernel, dom_name=dom_name,
        traffic=traffic, value_executed=value_executed,
    )
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _r(x, n=4):
    return None if x is None else round(x, n)


def summary(res, peak):
    """The compact figures of one workload (for the extra keys)."""
    dom = res["per_kernel"][res["dom_name"]]
    return {
        "config": {"B": res["wl"].B, "T": res["wl"].T, "H": res["wl"].H, "D": res["wl"].D,
                   "windows": res["windows"]},
        "steps": res["steps"],
        "ms_per_step": _r(res["ms_per_step"]),
        "value": _r(res["value"], 3),
        "pct_of_bf16_peak": _r(100.0 * res["value"] / peak, 2),
        "step_ms_median_events": _r(res["step_ms_median"]),
        "fwd_ms_median_events": _r(res["fwd_ms_median"]),
        "bwd_ms_median_events": _r(res["bwd_ms_median"]),
        "dominant_kernel": res["dom_name"],
        "dominant_frac": _r(dom["frac"]),
        "dominant_avg_us": _r(dom["avg_us"], 2),
        "kernels": {k: {"avg_us": _r(v["avg_us"], 2), "frac": _r(v["frac"])}
                    for k, v in res["per_kernel"].items()},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sample-steps", type=int, default=2,
                    help="untimed steps before the timed region that record every kernel's launches")
    ap.add_argument("--workload", default="sssl_stack")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other single-GPU workloads (s_layer, l_layer, long)")
    ap.add_argument("--extra-steps", type=int, default=20,
                    help="timed steps of each extra workload (at least --steps)")
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

    from workloads import workload
    wl = workload(args.workload)

    # the CPU baseline first: its worker processes start before anything touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        import oracle   # the library is not loaded yet: the windows from the oracle's layer rule
        windows = ([wl.explicit_window] * wl.n_layer if wl.explicit_window is not None
                   else oracle.layer_windows(wl.pattern, wl.n_layer, wl.T))
        print(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, windows, args.cpu_seconds)
        print(f"[bench] cpu baseline: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} processes",
              file=sys.stderr, flush=True)

    import torch
    import sliding_window_causal_qk_amd as sw

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cus, clk = ctypes_device_info(sw)
    peak_derived = cus * BF16_FLOP_PER_CLK_CU * clk * 1e3 / 1e12 if cus and clk else None
    print(f"[bench] device: {cus} compute units, peak clock {clk / 1e3:.0f} MHz -> bf16 dense peak "
          f"{peak_derived:.1f} TFLOP/s (published {PEAK_BF16_TFLOPS:.0f})", file=sys.stderr, flush=True)

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

    main_res = measure(wl, args, sw, torch, dev)
    extras = {}
    if not args.no_extra and args.workload == "sssl_stack":
        for name in EXTRA_WORKLOADS:
            extras[name] = summary(measure(workload(name), args, sw, torch, dev, want_traffic=False),
                                   PEAK_BF16_TFLOPS)

    r = main_res
    B, T, H, D, H_kv = wl.B, wl.T, wl.H, wl.D, wl.kv_heads
    per_kernel = r["per_kernel"]
    dom_name = r["dom_name"]
    dom = per_kernel[dom_name]
    roofline = {"kernel": dom_name, "bound": dom["bound"], "achieved": round(dom["achieved"], 3),
                "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4),
                "traffic": r["traffic"],
                "work_per_launch": dom["work_per_launch"], "work_unit": dom["work_unit"],
                "avg_launch_us": round(dom["avg_us"], 2)}
    out = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "H_kv": H_kv, "D": D, "rope": wl.rope,
                   "ve_gate": wl.ve_gate,
                   "pattern": wl.pattern,
                   "n_layer": len(r["windows"]), "windows": r["windows"], "eps": wl.eps,
                   "flop_convention": "F14 = 14*D*N_vis per (batch, head, layer)",
                   "flops_per_step": r["flops_step"], "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * r["value"] / PEAK_BF16_TFLOPS, 2),
        "peak_bf16_published_tflops": PEAK_BF16_TFLOPS,
        "peak_bf16_derived_tflops": _r(peak_derived, 1),
        "device": {"compute_units": cus, "peak_clock_mhz": clk / 1e3 if clk else None,
                   "bf16_flop_per_clk_per_cu": BF16_FLOP_PER_CLK_CU},
        "value_f12": round(r["flops12_step"] / (r["ms_per_step"] * 1e-3) / 1e12, 3),
        "value_executed_mfma": _r(r["value_executed"], 3),
        # medians over the timed steps of HIP events on the launch stream
        "step_ms_median_events": round(r["step_ms_median"], 4),
        "fwd_ms_median_events": round(r["fwd_ms_median"], 4),
        "bwd_ms_median_events": round(r["bwd_ms_median"], 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in per_kernel.items()},
        "kernels_timing": (f"HIP events on the launch stream: {dom_name} over the timed region, the "
                           f"other kernels over {args.sample_steps} untimed steps just before it"),
        "kernel_sources_sha": kernel_sources_sha(),
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


def ctypes_device_info(sw):
    import ctypes
    cus, clk = ctypes.c_int(), ctypes.c_int()
    if sw.lib().attn_device_info(0, ctypes.byref(cus), ctypes.byref(clk)) != 0:
        return None, None
    return cus.value, clk.value


if __name__ == "__main__":
    main()
