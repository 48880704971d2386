#!/usr/bin/env python3
"""Benchmark of the multi-adapter LoRA apply path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama7b_prefill]
                    [--extra llama7b_decode,qwen32b_decode]

One step is one pass of the whole hot path over one batch: the device plan
(lora_plan_prepare) and, for every group of modules of the workload's layer,
lora_apply_group (a shrink launch and an expand launch).
Steps rotate over L "layer sets" (each with its own adapter weights, x and y,
like the layers of a model) so that the bytes the kernels read come from HBM
rather than from the 256 MB Infinity Cache.  Inputs are resident
in HBM before timing starts.  Prints one JSON line.

The headline ("value") is the Llama-7B-shaped prefill (segment-grouped SGMV,
32 requests of 128..2048 tokens, q/k/v/o 4096->4096, ranks 8..64 padded to 64):
the largest workload of the metric that fits one GPU.  The two decode (BGMV)
workloads, Llama-7B q/v at 256 tokens and Qwen3-32B q/k/v/o at 512 tokens, are
measured after it with their own step counts and reported under their names.

Passes over the same K steps (after W warm-up steps):
  eager      library calls from Python, one step after the other ("value");
  graph      the calls of one rotation captured into a HIP graph and replayed,
             as a serving engine replays its decode step (--launch graph makes
             this "value");
  plan_amortized  one lora_plan_prepare, then the K steps' applies only (the
             layers of a model share one batch and its slot indices);
  fused      (decode batches) lora_apply_group_fused: each group's shrink and
             expand in one launch; and its plan_amortized form, one
             lora_plan_prepare, then the K steps' fused applies;
  step_spread     an event after each step: p10 / p50 / p90 step times;
  kernels    per-dispatch start / stop events the library records with each
             of its dispatches (hipExtLaunchKernelGGL): kernel times.

roofline   the kernel with the largest share of the step: its algorithmic bytes /
           its kernel time against the 8 TB/s HBM peak ("frac"), its fraction of
           a measured 1 GiB device copy (copy_GBps, read plus write), and, flat
           beside them, its algorithmic flops per second against the 2.5 PFLOP/s
           dense bf16 MFMA peak ("mfma_frac") with rocprofv3's MfmaUtil reading
           ("mfma_util_pct", from the committed counter summary when the kernel
           source is unchanged); "traffic" is the calibrated FETCH_SIZE +
           WRITE_SIZE of the same kernel, from its committed counter summary
cpu_baseline  the CPU oracle on the host cores over a bounded sample of the
           headline workload (rank 0, one GPU only): all threads, and one thread
           on a smaller sample; nproc and the CPU model

saved_module  the saved-module product (modules_to_save) on the headline batch,
           every adapter saving o_proj: the dense segmented GEMM on the matrix
           cores, its TFLOP/s against the dense bf16 peak

--workload churn [--prefetch] times adapter uploads with the applies instead
(see churn and churn_prefetch below); its "h2d" carries the upload rate beside
copy_GBps, back-to-back pinned copies of one adapter's size on the same link.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFS = 2500.0     # dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="llama7b_prefill",
                   choices=["llama7b_decode", "qwen32b_decode", "llama7b_prefill", "churn"])
    p.add_argument("--extra", default="llama7b_decode,qwen32b_decode",
                   type=lambda v: [w for w in v.split(",") if w],
                   help="further workloads measured after the headline one and reported as "
                        "extra keys (empty: none)")
    p.add_argument("--max-tokens", type=int, default=0,
                   help="token capacity of the slot ctx (default: the batch's own size)")
    p.add_argument("--extra-steps", type=int, default=2000)
    p.add_argument("--extra-warmup", type=int, default=200)
    p.add_argument("--no-saved", dest="saved", action="store_false",
                   help="skip the saved-module (modules_to_save) measurement on the headline batch")
    p.add_argument("--saved-only", action="store_true",
                   help="measure only the saved-module product on the prefill batch")
    p.add_argument("--churn-steps", type=int, default=50)
    p.add_argument("--prefetch", action="store_true",
                   help="churn: upload the next step's misses while the current step computes "
                        "(slots declared per plan, spare slots beyond the per-step cap)")
    p.add_argument("--churn-slots", type=int, default=192,
                   help="churn --prefetch: GPU slots (the per-step cap stays 128)")
    p.add_argument("--layer-bytes", type=float, default=1.2e9,
                   help="minimum footprint of the rotated layer sets (bytes)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--shared-x", action="store_true",
                   help="the members of a group read one x buffer, as q, k and v read the layer "
                        "input (the grouped shrink then fetches x from HBM once per group)")
    p.add_argument("--launch", choices=["graph", "eager"], default="eager",
                   help="which timed pass gives value: eager calls or graph replays")
    p.add_argument("--no-kernel-timing", action="store_true",
                   help="time the steps without per-dispatch kernel events (roofline then null)")
    p.add_argument("--calib-copy", action="store_true",
                   help="run only a plain device copy of known size (counter calibration)")
    return p.parse_args()


# Modules applied in one grouped launch: projections that read the same layer
# input are applied together (q and v; q, k and v), the output projection alone.
GROUPS = {"llama7b_decode": [["q_proj", "v_proj"]],
          "qwen32b_decode": [["q_proj", "k_proj", "v_proj"], ["o_proj"]],
          "llama7b_prefill": [["q_proj", "k_proj", "v_proj"], ["o_proj"]]}


def workload(name):
    from lora_adapter_application_amd import synth
    return {"llama7b_decode": synth.llama7b_decode, "qwen32b_decode": synth.qwen32b_decode,
            "llama7b_prefill": synth.llama7b_prefill}[name]()


def calib_copy(steps):
    import torch
    n = 1 << 30                                   # 1 GiB read + 1 GiB written per copy
    a = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                      "ms_per_copy": dt * 1e3, "GBps_read_plus_write": 2 * n / dt / 1e9}))


def measured_copy_gbps(reps=10):
    """Read-plus-write rate of a 1 GiB device copy (torch), the practical ceiling
    the dominant kernel is also compared with, beside the 8 TB/s spec."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    e1.synchronize()
    gbps = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbps


def measured_h2d_gbps(nbytes=7897088, bufs=16, reps=32):
    """Rate of back-to-back pinned host to device copies of one adapter's size
    (torch, current stream): the link's practical ceiling for uploads."""
    import torch
    src = [torch.empty(nbytes, dtype=torch.uint8).pin_memory() for _ in range(bufs)]
    dst = torch.empty(2 * nbytes, dtype=torch.uint8, device="cuda")
    for i in range(4):
        dst[(i & 1) * nbytes:((i & 1) + 1) * nbytes].copy_(src[i % bufs], non_blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        dst[(i & 1) * nbytes:((i & 1) + 1) * nbytes].copy_(src[i % bufs], non_blocking=True)
    e1.record()
    e1.synchronize()
    gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def kernel_source_sha():
    p = os.path.join(ROOT, "lora_adapter_application_amd", "csrc", "lora_kernels.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()


def profile_figure(kind, kernel, wl_name, key):
    """A figure from a committed counter summary (profiles/<kind>_<kernel>_<workload>.json),
    if the kernel source is still the one the counters were taken on; else None."""
    p = os.path.join(ROOT, "profiles", f"{kind}_{kernel}_{wl_name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return d.get(key)


def traffic_from_profiles(kernel, wl_name):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, calibrated) of the kernel."""
    return profile_figure("traffic", kernel, wl_name, "hbm_bytes_per_launch")


def measure(wl_name, args, K, W, kernel_timing=True, launch="eager"):
    """Time K steps of one workload (after W warm-up steps) and return its record.

    A step is lora_plan_prepare of the batch and one lora_apply_group per module
    group, on one of L rotated layer sets.  Passes over the same K steps:
      eager        the library calls from Python, one step after the other
      graph        the calls of one rotation captured into a HIP graph, replayed
      amortized    one lora_plan_prepare before the K steps, then only the applies
                   (the layers of a model share the batch's slot indices)
      spread       an event after each step (p10 / p50 / p90)
      kernels      per-dispatch start / stop events (kernel times, roofline)"""
    import torch
    from lora_adapter_application_amd import binding
    dev = torch.device("cuda:0")
    wl = workload(wl_name)
    T = wl.n_tokens
    S, R = wl.max_loras, wl.max_rank
    mods = wl.modules
    b = 2                                                   # bf16
    names = [m.name for m in mods]
    groups = [[names.index(n) for n in g] for g in GROUPS[wl.name]]
    # with --shared-x, the first member of each group whose members have one d_in
    # owns the x buffer the whole group reads
    x_owner = list(range(len(mods)))
    for g in groups:
        if args.shared_x and len({mods[j].d_in for j in g}) == 1:
            for j in g:
                x_owner[j] = g[0]
    # rotation depth
    per_set = sum(S * R * (m.d_in + m.d_out) * b + T * 2 * m.d_out * b
                  + (T * m.d_in * b if x_owner[j] == j else 0) for j, m in enumerate(mods))
    L = max(1, math.ceil(args.layer_bytes / per_set))
    log(f"workload {wl.name}: T={T} S={S} R={R} modules={[(m.name, m.d_in, m.d_out) for m in mods]}"
        f" layer sets={L} ({L * per_set / 1e9:.2f} GB) steps={K} warmup={W}")

    def dev_bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    shapes = [(m.d_in, m.d_out) for _ in range(L) for m in mods]
    slots = binding.Slots(S, R, shapes, "bf16", max_tokens=max(T, args.max_tokens))
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260101)
    for k, ad in enumerate(wl.adapters):
        A_t, B = [], []
        for l in range(L):
            for m in mods:
                if l == 0:
                    A_t.append(dev_bits(ad.At[m.name]))
                    B.append(dev_bits(ad.B[m.name]))
                else:
                    bound = 1.0 / math.sqrt(m.d_in)
                    A_t.append(((torch.rand(ad.r, m.d_in, generator=gen, device=dev) * 2 - 1)
                                * bound).to(torch.bfloat16))
                    B.append((torch.randn(ad.r, m.d_out, generator=gen, device=dev) * 0.01)
                             .to(torch.bfloat16))
        slots.load(k, A_t, B, ad.r, ad.lora_alpha, ad.use_rslora)
        slots.sync_loads()
        del A_t, B
    idx = torch.from_numpy(wl.idx).to(dev)
    xs, ys = [], []
    for l in range(L):
        for j, m in enumerate(mods):
            if x_owner[j] != j:
                xs.append(xs[l * len(mods) + x_owner[j]])
            elif l == 0:
                xs.append(dev_bits(wl.x[m.name]))
            else:
                xs.append(torch.randn(T, m.d_in, generator=gen, device=dev).to(torch.bfloat16))
            if l == 0:
                ys.append(dev_bits(wl.y[m.name]))
            else:
                ys.append(torch.randn(T, m.d_out, generator=gen, device=dev).to(torch.bfloat16))
    torch.cuda.synchronize()

    nm = len(mods)
    ng = len(groups)

    # the library calls of one step per layer set, arguments marshalled once
    # (per stream: the eager passes use the current stream, the graph capture its own)
    def bind_all(stream=None, prepare=True, fused=False):
        return [slots.bind_step([([l * nm + j for j in g], [xs[l * nm + j] for j in g],
                                  [ys[l * nm + j] for j in g]) for g in groups], idx, stream,
                                prepare=prepare, fused=fused)
                for l in range(L)]
    bound = bind_all()
    bound_np = bind_all(prepare=False)

    def step(i):
        bound[i % L]()

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    # eager: K steps, nothing but the library calls
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    # fused decode: each group's shrink and expand in one launch (bf16 batches of
    # at most 1024 tokens; lora_apply_group_fused)
    fused_s = fused_amort_s = None
    if T <= 1024:
        bound_f = bind_all(fused=True)
        for i in range(W):
            bound_f[i % L]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            bound_f[(W + i) % L]()
        torch.cuda.synchronize()
        fused_s = time.perf_counter() - t0
        del bound_f
        # the same with the plan amortized over the layers: one lora_plan_prepare,
        # then K steps of fused applies (the first forms the plan inline and
        # publishes it, the others read it)
        bound_fa = bind_all(prepare=False, fused=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        slots.prepare(idx)
        for i in range(K):
            bound_fa[(W + i) % L]()
        torch.cuda.synchronize()
        fused_amort_s = time.perf_counter() - t0
        del bound_fa
    # plan amortized over the layers: one lora_plan_prepare, then K steps of applies
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    slots.prepare(idx)
    for i in range(K):
        bound_np[(W + i) % L]()
    torch.cuda.synchronize()
    amort_s = time.perf_counter() - t0
    # graph: the L steps of one rotation (and the K mod L first ones) captured once;
    # K steps = K // L replays of the first graph and one of the second
    slots.sync_loads()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    bound_cap = bind_all(cap)
    graphs = []
    for n_steps in (L, K % L):
        if n_steps == 0 or (n_steps == L and K < L):
            graphs.append(None)
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(n_steps):
                bound_cap[i % L]()
        graphs.append(g)
    for g in graphs:                # one untimed replay each
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K // L):
        graphs[0].replay()
    if graphs[1] is not None:
        graphs[1].replay()
    torch.cuda.synchronize()
    graph_s = time.perf_counter() - t0
    del graphs
    # step-time spread: the K steps once more, an event recorded after each
    # (events made before the pass); each step's time is the gap to the
    # previous event, so the distribution includes one event's cost per step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(K):
        step(W + i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(K)])
    step_spread = {"p10_us": round(float(np.percentile(per_step, 10)), 3),
                   "p50_us": round(float(np.percentile(per_step, 50)), 3),
                   "p90_us": round(float(np.percentile(per_step, 90)), 3),
                   "pass": "eager, an event after each step"}
    del evs
    elapsed = graph_s if launch == "graph" else eager_s
    if kernel_timing:
        # the same K steps again with per-dispatch kernel events (their host cost
        # would distort the step time above, so they get a pass of their own);
        # the events are created before this pass starts
        slots.profile_begin(K * (2 * ng + 2))
        torch.cuda.synchronize()
        for i in range(K):
            step(W + K + i)
        torch.cuda.synchronize()

    act = (wl.idx >= 0) & (wl.idx < S)
    T_act = int(act.sum())
    used = np.unique(wl.idx[act])
    sum_r = int(sum(wl.adapters[k].r for k in used))
    roofline, kernels = None, None
    if kernel_timing:
        prof = slots.profile_end()
        n = prof["launches"]
        tot = prof["total_ms"]
        # algorithmic bytes of one launch of each group: the shrink reads x once per
        # buffer (once per group with --shared-x) plus each used slot's A^T; the
        # expand reads and writes y and reads each used slot's B
        shrink_bytes = [sum(b * mods[j].d_in * ((T_act if x_owner[j] == j else 0) + sum_r) for j in g)
                        for g in groups]
        expand_bytes = [sum(b * mods[j].d_out * (2 * T_act + sum_r) for j in g) for g in groups]
        # a fused decode launch does one group's shrink and expand
        group_bytes = {"shrink": shrink_bytes, "expand": expand_bytes,
                       "fused": [a + b for a, b in zip(shrink_bytes, expand_bytes)]}
        rsum = int(sum(wl.adapters[k].r for k in wl.idx[act]))    # true ranks of the active tokens
        flops = [2 * (m.d_in + m.d_out) * rsum for m in mods]
        # algorithmic flops of each kind per step (true ranks; the expand's MFMAs
        # also contract h's low half, which is not counted)
        kind_flops = {"shrink": float(sum(2 * m.d_in * rsum for m in mods)),
                      "expand": float(sum(2 * m.d_out * rsum for m in mods))}
        kind_flops["fused"] = kind_flops["shrink"] + kind_flops["expand"]

        def avg_us(kind):
            return tot[kind] / n[kind] * 1e3 if n[kind] else None
        kernels = {
            "groups": [[names[j] for j in g] for g in groups],
            "timed_dispatches": n, "untimed_dispatches": prof["untimed"],
            "plan": {"avg_us": avg_us("plan"), "per_step_us": tot["plan"] / K * 1e3},
            "step_alg_bytes": float(sum(shrink_bytes) + sum(expand_bytes)),
            "step_alg_flops": float(sum(flops)),
        }
        for kind in ("shrink", "expand", "fused"):
            if n[kind]:
                step_bytes = float(sum(group_bytes[kind]))
                tfs = kind_flops[kind] * K / (tot[kind] * 1e-3) / 1e12
                kernels["lora_" + kind] = {
                    "avg_us": avg_us(kind), "per_step_us": tot[kind] / K * 1e3,
                    "alg_bytes_per_step": step_bytes,
                    "GBps": float(step_bytes * K / (tot[kind] * 1e-3) / 1e9),
                    "hbm_frac": round(float(step_bytes * K / (tot[kind] * 1e-3) / 1e9) / HBM_PEAK_GBS, 4),
                    "alg_flops_per_step": kind_flops[kind], "TFLOPs": round(tfs, 2),
                    "mfma_frac": round(tfs / BF16_MFMA_PEAK_TFS, 5),
                    "mfma_util_pct": profile_figure("mfma", "lora_" + kind, wl.name, "mfma_util_pct")}
        dom = max(("shrink", "expand", "fused"), key=lambda k: tot[k])
        dom_bytes = group_bytes[dom]
        achieved = sum(dom_bytes) * K / (tot[dom] * 1e-3) / 1e9      # GB/s
        kname = "lora_" + dom
        traffic = traffic_from_profiles(kname, wl.name)
        # flat fields only: the %MFMA half of the metric beside the HBM fraction
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic,
                    "alg_bytes_per_launch": float(np.mean(dom_bytes)),
                    "avg_launch_us": avg_us(dom),
                    "mfma_frac": kernels[kname]["mfma_frac"],
                    "mfma_TFLOPs": kernels[kname]["TFLOPs"],
                    "mfma_peak_TFLOPs": BF16_MFMA_PEAK_TFS,
                    "mfma_util_pct": kernels[kname]["mfma_util_pct"],
                    "mfma_flops": "algorithmic, true ranks"}
        log("kernels:", json.dumps(kernels))
    rec = {
        "wl": wl, "T": T, "T_act": T_act, "K": K, "L": L,
        "value": T * K / elapsed, "ms_per_step": elapsed / K * 1e3,
        "config": {"workload": wl.name, "tokens": T, "active_tokens": T_act,
                   "modules": [f"{m.name} {m.d_in}->{m.d_out}" for m in mods],
                   "max_loras": S, "max_rank": R, "ranks": sorted({a.r for a in wl.adapters if a}),
                   "layer_sets_rotated": L, "groups": [[names[j] for j in g] for g in groups],
                   "shared_x": bool(args.shared_x),
                   "launch": "hip_graph" if launch == "graph" else "eager",
                   "kernel_timing": "per-dispatch events" if kernel_timing else "none",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "eager": {"ms_per_step": round(eager_s / K * 1e3, 5), "value": round(T * K / eager_s, 1)},
        "graph": {"ms_per_step": round(graph_s / K * 1e3, 5), "value": round(T * K / graph_s, 1)},
        "fused": None if fused_s is None else {
            "ms_per_step": round(fused_s / K * 1e3, 5), "value": round(T * K / fused_s, 1),
            "pass": "lora_apply_group_fused: each group's shrink and expand in one launch",
            "plan_amortized": {"ms_per_step": round(fused_amort_s / K * 1e3, 5),
                               "value": round(T * K / fused_amort_s, 1),
                               "pass": "one lora_plan_prepare, then the K steps' fused applies"}},
        "plan_amortized": {"ms_per_step": round(amort_s / K * 1e3, 5),
                           "value": round(T * K / amort_s, 1),
                           "pass": "one lora_plan_prepare, then the K steps' applies"},
        "step_spread": step_spread,
        "kernels": kernels,
    }
    slots.close()
    del xs, ys, bound, bound_np, bound_cap
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def measure_saved(wl, K, W):
    """Saved modules ("modules_to_save") on the headline batch: every adapter also
    saves a whole o_proj (4096 x 4096, random bf16 weights drawn on the device), so
    the o_proj launch writes x . W_k^T for all tokens in place of the base output.
    Only that module is applied; the saved-module kernel is timed with per-dispatch
    events over K launches.  Algorithmic flops: 2 d_in d_out per token; bytes: x
    read, y written, each used slot's W read once."""
    import torch
    from lora_adapter_application_amd import binding
    dev = torch.device("cuda:0")
    m = next(mm for mm in wl.modules if mm.name == "o_proj")
    T = wl.n_tokens
    S = binding.Slots(wl.max_loras, wl.max_rank, [(m.d_in, m.d_out)], "bf16", max_tokens=T)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260202)
    keep = []
    for k, ad in enumerate(wl.adapters):
        S.load(k, [None], [None], ad.r, ad.lora_alpha, ad.use_rslora)   # saves o_proj only
        Wk = (torch.randn(m.d_out, m.d_in, generator=gen, device=dev) / math.sqrt(m.d_in)).to(torch.bfloat16)
        keep.append(Wk)
        S.load_saved(k, 0, Wk)
    S.sync_loads()
    idx = torch.from_numpy(wl.idx).to(dev)
    x = torch.from_numpy(np.ascontiguousarray(wl.x[m.name]).view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.zeros(T, m.d_out, dtype=torch.bfloat16, device=dev)
    S.prepare(idx)
    for _ in range(W):
        S.apply_group([0], [x], [y], idx)
    torch.cuda.synchronize()
    S.profile_begin(K * 4)
    for _ in range(K):
        S.apply_group([0], [x], [y], idx)
    prof = S.profile_end()
    S.close()
    n = prof["launches"]["saved"]
    us = prof["total_ms"]["saved"] / n * 1e3
    used = np.unique(wl.idx[(wl.idx >= 0) & (wl.idx < wl.max_loras)])
    flops = 2.0 * T * m.d_in * m.d_out
    nbytes = 2.0 * (T * m.d_in + T * m.d_out + len(used) * m.d_in * m.d_out)
    tfs = flops / (us * 1e-6) / 1e12
    # the launch stages x and W through LDS when every member's d_in is a multiple of 64
    kernel = "saved_bf16_quad_kernel" if m.d_in % 64 == 0 else "saved_bf16_kernel"
    del keep, x, y
    torch.cuda.empty_cache()
    return {"workload": f"{wl.name} batch ({T} tokens), every adapter saving o_proj "
                        f"{m.d_in}->{m.d_out}",
            "kernel": kernel, "launches": n, "avg_launch_us": round(us, 2),
            "alg_flops_per_launch": flops, "TFLOPs": round(tfs, 1),
            "mfma_frac": round(tfs / BF16_MFMA_PEAK_TFS, 4),
            "alg_bytes_per_launch": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bound": "mfma"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards "
              "by replicating slot pools per GPU with no exchange, which this benchmark does "
              "not measure.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy:
        calib_copy(args.steps)
        return

    from lora_adapter_application_amd import binding
    binding.load_library()
    if args.workload == "churn":
        if args.prefetch:
            churn_prefetch(args)
        else:
            churn(args)
        return
    if args.saved_only:
        saved = measure_saved(workload("llama7b_prefill"), args.steps, args.warmup)
        print(json.dumps({"metric": "saved-module product TFLOP/s", "value": saved["TFLOPs"],
                          "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "saved_module": saved}), flush=True)
        return
    rec = measure(args.workload, args, args.steps, args.warmup,
                  kernel_timing=not args.no_kernel_timing, launch=args.launch)
    if rec["roofline"] is not None:
        copy_gbps = measured_copy_gbps()
        rec["roofline"]["copy_GBps"] = round(copy_gbps, 1)
        rec["roofline"]["frac_of_copy"] = round(rec["roofline"]["achieved"] / copy_gbps, 4)
    # the other single-GPU workloads of the metric (decode BGMV), each with its
    # own step count: their steps take microseconds
    extras = {}
    for name in args.extra:
        if name == args.workload:
            continue
        e = measure(name, args, args.extra_steps, args.extra_warmup,
                    kernel_timing=not args.no_kernel_timing, launch=args.launch)
        extras[name] = {"value": round(e["value"], 1), "unit": "tokens/s",
                        "ms_per_step": round(e["ms_per_step"], 5), "steps": e["K"],
                        "config": e["config"], "roofline": e["roofline"],
                        "graph": e["graph"], "plan_amortized": e["plan_amortized"],
                        "fused": e["fused"],
                        "step_spread": e["step_spread"]}
    saved = None
    if args.saved and rec["wl"].name == "llama7b_prefill" and not args.no_kernel_timing:
        saved = measure_saved(rec["wl"], args.steps, args.warmup)
        log("saved_module:", json.dumps(saved))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(rec["wl"], args.cpu_seconds)

    out = {
        "metric": "multi-LoRA tokens/s",
        "value": round(rec["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
        "eager": rec["eager"],
        "graph": rec["graph"],
        "plan_amortized": rec["plan_amortized"],
        "fused": rec["fused"],
        "step_spread": rec["step_spread"],
        "kernels": rec["kernels"],
    }
    for name, e in extras.items():
        out[name] = e
    if saved is not None:
        out["saved_module"] = saved
    print(json.dumps(out), flush=True)


def churn(args):
    """Mixed batches with slot churn: 128 slots, a 200-adapter pinned host pool,
    host LRU residency, misses loaded with lora_slot_load before each step (the
    "CPU hit = H2D upload" tier), then the five modules applied in three groups.
    Cold start: step 0 loads 128 adapters."""
    import torch
    from lora_adapter_application_amd import binding, synth
    from lora_adapter_application_amd.lru import SlotLRU
    mods = synth.CHURN_MODULES
    names = [m.name for m in mods]
    groups = [["q_proj", "v_proj"], ["gate_proj", "up_proj"], ["down_proj"]]
    pool = synth.churn_pool_device()
    slots = binding.Slots(128, 64, [(m.d_in, m.d_out) for m in mods], "bf16", max_tokens=8192)
    lru = SlotLRU(128)
    t_load = t_apply = 0.0
    t_load_warm = t_apply_warm = 0.0
    tokens = tokens_warm = 0
    redraws = 0
    per_miss = []
    for step in range(args.churn_steps):
        ids, rd, x, y = synth.churn_step_device(step)
        redraws += rd
        slot_idx, loads = lru.plan_step(ids)
        idx = torch.from_numpy(slot_idx).cuda()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for slot, a in loads:
            slots.load(slot, [pool.At[n][a] for n in names], [pool.B[n][a] for n in names], 64, 128.0)
        slots.sync_loads()
        t1 = time.perf_counter()
        slots.prepare(idx)
        for g in groups:
            mi = [names.index(n) for n in g]
            slots.shrink_group(mi, [x[n] for n in g])
            slots.expand_group(mi, [y[n] for n in g])
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        t_load += t1 - t0
        t_apply += t2 - t1
        tokens += ids.shape[0]
        if loads:
            per_miss.append((t1 - t0) / len(loads))
        if step > 0:
            t_load_warm += t1 - t0
            t_apply_warm += t2 - t1
            tokens_warm += ids.shape[0]
        del x, y
    st = lru.stats
    bytes_loaded = slots.stats()["bytes_loaded"]
    link = measured_h2d_gbps()
    h2d_rate = bytes_loaded / t_load / 1e9 if t_load else None
    out = {
        "metric": "multi-LoRA tokens/s",
        "value": round(tokens / (t_load + t_apply), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.churn_steps, "warmup": 0,
        "ms_per_step": round((t_load + t_apply) / args.churn_steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "churn", "tokens_per_step": 8192,
                   "modules": [f"{m.name} {m.d_in}->{m.d_out}" for m in mods],
                   "groups": groups, "max_loras": 128, "max_rank": 64, "pool_adapters": 200,
                   "zipf": 0.9, "cold_start": True, "parallelism": "none (1 GPU)"},
        "apply_only_tokens_per_s": round(tokens / t_apply, 1),
        "steady_state": {"steps": args.churn_steps - 1,
                         "load_plus_apply_tokens_per_s": round(tokens_warm / (t_load_warm + t_apply_warm), 1),
                         "apply_only_tokens_per_s": round(tokens_warm / t_apply_warm, 1),
                         "ms_per_step": round((t_load_warm + t_apply_warm) / (args.churn_steps - 1) * 1e3, 4)},
        "h2d": {"bytes": bytes_loaded, "seconds": round(t_load, 6),
                "GBps": round(h2d_rate, 2) if h2d_rate else None,
                "copy_GBps": round(link, 2),
                "frac_of_copy": round(h2d_rate / link, 3) if h2d_rate else None,
                "adapter_h2d_seconds_mean": round(float(np.mean(per_miss)), 7) if per_miss else None,
                "bytes_per_adapter": bytes_loaded // max(st.misses, 1)},
        "lru": {"hits": st.hits, "misses": st.misses, "evictions": st.evictions,
                "reloads_after_eviction": st.reloads_after_eviction,
                "thrash_ratio": round(st.thrash_ratio, 4), "capped_redraws": redraws},
    }
    print(json.dumps(out), flush=True)
    slots.close()


def churn_prefetch(args):
    """The churn workload as a pipeline: the misses of step s+1 are uploaded
    while step s computes.  The LRU schedule (host control plane, decided from
    the adapter ids alone) and every step's inputs are prepared before timing.
    Timed twice on the same schedule and the same slot count:
      prefetch: each plan declares its slots (lora_plan_prepare_slots), so a
                load waits only for the batches that read its slot, and the
                LRU evicts slots the step in flight reads only as a last resort;
      serial:   undeclared plans, so every load waits for all batches issued
                before it, and the uploads of step s+1 follow step s.
    Cold start: step 0's misses are part of the timed region."""
    import torch
    from lora_adapter_application_amd import binding, synth
    from lora_adapter_application_amd.lru import SlotLRU
    mods = synth.CHURN_MODULES
    names = [m.name for m in mods]
    groups = [[names.index(n) for n in g] for g in (["q_proj", "v_proj"], ["gate_proj", "up_proj"],
                                                     ["down_proj"])]
    n_slots = args.churn_slots
    N = args.churn_steps
    pool = synth.churn_pool_device()
    steps = [synth.churn_step_device(s) for s in range(N)]
    lru = SlotLRU(n_slots)
    sched = []
    prev_used = set()
    for s, (ids, _, x, y) in enumerate(steps):
        slot_idx, loads = lru.plan_step(ids, avoid=prev_used)
        used = sorted({int(v) for v in slot_idx[slot_idx >= 0]})
        sched.append((torch.from_numpy(slot_idx).cuda(), used, loads, x, y))
        prev_used = set(used)
    st = lru.stats
    torch.cuda.synchronize()

    def run(declared):
        slots = binding.Slots(n_slots, 64, [(m.d_in, m.d_out) for m in mods], "bf16", max_tokens=8192)

        def issue(loads):
            for slot, a in loads:
                slots.load(slot, [pool.At[n][a] for n in names], [pool.B[n][a] for n in names], 64, 128.0)

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        issue(sched[0][2])
        for s in range(N):
            idx, used, _, x, y = sched[s]
            slots.prepare(idx, used_slots=used if declared else None)
            for g in groups:
                slots.apply_group(g, [x[names[j]] for j in g], [y[names[j]] for j in g], idx)
            if s + 1 < N:
                issue(sched[s + 1][2])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        bytes_loaded = slots.stats()["bytes_loaded"]
        slots.close()
        return dt, bytes_loaded

    run(True)                                  # warm-up pass (untimed): allocator, code objects
    t_pre, bytes_loaded = run(True)
    t_ser, _ = run(False)
    link = measured_h2d_gbps()
    tokens = sum(int(step[0].shape[0]) for step in steps)
    out = {
        "metric": "multi-LoRA tokens/s",
        "value": round(tokens / t_pre, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": N, "warmup": 0,
        "ms_per_step": round(t_pre / N * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "churn_prefetch", "tokens_per_step": 8192,
                   "modules": [f"{m.name} {m.d_in}->{m.d_out}" for m in mods],
                   "groups": [[names[j] for j in g] for g in groups], "max_loras": n_slots,
                   "per_step_cap": 128, "max_rank": 64, "pool_adapters": 200, "zipf": 0.9,
                   "cold_start": True, "parallelism": "none (1 GPU)"},
        "serial": {"value": round(tokens / t_ser, 1), "ms_per_step": round(t_ser / N * 1e3, 4)},
        "h2d": {"bytes": bytes_loaded, "GBps_over_prefetch_run": round(bytes_loaded / t_pre / 1e9, 2),
                "copy_GBps": round(link, 2)},
        "lru": {"hits": st.hits, "misses": st.misses, "evictions": st.evictions,
                "reloads_after_eviction": st.reloads_after_eviction,
                "thrash_ratio": round(st.thrash_ratio, 4)},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, seconds):
    """The oracle on the host over whole layers of the workload until ~`seconds` pass."""
    import oracle
    from lora_adapter_application_amd import synth
    threads = oracle.max_threads()
    ads = {m.name: synth.oracle_adapters(wl, m.name) for m in wl.modules}
    T = wl.n_tokens
    rows = np.arange(T)
    if wl.name == "llama7b_prefill":                     # a bounded sample of the batch
        rows = np.random.default_rng(0).choice(T, size=min(T, 2048), replace=False)
        rows.sort()
    layers = 0
    t0 = time.perf_counter()
    while True:
        for m in wl.modules:
            oracle.apply(oracle.BF16, wl.x[m.name][rows], wl.y[m.name][rows], wl.idx[rows],
                         ads[m.name])
        layers += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    # one thread on a smaller sample, about a third of the time
    rows1 = rows[:256]
    layers1 = 0
    t1 = time.perf_counter()
    while True:
        for m in wl.modules:
            oracle.apply(oracle.BF16, wl.x[m.name][rows1], wl.y[m.name][rows1], wl.idx[rows1],
                         ads[m.name], n_threads=1)
        layers1 += 1
        dt1 = time.perf_counter() - t1
        if dt1 >= seconds / 3:
            break
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(layers * len(rows) / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{layers} layer passes of {len(rows)} tokens of {wl.name} "
                      f"({len(wl.modules)} modules each), fp64 scalar C, OpenMP over tokens, "
                      f"{dt:.1f} s",
            "single_thread": {"value": round(layers1 * len(rows1) / dt1, 1), "unit": "tokens/s",
                              "sample": f"{layers1} layer passes of {len(rows1)} tokens, 1 thread, "
                                        f"{dt1:.1f} s"},
            "nproc": os.cpu_count(), "cpu_model": cpu_model}


if __name__ == "__main__":
    main()
