#!/usr/bin/env python3
"""Throughput of the exact attention forward (or backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--pass fwd|bwd]

One step = one fa_fwd call over the whole batch of the workload (default:
B=2, H=32, N=4096, d=128, bf16, causal), inputs already resident in device
memory.  Prints ONE JSON line with the throughput (FLOPs by 4*B*H*N^2*d,
halved for causal), the roofline figures of the kernel, and the CPU oracle
timed on the host as a reported baseline.

``--pass bwd`` times one fa_bwd call per step instead (the forward runs once,
untimed, to produce O and LSE); FLOPs are counted as the five products of the
gradient, 2.5x the forward's.

``--pass decode`` times one fa_decode_paged call per step (one query token
per request against a paged KV cache); it is bandwidth-bound, so the figure
is GB/s of algorithmic bytes (every cached K and V row once, q, O and LSE)
against the 8 TB/s HBM peak.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s (bf16, N=4096 d=128 causal) and % of MFMA peak"
METRIC_BWD = "bwd attention TFLOP/s (bf16, N=4096 d=128 causal) and % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}   # MI355X dense MFMA peaks
CSRC = os.path.join(ROOT, "exact_attention_92_amd", "csrc")
# Sources each pass's kernels are built from (the PMC summaries record their hash).
KERNEL_SRCS = {"fwd": ["fa_fwd.hip", "fa_device.h", "gen_fwd_d128_loop.py"],
               "bwd": ["fa_bwd.hip", "fa_bwd_kernels.h", "fa_device.h"],
               "fp8": ["fa_fwd_fp8.hip", "fa_device.h"],
               "decode": ["fa_decode.hip", "fa_device.h"]}
PMC_SUMMARY = {"fwd": os.path.join(ROOT, "profiles", "fa_fwd_bf16_b2h32_n4096_d128_causal_pmc.md"),
               "bwd": os.path.join(ROOT, "profiles", "fa_bwd_bf16_b2h32_n4096_d128_causal_pmc.md"),
               "fp8": os.path.join(ROOT, "profiles", "fa_fwd_fp8_b2h32_n4096_d128_causal_pmc.md"),
               "decode": os.path.join(ROOT, "profiles",
                                      "fa_decode_paged_b32h32_d128_bs64_len1k8k_pmc.md")}
HBM_PEAK_GBS = 8000.0


def fwd_kernel_name(wl, general):
    """The forward kernel fa_fwd and friends dispatch this workload to."""
    if wl.dtype == "bf16" and not general and wl.d == 128 and wl.scale > 0 \
            and os.environ.get("FA92_FWD_D128", "1")[:1] != "0":
        return "fa_fwd_d128_kernel"
    name = {"bf16": "fa_fwd_bf16_kernel", "f32": "fa_fwd_f32_kernel",
            "fp8": "fa_fwd_fp8_kernel"}[wl.dtype]
    if wl.tile_gain is not None:
        name += " (per-tile scales)"
    return name + (" (general layout)" if general else "")


def kernel_source_hash(which="fwd"):
    h = hashlib.sha256()
    for name in KERNEL_SRCS[which]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(which="fwd"):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel source; otherwise None."""
    try:
        text = open(PMC_SUMMARY[which]).read()
    except OSError:
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(which):
        return None
    return rec.get("hbm_bytes_per_launch")


def oracle_threads(cores, heads):
    """Threads the oracle runs on: one worker per head (single-threaded BLAS)
    up to ``cores``; a single head runs serially with BLAS's own threads."""
    if heads > 1:
        used = min(cores, heads)
        return used, f"{used} worker threads with single-threaded BLAS"
    return cores, f"one head, serial, BLAS threads (up to {cores})"


def cpu_baseline(x, wl, o_gpu):
    """Time the oracle on the host (all heads of the workload) and check the
    GPU output against it on the same bytes."""
    from fa_inputs import inputs_f64
    from oracle import attention_ref
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    q, k, v = inputs_f64(x)
    t0 = time.perf_counter()
    Or, Lr = attention_ref(q, k, v, wl.scale, wl.mask_kind, x["kv_lens"], workers=cores)
    dt = time.perf_counter() - t0
    err = np.abs(o_gpu - Or)
    parity = {"o_max_abs": float(err.max()),
              "o_rel_frobenius": float(np.linalg.norm(o_gpu - Or) / np.linalg.norm(Or))}
    used, how = oracle_threads(cores, wl.B * wl.H)
    return {"value": wl.flops() / dt / 1e12, "unit": "TFLOP/s", "cores": used,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole workload ({wl.B * wl.H} heads, all rows), fp64 NumPy/BLAS, "
                      f"{how}"}, parity


def cpu_baseline_window(x, wl, o_gpu_rows, rows):
    """Time the general oracle on a row sample of a sliding-window workload
    (every head, the query rows ``rows``) and check the GPU rows against it;
    the rate credits 4*d flops per visible (query, key) pair of the sample."""
    from fa_inputs import inputs_f64
    from oracle import attention_general_ref
    q, k, v = inputs_f64(x)
    t0 = time.perf_counter()
    Or, Lr = attention_general_ref(q, k, v, wl.scale, wl.mask_kind, wl.window_left,
                                   x["kv_lens"], rows=rows)
    dt = time.perf_counter() - t0
    a = rows                    # N_q = N_k: query r sits at key position r
    lo = np.maximum(0, a - wl.window_left) if wl.window_left >= 0 else np.zeros_like(a)
    hi = a + 1 if (wl.mask_kind & 1) else np.full_like(a, wl.N)
    flops = 4.0 * wl.d * wl.B * wl.H * float(np.sum(hi - lo))
    err = np.abs(o_gpu_rows - Or)
    parity = {"o_max_abs": float(err.max()),
              "o_rel_frobenius": float(np.linalg.norm(o_gpu_rows - Or) / np.linalg.norm(Or)),
              "rows_checked": int(len(rows) * wl.B * wl.H)}
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{len(rows)} evenly spaced query rows of each of the {wl.B * wl.H} "
                      "heads (full key rows, masked), fp64 NumPy/BLAS"}, parity


def cpu_baseline_varlen(x, wl, o_gpu, nseq=4):
    """Time the packed-sequence oracle on the first ``nseq`` sequences (all
    heads) and check the GPU rows of those sequences against it."""
    from fa_inputs import to_f64
    from oracle import attention_varlen_ref
    cu_q, cu_k = x["cu_q"][:nseq + 1], x["cu_k"][:nseq + 1]
    q = to_f64(x["q"][:cu_q[-1]])
    k, v = to_f64(x["k"][:cu_k[-1]]), to_f64(x["v"][:cu_k[-1]])
    t0 = time.perf_counter()
    Or, _ = attention_varlen_ref(q, k, v, cu_q, cu_k, wl.scale, wl.mask_kind, wl.window_left)
    dt = time.perf_counter() - t0
    n = np.diff(cu_q).astype(np.float64)
    pairs = n * (n + 1) / 2.0 if wl.mask_kind & 1 else n * n
    flops = 4.0 * wl.H * wl.d * float(pairs.sum())
    og = o_gpu[:cu_q[-1]]
    parity = {"o_max_abs": float(np.abs(og - Or).max()),
              "o_rel_frobenius": float(np.linalg.norm(og - Or) / np.linalg.norm(Or)),
              "rows_checked": int(cu_q[-1]) * wl.H}
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"the first {nseq} of the {wl.B} packed sequences (lengths "
                      f"{np.diff(cu_q).tolist()}), all {wl.H} heads, fp64 NumPy/BLAS"}, parity


def cpu_baseline_bwd(x, wl, g):
    """Time the backward oracle on the host (all heads) and check the GPU
    gradients against it on the same bytes."""
    from fa_inputs import to_f64
    from oracle import attention_bwd_ref
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    ref = attention_bwd_ref(q, k, v, do, wl.scale, wl.mask_kind, x["kv_lens"], workers=cores)
    dt = time.perf_counter() - t0
    parity = {}
    for name, want in zip(("dq", "dk", "dv"), ref[:3]):
        parity[f"{name}_rel_frobenius"] = float(np.linalg.norm(g[name] - want) /
                                                np.linalg.norm(want))
    used, how = oracle_threads(cores, wl.B * wl.H)
    return {"value": wl.bwd_flops() / dt / 1e12, "unit": "TFLOP/s", "cores": used,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole workload ({wl.B * wl.H} heads, all rows), fp64 NumPy/BLAS, "
                      f"{how}"}, parity


def decode_bench(args):
    """One fa_decode_paged call per step over a paged-KV decode batch."""
    import torch

    import exact_attention_92_amd as fa
    from fa_inputs import DECODE_WORKLOADS, bf16_bits_to_f32, make_paged_decode
    name = args.workload or "decode_b32h32_d128_bs64_len1k8k"
    wl = DECODE_WORKLOADS[name]
    x = make_paged_decode(wl.B, wl.H, wl.d, wl.block_size, wl.len_range, wl.seed, wl.spare)
    dev = torch.device("cuda:0")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, kp, vp = bf(x["q"]), bf(x["k_pool"]), bf(x["v_pool"])
    tab = torch.from_numpy(x["block_tables"]).to(dev)
    lens = torch.from_numpy(x["seq_lens"]).to(dev)
    o = torch.empty((wl.B, wl.H, wl.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.B, wl.H), dtype=torch.float32, device=dev)
    need = fa.fa_decode_paged_workspace_bytes(wl.B, wl.H, wl.d, wl.block_size, tab.shape[1])
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.fa_decode_paged(q, kp, vp, tab, lens, o, lse, ws, wl.scale, stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    avg_ms = float(np.mean(launch_ms))
    ntok = int(x["seq_lens"].astype(np.int64).sum())
    nbytes = ntok * wl.H * wl.d * 2 * 2 + 2 * wl.B * wl.H * wl.d * 2 + wl.B * wl.H * 4
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    rec = {
        "metric": f"paged-KV decode GB/s ({wl.name})",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "d": wl.d,
                   "block_size": wl.block_size, "len_range": list(wl.len_range),
                   "cached_tokens": ntok, "bytes_per_step": nbytes,
                   "device": torch.cuda.get_device_name(dev)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode"),
                     "kernel": "fa_decode_split_kernel + fa_decode_combine_kernel (one call)",
                     "avg_launch_us": round(avg_ms * 1e3, 2),
                     "min_launch_us": round(min(launch_ms) * 1e3, 2)},
        "cpu_baseline": None, "pass": "decode",
    }
    if not args.no_cpu_baseline:
        from oracle.paged_decode_ref import paged_decode_ref
        f = bf16_bits_to_f32
        kp32, vp32 = f(x["k_pool"]), f(x["v_pool"])
        t0 = time.perf_counter()
        Or, Lr = paged_decode_ref(f(x["q"]), kp32, vp32, x["block_tables"], x["seq_lens"],
                                  wl.scale)
        dt = time.perf_counter() - t0
        og = o.float().cpu().numpy().astype(np.float64)
        rec["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"the whole batch ({wl.B} requests x {wl.H} heads), "
                                         "fp64 NumPy, one thread"}
        rec["parity_vs_oracle"] = {"o_max_abs": float(np.abs(og - Or).max()),
                                   "o_rel_frobenius": float(np.linalg.norm(og - Or) /
                                                            np.linalg.norm(Or))}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "decode"), default="fwd")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run 3 plain device copies of this many MiB (a known-size "
                         "reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention forward here runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.which == "decode":
        decode_bench(args)
        return

    import exact_attention_92_amd as fa
    from fa_inputs import (BENCH_WORKLOAD, FP8_WORKLOADS, GENERAL_WORKLOADS, WORKLOADS,
                           bf16_bits_to_f32, make_bwd_inputs, make_inputs)

    wl = {**WORKLOADS, **FP8_WORKLOADS, **GENERAL_WORKLOADS}[args.workload or BENCH_WORKLOAD]
    general = wl.name in GENERAL_WORKLOADS
    bwd = args.which == "bwd"
    if bwd and wl.dtype != "bf16":
        print("--pass bwd runs the bf16 backward; pick a bf16 workload", file=sys.stderr)
        sys.exit(2)
    x = make_bwd_inputs(wl) if bwd else make_inputs(wl)
    dev = torch.device("cuda:0")

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
    varlen = wl.layout == "varlen"
    kv = None if varlen or x["kv_lens"] is None else torch.from_numpy(x["kv_lens"]).to(dev)
    shape = tuple(q.shape) if varlen else (wl.B, wl.H, wl.N, wl.d)
    o = torch.empty(shape, dtype=torch.float32 if wl.dtype == "f32" else torch.bfloat16,
                    device=dev)
    lse = torch.empty((wl.H, q.shape[0]) if varlen else (wl.B, wl.H, wl.N),
                      dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if varlen:
        cu_q, cu_k = (torch.from_numpy(x[n]).to(dev) for n in ("cu_q", "cu_k"))

        def step():
            fa.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, wl.N, wl.scale, wl.mask_kind,
                             wl.window_left, stream.cuda_stream)
    elif general:
        if wl.layout == "bnhd":     # same values, stored [B, N, H, d]; [B, H, N, d] views
            q, k, v = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
            o = torch.empty((wl.B, wl.N, wl.H, wl.d), dtype=torch.bfloat16,
                            device=dev).permute(0, 2, 1, 3)

        def step():
            fa.fa_fwd_general(q, k, v, o, lse, wl.scale, wl.mask_kind, wl.window_left, kv,
                              stream.cuda_stream)
    elif wl.dtype == "fp8":
        qs, ks, vs = (up(x[n + "_descale"]) for n in "qkv")

        fp8_fn = fa.fa_fwd_fp8_tiled if x.get("fp8_tiled") else fa.fa_fwd_fp8

        def step():
            fp8_fn(q, k, v, qs, ks, vs, o, lse, wl.scale, wl.mask_kind, kv, stream.cuda_stream)
    else:
        fn = fa.fa_fwd if wl.dtype == "bf16" else fa.fa_fwd_f32

        def step():
            fn(q, k, v, o, lse, wl.scale, wl.mask_kind, kv, stream.cuda_stream)

    if bwd:
        # The forward runs once (untimed) to give O and LSE; a step is fa_bwd.
        step()
        do = up(x["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dps = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)

        def step():
            fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dps, wl.scale, wl.mask_kind, kv,
                      stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps; an event pair around every launch on the launch
    # stream gives the per-launch kernel duration as well.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = float(np.mean(launch_ms))

    flops = wl.bwd_flops() if bwd else wl.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    which = "fp8" if wl.dtype == "fp8" else args.which
    traffic = (measured_traffic(which)
               if wl.name in (BENCH_WORKLOAD, "fp8_b2h32_n4096_d128_causal") else None)
    metric = METRIC_BWD if bwd else METRIC
    if wl.name != BENCH_WORKLOAD:
        metric = f"{args.which} attention TFLOP/s ({wl.name})"
    rec = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "mask": {0: "none", 1: "causal", 2: "key_padding"}[wl.mask_kind],
                   **({"window_left": wl.window_left, "layout": wl.layout} if general else {}),
                   **({"seq_lens": np.diff(x["cu_q"]).tolist()} if varlen else {}),
                   "scale": wl.scale, "q_mult": wl.q_mult, "seed": wl.seed,
                   "flops_per_step": flops, "device": torch.cuda.get_device_name(dev)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": fwd_kernel_name(wl, general or varlen),
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "min_launch_us": round(min(launch_ms) * 1e3, 2)},
        "cpu_baseline": None,
    }
    if bwd:
        rec["pass"] = "bwd"
        rec["roofline"]["kernel"] = "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel (one fa_bwd call)"
        # The kernels execute 7 products (S and dP are formed in both), the
        # metric credits the 5 of the gradient.
        rec["roofline"]["executed_mfma_tflops"] = round(achieved * 7 / 5, 2)
    if not args.no_cpu_baseline and bwd:
        g = {}
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
            g[name] = bf16_bits_to_f32(bits).astype(np.float64)
        rec["cpu_baseline"], rec["parity_vs_oracle"] = cpu_baseline_bwd(x, wl, g)
    elif not args.no_cpu_baseline and varlen:
        bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
        rec["cpu_baseline"], rec["parity_vs_oracle"] = cpu_baseline_varlen(
            x, wl, bf16_bits_to_f32(bits).astype(np.float64))
    elif not args.no_cpu_baseline and wl.window_left >= 0:
        rows = np.unique(np.linspace(0, wl.N - 1, 1536).astype(np.int64))
        bits = o[:, :, torch.from_numpy(rows).to(dev)].contiguous().view(torch.int16)
        o_rows = bf16_bits_to_f32(bits.cpu().numpy().view(np.uint16)).astype(np.float64)
        rec["cpu_baseline"], rec["parity_vs_oracle"] = cpu_baseline_window(x, wl, o_rows, rows)
    elif not args.no_cpu_baseline:
        if o.dtype == torch.bfloat16:
            bits = o.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            o_host = bf16_bits_to_f32(bits).astype(np.float64)
        else:
            o_host = o.cpu().numpy().astype(np.float64)
        rec["cpu_baseline"], rec["parity_vs_oracle"] = cpu_baseline(x, wl, o_host)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
