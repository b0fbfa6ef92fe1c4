#!/usr/bin/env python3
"""Throughput of causal prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 7b_2659]

One step = one fa_prefill launch over the whole workload (32 heads x 2659
tokens x head_dim 128, causal, f16 in, f32 out by default), inputs resident in
HBM.  W untimed steps (default 300: after idle the device's power management
runs a transient, launches first fast, then up to ~30 % slower, settling
after about 300 launches of this size), then K steps back to back on one
stream, bracketed by device synchronisation and split into B bursts
(default 7 x 50) with a HIP event on the launch stream at every burst
boundary.  The time per step is the
median burst's time per launch (p10 / p90 / mean over bursts are reported
too, so the clock's sag under sustained load shows), warm L2 / MALL.  A cold
figure follows: launches each preceded by a 1 GiB scrub that evicts the
inputs from the caches, each timed on its own.  Prints one JSON line
(``--workload all``: one line per configuration).

A K/V producer workload (--workload kv_store_2659 etc.) times fa_store_kv
instead: one step = one launch storing the workload's K and V, rotating over
enough input/output sets that each launch streams from HBM; the figure is
algorithmic bytes (f32 read, f16 written, positions read) per second.

The reported throughput counts algorithmic FLOP only: 4 * head_dim per
visible (query, key) pair per query head (Q.K^T and P.V multiply-adds, x2),
not the masked upper triangle nor the padding of diagonal and tail tiles.
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

# MI355X published dense f16 matrix peak: 256 CUs x 4096 FLOP/clk x 2.4 GHz.
PEAK_F16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("prefill_attention_amd/csrc/fa_prefill_kernel.h", "prefill_attention_amd/csrc/fa_prefill_hd128.hip",
                  "prefill_attention_amd/csrc/fa_geometry.h")
STORE_SOURCES = ("prefill_attention_amd/csrc/fa_kv_store.hip",)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_prefill_kernel_traffic.json")
STORE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_store_kv_traffic.json")
# The producer's timed loop rotates over input/output sets whose total exceeds
# this many bytes, so every launch streams from HBM rather than from the
# 256 MB Infinity Cache (MALL) that a repeated 130 MB working set would hit.
STORE_ROTATION_BYTES = 1 << 30


def code_tokens(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed: what
    the compiler sees, so that a comment-only edit keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the kernel's code (comments and layout excluded)."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str, path: str = TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None.

    Valid only for the kernel source they were taken on (hash recorded with
    the numbers) and for the same workload.
    """
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(sources) or rec.get("workload") != workload_key:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, q, k, v, gpu_out, scale, budget_s: float = 12.0) -> dict:
    """Time the float64 oracle on whole heads of the workload, about budget_s of CPU work."""
    import numpy as np
    from oracle import attention_chunk_f64, attention_f64, parity_errors

    try:
        import threadpoolctl

        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:  # threadpoolctl absent: report the affinity set
        threads = len(os.sched_getaffinity(0))
    group = wl.n_q_heads // wl.n_kv_heads
    heads, t_used, worst, worst_rel = 0, 0.0, 0.0, 0.0
    gpu_np = gpu_out.float().cpu().numpy()
    while heads < wl.n_q_heads and t_used < budget_s:
        h = heads
        hk = h // group
        t0 = time.perf_counter()
        oracle_fn = attention_chunk_f64 if wl.chunked else attention_f64
        ref = oracle_fn(q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], scale, wl.causal)
        t_used += time.perf_counter() - t0
        err = parity_errors(gpu_np[:, h:h + 1], ref)
        worst = max(worst, err["max_abs"])
        worst_rel = max(worst_rel, err["rel_plain_max"])
        heads += 1
    flop = 4 * wl.head_dim * heads * wl.visible_pairs
    return {
        "value": flop / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {heads} of {wl.n_q_heads} query heads, all {wl.q_len} rows "
                  f"({flop / 1e9:.2f} GFLOP algorithmic) in {t_used:.1f} s; numpy float64, "
                  f"dense score matrix then mask",
        "seconds": round(t_used, 3),
        "gpu_vs_oracle_max_abs_on_sample": worst,
        "gpu_vs_oracle_plain_rel_on_sample": worst_rel,  # |g-o|/|o| over |o| >= 0.05
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def store_cpu_baseline(swl, k, v, pos, budget_s: float = 15.0) -> dict:
    """Time the oracle's K/V store (numpy) on whole tokens of the workload."""
    import numpy as np
    from oracle import store_kv

    cache = np.zeros((swl.cache_len, swl.n_kv_heads, swl.head_dim), dtype=np.uint16)
    kn, vn, pn = k.numpy(), v.numpy(), pos.numpy()
    done, t_used, chunk = 0, 0.0, max(1, min(swl.n_tokens, 256))
    while done < swl.n_tokens and t_used < budget_s:
        n = min(chunk, swl.n_tokens - done)
        t0 = time.perf_counter()
        store_kv(kn[done:done + n], vn[done:done + n], pn[done:done + n], cache, cache)
        t_used += time.perf_counter() - t0
        done += n
    nbytes = 2 * done * swl.row * 6 + 4 * done
    return {
        "value": nbytes / t_used / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {done} of {swl.n_tokens} tokens, K and V ({nbytes / 1e6:.1f} MB algorithmic) "
                  f"in {t_used:.1f} s; numpy, rounding by table search",
        "seconds": round(t_used, 3),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def store_bench(args, key) -> int:
    """Bench of the K/V producer (fa_store_kv): GB/s of algorithmic bytes."""
    import torch

    import prefill_attention_amd as fa
    from prefill_attention_amd.workloads import STORE_WORKLOADS, make_store_inputs

    swl = STORE_WORKLOADS[key]
    fa.load_library()
    dev = torch.device("cuda:0")
    k, v, pos = make_store_inputs(swl)
    per_set = 2 * k.numel() * 4 + 2 * swl.cache_len * swl.row * 2 + pos.numel() * 4
    n_sets = max(2, min(32, -(-STORE_ROTATION_BYTES // per_set)))
    sets = []
    for _ in range(n_sets):
        kc = torch.zeros(swl.cache_len, swl.n_kv_heads, swl.head_dim, dtype=torch.float16, device=dev)
        sets.append((k.to(dev), v.to(dev), pos.to(dev), kc, torch.zeros_like(kc)))
    stream = torch.cuda.Stream(device=dev)
    calls = [(a.data_ptr(), b.data_ptr(), p.data_ptr(), swl.n_tokens, swl.n_kv_heads, swl.head_dim,
              c.data_ptr(), d.data_ptr(), swl.cache_len, None, stream.cuda_stream)
             for a, b, p, c, d in sets]
    fa.store_kv(*sets[0][:5], stream=stream)  # checked call first
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            fa.fa_store_kv(*calls[i % n_sets])
        stream.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        statuses = [fa.fa_store_kv(*calls[i % n_sets]) for i in range(args.steps)]
        end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
    if any(statuses):
        print(f"bench.py: fa_store_kv returned {set(statuses)}", file=sys.stderr)
        return 1
    ms_per_step = start.elapsed_time(end) / args.steps
    gbs = swl.algorithmic_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": f"K/V store GB/s, algorithmic bytes ({swl.name})",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32->f16",
        "data": "synthetic",
        "config": {**swl.describe(), "workload_key": key, "rotating_sets": n_sets},
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(key, STORE_TRAFFIC_FILE, STORE_SOURCES),
            "bytes_per_launch": swl.algorithmic_bytes,
            "avg_launch_us": round(ms_per_step * 1e3, 3),
            "kernel_source_hash": kernel_source_hash(STORE_SOURCES),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = store_cpu_baseline(swl, k, v, pos)
    print(json.dumps(line), flush=True)
    return 0


def burst_split(steps: int, bursts: int) -> list:
    """Sizes of `bursts` near-equal bursts covering exactly `steps` launches."""
    b = max(1, min(bursts, steps))
    return [steps // b + (1 if i < steps % b else 0) for i in range(b)]


def percentile(xs, p: float) -> float:
    """Linear-interpolated percentile p (0..100) of a non-empty list."""
    s = sorted(xs)
    if len(s) == 1:
        return s[0]
    pos = (len(s) - 1) * p / 100.0
    lo = int(pos)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


def time_bursts(launch, stream, steps: int, warmup: int, bursts: int) -> dict:
    """Warm up, then time `steps` launches in bursts on `stream`.

    Every burst boundary carries a HIP event recorded on the launch stream,
    so the per-burst times are device times of back-to-back launches; the
    whole region is bracketed by device synchronisation.  Returns the
    per-launch milliseconds of each burst, their median / p10 / p90, the
    mean over all launches and the launch statuses.
    """
    import torch

    sizes = burst_split(steps, bursts)
    statuses = []
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            statuses.append(launch())
        stream.synchronize()
        events = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
        torch.cuda.synchronize()
        events[0].record(stream)
        for i, n in enumerate(sizes):
            for _ in range(n):
                statuses.append(launch())
            events[i + 1].record(stream)
        events[-1].synchronize()
        torch.cuda.synchronize()
    per_launch = [events[i].elapsed_time(events[i + 1]) / n for i, n in enumerate(sizes)]
    total = events[0].elapsed_time(events[-1])
    return {
        "burst_ms_per_launch": per_launch,
        "burst_sizes": sizes,
        "median": percentile(per_launch, 50.0),
        "p10": percentile(per_launch, 10.0),
        "p90": percentile(per_launch, 90.0),
        "mean": total / steps,
        "region_ms": total,
        "statuses": statuses,
    }


def time_cold(launch, stream, n: int, scrub_bytes: int = 1 << 30) -> list:
    """Per-launch milliseconds of n launches, each after a scrub of scrub_bytes.

    The scrub writes a buffer four times the size of the MI355X's 256 MB
    Infinity Cache, which evicts the inputs from the L2s and the MALL; only
    the launch itself lies between its two events.
    """
    import torch

    scrub = torch.empty(scrub_bytes // 4, dtype=torch.float32, device=stream.device)
    times = []
    with torch.cuda.stream(stream):
        for _ in range(n):
            scrub.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b))
    del scrub
    return times


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=350, help="timed launches (split into --bursts)")
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed launches first; after idle the device's power management boosts, then "
                         "dips (launches up to ~30 %% slower) and settles within about 300 launches")
    ap.add_argument("--bursts", type=int, default=7, help="bursts the timed launches are split into")
    ap.add_argument("--cold", type=int, default=10, metavar="N",
                    help="cold-cache launches after the warm bursts (0: skip)")
    ap.add_argument("--workload", default=None,
                    help="workload key (default: the headline one; 'all': one line per configuration)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--lib", default=None, metavar="PATH",
                    help="time this build of libfa_prefill.so (e.g. another tile geometry from "
                         "prefill_attention_amd.build --kv-tile/--waves/--out) instead of the in-tree one")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of attention, run --steps device-to-device copies of MIB MiB "
                         "(reference for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not supported "
              "(attention shards over heads with no exchange, but no multi-GPU path is built)",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.bursts < 1 or args.cold < 0:
        print("bench.py: --steps and --bursts must be >= 1, --warmup and --cold >= 0", file=sys.stderr)
        return 2

    import torch

    from prefill_attention_amd.workloads import HEADLINE, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "launches": args.steps}), flush=True)
        return 0
    from prefill_attention_amd.workloads import STORE_WORKLOADS

    if args.lib:
        import prefill_attention_amd as fa

        fa.load_library(os.path.abspath(args.lib))
    key = args.workload or HEADLINE
    if key in STORE_WORKLOADS:
        return store_bench(args, key)
    if key == "all":
        rc = 0
        for k in CONFIG_KEYS:
            rc = rc or attention_bench(args, k)
        return rc
    if key not in WORKLOADS:
        print(f"bench.py: unknown workload {key!r}; known: {sorted(WORKLOADS) + sorted(STORE_WORKLOADS)}",
              file=sys.stderr)
        return 2
    return attention_bench(args, key)


# The five configurations the throughput is reported on (``--workload all``).
CONFIG_KEYS = ("tiny", "7b_2k", "7b_2659", "gqa_4k", "long_16k")


def attention_bench(args, key) -> int:
    """Time one attention workload; print its JSON line."""
    import torch

    import prefill_attention_amd as fa
    from prefill_attention_amd.binding import FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32
    from prefill_attention_amd.workloads import HEADLINE, TORCH_DTYPES, WORKLOADS, make_inputs

    wl = WORKLOADS[key]
    fa.load_library()
    dev = torch.device("cuda:0")
    q, k, v = make_inputs(wl)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    scale = wl.scale
    out_dt = TORCH_DTYPES[wl.out_dtype]
    out = torch.empty((wl.q_len, wl.n_q_heads, wl.head_dim), dtype=out_dt, device=dev)
    stream = torch.cuda.Stream(device=dev)
    codes = {"f16": FA_DTYPE_F16, "bf16": FA_DTYPE_BF16, "f32": FA_DTYPE_F32}
    # One step = one call of the C entry point (argument marshalling done once,
    # so the timed loop is not bound by Python-side checks).
    if (wl.in_dtype, wl.out_dtype) != ("f16", "f32"):
        plan = fa.fa_prefill_chunk_plan(wl.n_q_heads, wl.n_kv_heads, wl.q_len, wl.seq_len, wl.head_dim,
                                        int(wl.causal))
        entry = fa.fa_prefill_ex
        call_args = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(), wl.n_q_heads,
                     wl.n_kv_heads, wl.q_len, wl.seq_len, wl.head_dim, scale, int(wl.causal),
                     codes[wl.in_dtype], codes[wl.out_dtype], stream.cuda_stream)
    elif wl.chunked:
        plan = fa.fa_prefill_chunk_plan(wl.n_q_heads, wl.n_kv_heads, wl.q_len, wl.seq_len, wl.head_dim,
                                        int(wl.causal))
        entry = fa.fa_prefill_chunk
        call_args = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(), wl.n_q_heads,
                     wl.n_kv_heads, wl.q_len, wl.seq_len, wl.head_dim, scale, int(wl.causal),
                     stream.cuda_stream)
    else:
        plan = fa.fa_prefill_plan(wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.head_dim, int(wl.causal))
        entry = fa.fa_prefill
        call_args = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(), wl.n_q_heads,
                     wl.n_kv_heads, wl.seq_len, wl.head_dim, scale, int(wl.causal), stream.cuda_stream)
    fa.attention(dq, dk, dv, scale, wl.causal, out=out, stream=stream)  # checked call first
    torch.cuda.synchronize()
    launch = lambda: entry(*call_args)  # noqa: E731
    t = time_bursts(launch, stream, args.steps, args.warmup, args.bursts)
    cold = time_cold(launch, stream, args.cold) if args.cold > 0 else []
    statuses = t["statuses"]
    if any(statuses):
        print(f"bench.py: the entry point returned {set(statuses)}", file=sys.stderr)
        return 1
    ms_per_step = t["median"]
    tflops = wl.flop / (ms_per_step * 1e-3) / 1e12
    tf = lambda ms: round(wl.flop / (ms * 1e-3) / 1e12, 2)  # noqa: E731

    traffic = measured_traffic(key) if not args.lib else None  # the record is the shipped build's
    min_bytes = (q.numel() + k.numel() + v.numel()) * 2 + out.numel() * out.element_size()
    line = {
        "metric": "causal FA prefill TFLOP/s + % f16 MFMA peak (S=2659, 32 heads, hd=128)"
        if key == HEADLINE else f"causal FA {'chunked ' if wl.chunked else ''}prefill TFLOP/s ({wl.name})",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.in_dtype,
        "data": "synthetic",
        "config": {**wl.describe(), "workload_key": key, "plan": plan.as_dict(),
                   **({"library": os.path.abspath(args.lib)} if args.lib else {})},
        "pct_peak": round(100.0 * tflops / PEAK_F16_TFLOPS, 2),
        "peak_basis": f"MI355X dense {wl.in_dtype} MFMA 256 CU x 4096 FLOP/clk x 2.4 GHz = 2516.6 TFLOP/s",
        "timing": {
            "protocol": f"{len(t['burst_sizes'])} bursts of {t['burst_sizes'][0]} back-to-back launches after "
                        f"{args.warmup} warm-up launches, HIP events on the launch stream; ms_per_step = "
                        f"median burst (warm L2/MALL; the power-management transient after idle settles "
                        f"within about 300 launches)",
            "burst_ms_per_launch": [round(x, 5) for x in t["burst_ms_per_launch"]],
            "ms_p10": round(t["p10"], 5),
            "ms_p90": round(t["p90"], 5),
            "ms_mean": round(t["mean"], 5),
            "tflops_p10_p90": [tf(t["p90"]), tf(t["p10"])],
            "cold_ms_median": round(percentile(cold, 50.0), 5) if cold else None,
            "cold_tflops": tf(percentile(cold, 50.0)) if cold else None,
            "cold_protocol": f"{len(cold)} launches, each after a 1 GiB scrub (inputs evicted from L2 and MALL), "
                             f"median" if cold else None,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": round(PEAK_F16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_F16_TFLOPS, 4),
            "traffic": traffic,
            "flop_per_launch": wl.flop,
            "avg_launch_us": round(ms_per_step * 1e3, 3),
            "min_hbm_bytes_per_launch": min_bytes,
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, q, k, v, out, scale)
    print(json.dumps(line), flush=True)
    return 0

if __name__ == "__main__":
    sys.exit(main())
