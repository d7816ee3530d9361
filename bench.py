"""Throughput of the tiled attention forward on one MI355X.

One step = one aule_attn_fwd call over the whole bf16 causal GQA batch (B=4, Hq=32, Hkv=8,
N=4096, head_dim=128, scale 1/sqrt(128), seeded N(0,1) inputs) — the full hot path of this
library on its headline workload. Inputs are resident in HBM before timing starts.

Prints ONE JSON line on stdout. `value` is causal-adjusted TFLOP/s (exact count of unmasked
query-key pairs, 4*d FLOP per pair per query head). The `roofline` object reports the
attention kernel's achieved rate (HIP events on the launch stream over the timed region)
against the MI355X dense bf16 MFMA peak; `cpu_baseline` times the CPU fp64 oracle on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Other workloads (--workload): the dense, varlen and long-context forward cases, the split-KV
decode case (GB/s against the HBM roofline) and the backward of the headline shape.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense, published
HBM_PEAK_GBS = 8000.0
# Sources each workload's kernels are built from: a traffic record taken on other sources is
# stale and not reported.
KERNEL_SOURCES = ["tiled_attention_02_amd/csrc/attn_fwd_mfma.hip",
                  "tiled_attention_02_amd/csrc/attn_mfma.h",
                  "tiled_attention_02_amd/csrc/attn_device.h",
                  "tiled_attention_02_amd/csrc/attn_problem.h",
                  "tiled_attention_02_amd/csrc/aule_attn_api.cpp"]
DECODE_SOURCES = ["tiled_attention_02_amd/csrc/attn_decode.hip",
                  "tiled_attention_02_amd/csrc/attn_decode_mfma.hip",
                  "tiled_attention_02_amd/csrc/attn_decode.h",
                  "tiled_attention_02_amd/csrc/attn_mfma.h",
                  "tiled_attention_02_amd/csrc/attn_device.h",
                  "tiled_attention_02_amd/csrc/aule_attn_api.cpp"]
BWD_SOURCES = ["tiled_attention_02_amd/csrc/attn_bwd_mfma.hip",
               "tiled_attention_02_amd/csrc/attn_bwd.hip",
               "tiled_attention_02_amd/csrc/attn_bwd.h",
               "tiled_attention_02_amd/csrc/attn_mfma.h",
               "tiled_attention_02_amd/csrc/attn_device.h",
               "tiled_attention_02_amd/csrc/aule_attn_api.cpp"]
F32_SOURCES = ["tiled_attention_02_amd/csrc/attn_fwd_f32_mfma.hip",
               "tiled_attention_02_amd/csrc/attn_mfma.h",
               "tiled_attention_02_amd/csrc/attn_device.h",
               "tiled_attention_02_amd/csrc/attn_problem.h",
               "tiled_attention_02_amd/csrc/aule_attn_api.cpp"]
F32_BWD_SOURCES = ["tiled_attention_02_amd/csrc/attn_bwd_f32_mfma.hip",
                   "tiled_attention_02_amd/csrc/attn_bwd.h",
                   "tiled_attention_02_amd/csrc/attn_mfma.h",
                   "tiled_attention_02_amd/csrc/attn_device.h",
                   "tiled_attention_02_amd/csrc/aule_attn_api.cpp"]
SHORT_SOURCES = ["tiled_attention_02_amd/csrc/attn_fwd_short.hip",
                 "tiled_attention_02_amd/csrc/attn_mfma.h",
                 "tiled_attention_02_amd/csrc/attn_device.h",
                 "tiled_attention_02_amd/csrc/attn_problem.h",
                 "tiled_attention_02_amd/csrc/aule_attn_api.cpp"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def sources_for(workload):
    from workloads import BWD_CONFIGS, CONFIGS, DECODE_CONFIGS, F32_CONFIGS, SHORT_CONFIGS
    dense = {**CONFIGS, **F32_CONFIGS}
    if workload in dense and dense[workload].dtype == "f32":
        return F32_SOURCES
    if workload in DECODE_CONFIGS:
        return DECODE_SOURCES
    if workload in SHORT_CONFIGS:
        return SHORT_SOURCES
    if workload in BWD_CONFIGS:
        return F32_BWD_SOURCES if BWD_CONFIGS[workload].dtype == "f32" else BWD_SOURCES
    return KERNEL_SOURCES


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE record of
    this workload, scaled by the copy-kernel calibration and summed over the launch's
    kernels; None when there is no record for the workload or it was taken on kernel
    sources that have changed since."""
    try:
        with open(TRAFFIC_RECORD) as f:
            records = json.load(f)["records"]
    except (OSError, ValueError, KeyError):
        return None
    for rec in records:
        if rec.get("workload") != workload:
            continue
        if rec.get("kernel_source_sha") != kernel_source_hash(sources_for(workload)):
            return None
        kib = rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]
        return int(kib * 1024)
    return None


def traffic_source(workload):
    """Where `traffic` comes from: it is not measured in this run but read from the committed
    counter record, and only when that record was taken on the current kernel sources."""
    sha = kernel_source_hash(sources_for(workload))
    if measured_traffic(workload) is None:
        return f"no rocprofv3 record in profiles/traffic.json for kernel sources {sha}"
    return (f"rocprofv3 FETCH_SIZE + WRITE_SIZE record in profiles/traffic.json, taken on kernel "
            f"sources {sha} (the current ones), scaled by a 256 MiB copy calibration")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3_bf16_causal_gqa")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload and report them on stderr")
    ap.add_argument("--print-kernel-hash", action="store_true",
                    help="print the hash of the kernel sources the workload's traffic record is keyed to")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def device_inputs(cfg, torch):
    from workloads import BwdConfig, DecodeConfig, DenseConfig, ShortConfig
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    if isinstance(cfg, BwdConfig):
        q, k, v = cfg.inputs()
        do = cfg.grad()
        t = lambda x: torch.from_numpy(x).to(device="cuda", dtype=tdt)
        return (t(q), t(k), t(v), t(do)), (q, k, v, do)
    if isinstance(cfg, (DenseConfig, DecodeConfig, ShortConfig)):
        q, k, v = cfg.inputs()
        t = lambda x: torch.from_numpy(x).to(device="cuda", dtype=tdt)
        return (t(q), t(k), t(v)), (q, k, v)
    qkv, cu = cfg.inputs()
    return (torch.from_numpy(qkv).to(device="cuda", dtype=tdt),
            torch.from_numpy(cu).to("cuda")), (qkv, cu)


def make_step(cfg, dev_inputs, torch):
    import tiled_attention_02_amd as aule
    from workloads import BwdConfig, DecodeConfig, DenseConfig, ShortConfig
    if isinstance(cfg, BwdConfig):
        # O and the row LSE come from one forward before the timed region; a step is the
        # backward alone (both of its kernels)
        q, k, v, do = dev_inputs
        o, lse = aule.flash_attention(q, k, v, causal=cfg.causal, scale=cfg.softmax_scale,
                                      return_lse=True)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        return lambda: aule.flash_attention_backward(q, k, v, o, do, lse, causal=cfg.causal,
                                                     scale=cfg.softmax_scale, grads=grads)
    if isinstance(cfg, DecodeConfig):
        q, k, v = dev_inputs
        out = torch.empty_like(q)
        B, Hq, Nq, d = q.shape
        need = aule.aule_attn_splitkv_workspace_size(B, Hq, k.shape[1], Nq, k.shape[2], d,
                                                     aule.dtype_code(q.dtype), 0)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)   # outside the timed region
        return lambda: aule.flash_attention_decode(q, k, v, causal=cfg.causal,
                                                   scale=cfg.softmax_scale, out=out, workspace=ws)
    if isinstance(cfg, (DenseConfig, ShortConfig)):
        q, k, v = dev_inputs
        out = torch.empty_like(q)
        return lambda: aule.flash_attention(q, k, v, causal=cfg.causal, scale=cfg.softmax_scale,
                                            out=out)
    from workloads import ModsConfig
    qkv, cu = dev_inputs
    T, _, H, d = qkv.shape
    out = torch.empty((T, H, d), dtype=qkv.dtype, device=qkv.device)
    max_len = int(max(cfg.lengths()))
    mods = {}
    if isinstance(cfg, ModsConfig):
        sl = cfg.slopes()
        mods = dict(window_size=(cfg.window_left, cfg.window_right), softcap=cfg.softcap,
                    alibi_slopes=None if sl is None else torch.from_numpy(sl).to("cuda"))
    return lambda: aule.flash_attn_varlen_qkvpacked_func(qkv, cu, max_len,
                                                         softmax_scale=cfg.softmax_scale,
                                                         causal=cfg.causal, out=out, **mods)


def time_steps(step, steps, warmup, torch, per_launch=False):
    """Wall-clock seconds per step and HIP-event seconds per step over exactly `steps` timed
    steps after `warmup` untimed ones. With `per_launch`, an event pair around every step (on
    the launch stream) also gives the per-launch durations (sorted, seconds)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()          # the stream the kernels are launched on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)] if per_launch else None
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        if marks:
            marks[i].record(stream)
        step()
    if marks:
        marks[steps].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launches = sorted(marks[i].elapsed_time(marks[i + 1]) / 1e3 for i in range(steps)) if marks else None
    return wall / steps, ev0.elapsed_time(ev1) / 1e3 / steps, launches


def cold_median(step, launches, torch, scrub_mib=512):
    """Median seconds of `launches` event-timed launches, each after a write of scrub_mib MiB
    that evicts the caches (the 256 MB Infinity Cache included)."""
    scrub = torch.empty(scrub_mib << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(launches):
        scrub.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    del scrub
    times.sort()
    return times[len(times) // 2]


def cpu_baseline(cfg, host_inputs, budget_s):
    """The CPU fp64 oracle on whole (batch, query head) slices of the workload, as many as
    fit in about budget_s seconds; scaled to TFLOP/s with the same FLOP count."""
    import numpy as np
    import oracle
    from workloads import BwdConfig, DecodeConfig, DenseConfig, ShortConfig
    threads = len(os.sched_getaffinity(0))
    if isinstance(cfg, ShortConfig):
        # whole batch entries (every head) through the oracle, as many as fit the budget
        q, k, v = host_inputs
        t0 = time.perf_counter()
        done = 0
        while done < cfg.batch and time.perf_counter() - t0 <= budget_s:
            b = done
            oracle.attention_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=cfg.causal,
                                 scale=cfg.softmax_scale)
            done += 1
        dt = time.perf_counter() - t0
        return {"value": cfg.flops() * done / cfg.batch / dt / 1e12, "unit": "TFLOP/s",
                "cores": threads, "kind": "oracle",
                "sample": f"{done} of {cfg.batch} batch entries (all heads), {dt:.1f} s"}
    if isinstance(cfg, BwdConfig):
        # whole (batch, query head) slices: the oracle's gradients of one query head against
        # its kv head, 10*d FLOP per unmasked pair like the GPU figure
        q, k, v, do = host_inputs
        G = cfg.heads_q // cfg.heads_kv
        n = cfg.seqlen
        pairs = n * (n + 1) // 2 if cfg.causal else n * n
        t0 = time.perf_counter()
        heads = 0
        for b in range(cfg.batch):
            for hq in range(cfg.heads_q):
                hk = hq // G
                oracle.attention_ref_bwd(q[b:b + 1, hq:hq + 1], k[b:b + 1, hk:hk + 1],
                                         v[b:b + 1, hk:hk + 1], do[b:b + 1, hq:hq + 1],
                                         causal=cfg.causal, scale=cfg.softmax_scale)
                heads += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            else:
                continue
            break
        dt = time.perf_counter() - t0
        return {"value": 10 * cfg.head_dim * pairs * heads / dt / 1e12, "unit": "TFLOP/s",
                "cores": threads, "kind": "oracle",
                "sample": f"{heads} of {cfg.batch * cfg.heads_q} (batch, query head) slices in "
                f"full, {dt:.1f} s"}
    if isinstance(cfg, DecodeConfig):
        # whole (batch, query head) slices against their kv head's cache; scaled to GB/s of
        # the workload's compulsory bytes like the GPU figure
        q, k, v = host_inputs
        G = cfg.heads_q // cfg.heads_kv
        total = cfg.batch * cfg.heads_q
        t0 = time.perf_counter()
        done = 0
        for b in range(cfg.batch):
            for hq in range(cfg.heads_q):
                hk = hq // G
                oracle.attention_ref_decode(q[b:b + 1, hq:hq + 1], k[b:b + 1, hk:hk + 1],
                                            v[b:b + 1, hk:hk + 1], causal=cfg.causal,
                                            scale=cfg.softmax_scale)
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": cfg.bytes_compulsory() * done / total / dt / 1e9, "unit": "GB/s",
                "cores": threads, "kind": "oracle",
                "sample": f"{done} of {total} (batch, query head) slices, {dt:.1f} s"}
    if not isinstance(cfg, DenseConfig):
        from workloads import ModsConfig, visible_pairs
        qkv, cu = host_inputs
        t0 = time.perf_counter()
        done_flops, seqs = 0, 0
        for s in range(len(cu) - 1):
            a, e = int(cu[s]), int(cu[s + 1])
            sub_cu = np.array([0, e - a], dtype=np.int32)
            L = e - a
            if isinstance(cfg, ModsConfig):
                sl = cfg.slopes()
                oracle.attention_ref_varlen_mods(qkv[a:e], sub_cu, causal=cfg.causal,
                                                 scale=cfg.softmax_scale,
                                                 window=(cfg.window_left, cfg.window_right),
                                                 softcap=cfg.softcap, alibi_slopes=sl)
                pairs = visible_pairs(L, cfg.causal, cfg.window_left, cfg.window_right)
            else:
                oracle.attention_ref_varlen(qkv[a:e], sub_cu, causal=cfg.causal, scale=cfg.softmax_scale)
                pairs = L * (L + 1) // 2 if cfg.causal else L * L
            done_flops += 4 * cfg.head_dim * cfg.heads * pairs
            seqs += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                "kind": "oracle", "sample": f"{seqs} of {len(cu) - 1} sequences, all heads, "
                f"{dt:.1f} s"}
    q, k, v = host_inputs
    G = cfg.heads_q // cfg.heads_kv
    n = cfg.seqlen
    pairs = n * (n + 1) // 2 if cfg.causal else n * n
    if n * n * 8 > (1 << 30):
        # a whole slice's fp64 score matrix would pass 1 GiB (8.6 GB at 32k tokens): the
        # oracle computes the sampled query rows of every head instead, and the full problem's
        # time is extrapolated from the sampled (query, key) pairs
        from workloads import sampled_rows
        rows = sampled_rows(n)
        sp = int(sum(r + 1 for r in rows)) if cfg.causal else rows.size * n
        t0 = time.perf_counter()
        heads = 0
        for b in range(cfg.batch):
            for hq in range(cfg.heads_q):
                hk = hq // G
                oracle.attention_ref_rows(q[b:b + 1, hq:hq + 1], k[b:b + 1, hk:hk + 1],
                                          v[b:b + 1, hk:hk + 1], rows, causal=cfg.causal,
                                          scale=cfg.softmax_scale)
                heads += 1
        dt = time.perf_counter() - t0
        sampled_pairs = sp * heads
        full_pairs = pairs * cfg.batch * cfg.heads_q
        return {"value": 4 * cfg.head_dim * sampled_pairs / dt / 1e12, "unit": "TFLOP/s",
                "cores": threads, "kind": "oracle",
                "sample": f"{rows.size} sampled query rows of each of {heads} (batch, query head) "
                f"slices, {dt:.1f} s",
                "extrapolated_full_s": round(dt * full_pairs / sampled_pairs, 1),
                "extrapolation": "sampled time x full pairs / sampled pairs (label only)"}
    t0 = time.perf_counter()
    heads = 0
    for b in range(cfg.batch):
        for hq in range(cfg.heads_q):
            hk = hq // G
            oracle.attention_ref(q[b:b + 1, hq:hq + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1],
                                 causal=cfg.causal, scale=cfg.softmax_scale)
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    flops = 4 * cfg.head_dim * pairs * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {cfg.batch * cfg.heads_q} (batch, query head) slices in full, "
            f"{dt:.1f} s"}


def main():
    args = parse()
    if args.print_kernel_hash:
        print(kernel_source_hash(sources_for(args.workload)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import (BWD_CONFIGS, CONFIGS, DECODE_CONFIGS, MODS_CONFIGS, SHORT_CONFIGS,
                           BwdConfig, DecodeConfig, ModsConfig, ShortConfig)
    from workloads import F32_CONFIGS, HARNESS_CONFIGS
    ALL = {**CONFIGS, **DECODE_CONFIGS, **BWD_CONFIGS, **MODS_CONFIGS, **SHORT_CONFIGS,
           **HARNESS_CONFIGS, **F32_CONFIGS}

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": max(1, args.steps)}), flush=True)
        return

    cfg = ALL[args.workload]
    dev_in, host_in = device_inputs(cfg, torch)
    step = make_step(cfg, dev_in, torch)
    wall_s, kern_s, launches = time_steps(step, args.steps, args.warmup, torch, per_launch=True)

    flops = cfg.flops()
    value = flops / wall_s / 1e12
    achieved = flops / kern_s / 1e12
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    line = {
        "metric": "attention fwd TFLOPS (causal-adjusted) and % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) inputs)",
        "config": {"workload": cfg.name, "desc": describe(cfg), "pct_of_peak": round(100 * value / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(cfg.name),
                     "traffic_source": traffic_source(cfg.name),
                     "kernel_ms": round(kern_s * 1e3, 4),
                     "launch_ms": {"median": round(launches[len(launches) // 2] * 1e3, 4),
                                   "min": round(launches[0] * 1e3, 4),
                                   "max": round(launches[-1] * 1e3, 4)},
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": cfg.bytes_compulsory()},
    }
    if hasattr(cfg, "pairs") and not isinstance(cfg, (DecodeConfig, ShortConfig)):
        # the exact unmasked-pair count, and the common convention that counts a causal
        # problem as half of the full square (B * N^2 / 2 pairs)
        line["config"]["flops_exact"] = flops
        half = half_convention_flops(cfg)
        if half is not None:
            line["config"]["flops_half_convention"] = half
            line["config"]["value_half_convention"] = round(half / wall_s / 1e12, 2)
    if cfg.dtype == "f32":
        line["metric"] = "attention fwd TFLOPS (causal-adjusted) and % of MI355X fp32 peak"
    if isinstance(cfg, ModsConfig):
        line["metric"] = "attention varlen fwd with window/softcap/ALiBi TFLOPS (visible pairs) and % of MI355X bf16 MFMA peak"
    if isinstance(cfg, BwdConfig):
        line["metric"] = ("attention bwd TFLOPS (causal-adjusted, 2.5x forward FLOPs) and % of MI355X "
                          + ("fp32 peak" if cfg.dtype == "f32" else "bf16 MFMA peak"))
    if isinstance(cfg, DecodeConfig):
        # reading the KV cache bounds this path: throughput against the HBM roofline
        gbs = cfg.bytes_compulsory() / kern_s / 1e9
        line["metric"] = "attention decode (split-KV) achieved HBM GB/s"
        line["value"] = round(cfg.bytes_compulsory() / wall_s / 1e9, 1)
        line["unit"] = "GB/s"
        line["config"]["pct_of_peak"] = round(100 * line["value"] / HBM_PEAK_GBS, 2)
        line["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)})
    if isinstance(cfg, ShortConfig):
        # 35 FLOP per compulsory byte, far left of the ridge: the HBM roofline bounds it
        gbs = cfg.bytes_compulsory() / kern_s / 1e9
        line["config"]["gbs_compulsory"] = round(cfg.bytes_compulsory() / wall_s / 1e9, 1)
        line["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)})
    if args.all:
        for name, c in ALL.items():
            if name == cfg.name:
                continue
            di, _ = device_inputs(c, torch)
            st = make_step(c, di, torch)
            # the pages' harness method: 20 warm-ups, then 100 launches, the median reported
            n = 100 if c.flops() < 1e12 else 20
            _, kt, ls = time_steps(st, n, 20, torch, per_launch=True)
            med = ls[len(ls) // 2]
            cold = cold_median(st, 21, torch)
            pk = MFMA_PEAK_TFLOPS[c.dtype]
            gbs = c.bytes_compulsory() / med / 1e9
            print(f"[bench] {name}: median {med * 1e3:.4f} ms/launch (mean {kt * 1e3:.4f}, cold-cache "
                  f"median {cold * 1e3:.4f}), {c.flops() / med / 1e12:.1f} TFLOP/s "
                  f"({100 * c.flops() / med / 1e12 / pk:.1f}% of {pk:.0f}), "
                  f"{gbs:.0f} GB/s compulsory ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)", file=sys.stderr)
            del di
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, host_in, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def half_convention_flops(cfg):
    """FLOPs with a causal problem counted as half the full square (4*d*Hq*B*N^2/2), the
    figure many reports quote; None for the workloads it does not apply to."""
    from workloads import BwdConfig, DenseConfig, ModsConfig, VarlenConfig
    if isinstance(cfg, ModsConfig) or not getattr(cfg, "causal", False):
        return None
    per_pair = 10 if isinstance(cfg, BwdConfig) else 4
    if isinstance(cfg, DenseConfig):
        return per_pair * cfg.head_dim * cfg.heads_q * cfg.batch * cfg.seqlen * cfg.seqlen // 2
    if isinstance(cfg, VarlenConfig):
        return per_pair * cfg.head_dim * cfg.heads * sum(int(l) ** 2 for l in cfg.lengths()) // 2
    return None


def describe(cfg):
    from workloads import BwdConfig, DecodeConfig, DenseConfig, ShortConfig
    if isinstance(cfg, ShortConfig):
        return (f"{cfg.dtype} short {'causal' if cfg.causal else 'non-causal'} B={cfg.batch} "
                f"Hq={cfg.heads_q} Hkv={cfg.heads_kv} Nq={cfg.seqlen_q} Nk={cfg.seqlen_k} "
                f"d={cfg.head_dim} scale={cfg.softmax_scale:.6g}")
    if isinstance(cfg, BwdConfig):
        return (f"{cfg.dtype} backward {'causal' if cfg.causal else 'non-causal'} B={cfg.batch} "
                f"Hq={cfg.heads_q} Hkv={cfg.heads_kv} N={cfg.seqlen} d={cfg.head_dim} "
                f"scale={cfg.softmax_scale:.6g}")
    if isinstance(cfg, DecodeConfig):
        return (f"{cfg.dtype} decode {'causal' if cfg.causal else 'non-causal'} B={cfg.batch} "
                f"Hq={cfg.heads_q} Hkv={cfg.heads_kv} Nq={cfg.seqlen_q} Nk={cfg.seqlen_k} "
                f"d={cfg.head_dim} scale={cfg.softmax_scale:.6g}")
    if isinstance(cfg, DenseConfig):
        return (f"{cfg.dtype} {'causal' if cfg.causal else 'non-causal'} B={cfg.batch} Hq={cfg.heads_q} "
                f"Hkv={cfg.heads_kv} N={cfg.seqlen} d={cfg.head_dim} scale={cfg.softmax_scale:.6g}")
    from workloads import ModsConfig
    extra = ""
    if isinstance(cfg, ModsConfig):
        extra = (f" window=({cfg.window_left},{cfg.window_right}) softcap={cfg.softcap:g} "
                 f"alibi={'geometric' if cfg.alibi else 'off'}")
    return (f"{cfg.dtype} varlen {'causal' if cfg.causal else 'non-causal'} {cfg.num_seqs} seqs "
            f"L~U[{cfg.len_lo},{cfg.len_hi}] H={cfg.heads} d={cfg.head_dim}{extra}")


if __name__ == "__main__":
    main()
