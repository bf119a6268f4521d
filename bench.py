#!/usr/bin/env python3
"""Throughput of the packed, ragged attention step over a paged KV cache on
one MI355X.

The default workload is the continuous-batching trace: a seeded
iteration-level scheduler's 200 iterations (8192-token budget, chunked
prefill, recompute preemption, 65,536-block pool), each running the whole
hot path -- slot translation + KV append (one launch), the fused attention
launch, the split merge -- for each of 32 layers (32 query / 8 KV heads,
head_dim 128, bf16).  One bench step is one pass over the whole trace; HIP
events on the library's stream bracket every iteration and every attention
launch.

The single-step workloads (--workload decode64, mixed, longshared, ...)
time K steps of one batch resident in HBM; before each, a 1 GiB read evicts
L2 and the Infinity Cache, so no step finds the previous one's KV on chip.

Prints ONE JSON line.  `value` is KV GB/s over the whole step (unique KV
bytes / step time); query tok/s, the attention kernel's roofline fraction
and the fp64 CPU oracle's rate on a sample of the same workload are
reported beside it.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_149_amd", "csrc", "pkv_kernels.hip")
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "packed-step attention: KV GB/s + query tok/s vs HBM/MFMA roofline, 1 GPU"

WORKLOADS = {
    "decode64": "config_decode64",
    "worked": "config_worked_step",
    "mixed": "config_mixed_chunked",
    "longshared": "config_long_shared",
    "prefillchunk": "config_prefill_chunk",
    "prefillfresh": "config_prefill_fresh",
    "tracestep": "config_trace_step",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (trace: passes over the whole trace; default 5, else 50)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps first (trace: default 1, else 5)")
    p.add_argument("--workload", default="trace", choices=sorted(WORKLOADS) + ["trace", "blockcopy", "swap", "prefixcache", "layer"])
    p.add_argument("--trace-steps", type=int, default=200, help="trace workload: scheduler steps")
    p.add_argument("--layer-batch", default="mixed", choices=sorted(WORKLOADS),
                   help="layer workload: the step whose rows the layer runs on")
    p.add_argument("--layers", type=int, default=32, help="trace workload: layers per step")
    p.add_argument("--trace-step-index", type=int, default=150,
                   help="tracestep workload: which step of the scheduler's trace to time")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-flush", action="store_true",
                   help="skip the 1 GiB read that evicts L2 and the Infinity Cache before each timed step")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time")
    p.add_argument("--narrow-waves", type=int, default=0, help="plan option (0 = library default)")
    p.add_argument("--min-wave-keys", type=int, default=0, help="plan option (0 = library default)")
    p.add_argument("--wide-tiles", type=int, default=-1, help="plan option: -1 auto, 0 never, 1 always")
    p.add_argument("--hbm-probe", action="store_true",
                   help="only measure plain streaming read and copy rates with torch kernels")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB fp32 copy kernel 5 times (HBM counter calibration)")
    args = p.parse_args()
    if args.steps is None:
        args.steps = 5 if args.workload == "trace" else 50
    if args.warmup is None:
        args.warmup = 1 if args.workload == "trace" else 5
    return args


def copy_calibration():
    """A plain elementwise copy of known size: reads and writes 2^30 bytes
    per launch, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": 5}), flush=True)


def hbm_probe():
    """Reference rates of plain torch kernels on this GPU: a sum over 4 GiB
    of bf16 (read-only) and an elementwise copy of 2 GiB."""
    import torch
    x = torch.ones(1 << 31, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(1 << 30, dtype=torch.bfloat16, device="cuda")
    res = {}
    for name, fn, nbytes in (("sum_read_4GiB", lambda: x.sum(dtype=torch.float32), 2 << 30 << 1),
                             ("copy_2GiB", lambda: y.copy_(x[: 1 << 30] * 1), 4 << 30)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        res[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    print(json.dumps({"hbm_probe_GBs": res}), flush=True)


def make_flush(dev, off: bool):
    """A read of 1 GiB that leaves L2 and the 256 MB Infinity Cache holding
    none of the step's data (a read, so the evicted lines are clean and no
    write-back lands in the timed step); it runs before every step, outside
    the step's events."""
    import torch
    if off:
        return lambda: None
    buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    return lambda: buf.sum()


def kernel_source_sha256() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, batch_name: str):
    """HBM bytes per attention launch from the committed rocprofv3 --pmc
    record for this workload (FETCH_SIZE and WRITE_SIZE, each scaled by the
    factor a plain copy kernel of known size gives), or None when there is
    no record, the record is of another batch (another trace step), or the
    kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_sha256() or rec.get("workload") != batch_name:
        return None
    return rec.get("traffic_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.hbm_probe:
        hbm_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this path has no "
              "multi-GPU form: the step shards by sequence with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_149_amd as pkv
    from paged_kv_cache_149_amd import accounting
    from synth import workloads as wl
    from synth.device import to_device

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "trace":
        run_trace(args)
        return
    if args.workload in ("blockcopy", "swap"):
        run_blocks(args)
        return
    if args.workload == "prefixcache":
        run_prefix(args)
        return
    if args.workload == "layer":
        run_layer(args)
        return
    dev = torch.device("cuda", 0)
    pkv.load_library()
    kw = {"index": args.trace_step_index} if args.workload == "tracestep" else {}
    batch = getattr(wl, WORKLOADS[args.workload])(**kw)
    log(f"workload {batch.name}: {batch.num_seqs} seqs, {batch.num_rows} rows, {batch.num_blocks} blocks")
    t = to_device(batch, dev)
    stream = torch.cuda.current_stream(dev)
    plan = pkv.pkv_plan(batch.cu_seqlens_q, batch.seq_lens, batch.num_q_heads, batch.num_kv_heads,
                        batch.head_dim, block_tables=batch.block_tables, num_blocks=batch.num_blocks,
                        options={"narrow_waves": args.narrow_waves, "min_wave_keys": args.min_wave_keys,
                                 "wide_tiles": args.wide_tiles},
                        device=dev, stream=stream)
    slots = torch.empty(batch.num_rows, dtype=torch.int64, device=dev)
    out = torch.empty_like(t["q"])
    torch.cuda.synchronize()

    new_ev = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(new_ev(), new_ev(), new_ev(), new_ev()) for _ in range(args.steps)]
    flush = make_flush(dev, args.no_flush)

    def step(i=None):
        if i is not None:
            ev[i][0].record(stream)
        pkv.pkv_slot_append_planned(t["k_new"], t["v_new"], t["cu_seqlens_q"], t["seq_lens"], t["block_tables"],
                                    t["k_cache"], t["v_cache"], plan, slot_mapping=slots, stream=stream)
        if i is not None:
            ev[i][1].record(stream)
        pkv.pkv_varlen_attention_main(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["scale"],
                                      plan, out=out, stream=stream)
        if i is not None:
            ev[i][2].record(stream)
        pkv.pkv_split_kv_reduce(plan, out, stream=stream)
        if i is not None:
            ev[i][3].record(stream)

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    for i in range(args.steps):
        flush()
        step(i)
    torch.cuda.synchronize()
    ms_step = float(np.mean([e[0].elapsed_time(e[3]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    log(f"step {ms_step:.4f} ms, attention launch {attn_ms:.4f} ms")

    nbytes = accounting.step_bytes(batch.cu_seqlens_q, batch.seq_lens, batch.block_tables,
                                   batch.num_q_heads, batch.num_kv_heads, batch.head_dim)
    flop = accounting.attention_flop(batch.cu_seqlens_q, batch.seq_lens, batch.num_q_heads, batch.head_dim)
    kv_gbs = nbytes["kv_unique"] / (ms_step * 1e-3) / 1e9
    launch_bytes = nbytes["total"]
    attn_gbs = launch_bytes / (attn_ms * 1e-3) / 1e9
    attn_tflops = flop / (attn_ms * 1e-3) / 1e12
    hbm_bound = launch_bytes / (HBM_PEAK_GBS * 1e9) >= flop / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
    kernel = "attention_mixed_kernel" if plan.num_wide_items > 0 else "attention_kernel"
    roof.update({"traffic": measured_traffic(args.workload, batch.name), "kernel": kernel, "avg_ms": round(attn_ms, 5),
                 "bytes_per_launch": launch_bytes, "flop_per_launch": flop})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(batch, args.cpu_seconds, nbytes)

    line = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": batch.name, "seqs": batch.num_seqs, "rows": batch.num_rows,
                   "q_heads": batch.num_q_heads, "kv_heads": batch.num_kv_heads,
                   "head_dim": batch.head_dim, "block_size": 16, "num_blocks": batch.num_blocks,
                   "kv_keys": int(plan.kv_keys), "items": int(plan.num_items),
                   "waves": int(plan.num_waves) + int(plan.num_wide_items),
                   "wave_keys": int(plan.wave_keys)},
        "query_tok_s": round(batch.num_rows / (ms_step * 1e-3), 1),
        "cache_flush_before_each_step": not args.no_flush,
        "kv_bytes_unique": nbytes["kv_unique"],
        "attention_flop": flop,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_trace(args):
    """The continuous-batching trace: the seeded scheduler's 200 iterations
    (Poisson(8) arrivals, prompts U{32..2048}, outputs log-uniform in
    [10, 2000], 8192-token budget with chunked prefill, recompute
    preemption, 65,536-block pool), each one packed step for every one of
    the 32 layers -- slot translation + append, the attention launch, the
    split merge -- each layer with its own K and V pools.

    One bench step is one pass over the whole trace.  Per iteration, every
    layer's Q/K/V rows are N(0,1) drawn on the device before the
    iteration's first event, and the iteration is planned on the host
    (pkv_plan into one of two pinned staging buffers) while the device still
    runs the previous ones.  HIP events on the stream bracket each
    iteration's layer loop and every attention launch."""
    import torch
    import paged_kv_cache_149_amd as pkv
    from paged_kv_cache_149_amd import accounting
    from synth import scheduler as sc

    dev = torch.device("cuda", 0)
    pkv.load_library()
    cfg = sc.TraceConfig(steps=args.trace_steps)
    t0 = time.perf_counter()
    steps, sch = sc.continuous_batching_trace(cfg)
    sched_s = time.perf_counter() - t0
    L, Hq, Hkv, D, NB = args.layers, 32, 8, 128, cfg.num_blocks
    n_it = len(steps)
    log(f"trace: {n_it} iterations, {L} layers, {NB}-block pool per layer, "
        f"{sch.preemptions} preemptions, {len(sch.finished)} requests finished (scheduler {sched_s:.2f} s)")
    kc = [torch.empty(NB, Hkv, 16, D, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    vc = [torch.empty(pkv.v_cache_shape(NB, Hkv, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    Tmax = max(st.num_rows for st in steps)
    qa = torch.empty(L, Tmax, Hq, D, dtype=torch.bfloat16, device=dev)
    ka = torch.empty(L, Tmax, Hkv, D, dtype=torch.bfloat16, device=dev)
    va = torch.empty(L, Tmax, Hkv, D, dtype=torch.bfloat16, device=dev)
    out = torch.empty(Tmax, Hq, D, dtype=torch.bfloat16, device=dev)
    slots = torch.empty(Tmax, dtype=torch.int64, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    stream = torch.cuda.current_stream(dev)
    scale = 1.0 / (D ** 0.5)

    # device metadata of every iteration, uploaded once; algorithmic work
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    meta = [(i32(st.cu_seqlens_q), i32(st.seq_lens), i32(st.block_tables)) for st in steps]
    att_bytes = np.zeros(n_it)
    app_bytes = np.zeros(n_it)
    kv_unique = np.zeros(n_it)
    flop = np.zeros(n_it)
    for i, st in enumerate(steps):
        nb_ = accounting.step_bytes(st.cu_seqlens_q, st.seq_lens, st.block_tables, Hq, Hkv, D)
        att_bytes[i], app_bytes[i], kv_unique[i] = nb_["total"], nb_["append"], nb_["kv_unique"]
        flop[i] = accounting.attention_flop(st.cu_seqlens_q, st.seq_lens, Hq, D)
    rows = np.array([st.num_rows for st in steps], dtype=np.float64)

    ws = [torch.empty(32 << 20, dtype=torch.uint8, device=dev)]
    staging = [torch.empty(4 << 20, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    pending = [None, None]  # the plan whose copy last read each staging buffer
    new_ev = lambda: torch.cuda.Event(enable_timing=True)
    ev_it = [(new_ev(), new_ev()) for _ in range(n_it)]
    ev_at = [[(new_ev(), new_ev()) for _ in range(L)] for _ in range(n_it)]
    kernels = set()

    def one_pass():
        plan_us = np.zeros(n_it)
        for i, st in enumerate(steps):
            T = st.num_rows
            qa[:, :T].normal_(generator=gen)
            ka[:, :T].normal_(generator=gen)
            va[:, :T].normal_(generator=gen)
            k = i % 2
            if pending[k] is not None:
                pending[k].event.synchronize()
            plan = pkv.pkv_plan(st.cu_seqlens_q, st.seq_lens, Hq, Hkv, D, block_tables=st.block_tables,
                                num_blocks=NB, device=dev, workspace=ws[0], staging=staging[k], stream=stream)
            pending[k] = plan
            ws[0] = plan.workspace
            plan_us[i] = plan.host_us
            kernels.add("attention_mixed_kernel" if plan.num_wide_items > 0 else "attention_kernel")
            cu, sl, bt = meta[i]
            ev_it[i][0].record(stream)
            for l in range(L):
                pkv.pkv_slot_append_planned(ka[l, :T], va[l, :T], cu, sl, bt, kc[l], vc[l], plan,
                                            slot_mapping=slots[:T], stream=stream)
                ev_at[i][l][0].record(stream)
                pkv.pkv_varlen_attention_main(qa[l, :T], kc[l], vc[l], bt, scale, plan, out=out[:T], stream=stream)
                ev_at[i][l][1].record(stream)
                pkv.pkv_split_kv_reduce(plan, out[:T], stream=stream)
            ev_it[i][1].record(stream)
        torch.cuda.synchronize()
        it_ms = np.array([a.elapsed_time(b) for a, b in ev_it])
        at_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in ev_at])
        return it_ms, at_ms, plan_us

    for w in range(args.warmup):
        one_pass()
        log(f"warmup pass {w + 1}/{args.warmup} done")
    it_all, at_all, plan_all = [], [], []
    for p in range(args.steps):
        it_ms, at_ms, plan_us = one_pass()
        it_all.append(it_ms)
        at_all.append(at_ms)
        plan_all.append(plan_us)
        log(f"pass {p + 1}/{args.steps}: {it_ms.sum():.1f} ms over {n_it} iterations "
            f"(attention launches {at_ms.sum():.1f} ms)")
    it_all = np.array(it_all)            # [pass, iteration]
    at_all = np.array(at_all)            # [pass, iteration, layer]
    plan_all = np.array(plan_all)

    sec_it = it_all.mean(axis=0) * 1e-3                  # per iteration, all layers
    pass_ms = it_all.sum(axis=1)
    t_hbm = (att_bytes + app_bytes) * L / (HBM_PEAK_GBS * 1e9)
    t_mfma = flop * L / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    dec = t_hbm >= t_mfma
    pre = ~dec
    # the attention launches alone: per-launch algorithmic bytes / FLOP over
    # their event-timed durations
    at_sec = at_all * 1e-3
    n_launch = at_all.size
    la_bytes = np.broadcast_to(att_bytes[None, :, None], at_all.shape)
    la_flop = np.broadcast_to(flop[None, :, None], at_all.shape)
    l_hbm = la_bytes / (HBM_PEAK_GBS * 1e9)
    l_mfma = la_flop / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    l_dec = l_hbm >= l_mfma
    achieved = la_bytes.sum() / at_sec.sum() / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("trace", f"cb-trace-{n_it}steps-{L}layers"),
            "kernel": "+".join(sorted(kernels)), "launches": int(n_launch),
            "avg_ms": round(float(at_all.mean()), 5), "bytes_per_launch": round(float(la_bytes.mean()), 1),
            "flop_per_launch": round(float(la_flop.mean()), 1),
            "frac_per_launch_bound": round(float(np.maximum(l_hbm, l_mfma).sum() / at_sec.sum()), 4),
            "decode_heavy_launches": {"n": int(l_dec.sum()),
                                      "hbm_frac": round(float(la_bytes[l_dec].sum() / at_sec[l_dec].sum()
                                                              / (HBM_PEAK_GBS * 1e9)), 4) if l_dec.any() else None},
            "prefill_heavy_launches": {"n": int((~l_dec).sum()),
                                       "mfma_frac": round(float(la_flop[~l_dec].sum() / at_sec[~l_dec].sum()
                                                                / (BF16_MFMA_PEAK_TFLOPS * 1e12)), 4)
                                       if (~l_dec).any() else None}}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = trace_cpu_baseline(steps, cfg, kv_unique, L, dev)
    res = {
        "metric": METRIC,
        "value": round(kv_unique.sum() * L / sec_it.sum() / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(pass_ms.mean()), 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"cb-trace-{n_it}steps-{L}layers", "step": "one pass over the whole trace",
                   "iterations": n_it, "layers": L, "budget": cfg.token_budget, "pool_blocks": NB,
                   "arrival_rate": cfg.arrival_rate, "preemptions": sch.preemptions,
                   "finished": len(sch.finished), "q_heads": Hq, "kv_heads": Hkv, "head_dim": D},
        "query_tok_s": round(rows.sum() / sec_it.sum(), 1),
        "total_rows": int(rows.sum()),
        "ms_per_iteration": round(float(sec_it.mean() * 1e3), 4),
        "pass_ms_min_max": [round(float(pass_ms.min()), 3), round(float(pass_ms.max()), 3)],
        "roofline_fraction": round(float(np.maximum(t_hbm, t_mfma).sum() / sec_it.sum()), 4),
        "decode_heavy": {"steps": int(dec.sum()),
                         "hbm_frac": round(float((att_bytes + app_bytes)[dec].sum() * L / sec_it[dec].sum()
                                                 / (HBM_PEAK_GBS * 1e9)), 4) if dec.any() else None},
        "prefill_heavy": {"steps": int(pre.sum()),
                          "mfma_frac": round(float(flop[pre].sum() * L / sec_it[pre].sum()
                                                   / (BF16_MFMA_PEAK_TFLOPS * 1e12)), 4) if pre.any() else None,
                          "ms": round(float(sec_it[pre].sum() * 1e3), 3) if pre.any() else None},
        "host_plan_us": {"mean": round(float(plan_all.mean()), 1), "max": round(float(plan_all.max()), 1),
                         "overlapped": "each iteration is planned while the device runs earlier ones"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def trace_cpu_baseline(steps, cfg, kv_unique, L, dev):
    """The fp64 oracle, untuned, on a bounded sample of the trace: every
    fourth sequence (packed order) of iterations n/8, n/2 and 7n/8 (25, 100
    and 175 of 200) with the host's BLAS threads, and every sixteenth
    sequence of iteration n/2 with one thread.  Values are the seeded counter generator's (pool tiles
    generated on the device by the generator's torch form, then copied to
    the host before timing).  The whole trace's oracle time is extrapolated
    from the sampled rate by KV bytes, and labelled so."""
    import dataclasses
    import torch
    import oracle
    from synth import workloads as wl
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits, threads = None, cores
    per_tok = 2 * 8 * 128 * 2

    def sampled(index, every):
        st = steps[index]
        b = wl.batch_from_metadata(f"trace-{index}", st.cu_seqlens_q, st.seq_lens, st.block_tables,
                                   cfg.num_blocks, seed=cfg.seed + 100 * index)
        sel = list(range(0, b.num_seqs, every))
        used = np.unique(np.concatenate([b.block_tables[s, :(int(b.seq_lens[s]) + 15) // 16] for s in sel]))
        idx = torch.from_numpy(used.astype(np.int64)).to(dev)
        pools = []
        for p in (b.k_pool, b.v_pool):
            tiles = p.to_device(dev)[idx].cpu().numpy().view(np.uint16)
            pools.append(_Dense({int(x): tiles[j] for j, x in enumerate(used)}, p.shape))
        b = dataclasses.replace(b, k_pool=pools[0], v_pool=pools[1])
        torch.cuda.empty_cache()
        nbytes = int(sum(int(b.seq_lens[s]) for s in sel)) * per_tok
        nrows = int(sum(int(b.cu_seqlens_q[s + 1] - b.cu_seqlens_q[s]) for s in sel))
        return b, sel, nbytes, nrows

    n = len(steps)
    picks = sorted({n // 8, n // 2, (7 * n) // 8})
    log(f"cpu baseline: oracle on every 4th sequence of trace iterations {picks}")
    tot_s, tot_b, tot_r = 0.0, 0, 0
    for index in picks:
        b, sel, nbytes, nrows = sampled(index, 4)
        t0 = time.perf_counter()
        oracle.packed_attention(b, sel)
        dt = time.perf_counter() - t0
        log(f"cpu baseline: iteration {index}: {len(sel)} sequences, {nbytes / 1e9:.3f} GB, {dt:.2f} s")
        tot_s, tot_b, tot_r = tot_s + dt, tot_b + nbytes, tot_r + nrows
    one = None
    if threadpool_limits is not None:
        b, sel, nbytes, nrows = sampled(n // 2, 16)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.packed_attention(b, sel)
            dt = time.perf_counter() - t0
        one = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "sample": f"every 16th sequence of iteration {n // 2} ({len(sel)} sequences, {nbytes / 1e9:.3f} GB "
                         f"of KV), {dt:.2f} s with one BLAS thread"}
        log(f"cpu baseline: one thread: {one['value']} GB/s")
    rate = tot_b / tot_s
    total_bytes = float(kv_unique.sum()) * L
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"every 4th sequence of trace iterations {picks}, one layer each "
                      f"({tot_b / 1e9:.3f} GB of KV, {tot_r} query rows, {tot_s:.2f} s; fp64 numpy, "
                      f"{threads} BLAS threads, host cores available: {cores})",
            "query_tok_s": round(tot_r / tot_s, 2),
            "extrapolated_trace_s": round(total_bytes / rate, 1),
            "extrapolated": "whole trace (all iterations, all layers) at the sampled rate, by KV bytes",
            "one_thread": one}


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def run_blocks(args):
    """Whole-block moves on one synthetic 16,384-block pool (8 kv heads,
    head_dim 128: 64 KiB of K and V per block): copy-on-write copies of 4,096
    disjoint random (src, dst) pairs in HBM, or a swap of 2,048 random blocks
    to pinned host memory and back.  K launches after W warm-ups, HIP events
    on the stream."""
    import torch
    import paged_kv_cache_149_amd as pkv
    dev = torch.device("cuda", 0)
    pkv.load_library()
    Hkv, D, nb = 8, 128, 16384
    kc = torch.empty(nb, Hkv, 16, D, dtype=torch.bfloat16, device=dev).normal_()
    vc = torch.empty(pkv.v_cache_shape(nb, Hkv, D), dtype=torch.bfloat16, device=dev).normal_()
    perm = np.random.default_rng(149100).permutation(nb).astype(np.int32)
    blk = 2 * Hkv * 16 * D * 2
    stream = torch.cuda.current_stream(dev)

    def timed(fn, k):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    base = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if args.workload == "blockcopy":
        n = 4096
        pairs = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).copy()).to(dev)
        ms = timed(lambda: pkv.pkv_copy_blocks(kc, vc, pairs), args.steps)
        moved = 2 * n * blk
        gbs = moved / (ms * 1e-3) / 1e9
        res = {"metric": "kv block copy-on-write: GB/s moved vs HBM roofline, 1 GPU", "value": round(gbs, 1),
               "unit": "GB/s", "ms_per_step": round(ms, 5), **base,
               "config": {"workload": f"blockcopy-{n}pairs-{Hkv}kv-pool{nb}", "pairs": n, "block_bytes": blk},
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                            "kernel": "copy_blocks_kernel", "bytes_per_launch": moved}}
    else:
        n = 2048
        blocks = torch.from_numpy(perm[:n].copy()).to(dev)
        host = torch.empty(pkv.swap_bytes(Hkv, n) // 2, dtype=torch.int16, pin_memory=True)
        ms_out = timed(lambda: pkv.pkv_swap_out(kc, vc, blocks, host), args.steps)
        ms_in = timed(lambda: pkv.pkv_swap_in(host, blocks, kc, vc), args.steps)
        nbytes = n * blk
        out_gbs, in_gbs = nbytes / (ms_out * 1e-3) / 1e9, nbytes / (ms_in * 1e-3) / 1e9
        rt = 2 * nbytes / ((ms_out + ms_in) * 1e-3) / 1e9
        # an 8,192-token context over 32 layers at 4 KiB per token per layer
        ctx = 8192 * 32 * 4096
        res = {"metric": "kv swap to pinned host memory: GB/s per direction vs PCIe, 1 GPU", "value": round(rt, 1),
               "unit": "GB/s", "ms_per_step": round(ms_out + ms_in, 5), **base,
               "config": {"workload": f"swap-{n}blocks-{Hkv}kv-pool{nb}", "blocks": n, "bytes_each_way": nbytes},
               "out_GBs": round(out_gbs, 1), "in_GBs": round(in_gbs, 1),
               "ms_8k_context_32_layers_round_trip": round(ctx / (out_gbs * 1e9) * 1e3 + ctx / (in_gbs * 1e9) * 1e3, 2),
               "roofline": {"bound": "pcie", "achieved": round(rt, 1), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                            "frac": round(rt / PCIE_PEAK_GBS, 4), "traffic": None,
                            "kernel": "swap_kernel", "bytes_per_launch": nbytes}}
    print(json.dumps(res), flush=True)


def run_prefix(args):
    """Prefix caching on the worked example of 11.2.4, sixteen times over: 16
    requests share a 2,010-token prompt and add 200 tokens each (8 kv heads,
    32 query heads, head_dim 128).  Cold: no cache, all 16 prefill their
    2,210 tokens in one packed step.  Warm: an earlier request registered
    the prompt; each request hits 125 blocks (2,000 tokens) in the library's
    pool and its step prefills 210 rows against 2,210 keys.  Both steps are
    append + attention + merge, timed as in the main workload; the host
    pool work (match, allocate, register) is timed on its own: it runs once
    per request, while the step runs once per layer.  `value` is prompt
    tokens (cached + computed) per second of the warm step."""
    import torch
    import paged_kv_cache_149_amd as pkv
    from paged_kv_cache_149_amd import accounting
    dev = torch.device("cuda", 0)
    pkv.load_library()
    R, shared_n, own_n, Hq, Hkv, D = 16, 2010, 200, 32, 8, 128
    total = shared_n + own_n
    rng = np.random.default_rng(149200)
    shared = rng.integers(0, 50000, size=shared_n, dtype=np.int32)
    prompts = [np.concatenate([shared, rng.integers(0, 50000, size=own_n, dtype=np.int32)]) for _ in range(R + 1)]
    nb = (R + 1) * 140
    pool = pkv.BlockPool(nb)
    cap = 140
    kc = torch.empty(nb, Hkv, 16, D, dtype=torch.bfloat16, device=dev).normal_()
    vc = torch.empty(pkv.v_cache_shape(nb, Hkv, D), dtype=torch.bfloat16, device=dev).normal_()
    stream = torch.cuda.current_stream(dev)
    scale = 1.0 / np.sqrt(D)

    # the request that fills the cache, then finishes
    row0 = np.full(cap, -1, np.int32)
    pool.append_slots(row0, 0, total)
    pool.register_prefix(prompts[0], row0)
    pool.release(row0[:139][::-1])

    # warm admission: host-side pool work for 16 requests
    t0 = time.perf_counter()
    rows_w, cached = [], []
    for r in range(R):
        row = np.full(cap, -1, np.int32)
        c = pool.match_prefix(prompts[r + 1], row)
        pool.append_slots(row, c, total - c)
        rows_w.append(row), cached.append(c)
    host_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    for r in range(R):
        pool.register_prefix(prompts[r + 1], rows_w[r])
    register_ms = (time.perf_counter() - t0) * 1e3
    assert all(c == 2000 for c in cached)
    # cold: the same requests, each in blocks of its own
    cold_pool = pkv.BlockPool(nb)
    rows_c = []
    for r in range(R):
        row = np.full(cap, -1, np.int32)
        cold_pool.append_slots(row, 0, total)
        rows_c.append(row)

    def setup(rows, q_len):
        cu = np.arange(R + 1, dtype=np.int32) * q_len
        sl = np.full(R, total, np.int32)
        bt = np.stack(rows)
        T = int(cu[-1])
        g = torch.Generator(device=dev).manual_seed(149201)
        mk = lambda h: torch.randn(T, h, D, device=dev, generator=g).to(torch.bfloat16)
        t = {"q": mk(Hq), "k_new": mk(Hkv), "v_new": mk(Hkv), "cu": torch.from_numpy(cu).to(dev),
             "sl": torch.from_numpy(sl).to(dev), "bt": torch.from_numpy(bt).to(dev)}
        plan = pkv.pkv_plan(cu, sl, Hq, Hkv, D, block_tables=bt, num_blocks=nb, device=dev, stream=stream)
        return cu, sl, bt, t, plan

    def timed(cu, sl, bt, t, plan):
        slots = torch.empty(t["q"].shape[0], dtype=torch.int64, device=dev)
        out = torch.empty_like(t["q"])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]

        def step(i=None):
            pkv.pkv_slot_append_planned(t["k_new"], t["v_new"], t["cu"], t["sl"], t["bt"], kc, vc, plan,
                                        slot_mapping=slots, stream=stream)
            if i is not None:
                ev[i][0].record(stream)
            pkv.pkv_varlen_attention_main(t["q"], kc, vc, t["bt"], scale, plan, out=out, stream=stream)
            if i is not None:
                ev[i][1].record(stream)
            pkv.pkv_split_kv_reduce(plan, out, stream=stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - a) * 1e3 / args.steps
        attn = float(np.mean([x.elapsed_time(y) for x, y in ev]))
        flop = accounting.attention_flop(cu, sl, Hq, D)
        return ms, attn, flop

    log("prefix cache: cold step, 16 x 2210 rows")
    cold_ms, cold_attn, cold_flop = timed(*setup(rows_c, total))
    log("prefix cache: warm step, 16 x 210 rows over 2210 keys")
    warm_ms, warm_attn, warm_flop = timed(*setup(rows_w, total - 2000))
    tflops = warm_flop / (warm_attn * 1e-3) / 1e12
    res = {"metric": "prefix-cached prefill step: prompt tokens served per second, 1 GPU",
           "value": round(R * total / (warm_ms * 1e-3), 1), "unit": "tok/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(warm_ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"prefix-{R}req-{shared_n}shared-{own_n}own", "requests": R,
                      "cached_tokens_each": 2000, "rows_each_warm": total - 2000, "keys_each": total},
           "cold_ms_per_step": round(cold_ms, 5), "cold_tok_s": round(R * total / (cold_ms * 1e-3), 1),
           "warm_over_cold_step": round(warm_ms / cold_ms, 4),
           "rows_fraction": round((total - 2000) / total, 4),
           "host_us_per_request": {"match_and_allocate": round(host_ms * 1e3 / R, 2),
                                   "register": round(register_ms * 1e3 / R, 2)},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "attention (warm step)", "avg_ms": round(warm_attn, 5),
                        "flop_per_launch": warm_flop, "cold_avg_ms": round(cold_attn, 5),
                        "cold_TFLOPs": round(cold_flop / (cold_attn * 1e-3) / 1e12, 2)}}
    print(json.dumps(res), flush=True)


def run_layer(args):
    """One packed attention layer (hidden 4096, 32 query / 8 KV heads of
    128) on the rows of a step workload: the fused QKV projection with RoPE,
    the paged step (append, attention, merge) and the output projection,
    each launch bracketed by HIP events; L2 and the Infinity Cache evicted
    before every step.  Weights are random N(0, 1/fan_in) bf16."""
    import torch
    import paged_kv_cache_149_amd as pkv
    from paged_kv_cache_149_amd import accounting
    from synth import workloads as wl
    from synth.device import to_device
    dev = torch.device("cuda", 0)
    pkv.load_library()
    batch = getattr(wl, WORKLOADS[args.layer_batch])()
    T, Hq, Hkv, D, hidden = batch.num_rows, batch.num_q_heads, batch.num_kv_heads, batch.head_dim, 4096
    log(f"layer on {batch.name}: {T} rows, hidden {hidden}")
    t = to_device(batch, dev)
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev).manual_seed(149300)
    x = torch.randn(T, hidden, device=dev, generator=g).to(torch.bfloat16)
    w_qkv = (torch.randn((Hq + 2 * Hkv) * D, hidden, device=dev, generator=g) / hidden ** 0.5).to(torch.bfloat16)
    w_o = (torch.randn(hidden, Hq * D, device=dev, generator=g) / (Hq * D) ** 0.5).to(torch.bfloat16)
    plan = pkv.pkv_plan(batch.cu_seqlens_q, batch.seq_lens, Hq, Hkv, D, block_tables=batch.block_tables,
                        num_blocks=batch.num_blocks, device=dev, stream=stream)
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    attn = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)
    flush = make_flush(dev, args.no_flush)
    new_ev = lambda: torch.cuda.Event(enable_timing=True)
    names = ["qkv_rope", "append", "attention", "merge", "o_proj"]
    ev = [[new_ev() for _ in range(len(names) + 1)] for _ in range(args.steps)]

    def step(i=None):
        mark = (lambda k: ev[i][k].record(stream)) if i is not None else (lambda k: None)
        mark(0)
        q, k_new, v_new = pkv.pkv_qkv_rope(x, w_qkv, t["cu_seqlens_q"], t["seq_lens"], Hq, Hkv, stream=stream)
        mark(1)
        pkv.pkv_slot_append_planned(k_new, v_new, t["cu_seqlens_q"], t["seq_lens"], t["block_tables"],
                                    t["k_cache"], t["v_cache"], plan, slot_mapping=slots, stream=stream)
        mark(2)
        pkv.pkv_varlen_attention_main(q, t["k_cache"], t["v_cache"], t["block_tables"], t["scale"], plan,
                                      out=attn, stream=stream)
        mark(3)
        pkv.pkv_split_kv_reduce(plan, attn, stream=stream)
        mark(4)
        pkv.pkv_linear(attn.view(T, Hq * D), w_o, out=y, stream=stream)
        mark(5)

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush()
        step(i)
    torch.cuda.synchronize()
    ms = {n: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in ev])) for k, n in enumerate(names)}
    layer_ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in ev]))
    qkv_flop = 2.0 * T * hidden * (Hq + 2 * Hkv) * D
    o_flop = 2.0 * T * Hq * D * hidden
    nbytes = accounting.step_bytes(batch.cu_seqlens_q, batch.seq_lens, batch.block_tables, Hq, Hkv, D)
    flop = accounting.attention_flop(batch.cu_seqlens_q, batch.seq_lens, Hq, D)
    kern = {
        "qkv_rope": {"TFLOP/s": qkv_flop / (ms["qkv_rope"] * 1e-3) / 1e12, "flop": qkv_flop},
        "attention": {"GB/s": nbytes["total"] / (ms["attention"] * 1e-3) / 1e9,
                      "TFLOP/s": flop / (ms["attention"] * 1e-3) / 1e12},
        "o_proj": {"TFLOP/s": o_flop / (ms["o_proj"] * 1e-3) / 1e12, "flop": o_flop},
    }
    dominant = max(("qkv_rope", "attention", "o_proj"), key=lambda n: ms[n])
    if dominant == "attention":
        hbm = nbytes["total"] / (HBM_PEAK_GBS * 1e9) >= flop / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        a = kern["attention"]["GB/s" if hbm else "TFLOP/s"]
        peak = HBM_PEAK_GBS if hbm else BF16_MFMA_PEAK_TFLOPS
        roof = {"bound": "hbm" if hbm else "mfma", "achieved": round(a, 1), "peak": peak,
                "unit": "GB/s" if hbm else "TFLOP/s", "frac": round(a / peak, 4), "kernel": "attention"}
    else:
        a = kern[dominant]["TFLOP/s"]
        roof = {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / BF16_MFMA_PEAK_TFLOPS, 4), "kernel": f"linear_kernel ({dominant})"}
    roof.update({"traffic": None, "avg_ms": round(ms[dominant], 5)})
    res = {"metric": "packed attention layer (QKV+RoPE, paged step, O projection): rows/s, 1 GPU",
           "value": round(T / (layer_ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(layer_ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"layer-h{hidden}-{batch.name}", "rows": T, "hidden": hidden, "q_heads": Hq,
                      "kv_heads": Hkv, "head_dim": D},
           "ms_per_launch": {n: round(v, 5) for n, v in ms.items()},
           "kernels": {n: {k: round(v, 2) if isinstance(v, float) and k != "flop" else v for k, v in d.items()}
                       for n, d in kern.items()},
           "cache_flush_before_each_step": not args.no_flush, "roofline": roof}
    print(json.dumps(res), flush=True)


def cpu_baseline(batch, seconds, nbytes):
    """The fp64 oracle, untuned, on the host cores: whole-batch passes of
    the same step (inputs materialised first, outside the clock)."""
    import oracle
    from synth import workloads as wl
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = cores
    log("cpu baseline: materialising the pool for the oracle")
    import dataclasses
    b = dataclasses.replace(batch, k_pool=_materialize_used(batch.k_pool, batch),
                            v_pool=_materialize_used(batch.v_pool, batch))
    reps, t_total = 0, 0.0
    while t_total < seconds and reps < 100:
        t0 = time.perf_counter()
        oracle.packed_attention(b)
        t_total += time.perf_counter() - t0
        reps += 1
    per = t_total / reps
    log(f"cpu baseline: {reps} oracle passes, {per:.3f} s each")
    return {"value": round(nbytes["kv_unique"] / per / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{reps} full passes of the same {batch.num_rows}-row step "
                                        f"(fp64 numpy, {per:.3f} s per pass, host cores available: {cores})",
            "query_tok_s": round(batch.num_rows / per, 2)}


class _Dense:
    """Pool view backed by a dict of materialised tiles (the blocks the
    batch references), so the oracle's reads cost no generation time."""

    def __init__(self, tiles, shape):
        self.tiles, self.shape = tiles, shape

    def __getitem__(self, key):
        if isinstance(key, tuple):
            return self.tiles[int(key[0])][key[1]]
        a = np.asarray(key)
        if a.ndim == 0:
            return self.tiles[int(a)]
        return np.stack([self.tiles[int(x)] for x in a.reshape(-1)])


def _materialize_used(pool, batch):
    if isinstance(pool, np.ndarray):
        return pool
    used = np.unique(batch.block_tables[batch.block_tables >= 0])
    arr = pool.tiles(used)
    return _Dense({int(b): arr[i] for i, b in enumerate(used)}, pool.shape)


if __name__ == "__main__":
    main()
