"""Decode-step throughput of the HashEvict path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long_128k]

One step = one decode step of one attention layer over all sequences and KV
heads of the workload: encode the queries, score every cached key code,
evict, write the new token, attend (the whole hot path).  Steps rotate over
L independent layer caches so the rotating working set (>= 512 MB) does not
fit the 256 MB last-level cache: every step reads its K/V from HBM.
Inputs are synthetic (seeded), already resident in HBM when timing starts.

Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, AMD public spec
MALL_BYTES = 256 << 20
HOLD_CYCLES = 1_000_000     # spin of torch.cuda._sleep before a timed region (well under 1 ms)
DEFAULT_WORKLOAD = "long_128k"


def step_bytes(shape, budgets, value_bits: int = 0) -> int:
    """Algorithmic HBM bytes of one decode step: per cached slot and KV head the
    code (b/8 bytes), the K row (d * kv bytes) and the V row (d * kv bytes, or
    d codes of value_bits bits and a 4-byte scale) are read; per KV head the new k, v, code
    and position are written; q is read and out written (fp32)."""
    es = 2 if shape.kv_dtype == "bf16" else 4
    cb = shape.n_bits // 8
    H, d = shape.n_kv_heads, shape.head_dim
    slots = int(sum(int(s) for s in budgets)) * H
    vrow = d * value_bits // 8 + 4 if value_bits else d * es
    per_slot = cb + d * es + vrow
    writes = shape.batch * H * (d * es + vrow + cb + 4)
    qo = shape.batch * shape.n_q_heads * d * 4 * 2
    return slots * per_slot + writes + qo


def load_traffic(workload: str, schedule: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, or None if the
    kernel source changed since they were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
        rec = data.get(f"{workload}/{schedule}")
        from lsh_eviction_amd.profiling import kernel_source_hash
        if rec and rec.get("kernel_hash") == kernel_source_hash():
            return rec.get("bytes_per_launch")
    except Exception:
        return None
    return None


def make_layer_inputs(shape, P, layer: int, seed: int):
    """Prompt K, V of one layer on the GPU with the datagen recipe (R and the key
    channel scales are the workload's; the draws come from a torch generator)."""
    import torch
    B, H, d = shape.batch, shape.n_kv_heads, shape.head_dim
    n_max = int(P.prompt_lens.max())
    g = torch.Generator(device="cuda")
    g.manual_seed(seed * 1000 + layer)
    dt = torch.bfloat16 if shape.kv_dtype == "bf16" else torch.float32
    scale = torch.from_numpy(P.key_scale).cuda()
    K = torch.randn((B, H, n_max, d), generator=g, device="cuda", dtype=torch.float32)
    K.mul_(scale[None, :, None, :])
    K = K.to(dt)
    V = torch.randn((B, H, n_max, d), generator=g, device="cuda", dtype=torch.float32).to(dt)
    return K, V


def copy_bandwidth(mib: int = 1024, reps: int = 10) -> float:
    """GB/s of torch's device copy (read + write bytes), the practical ceiling of
    a streaming kernel on this part."""
    import torch
    src = torch.empty((mib << 20) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * (mib << 20) * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, budget_s: float = 15.0):
    """The oracle's decode step timed on one host core on a bounded sample: the
    first sequence of the workload with all its KV heads, its cache filled with
    the first `budget` prompt tokens (the same slot count the GPU cache holds;
    the time of a decode step does not depend on which tokens the slots hold).
    The timing thread is pinned to one core of the process's CPU set for the
    timed loop (the oracle itself is single-threaded), then unpinned."""
    import oracle
    from lsh_eviction_amd import datagen
    oracle.lib()
    n, s = datagen.lengths(shape)
    S1 = int(s[0])
    one = shape.scaled(batch=1, prompt_range=None, budget_frac=None, prompt=S1, budget=S1)
    P = datagen.prompt(one)
    D = datagen.decode(one, steps=256, key_scale=P.key_scale if one.key_outliers else None)
    orc = oracle.OracleCache(P.R, P.budgets, one.n_q_heads, one.n_kv_heads)
    orc.prefill(P.K, P.V, P.prompt_lens, oracle.TRUNCATE)
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})   # pid 0: this (the calling) thread
    try:
        t0 = time.perf_counter()
        steps = 0
        while steps < 256:
            orc.decode_step(D.q[steps], D.k[steps], D.v[steps])
            steps += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, set(allowed))
    per_seq_step = dt / steps
    rate = 1.0 / (per_seq_step * shape.batch)   # a workload step covers `batch` sequences
    return {"value": round(rate, 4), "unit": "decode steps/s", "cores": 1, "kind": "oracle",
            "pinned_core": core, "nproc": os.cpu_count(), "cpus_allowed": len(allowed), "cpu_model": cpu_model(),
            "sample": f"1 sequence x {one.n_kv_heads} KV heads x {S1} slots (G={one.group}, d={one.head_dim}), "
                      f"{steps} decode steps in {dt:.1f} s on one thread pinned to core {core}, scaled to "
                      f"{shape.batch} sequence(s) per workload step"}


def host_link_bandwidth(mib: int = 512, reps: int = 5) -> float:
    """GB/s of a host-to-device copy from pinned host memory: the ceiling of a
    kernel that streams pinned host memory over the host link."""
    import torch
    src = torch.empty((mib << 20) // 4, dtype=torch.float32, pin_memory=True)
    dst = torch.empty(src.shape, dtype=torch.float32, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    return (mib << 20) * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def run_tier(args, shape, n, budgets, P, kvd, sched, make_layer_inputs):
    """Tiered decode: one cache whose evicted and dropped tokens go to a host
    tier in pinned memory; a step is hkv_decode_step followed by
    hkv_attend_tiered (attention over cache and tier, the tier streamed over the
    host link).  Prints one JSON line of its own."""
    import numpy as np
    import torch
    from lsh_eviction_amd import hkv
    n_max = int(n.max())
    cap = n_max + args.steps + args.warmup + 8
    pol = {"stream": hkv.HKV_PREFILL_STREAM, "truncate": hkv.HKV_PREFILL_TRUNCATE}[args.prefill]
    c = hkv.Cache(shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_bits, kvd,
                  budgets, P.R, prefill_policy=pol, decode_schedule=sched, max_prompt=n_max, chunk=args.chunk,
                  tier_capacity=cap)
    c.attach_tier()
    K, V = make_layer_inputs(shape, P, 0, shape.index)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    c.prefill(K, V, n)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    del K, V
    g = torch.Generator(device="cuda")
    g.manual_seed(shape.index + 7)
    dt = torch.bfloat16 if shape.kv_dtype == "bf16" else torch.float32
    POOL = 8
    qs = torch.randn((POOL, shape.batch, shape.n_q_heads, shape.head_dim), generator=g, device="cuda")
    ks = torch.randn((POOL, shape.batch, shape.n_kv_heads, shape.head_dim), generator=g, device="cuda").to(dt)
    vs = torch.randn((POOL, shape.batch, shape.n_kv_heads, shape.head_dim), generator=g, device="cuda").to(dt)
    out = torch.empty((shape.batch, shape.n_q_heads, shape.head_dim), device="cuda")
    tout = torch.empty_like(out)
    ev = torch.empty((shape.batch, shape.n_kv_heads), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    # every argument is checked once here; the timed calls skip the checks
    for p in range(POOL):
        c.check_step_args(qs[p], ks[p], vs[p], out, ev)
        c.check_step_args(qs[p], ks[p], vs[p], tout, ev)

    def step(i):
        c.decode_step(qs[i % POOL], ks[i % POOL], vs[i % POOL], out, ev, stream, check=False)
        c.attend_tiered(qs[i % POOL], tout, stream, check=False)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / args.steps
    # the tiered attention alone (the tier no longer changes)
    a2, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a2.record(stream)
    for i in range(args.steps):
        c.attend_tiered(qs[i % POOL], tout, stream, check=False)
    b2.record(stream)
    torch.cuda.synchronize()
    ms_att = a2.elapsed_time(b2) / args.steps
    cnt = hkv.to_numpy(c.tier_counts()).astype(np.int64)
    rows = int(np.minimum(cnt, cap).sum())
    es = 2 if shape.kv_dtype == "bf16" else 4
    tier_bytes = rows * 2 * shape.head_dim * es
    link = host_link_bandwidth()
    achieved = tier_bytes / (ms_att * 1e-3) / 1e9
    rec = {
        "metric": "tiered decode steps/s (decode step + attention over HBM cache and host tier)",
        "value": round(1000.0 / ms_step, 2), "unit": "tiered decode steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "data": "synthetic",
        "config": {"workload": args.config, "prefill_rule": args.prefill, "tier_capacity": cap,
                   "tier_rows_per_head_mean": round(rows / (shape.batch * shape.n_kv_heads), 1)},
        "roofline": {"bound": "host link", "achieved": round(achieved, 1), "peak": round(link, 1), "unit": "GB/s",
                     "frac": round(achieved / link, 4), "traffic": None},
        "attend_tiered_ms": round(ms_att, 4), "tier_bytes_per_attend": tier_bytes,
        "host_link_h2d_gbs": round(link, 1), "prefill_ms_with_tier_spill": round(prefill_ms, 2),
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD)
    ap.add_argument("--schedule", default="fused", choices=["fused", "split"])
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--value-bits", type=int, default=0, choices=[0, 4, 8],
                    help="8 or 4: values kept as codes of that width with a per-row scale (a different workload)")
    ap.add_argument("--prefill", default="stream", choices=["stream", "truncate", "query", "chunk"],
                    help="prefill rule of the layer caches (timed per layer, not part of a step)")
    ap.add_argument("--layers", type=int, default=0, help="layer caches rotated (0 = enough to exceed the MALL twice)")
    ap.add_argument("--graph", action="store_true", help="replay the steps of one rotation as a HIP graph")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--tier", action="store_true",
                    help="tiered decode: evictions kept in a pinned host tier, attention over both tiers")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only-timed", action="store_true",
                    help="launch only the warm-up and timed steps (no 50-step blocks, no warm single-cache run): "
                         "for counter runs")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the decode step runs on one GPU (it has no cross-GPU path); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.tier and args.prefill not in ("stream", "truncate"):
        print(json.dumps({"error": "--tier takes --prefill stream or truncate"}))
        sys.exit(2)

    import numpy as np
    import torch
    from lsh_eviction_amd import configs, datagen, hkv

    shape = configs.BY_NAME[args.config]
    torch.cuda.set_device(0)
    n, budgets = datagen.lengths(shape)
    per_step = step_bytes(shape, budgets, args.value_bits)
    L = args.layers or max(1, math.ceil(2 * MALL_BYTES / per_step))
    kvd = hkv.HKV_BF16 if shape.kv_dtype == "bf16" else hkv.HKV_F32
    sched = hkv.HKV_DECODE_FUSED if args.schedule == "fused" else hkv.HKV_DECODE_SPLIT
    P = datagen.prompt(shape.scaled(prompt=1, prompt_range=None, budget_frac=None, budget=1, batch=1))
    P.prompt_lens, P.budgets = n, budgets
    n_max = int(n.max())
    if args.tier:
        run_tier(args, shape, n, budgets, P, kvd, sched, make_layer_inputs)
        return

    caches, prefill_ms = [], []
    kept = None      # chunk rule: layer 0 scores its chunks, later layers reuse its kept lists
    for layer in range(L):
        pol = {"stream": hkv.HKV_PREFILL_STREAM, "truncate": hkv.HKV_PREFILL_TRUNCATE,
               "query": hkv.HKV_PREFILL_QUERY, "chunk": hkv.HKV_PREFILL_CHUNK}[args.prefill]
        c = hkv.Cache(shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_bits, kvd,
                      budgets, P.R, prefill_policy=pol, decode_schedule=sched, max_prompt=n_max, chunk=args.chunk,
                      value_bits=args.value_bits)
        K, V = make_layer_inputs(shape, P, layer, shape.index)
        Q = None
        if args.prefill == "query":
            gq = torch.Generator(device="cuda")
            gq.manual_seed(shape.index * 1000 + 500 + layer)
            Q = torch.randn((shape.batch, shape.n_q_heads, n_max, shape.head_dim), generator=gq, device="cuda")
        elif args.prefill == "chunk" and kept is None:
            gq = torch.Generator(device="cuda")
            gq.manual_seed(shape.index * 1000 + 600)
            Q = torch.randn((shape.batch, shape.n_q_heads, shape.head_dim), generator=gq, device="cuda")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r = c.prefill(K, V, n, Q=Q, reuse=kept)
        if args.prefill == "chunk" and kept is None:
            kept = r
        e1.record()
        torch.cuda.synchronize()
        prefill_ms.append(e0.elapsed_time(e1))
        del K, V, Q
        caches.append(c)
    # The prompt tensors stay in torch's allocator cache: device memory given
    # back to the driver here is cleared in the background while the timed
    # steps run, and slows the first ~600 of them by about 1 µs each.

    # decode inputs: a pool of distinct steps, resident on the GPU
    POOL = 16
    g = torch.Generator(device="cuda")
    g.manual_seed(shape.index + 7)
    dt = torch.bfloat16 if shape.kv_dtype == "bf16" else torch.float32
    scale = torch.from_numpy(P.key_scale).cuda()
    qs = torch.randn((POOL, shape.batch, shape.n_q_heads, shape.head_dim), generator=g, device="cuda")
    ks = (torch.randn((POOL, shape.batch, shape.n_kv_heads, shape.head_dim), generator=g, device="cuda")
          * scale[None, None]).to(dt)
    vs = torch.randn((POOL, shape.batch, shape.n_kv_heads, shape.head_dim), generator=g, device="cuda").to(dt)
    outs = torch.empty((L, shape.batch, shape.n_q_heads, shape.head_dim), device="cuda")
    evs = torch.empty((L, shape.batch, shape.n_kv_heads), dtype=torch.int32, device="cuda")

    stream = torch.cuda.current_stream()

    # every argument is checked once here; the timed calls skip the checks
    for l in range(L):
        for p in range(POOL):
            caches[l].check_step_args(qs[p], ks[p], vs[p], outs[l], evs[l])

    def one(i):
        l = i % L
        p = i % POOL
        caches[l].decode_step(qs[p], ks[p], vs[p], outs[l], evs[l], stream, check=False)

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(L):
                    caches[i].decode_step(qs[i % POOL], ks[i % POOL], vs[i % POOL], outs[i], evs[i], s, check=False)
        torch.cuda.synchronize()

    K_ = args.steps
    t_wall = time.perf_counter()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # A bounded spin kernel holds the stream while the host enqueues the
    # warm-up and the timed launches; the warm-up steps then run back to back
    # right before the start event, so the region measures the GPU's steps
    # back to back and not the host's first launch latency.
    torch.cuda.synchronize()
    torch.cuda._sleep(HOLD_CYCLES)
    for i in range(args.warmup):
        one(i)
    if graph is not None:
        reps = max(1, K_ // L)
        K_ = reps * L
        e_start.record(stream)
        for r in range(reps):
            graph.replay()
        e_end.record(stream)
        torch.cuda.synchronize()
        total_ms = e_start.elapsed_time(e_end)
        kern_ms = total_ms / K_
    else:
        # the steps back to back, bracketed by events on the stream they run on
        e_start.record(stream)
        for i in range(K_):
            one(i)
        e_end.record(stream)
        torch.cuda.synchronize()
        total_ms = e_start.elapsed_time(e_end)
        # the fused schedule is one kernel launch per step: its average launch
        # duration is the region's time over the launches (gaps included)
        kern_ms = total_ms / K_
    # spread: the same steps in blocks of 50, each block bracketed by events
    blocks = []
    for j in range(0, 0 if args.only_timed else min(K_, 1000) - 49, 50):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(j, j + 50):
            one(i)
        b.record(stream)
        blocks.append((a, b))
    # warm: one layer cache only, so the step's bytes may stay in the 256 MB MALL
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    KW = 0 if args.only_timed else min(K_, 500)
    w0.record(stream)
    for i in range(KW):
        caches[0].decode_step(qs[i % POOL], ks[i % POOL], vs[i % POOL], outs[0], evs[0], stream, check=False)
    w1.record(stream)
    torch.cuda.synchronize()
    block_us = sorted(a.elapsed_time(b) * 1e3 / 50 for a, b in blocks)
    warm_us = w0.elapsed_time(w1) * 1e3 / KW if KW else None
    wall = time.perf_counter() - t_wall
    copy_gbs = copy_bandwidth()

    ms_per_step = total_ms / K_
    value = 1000.0 / ms_per_step
    achieved = per_step / (kern_ms * 1e-3) / 1e9
    traffic = load_traffic(args.config, args.schedule + (f"/v{args.value_bits}" if args.value_bits else ""))
    rec = {
        "metric": "decode steps/s (LSH score+evict+attend) & % HBM peak, 8B-shape 128K ctx",
        "value": round(value, 1),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.kv_dtype if args.value_bits == 0 else f"{shape.kv_dtype}+i{args.value_bits}",
        "data": "synthetic",
        "config": {"workload": shape.name, "batch": shape.batch, "n_q_heads": shape.n_q_heads,
                   "n_kv_heads": shape.n_kv_heads, "head_dim": shape.head_dim, "n_bits": shape.n_bits,
                   "kv_storage": shape.kv_dtype, "budget_slots": int(budgets.sum()),
                   "prompt_tokens": int(n.sum()), "layers_rotated": L, "schedule": args.schedule,
                   "chunk": caches[0].chunk, "graph": bool(args.graph), "value_bits": args.value_bits},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "bytes_per_step": per_step,
        "kernel_us": round(kern_ms * 1e3, 3),
        "kernel": "k_decode_fused" if args.schedule == "fused" else "all kernels of the split step",
        "hbm_frac_of_step": round(per_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "us_per_step_median_of_50_step_blocks": round(float(np.median(block_us)), 3) if block_us else None,
        "warm_us_per_step_one_cache": round(warm_us, 3) if warm_us else None,
        "copy_gbs": round(copy_gbs, 1),
        "frac_of_copy": round(achieved / copy_gbs, 4),
        "prefill_ms_per_layer": round(float(np.mean(prefill_ms)), 2),
        "prefill_rule": args.prefill,
        **({"prefill_ms_scored_then_reused": [round(float(x), 2) for x in prefill_ms]}
           if args.prefill == "chunk" else {}),
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(shape, args.cpu_seconds)
    for c in caches:
        c.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
