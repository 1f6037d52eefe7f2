#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

One step = one decode token for every sequence of the batch, through the whole
hot path: host slot allocation (allocate-on-fill, copy-on-write), block copies,
block-table / length / slot upload, cache_append, paged decode attention
(partition + merge kernels) and the pool's fragmentation accounting.  Inputs
are synthetic and seeded (see synth/), resident in HBM before timing starts.

Prints one JSON line.  `value` is the step's algorithmic bytes (K/V read by
attention, q, out, table entries, lengths, plus cache_append's reads and
writes) per second of wall-clock step time; `roofline` is the decode
operation alone, timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
DEFAULT_STEPS = 50    # timed steps
DEFAULT_WARMUP = 10   # untimed warm-up steps


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    ap.add_argument("--config", default="long", help="tiny|small_mha|gqa|long|prefix|mha|beam|prefill|prefill_chunk|admission|admission_small")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--layout", default="head_major", choices=["head_major", "token_major"],
                    help="key cache order inside a block: [Hkv, P, D] or [P, Hkv, D]")
    ap.add_argument("--sweep-block-sizes", default="",
                    help="comma-separated block sizes: one decode JSON line per size (block-size study)")
    ap.add_argument("--no-share", action="store_true",
                    help="decode without the shared-block array (sequences that share blocks "
                         "read them once per sequence instead of once per pack)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle baseline (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the steps, run one device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(lengths, hq, hkv, d, p, s):
    kv = int(np.sum(lengths)) * hkv * d * 2 * s
    qo = 2 * len(lengths) * hq * d * s
    table = 4 * int(np.sum(-(-np.asarray(lengths) // p)))
    return kv + qo + table + 4 * len(lengths)


def append_bytes(b, hkv, d, s):
    return 2 * 2 * b * hkv * d * s + 4 * b


def measured_traffic(cfg_name, root):
    """HBM bytes per decode from the committed counter summary, if it was taken
    on the current decode kernel source (else None)."""
    import hashlib
    path = os.path.join(root, "profiles", f"paged_decode_{cfg_name}_traffic.json")
    src = os.path.join(root, "paged_kv_cache_399_amd", "csrc", "decode_kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != digest:
        return None
    return int(rec["traffic_bytes_per_decode"])


def run_beam(args):
    """Fan-out workload: prompts forked into several sequences; the first decode
    step copies every shared partly filled block (copy-on-write)."""
    import torch
    from synth import BEAM_CONFIGS, make_beam_workload
    from paged_kv_cache_399_amd import copy_blocks
    from paged_kv_cache_399_amd.session import PagedKVCache

    cfg = BEAM_CONFIGS[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    nsteps = 1 + args.warmup + args.steps
    w = make_beam_workload(cfg, args.seed, dev, steps=nsteps)
    b, hq, hkv, d, p = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    s = 2 if cfg.dtype == "bf16" else 4
    kv = PagedKVCache(w.num_blocks, p, hkv, d, w.torch_dtype, dev, w.free_order, fill=0.0,
                      share_blocks=not args.no_share)
    roots = kv.new_sequences(cfg.groups)
    slots, _ = kv.pool.append_slots(roots, w.prompt_lengths)
    kv.write_slots(torch.from_numpy(slots).to(dev), w.prompt_k, w.prompt_v)
    seqs = []
    for r in roots:
        seqs += [r] + [kv.fork(r) for _ in range(cfg.fanout - 1)]
    lens = np.repeat(w.prompt_lengths, cfg.fanout)
    max_len = int(lens.max()) + nsteps
    meta = kv.prepare(seqs, -(-max_len // p), hq, max_len, int(lens.sum()) + b * nsteps)
    out = torch.empty_like(w.q)
    stream = torch.cuda.current_stream()
    # first step: every sharer but the last copies its prompt's partial block
    step_slots, cow = kv.pool.append_slots(meta.seqs, np.ones(b, np.int32))
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    copy_blocks(kv.k_cache, kv.v_cache, cow, stream)
    c1.record(stream)
    meta.max_len, meta.total = kv.pool.block_table_upload(meta.seqs, meta.max_blocks, meta.table,
                                                          meta.lens, step_slots, meta.slots, stream,
                                                          d_shared_prev=meta.shared)
    meta.uploaded = True
    from paged_kv_cache_399_amd import cache_append
    cache_append(kv.k_cache, kv.v_cache, w.step_k[0], w.step_v[0], meta.slots, stream)
    kv.attend(meta, w.q, out, stream=stream)
    torch.cuda.synchronize()
    first_copy_ms = c0.elapsed_time(c1)
    # the same copies again, back to back (idempotent), for a bandwidth figure
    reps = 20
    c0.record(stream)
    for _ in range(reps):
        copy_blocks(kv.k_cache, kv.v_cache, cow, stream)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / reps
    block_bytes = hkv * p * d * s * 2                       # K and V of one block
    copy_bytes = 2 * len(cow) * block_bytes                 # read + write
    for i in range(args.warmup):
        kv.append_decode_tokens(meta, w.step_k[1 + i], w.step_v[1 + i], stream)
        kv.attend(meta, w.q, out, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        kv.append_decode_tokens(meta, w.step_k[1 + args.warmup + i], w.step_v[1 + args.warmup + i], stream)
        kv.attend(meta, w.q, out, stream=stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        kv.attend(meta, w.q, out, stream=stream)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / args.steps
    # the same decode split as a model step would run it over its layers: the
    # plan once (timed alone, `steps` calls), then `steps` planned calls
    # (partition + merge) on that plan
    kv.plan(meta, stream=stream)
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(args.steps):
        kv.plan(meta, stream=stream)
    d1.record(stream)
    torch.cuda.synchronize()
    plan_ms = d0.elapsed_time(d1) / args.steps
    d0.record(stream)
    for _ in range(args.steps):
        kv.attend(meta, w.q, out, stream=stream, planned=True)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_planned_ms = d0.elapsed_time(d1) / args.steps
    final = lens + nsteps
    dbytes = decode_bytes(final, hq, hkv, d, p, s)
    # unique K/V: prompts once, each sequence's own tokens once
    ubytes = dbytes - (int(final.sum()) - int(w.prompt_lengths.sum()) - b * nsteps) * hkv * d * 2 * s
    st = kv.pool.stats()
    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + decode tokens/s",
        "value": round(dbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_decode", "groups": cfg.groups, "fanout": cfg.fanout,
                   "batch": b, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                   "block_size": p, "prompt_lengths": f"uniform [{cfg.length_lo},{cfg.length_hi}]",
                   "seed": args.seed, "shared_blocks_read_once_per_pack": not args.no_share,
                   "parallelism": "single GPU"},
        "decode_tokens_per_s": round(b / (ms_step * 1e-3), 1),
        "decode_ms": round(dec_ms, 4),
        "decode_ms_planned": round(dec_planned_ms, 4),
        "plan_ms": round(plan_ms, 4),
        "decode_bytes_per_step": int(dbytes),
        "decode_unique_bytes": int(ubytes),
        "unique_GB_per_s": round(ubytes / (dec_planned_ms * 1e-3) / 1e9, 1),
        "unique_GB_per_s_with_plan": round(ubytes / (dec_ms * 1e-3) / 1e9, 1),
        "fragmentation": round(st["fragmentation"], 6),
        "copy_on_write": {"pairs": int(len(cow)), "first_step_ms": round(first_copy_ms, 4),
                          "ms": round(copy_ms, 4),
                          "GB_per_s": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1)},
        "GB_per_s_with_plan": round(dbytes / (dec_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(dbytes / (dec_planned_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dbytes / (dec_planned_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": PLANNED_KERNELS},
    }
    print(json.dumps(result), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0
# what roofline.achieved times: the per-layer decode on a plan made once per step
PLANNED_KERNELS = ("paged_attention_decode_planned (partition + merge launches; the plan, "
                   "once per step for every layer, is timed apart as plan_ms)")


def run_prefill(args):
    """Chunked / whole-prompt prefill: append the new tokens, then causal attention
    from each of them; matrix-core bound, reported in TFLOP/s."""
    import torch
    from synth import PREFILL_CONFIGS, make_prefill_workload
    from paged_kv_cache_399_amd import paged_attention_prefill
    from paged_kv_cache_399_amd.session import PagedKVCache

    cfg = PREFILL_CONFIGS[args.config]
    if args.block_size:
        cfg = dataclasses.replace(cfg, block_size=args.block_size)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = make_prefill_workload(cfg, args.seed, dev)
    b, hq, hkv, d, p = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    kv = PagedKVCache(w.num_blocks, p, hkv, d, torch.bfloat16, dev, w.free_order, fill=0.0,
                      layout=args.layout)
    seqs = kv.new_sequences(b)
    if cfg.context:
        slots, _ = kv.pool.append_slots(seqs, [cfg.context] * b)
        kv.write_slots(torch.from_numpy(slots).to(dev), w.ctx_k, w.ctx_v)
    total = cfg.context + cfg.new
    m = kv.prepare(seqs, -(-total // p), hq, total, b * total)
    out = torch.empty_like(w.q)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kv.extend(m, [cfg.new] * b, w.new_k, w.new_v, w.q, out, stream=stream)
    torch.cuda.synchronize()
    extend_ms = (time.perf_counter() - t0) * 1e3
    # the attention alone, back to back on the final state
    for _ in range(args.warmup):
        paged_attention_prefill(out, w.q, kv.k_cache, kv.v_cache, m.table, m.lens, m.query_start,
                                cfg.new, stream=stream, layout=kv.layout)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        paged_attention_prefill(out, w.q, kv.k_cache, kv.v_cache, m.table, m.lens, m.query_start,
                                cfg.new, stream=stream, layout=kv.layout)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    keys_seen = b * sum(cfg.context + i + 1 for i in range(cfg.new))      # causal
    flops = 4.0 * d * hq * keys_seen
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "paged prefill attention: TFLOP/s (% of dense bf16 matrix-core peak)",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": b, "context": cfg.context, "new_tokens": cfg.new,
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d, "block_size": p,
                   "k_layout": args.layout, "seed": args.seed, "parallelism": "single GPU"},
        "tokens_per_s": round(b * cfg.new / (ms * 1e-3), 1),
        "extend_ms_first_call": round(extend_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_attention_prefill"},
    }
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        result["cpu_baseline"] = prefill_cpu_baseline(w, cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def prefill_cpu_baseline(w, cfg, budget_s):
    """The float64 oracle's prefill on host cores over whole sequences until the budget is spent."""
    from oracle import attention as oatt
    from synth import bf16_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    spent, flops, done = 0.0, 0.0, 0
    for bi in range(cfg.batch):
        rows = slice(bi * cfg.new, (bi + 1) * cfg.new)
        k = np.concatenate([bf16_bits(w.ctx_k[bi * cfg.context:(bi + 1) * cfg.context]), bf16_bits(w.new_k[rows])])
        v = np.concatenate([bf16_bits(w.ctx_v[bi * cfg.context:(bi + 1) * cfg.context]), bf16_bits(w.new_v[rows])])
        q = bf16_bits(w.q[rows])
        t0 = time.perf_counter()
        oatt.prefill(q, k, v)
        spent += time.perf_counter() - t0
        flops += 4.0 * cfg.head_dim * cfg.num_q_heads * sum(cfg.context + i + 1 for i in range(cfg.new))
        done += 1
        if spent >= budget_s:
            break
    return {"value": round(flops / spent / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences, float64 numpy causal attention, {spent:.1f}s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}


def run_admission(args):
    """Replay a synthetic request trace under paged blocks and under up-front
    reservation on the same KV slots (host only: the library's block pool)."""
    from synth import ADMISSION_CONFIGS, make_admission_trace
    from paged_kv_cache_399_amd import admission
    cfg = ADMISSION_CONFIGS[args.config]
    pr, ou, mx, fo = make_admission_trace(cfg, args.seed)
    cap = cfg.num_blocks * cfg.block_size
    t0 = time.perf_counter()
    pg = admission.run_paged(cfg.num_blocks, cfg.block_size, pr, ou, fo)
    t_paged = time.perf_counter() - t0
    rs = admission.run_reserved(cap, pr, ou, mx)
    sp, sr = pg.summary(), rs.summary()
    result = {
        "metric": "admission: mean sequences resident per step, paged blocks vs up-front reservation",
        "value": round(sp["mean_running"], 2),
        "unit": "sequences",
        "n_gpus": 1, "steps": sp["steps"], "warmup": 0,
        "ms_per_step": round(t_paged * 1e3 / max(sp["steps"], 1), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int64", "data": "synthetic",
        "config": {"workload": cfg.name, "requests": cfg.n_requests,
                   "prompt": f"loguniform [{cfg.prompt_lo},{cfg.prompt_hi}]",
                   "output": f"loguniform [{cfg.output_lo},{cfg.output_hi}]",
                   "max_output": cfg.max_output, "num_blocks": cfg.num_blocks,
                   "block_size": cfg.block_size, "kv_slots": cap, "seed": args.seed,
                   "parallelism": "host only"},
        "paged": sp,
        "reserved": sr,
        "resident_ratio": round(sp["mean_running"] / max(sr["mean_running"], 1e-9), 3),
        "host_us_per_step_paged": round(t_paged * 1e6 / max(sp["steps"], 1), 1),
        "roofline": None,
    }
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        from oracle import admission as oad
        n = 50
        while True:
            t0 = time.perf_counter()
            oad.paged(cfg.num_blocks, cfg.block_size, pr, ou, fo, max_steps=n)
            dt = time.perf_counter() - t0
            if dt > args.cpu_seconds / 4 or n >= sp["steps"]:
                break
            n = min(sp["steps"], n * 4)
        result["cpu_baseline"] = {"value": round(n / dt, 2), "unit": "steps/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"first {n} steps of the paged replay ({dt:.1f} s)"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                          "multi-GPU runs are not supported (use --gpus 1)"}))
        sys.exit(2)
    import torch
    from synth import BEAM_CONFIGS, CONFIGS, make_workload
    from paged_kv_cache_399_amd.session import PagedKVCache
    if args.config in BEAM_CONFIGS:
        return run_beam(args)
    from synth import PREFILL_CONFIGS
    if args.config in PREFILL_CONFIGS:
        return run_prefill(args)
    from synth import ADMISSION_CONFIGS
    if args.config in ADMISSION_CONFIGS:
        return run_admission(args)
    cfg = CONFIGS[args.config]
    if args.sweep_block_sizes:
        # one line per block size, same schema, no CPU baseline; each size in
        # a fresh child process so allocator state does not carry over (this
        # process never touches the GPU)
        import subprocess
        rc = 0
        for p in [int(x) for x in args.sweep_block_sizes.split(",")]:
            cmd = [sys.executable, os.path.abspath(__file__), "--config", args.config,
                   "--block-size", str(p), "--steps", str(args.steps), "--warmup", str(args.warmup),
                   "--seed", str(args.seed), "--layout", args.layout, "--no-cpu-baseline"]
            rc = rc or subprocess.run(cmd).returncode
        sys.exit(rc)
    if args.block_size:
        cfg = cfg.with_block_size(args.block_size)
    print(json.dumps(run_decode(args, cfg, cpu=True)), flush=True)


def run_decode(args, cfg, cpu):
    import torch
    from synth import make_workload
    from paged_kv_cache_399_amd.session import PagedKVCache
    dev = "cuda:0"
    torch.cuda.set_device(0)
    nsteps = args.warmup + args.steps
    t_setup = time.perf_counter()
    w = make_workload(cfg, args.seed, dev, extra_steps=nsteps)
    b, hq, hkv, d, p = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    s = 2 if cfg.dtype == "bf16" else 4
    # a workload with a fixed pool (tiny: 16 blocks) holds only so many appended tokens
    need = int(np.sum(-(-(w.lengths + nsteps) // p)))
    if cfg.prefix_len == 0 and need > w.num_blocks:
        fit = 0
        while int(np.sum(-(-(w.lengths + fit + 1) // p))) <= w.num_blocks:
            fit += 1
        print(json.dumps({"error": f"{cfg.name}: its {w.num_blocks}-block pool holds {fit} decode steps "
                                   f"after the context, not warmup + steps = {nsteps} "
                                   f"(e.g. --steps {max(fit - 1, 1)} --warmup 1)"}), flush=True)
        sys.exit(2)
    kv = PagedKVCache(w.num_blocks, p, hkv, d, w.torch_dtype, dev, w.free_order, fill=0.0,
                      layout=args.layout, share_blocks=not args.no_share)
    if cfg.prefix_len:
        root = kv.new_sequences(1)[0]
        kv.write([root], [cfg.prefix_len], w.prefix_k, w.prefix_v)
        seqs = [root] + [kv.fork(root) for _ in range(b - 1)]
    else:
        seqs = kv.new_sequences(b)
    priv = (w.lengths - cfg.prefix_len).astype(np.int64)
    # prefill every generated token; the timed steps then append one token each
    slots, cow = kv.pool.append_slots(seqs, priv)
    assert len(cow) == 0
    d_slots = torch.from_numpy(slots).to(dev)
    # load the bulk-append kernel once outside the timed prefill: every slot
    # negative, so nothing is written
    skip = torch.full((4096,), -1, dtype=torch.int32, device=dev)
    kv.write_slots(skip, w.ctx_k[:0].new_zeros((4096, hkv, d)), w.ctx_v[:0].new_zeros((4096, hkv, d)))
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    kv.write_slots(d_slots, w.ctx_k, w.ctx_v)
    p1.record()
    torch.cuda.synchronize()
    prefill_ms = p0.elapsed_time(p1)
    prefill_bytes = 2 * 2 * int(priv.sum()) * hkv * d * s + 4 * int(priv.sum())
    max_len = int(w.lengths.max()) + nsteps
    total = int(w.lengths.sum()) + b * nsteps
    meta = kv.prepare(seqs, -(-max_len // p), hq, max_len, total)
    out = torch.empty_like(w.q)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s: {cfg.name} B={b} Hq={hq} Hkv={hkv} "
        f"D={d} P={p} tokens={int(w.lengths.sum())} blocks={w.num_blocks}")

    if args.calibrate_copy_mib:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    frag = []
    host_s = [0.0]

    def step(i):
        h0 = time.perf_counter()
        kv.append_decode_tokens(meta, w.step_k[i], w.step_v[i], stream)
        host_s[0] += time.perf_counter() - h0
        kv.attend(meta, w.q, out, stream=stream)
        frag.append(kv.pool.stats()["fragmentation"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    # timed region 1: whole steps (host allocation + uploads + kernels), no
    # events inside the loop so nothing is added between the step's launches
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    host_s[0] = 0.0
    t0 = time.perf_counter()
    s0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    s1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_step = s0.elapsed_time(s1) / args.steps
    # timed region 2: the decode operation alone, `steps` back-to-back calls on
    # the final state, HIP events on the stream its kernels run on
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(args.steps):
        kv.attend(meta, w.q, out, stream=stream)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / args.steps
    # the same decode split as a model step would run it over its layers: the
    # plan once (timed alone, `steps` calls), then `steps` planned calls
    # (partition + merge) on that plan
    kv.plan(meta, stream=stream)
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(args.steps):
        kv.plan(meta, stream=stream)
    d1.record(stream)
    torch.cuda.synchronize()
    plan_ms = d0.elapsed_time(d1) / args.steps
    d0.record(stream)
    for _ in range(args.steps):
        kv.attend(meta, w.q, out, stream=stream, planned=True)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_planned_ms = d0.elapsed_time(d1) / args.steps
    # timed region 3: cold caches -- a 1 GiB scratch write (beyond L2 and the
    # 256 MB Infinity Cache) before each call, every call timed on its own,
    # median reported
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(args.steps):
        scratch.fill_(1)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        kv.attend(meta, w.q, out, stream=stream)
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    del scratch
    cold_ms = float(np.median(cold))
    # timed region 4: the same decode replayed from a HIP graph (plan,
    # partition and merge captured once), `steps` back-to-back replays
    graph = kv.capture_attend(meta, w.q, out)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step wall, {gpu_ms_step:.3f} ms/step "
        f"on the stream, decode alone {dec_ms:.3f} ms (cold caches, median: {cold_ms:.3f} ms)")

    # algorithmic bytes: steps averaged over their growing contexts; the
    # decode-alone loop runs at the final lengths
    base = w.lengths.astype(np.int64)
    sbytes = np.mean([decode_bytes(base + args.warmup + i + 1, hq, hkv, d, p, s)
                      for i in range(args.steps)])
    dbytes = decode_bytes(base + args.warmup + args.steps, hq, hkv, d, p, s)
    abytes = append_bytes(b, hkv, d, s)
    step_gbs = (sbytes + abytes) / (ms_step * 1e-3) / 1e9
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9
    dec_planned_gbs = dbytes / (dec_planned_ms * 1e-3) / 1e9
    final = base + args.warmup + args.steps
    table_bytes = 4 * int(np.sum(-(-final // p)))
    # every decode this process ran: the steps at their growing lengths, then
    # the back-to-back, cold-cache and graph-replay loops (1 + steps replays)
    # at the final ones; per-dispatch hardware counters average over these
    per_call = [decode_bytes(base + i + 1, hq, hkv, d, p, s) for i in range(nsteps)]
    per_call += [dbytes] * (4 * args.steps + 1)
    extra = {}
    if cfg.prefix_len:
        # the shared prefix lives in HBM once: K/V bytes with the prefix counted once
        uniq_tokens = cfg.prefix_len + int(np.sum(final - cfg.prefix_len))
        ubytes = dbytes - (int(final.sum()) - uniq_tokens) * hkv * d * 2 * s
        extra["decode_unique_bytes"] = int(ubytes)
        extra["unique_GB_per_s"] = round(ubytes / (dec_planned_ms * 1e-3) / 1e9, 1)
        extra["unique_GB_per_s_with_plan"] = round(ubytes / (dec_ms * 1e-3) / 1e9, 1)

    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + decode tokens/s",
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}_decode", "batch": b, "num_q_heads": hq, "num_kv_heads": hkv,
            "head_dim": d, "block_size": p, "context_tokens": int(base.sum()),
            "max_context": int(base.max()), "seed": args.seed,
            "lengths": cfg.length_rule + (f" [{cfg.length_lo},{cfg.length_hi}]" if cfg.length_hi else ""),
            "prefix_len": cfg.prefix_len, "k_layout": args.layout,
            "shared_blocks_read_once_per_pack": not args.no_share, "parallelism": "single GPU",
        },
        "decode_tokens_per_s": round(b / (ms_step * 1e-3), 1),
        "decode_tokens_per_s_stream": round(b / (gpu_ms_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "decode_ms": round(dec_ms, 4),
        "decode_ms_planned": round(dec_planned_ms, 4),
        "plan_ms": round(plan_ms, 4),
        "decode_ms_cold_median": round(cold_ms, 4),
        "decode_ms_graph": round(graph_ms, 4),
        "GB_per_s_cold": round(dbytes / (cold_ms * 1e-3) / 1e9, 1),
        "gpu_ms_per_step": round(gpu_ms_step, 4),
        "decode_bytes_per_step": int(dbytes),
        "decode_calls": len(per_call),
        "decode_bytes_mean_per_call": int(round(float(np.mean(per_call)))),
        "block_table_bytes_read": table_bytes,
        "append_host_ms_per_step": round(host_s[0] * 1e3 / args.steps, 4),
        **extra,
        "fragmentation": round(float(np.mean(frag)), 6),
        "cache_append_prefill": {"tokens": int(priv.sum()), "ms": round(prefill_ms, 3),
                                 "GB_per_s": round(prefill_bytes / (prefill_ms * 1e-3) / 1e9, 1)},
        "GB_per_s_with_plan": round(dec_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(dec_planned_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_planned_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name, os.path.dirname(os.path.abspath(__file__))),
                     "kernel": PLANNED_KERNELS},
    }
    if cpu and not args.no_cpu_baseline and args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, cfg, args.cpu_seconds)
    return result


def cpu_baseline(w, cfg, budget_s):
    """The float64 oracle on host cores, over as many whole sequences as fit the budget."""
    import torch
    from oracle import attention as oatt
    from synth import bf16_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    hb = (lambda t: bf16_bits(t)) if cfg.dtype == "bf16" else (lambda t: t.cpu().numpy())
    order = np.random.default_rng(11).permutation(cfg.batch)
    s = 2 if cfg.dtype == "bf16" else 4
    spent, nbytes, done, toks = 0.0, 0, 0, 0
    for bi in order:
        k, v = w.seq_kv(int(bi))
        hk, hv, hq_ = hb(k), hb(v), hb(w.q[int(bi)])
        t0 = time.perf_counter()
        oatt.decode(hq_, hk, hv)
        spent += time.perf_counter() - t0
        L = hk.shape[0]
        nbytes += L * cfg.num_kv_heads * cfg.head_dim * 2 * s + 2 * cfg.num_q_heads * cfg.head_dim * s
        toks += L
        done += 1
        if spent >= budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences ({toks} context tokens), float64 numpy "
                      f"attention per sequence and KV head, {spent:.1f}s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "blas_threads": int(threads)}


if __name__ == "__main__":
    main()
