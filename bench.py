"""Benchmark: paged decode attention on one MI355X.

One step = the decode step of a batch: pa_cache_write of one new token per
sequence (its slots from the block allocator), then pa_decode over every
sequence's paged K/V. Default workload: the LLaMA-13B-shaped decode layer
(64 sequences, 40 MHA heads of 128, bf16 KV, blocks of 16, lengths uniform on
[1, 2048], pool 1.1x the need with random block placement).

Prints ONE JSON line. ``value`` is KV GB/s over the whole step: the
algorithmic KV bytes (each valid token's K and V once per KV head) divided by
the step time. ``roofline`` reports the decode call (its kernels, measured
with HIP events on the launch stream) against the 8 TB/s HBM peak.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
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

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")

WORKLOAD_TEXT = {
    "llama13b": "LLaMA-13B-shaped decode layer: 64 seqs, 40 MHA heads x 128, bf16 KV, "
                "block 16, lengths U[1,2048], pool 1.1x need, random placement",
    "llama70b": "Llama-2-70B-shaped GQA decode layer: 256 seqs, 64 q / 8 KV heads x 128, "
                "bf16 KV, block 16, lengths log-uniform [128,8192]",
    "prefix": "prefix-cached batch: 256 reqs sharing a 1024-token prefix (64 blocks), "
              "tails U[16,512], 40 heads x 128, bf16, block 16",
    "cow": "parallel sampling: 32 prompts x 3 samples sharing 512-token prompts, "
           "tails U[1,256], 40 heads x 128, bf16, block 16",
    "cow504": "parallel sampling, 504-token prompts (partial block copied on write)",
    "beam": "beam search width 4: 32 groups on 512-token prompts, U[1,256] steps",
    "tiny": "tiny fp32: 2 seqs (7, 11), 4 heads x 64, block 4",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "cache_ops.hip", "device.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_316_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per decode call from committed rocprofv3 PMC runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_decode_call")


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, on the first sequences of the batch until ~budget_s."""
    import numpy as np
    from oracle.expected import decode_out
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes
    lens = wl.seq_lens
    import contextlib
    ctx = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
    n = 0
    with ctx:
        t0 = time.perf_counter()
        while n < len(lens) and time.perf_counter() - t0 < budget_s:
            decode_out(wl, [n])
            n += 1
    dt = time.perf_counter() - t0
    nbytes = float(lens[:n].sum()) * per_tok
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} of {len(lens)} sequences ({int(lens[:n].sum())} tokens, "
                      f"all {wl.num_q_heads} heads), fp64 NumPy, {dt:.1f} s; "
                      f"tokens/s = {n / dt:.3f}",
            "tokens_per_s": round(n / dt, 4), "seconds": round(dt, 3),
            "os_cpu_count": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama13b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--workers", type=int, default=0, help="decode wavefronts (0 = default)")
    ap.add_argument("--replicas", type=int, default=2, help="pool replicas rotated between steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(decode shards by sequences or heads with no exchange inside attention).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_316_amd as pkv
    import workloads
    from paged_kv_cache_316_amd.runner import WriteBatch, apply_events, run_script, split_phases

    torch.cuda.set_device(0)
    t0 = time.time()
    wl = workloads.make(args.workload, "full")
    log(f"workload {args.workload}: {len(wl.decode_seqs)} seqs, drawn in {time.time() - t0:.1f} s")
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def dev(a):
        if wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(dt)

    # set-up through the library: allocator -> copies / cache writes (untimed)
    alloc = pkv.BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    phases = split_phases(run_script(alloc, wl.ops))
    rows_k, rows_v = dev(wl.rows_k), dev(wl.rows_v)
    pool0 = pkv.KVPool.empty(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, dt)
    for name in ("setup", "prefill"):
        apply_events(pool0, phases.get(name, []), rows_k, rows_v)
    dec_events = phases["decode"]
    copies = [e for e in dec_events if e[0] == "copy"]
    writes = [e for e in dec_events if e[0] == "write"]
    slots = np.concatenate([e[1] for e in writes])
    rows = np.concatenate([e[2] for e in writes])
    step_write = WriteBatch(slots, rows, rows_k, rows_v)
    if copies:  # copy-on-write caused by the decode tokens happens before the timed steps
        apply_events(pool0, copies, rows_k, rows_v)
    del rows_k, rows_v
    pools = [pool0] + [pkv.KVPool(pool0.k.clone(), pool0.v.clone()) for _ in range(args.replicas - 1)]
    tables, lens = alloc.batch_tables(wl.decode_seqs)
    tables_d = torch.from_numpy(tables).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    q = dev(wl.q)
    S, Hq = len(wl.decode_seqs), wl.num_q_heads
    plans = [pkv.DecodePlan(p, S, Hq, args.workers) for p in pools]
    torch.cuda.synchronize()
    log(f"set-up done in {time.time() - t0:.1f} s")

    kv_bytes = float(lens.astype(np.int64).sum()) * 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        p = pools[i % len(pools)]
        if ev is not None:
            ev[0].record(stream)
        step_write.run(p)
        if ev is not None:
            ev[1].record(stream)
        pkv.decode(q, p, tables_d, lens_d, wl.scale, args.workers, plan=plans[i % len(pools)])
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = t_total * 1e3 / args.steps
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    decode_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    dec_avg_s = float(decode_ms.mean()) * 1e-3

    achieved = kv_bytes / dec_avg_s / 1e9
    traffic = load_traffic(args.workload)
    result = {
        "metric": "paged decode attention: KV GB/s read (% of HBM peak) and decode tokens/s",
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "num_seqs": S, "num_q_heads": Hq,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, "tokens": int(lens.sum()),
                   "kv_bytes_per_step": int(kv_bytes), "pool_replicas": len(pools),
                   "accumulation": "fp32", "decode_workers": args.workers or "default (8 per CU)"},
        "pct_hbm_peak": round(100 * kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "decode_kv_gbps": round(achieved, 2),
        "decode_us": {"mean": round(float(decode_ms.mean()) * 1e3, 2),
                      "p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(decode_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 2)},
        "cache_write_us": round(float(write_ms.mean()) * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "pa_decode (balanced split kernel + LSE combine kernel)"},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
