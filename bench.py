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
MODEL_LAYERS = {"llama13b": 40, "llama70b": 80, "prefix": 40, "cow": 40, "cow504": 40, "beam": 40,
                "tiny": 1, "llama13b_fp8": 40, "llama70b_fp8": 80}

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
    "llama13b_fp8": "LLaMA-13B-shaped decode layer with an FP8 (OCP E4M3) KV cache: 64 seqs, "
                    "40 MHA heads x 128, scale 2^-6 per pool, bf16 q/out, block 16, "
                    "lengths U[1,2048], random placement",
    "llama70b_fp8": "Llama-2-70B-shaped GQA decode layer with an FP8 (OCP E4M3) KV cache: 256 "
                    "seqs, 64 q / 8 KV heads x 128, scale 2^-6 per pool, bf16 q/out, block 16, "
                    "lengths log-uniform [128,8192]",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


KERNEL_SOURCES = {
    "decode": ("decode.hip", "device.h"),
    "cache_ops": ("cache_ops.hip", "device.h"),
    "prefill": ("prefill.hip", "device.h"),
    "prefix_shared": ("prefix.hip", "decode.hip", "device.h"),
}


def kernel_source_hash(kind: str = "decode") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_cache_316_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kind: str = "decode"):
    """HBM bytes per call from committed rocprofv3 PMC runs, if they were taken on
    the current kernel sources; else None."""
    name = f"traffic_{workload}.json" if kind == "decode" else f"traffic_{kind}_{workload}.json"
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return t.get("bytes_per_call", t.get("bytes_per_decode_call"))


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, sequence by sequence through the batch (starting
    over when it is done) until ~budget_s have passed."""
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
    n, tokens = 0, 0
    with ctx:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            s = n % len(lens)
            decode_out(wl, [s])
            tokens += int(lens[s])
            n += 1
    dt = time.perf_counter() - t0
    nbytes = float(tokens) * per_tok
    passes = n / len(lens)
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} sequence decodes ({passes:.2f} passes over the {len(lens)} "
                      f"sequences of the batch, {tokens} cached tokens read, all "
                      f"{wl.num_q_heads} heads), fp64 NumPy, {dt:.1f} s; "
                      f"tokens/s = {n / dt:.3f}",
            "tokens_per_s": round(n / dt, 4), "seconds": round(dt, 3),
            "os_cpu_count": os.cpu_count()}


class Loaded:
    """A workload set up on the GPU through the library, ready for timed steps."""

    def __init__(self, name, replicas):
        import numpy as np
        import torch

        import paged_kv_cache_316_amd as pkv
        import workloads
        from paged_kv_cache_316_amd.runner import WriteBatch, apply_events, run_script, split_phases

        t0 = time.time()
        self.name = name
        wl = self.wl = workloads.make(name, "full")
        log(f"workload {name}: {len(wl.decode_seqs)} seqs, drawn in {time.time() - t0:.1f} s")
        self.dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

        def dev(a):
            if wl.dtype == "f32":
                return torch.from_numpy(np.ascontiguousarray(a)).cuda()
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(self.dt)

        # set-up through the library: allocator -> copies / cache writes (untimed)
        alloc = pkv.BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
        phases = split_phases(run_script(alloc, wl.ops))
        rows_k, rows_v = dev(wl.rows_k), dev(wl.rows_v)
        pool_dt = {"f32": torch.float32, "bf16": torch.bfloat16,
                   "fp8_e4m3": torch.float8_e4m3fn}[wl.pool_dtype]
        pool0 = pkv.KVPool.empty(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, pool_dt,
                                 k_scale=wl.k_scale, v_scale=wl.v_scale)
        apply_events(pool0, phases.get("setup", []), rows_k, rows_v)

        def batch(events):
            w = [e for e in events if e[0] == "write"]
            return WriteBatch(np.concatenate([e[1] for e in w]), np.concatenate([e[2] for e in w]),
                              rows_k, rows_v)

        # the prefill chunk writes (if any) are a timed step of their own
        self.prefill_write = batch(phases["prefill"]) if phases.get("prefill") else None
        if self.prefill_write is not None:
            self.prefill_write.run(pool0)
        dec_events = phases["decode"]
        self.decode_write = batch(dec_events)
        copies = [e for e in dec_events if e[0] == "copy"]
        if copies:  # copy-on-write caused by the decode tokens happens before the timed steps
            apply_events(pool0, copies, rows_k, rows_v)
        self.decode_write.run(pool0)
        del rows_k, rows_v
        self.pools = [pool0] + [pkv.KVPool(pool0.k.clone(), pool0.v.clone(), wl.k_scale, wl.v_scale)
                                for _ in range(replicas - 1)]
        tables, lens = alloc.batch_tables(wl.decode_seqs)
        self.lens = lens
        self.tables_d = torch.from_numpy(tables).cuda()
        self.lens_d = torch.from_numpy(lens).cuda()
        self.q = dev(wl.q)
        if wl.prefill_seqs:
            C = wl.prefill_len
            idx = [wl.decode_seqs.index(x) for x in wl.prefill_seqs]
            self.p_tables = self.tables_d[torch.tensor(idx, device="cuda")].contiguous()
            p_lens = np.array([int(wl.prefill_start[j]) + C for j in range(len(idx))], np.int64)
            self.p_lens_d = torch.from_numpy(p_lens.astype(np.int32)).cuda()
            self.p_loc = torch.arange(0, (len(idx) + 1) * C, C, dtype=torch.int32, device="cuda")
            self.p_q = dev(wl.prefill_q)
            # visible keys summed over chunk rows: row i of a chunk ending at P sees P - C + i + 1
            self.p_keys = int(sum(C * (P - C) + C * (C + 1) // 2 for P in p_lens))
        torch.cuda.synchronize()
        log(f"set-up done in {time.time() - t0:.1f} s")

    @property
    def kv_bytes(self):
        wl = self.wl
        return float(self.lens.astype("int64").sum()) * 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes


def _stats_us(ms):
    import numpy as np
    return {"samples": int(len(ms)), "mean": round(float(ms.mean()) * 1e3, 2),
            "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
            "p50": round(float(np.percentile(ms, 50)) * 1e3, 2),
            "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)}


EVENT_SAMPLES = 60  # event-recorded calls per row, in a pass of their own
# Extra rows run a few tens of steps right after seconds of host-side set-up
# with the GPU idle; measured that way the shortest of them (the FP8 decode,
# ~10 ms of work in all) read 8 % slow against the same call after a longer
# run of steps. Their warmup therefore also lasts at least this long. The
# main row keeps exactly --warmup steps.
EXTRA_ROW_WARM_S = 0.25
_warm_s = 0.0


def time_steps(step, steps, warmup, event_samples=EVENT_SAMPLES):
    """Run warmup steps (at least `warmup`, and for the extra rows at least
    _warm_s seconds of them), then exactly `steps` timed steps bracketed by
    synchronisation, with no events among them. Then, in a separate pass,
    `event_samples` more steps that each record 3 events on the launch stream
    (before, between the step's two calls, after): the per-call durations are
    taken from those. (An event record costs about 3 us of stream time on this
    device, so the timed steps carry none.)"""
    import numpy as np
    import torch
    for i in range(warmup):
        step(i, None)
    torch.cuda.synchronize()
    if _warm_s > 0:
        t0, i = time.perf_counter(), warmup
        while time.perf_counter() - t0 < _warm_s:
            for _ in range(8):
                step(i, None)
                i += 1
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(i, None)
    torch.cuda.synchronize()
    total = time.perf_counter() - t_start
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(event_samples)]
    for k in range(event_samples):
        step(steps + k, evs[k])
    torch.cuda.synchronize()
    first = np.array([e[0].elapsed_time(e[1]) for e in evs])
    second = np.array([e[1].elapsed_time(e[2]) for e in evs])
    return total * 1e3 / steps, first, second


def decode_step_fn(ld, workers):
    import torch
    import paged_kv_cache_316_amd as pkv
    S, Hq = len(ld.wl.decode_seqs), ld.wl.num_q_heads
    plans = [pkv.DecodePlan(p, S, Hq, workers) for p in ld.pools]
    stream = torch.cuda.current_stream()

    def step(i, ev):
        p = ld.pools[i % len(ld.pools)]
        if ev is not None:
            ev[0].record(stream)
        ld.decode_write.run(p)
        if ev is not None:
            ev[1].record(stream)
        pkv.decode(ld.q, p, ld.tables_d, ld.lens_d, ld.wl.scale, workers, plan=plans[i % len(ld.pools)])
        if ev is not None:
            ev[2].record(stream)
    return step


def prefill_step_fn(ld):
    import torch
    import paged_kv_cache_316_amd as pkv
    out = torch.empty_like(ld.p_q)
    stream = torch.cuda.current_stream()

    def step(i, ev):
        p = ld.pools[i % len(ld.pools)]
        if ev is not None:
            ev[0].record(stream)
        ld.prefill_write.run(p)
        if ev is not None:
            ev[1].record(stream)
        pkv.prefill_chunk(ld.p_q, ld.p_loc, ld.p_lens_d, p, ld.p_tables, ld.wl.prefill_len,
                          ld.wl.scale, out=out)
        if ev is not None:
            ev[2].record(stream)
    return step


def unique_kv_bytes(ld):
    """Bytes of the distinct physical blocks the batch reads (each block's
    filled tokens once), against the logical bytes of the per-sequence reads."""
    import numpy as np
    wl = ld.wl
    B = wl.block_size
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes
    tables = ld.tables_d.cpu().numpy()
    filled = {}
    for i, L in enumerate(ld.lens):
        L = int(L)
        for j in range(-(-L // B)):
            b = int(tables[i, j])
            filled[b] = max(filled.get(b, 0), min(B, L - j * B))
    return float(sum(filled.values())) * per_tok


GROUP_SIZE = {"cow": 3, "cow504": 3, "beam": 4}  # samples per prompt, beam width


def shared_block_row(ld, steps, warmup, workers):
    """A batch of forked sequences (parallel samples, beams): plain pa_decode,
    which reads every shared block once per sequence, beside pa_decode_grouped,
    which reads a group's common blocks once for the group. Unique bytes: each
    distinct physical block's filled tokens once."""
    import numpy as np
    import torch
    import paged_kv_cache_316_amd as pkv
    wl = ld.wl
    row = decode_row(ld, steps, warmup, workers)
    uniq = unique_kv_bytes(ld)
    t = row["decode_us"]["mean"] * 1e-6
    # grouped: the shared prefix of each group from the host tables
    M = GROUP_SIZE[ld.name]
    S = len(wl.decode_seqs)
    pl = pkv.group_prefix_lens(ld.tables_d.cpu().numpy(), ld.lens, M, wl.block_size)
    pl_d = torch.from_numpy(pl).cuda()
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes
    grouped_bytes = float(pl[::M].astype(np.int64).sum() +
                          (ld.lens.astype(np.int64) - pl).sum()) * per_tok
    out = torch.empty_like(ld.q)
    ws = torch.empty(pkv.decode_grouped_workspace_bytes(S, wl.num_q_heads, wl.num_kv_heads,
                                                        wl.head_dim, workers),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, ev):
        p = ld.pools[i % len(ld.pools)]
        if ev is not None:
            ev[0].record(stream)
        ld.decode_write.run(p)
        if ev is not None:
            ev[1].record(stream)
        pkv.decode_grouped(ld.q, p, ld.tables_d, ld.lens_d, pl_d, M, wl.scale, workers, out=out,
                           workspace=ws)
        if ev is not None:
            ev[2].record(stream)
    ms_step, _, g_ms = time_steps(step, steps, warmup)
    tg = float(g_ms.mean()) * 1e-3
    return {"workload": WORKLOAD_TEXT[ld.name], "num_seqs": S, "group_size": M,
            "logical_kv_bytes": int(ld.kv_bytes), "unique_kv_bytes": int(uniq),
            "grouped_kv_bytes": int(grouped_bytes),
            "shared_read_share": round(1 - uniq / ld.kv_bytes, 4),
            "plain_decode": {"ms_per_step": row["ms_per_step"], "decode_us": row["decode_us"],
                             "logical_kv_gbps": round(ld.kv_bytes / t / 1e9, 2),
                             "unique_kv_gbps": round(uniq / t / 1e9, 2)},
            "grouped_decode": {"ms_per_step": round(ms_step, 5),
                               "tokens_per_s": round(S / (ms_step * 1e-3), 1),
                               "decode_us": _stats_us(g_ms),
                               "grouped_kv_gbps": round(grouped_bytes / tg / 1e9, 2),
                               "unique_kv_gbps": round(uniq / tg / 1e9, 2),
                               "logical_kv_gbps": round(ld.kv_bytes / tg / 1e9, 2)},
            "speedup_grouped_vs_plain": round(t / tg, 3),
            "roofline": {"bound": "hbm", "achieved": round(uniq / tg / 1e9, 2),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(uniq / tg / 1e9 / HBM_PEAK_GBPS, 4),
                         "kernel": "pa_decode_grouped (grouped MFMA decode + LSE combine)",
                         "note": "achieved on the batch's unique physical bytes; the grouped "
                                 "call itself must read grouped_kv_bytes (a group's common "
                                 "blocks once, each member's later blocks once)"}}


def shared_prefix_blocks(ld):
    """Blocks every table row starts with (the prefix-cache hits), checked on the host."""
    wl = ld.wl
    P = wl.meta["prefix_tokens"] // wl.block_size
    t = ld.tables_d.cpu().numpy()
    if not ((t[:, :P] == t[0, :P]).all() and (ld.lens >= P * wl.block_size).all()):
        raise RuntimeError("workload rows do not share their first blocks")
    return P


def shared_prefix_step_fn(ld, workers, P):
    import torch
    import paged_kv_cache_316_amd as pkv
    wl = ld.wl
    S = len(wl.decode_seqs)
    out = torch.empty_like(ld.q)
    n = pkv.decode_shared_prefix_workspace_bytes(S, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                 wl.block_size, P, workers)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, ev):
        p = ld.pools[i % len(ld.pools)]
        if ev is not None:
            ev[0].record(stream)
        ld.decode_write.run(p)
        if ev is not None:
            ev[1].record(stream)
        pkv.decode_shared_prefix(ld.q, p, ld.tables_d, ld.lens_d, P, wl.scale, workers, out=out,
                                 workspace=ws)
        if ev is not None:
            ev[2].record(stream)
    return step


def shared_prefix_row(ld, steps, warmup, workers):
    """The prefix-cached batch through pa_decode_shared_prefix, beside pa_decode
    on the same batch. Unique bytes: the shared blocks once plus every tail."""
    wl = ld.wl
    P = shared_prefix_blocks(ld)
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes
    Lp = P * wl.block_size
    unique = float(Lp + (ld.lens.astype("int64") - Lp).sum()) * per_tok
    plain = decode_row(ld, steps, warmup, workers)
    ms_step, w_ms, d_ms = time_steps(shared_prefix_step_fn(ld, workers, P), steps, warmup)
    t = float(d_ms.mean()) * 1e-3
    achieved = unique / t / 1e9
    S = len(wl.decode_seqs)
    return {"workload": WORKLOAD_TEXT[ld.name], "shared_blocks": P,
            "ms_per_step": round(ms_step, 5), "tokens_per_s": round(S / (ms_step * 1e-3), 1),
            "decode_us": _stats_us(d_ms), "cache_write_us": round(float(w_ms.mean()) * 1e3, 2),
            "logical_kv_bytes": int(ld.kv_bytes), "unique_kv_bytes": int(unique),
            "logical_kv_gbps": round(ld.kv_bytes / t / 1e9, 2),
            "plain_decode": {"ms_per_step": plain["ms_per_step"], "decode_us": plain["decode_us"],
                             "logical_kv_gbps": plain["decode_kv_gbps"],
                             "unique_kv_gbps": round(unique / (plain["decode_us"]["mean"] * 1e-6)
                                                     / 1e9, 2)},
            "speedup_vs_plain_decode": round(plain["decode_us"]["mean"] / (t * 1e6), 3),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic(ld.name, "prefix_shared"),
                         "kernel": "pa_decode_shared_prefix (suffix decode + prefix MFMA pass + merge), "
                                   "unique bytes over the whole call"}}


def mixed_step_inputs(ld):
    """One scheduler step of a workload with prefill chunks: the chunked
    sequences give their chunk rows, every other sequence its decode row
    (decode sequences first)."""
    import torch
    wl = ld.wl
    C = wl.prefill_len
    pre = [wl.decode_seqs.index(x) for x in wl.prefill_seqs]
    dec = [i for i in range(len(wl.decode_seqs)) if i not in pre]
    nd = len(dec)
    order = torch.tensor(dec + pre, device="cuda")
    q = torch.cat([ld.q[order[:nd]], ld.p_q]).contiguous()
    loc = torch.tensor(list(range(nd + 1)) + [nd + C * (j + 1) for j in range(len(pre))],
                       dtype=torch.int32, device="cuda")
    lens = torch.cat([ld.lens_d[order[:nd]], ld.p_lens_d]).contiguous()
    tables = ld.tables_d[order].contiguous()
    return q, loc, lens, tables, nd, dec


def mixed_row(ld, steps, warmup, workers):
    """pa_attention_mixed on one step of the Llama-2-70B-shaped batch: 248
    decode rows and 8 prefill chunks of 512 rows, beside the two separate calls."""
    import numpy as np
    import torch
    import paged_kv_cache_316_amd as pkv
    wl = ld.wl
    q, loc, lens, tables, nd, dec = mixed_step_inputs(ld)
    C = wl.prefill_len
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_bytes(nd, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                workers), dtype=torch.uint8, device="cuda")
    qd, td, lsd = q[:nd].contiguous(), tables[:nd].contiguous(), lens[:nd].contiguous()
    qp, tp, lsp = q[nd:].contiguous(), tables[nd:].contiguous(), lens[nd:].contiguous()
    locp = (loc[nd:] - nd).contiguous()
    dplans = {id(p): pkv.DecodePlan(p, nd, wl.num_q_heads, workers) for p in ld.pools}
    pout = torch.empty_like(qp)
    stream = torch.cuda.current_stream()

    def timed(fn):
        def step(i, ev):
            p = ld.pools[i % len(ld.pools)]
            if ev is not None:
                ev[0].record(stream)
                ev[1].record(stream)
            fn(p)
            if ev is not None:
                ev[2].record(stream)
        return time_steps(step, steps, warmup)[2]  # per-call durations

    m_ms = timed(lambda p: pkv.attention_mixed(q, loc, lens, p, tables, nd, C, wl.scale, workers,
                                               out=out, workspace=ws))
    d_ms = timed(lambda p: pkv.decode(qd, p, td, lsd, wl.scale, workers, plan=dplans[id(p)]))
    p_ms = timed(lambda p: pkv.prefill_chunk(qp, locp, lsp, p, tp, C, wl.scale, out=pout))
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elt_bytes
    kv_bytes = float(ld.lens[dec].astype("int64").sum()) * per_tok
    flops = 4.0 * wl.head_dim * wl.num_q_heads * ld.p_keys
    t = float(m_ms.mean()) * 1e-3
    t_hbm = kv_bytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    rows = nd + len(wl.prefill_seqs) * C
    return {"workload": WORKLOAD_TEXT[ld.name] + "; one step: the 8 chunked sequences give "
                        "512-row chunks, the other 248 their decode row",
            "decode_rows": nd, "prefill_rows": rows - nd, "mixed_us": _stats_us(m_ms),
            "rows_per_s": round(rows / t, 1),
            "separate_calls_us": {"decode": _stats_us(d_ms), "prefill": _stats_us(p_ms),
                                  "sum_mean": round(float(d_ms.mean() + p_ms.mean()) * 1e3, 2)},
            "decode_kv_bytes": int(kv_bytes), "prefill_flops": flops,
            "roofline": {"bound": "hbm+mfma", "ideal_us": round(max(t_hbm, t_mfma) * 1e6, 2),
                         "hbm_us_at_peak": round(t_hbm * 1e6, 2),
                         "mfma_us_at_peak": round(t_mfma * 1e6, 2),
                         "frac": round(max(t_hbm, t_mfma) / t, 4),
                         "note": "ideal = the larger of the decode rows' bytes at 8 TB/s and the "
                                 "chunks' flops at 2.5 PFLOP/s (perfect overlap)"}}


def spec_verify_row(ld, steps, warmup, workers, k=4):
    """Speculative-decoding verification on the Llama-2-70B-shaped batch: every
    sequence checks k draft tokens in one call ("vLLM PagedAttention
    explained" section 7.5, "vLLM inference engine deep dive" section 5.2: the
    target model verifies the draft model's tokens in one pass), its last k
    positions taken as causal chunk rows (section 7.2 of the first page).
    pa_attention_mixed runs such short chunks as one multi-row decode (each
    K/V row read once for all k rows); beside it the same rows on the
    chunked-prefill kernel (bf16 pools only) and the plain decode of the batch
    (one row per sequence)."""
    import numpy as np
    import torch
    import paged_kv_cache_316_amd as pkv
    wl = ld.wl
    S = len(wl.decode_seqs)
    rng = np.random.default_rng(77)
    q = torch.from_numpy(rng.standard_normal((S * k, wl.num_q_heads, wl.head_dim))
                         .astype(np.float32)).to(torch.bfloat16).cuda()
    loc = torch.arange(0, S * k + 1, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(16, pkv.attention_mixed_workspace_bytes(0, S, wl.num_q_heads,
                                                                 wl.num_kv_heads, wl.head_dim, k,
                                                                 workers)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(call):
        def step(i, ev):
            p = ld.pools[i % len(ld.pools)]
            if ev is not None:
                ev[0].record(stream)
                ev[1].record(stream)
            call(p)
            if ev is not None:
                ev[2].record(stream)
        return time_steps(step, steps, warmup)[2]
    v_ms = timed(lambda p: pkv.attention_mixed(q, loc, ld.lens_d, p, ld.tables_d, 0, k, wl.scale,
                                               workers, out=out, workspace=ws))
    # the chunked-prefill kernel reads bf16 pools only
    pf_ms = (None if wl.pool_dtype == "fp8_e4m3" else
             timed(lambda p: pkv.prefill_chunk(q, loc, ld.lens_d, p, ld.tables_d, k, wl.scale,
                                               out=out)))
    _, _, d_ms = time_steps(decode_step_fn(ld, workers), steps, warmup)
    t = float(v_ms.mean()) * 1e-3
    gbps = ld.kv_bytes / t / 1e9
    lens = ld.lens.astype("int64")
    pairs = int(sum(int(L) * k - k * (k - 1) // 2 for L in lens))  # visible (row, key) pairs
    return {"workload": WORKLOAD_TEXT[ld.name] + f"; every sequence verifies {k} draft tokens "
                        "(its last positions as causal chunk rows)",
            "draft_rows_per_seq": k, "verify_us": _stats_us(v_ms),
            "prefill_kernel_path_us": None if pf_ms is None else _stats_us(pf_ms),
            "decode_us": _stats_us(d_ms),
            "verify_over_decode": round(float(v_ms.mean() / d_ms.mean()), 3),
            "kv_bytes": int(ld.kv_bytes), "flops": 4.0 * wl.head_dim * wl.num_q_heads * pairs,
            "draft_tokens_per_s": round(S * k / t, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "kernel": "pa_attention_mixed, multi-row decode (k x G = 32 columns "
                                   "per (sequence, KV head) on a pair of waves sharing each "
                                   "K/V tile in LDS) + combine"}}


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction


def swap_row(ld, reps=5):
    """pa_swap_blocks of a preemption-sized batch of blocks (the longest
    sequences' blocks until 1024 blocks, ~335 MB) out to a pinned host pool and
    back in, beside one contiguous device<->pinned copy of the same bytes by
    the copy engine (torch's copy_)."""
    import numpy as np
    import torch
    import paged_kv_cache_316_amd as pkv
    wl = ld.wl
    tables = ld.tables_d.cpu().numpy()
    B = wl.block_size
    blocks = []
    for i in np.argsort(-ld.lens):
        blocks += [int(b) for b in tables[i, :-(-int(ld.lens[i]) // B)]]
        if len(blocks) >= 1024:
            break
    blocks = sorted(set(blocks))[:1024]
    n = len(blocks)
    pool = ld.pools[0]
    host = pkv.KVPool.empty_host(n, wl.num_kv_heads, B, wl.head_dim, pool.dtype)
    out_pairs = np.array([(b, j) for j, b in enumerate(blocks)], dtype=np.int32)
    in_pairs = out_pairs[:, ::-1].copy()
    block_bytes = 2 * wl.num_kv_heads * B * wl.head_dim * pool.k.element_size()
    nbytes = n * block_bytes
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    t_out = timed(lambda: pkv.swap_out(pool, host, out_pairs))
    t_in = timed(lambda: pkv.swap_in(pool, host, in_pairs))
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hbuf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    t_d2h = timed(lambda: hbuf.copy_(dbuf, non_blocking=True))
    t_h2d = timed(lambda: dbuf.copy_(hbuf, non_blocking=True))
    del dbuf, hbuf, host
    gbps = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    return {"blocks": n, "bytes": nbytes, "block_bytes": block_bytes,
            "swap_out_ms": round(t_out, 3), "swap_in_ms": round(t_in, 3),
            "swap_out_gbps": gbps(t_out), "swap_in_gbps": gbps(t_in),
            "copy_engine_contiguous_gbps": {"d2h": gbps(t_d2h), "h2d": gbps(t_h2d)},
            "roofline": {"bound": "host link", "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                         "frac_out": round(gbps(t_out) / HOST_LINK_PEAK_GBPS, 4),
                         "frac_in": round(gbps(t_in) / HOST_LINK_PEAK_GBPS, 4),
                         "note": "peak = PCIe 5.0 x16 per direction; the copy engine's contiguous "
                                 "rate is the practical ceiling"}}


def stream_read_ceiling(gib: int = 4):
    """Best streaming-read rate (GB/s) of pa_probe_stream_read over a few grid sizes."""
    import torch
    import paged_kv_cache_316_amd as pkv
    buf = torch.ones(gib << 28, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best, best_grid = 0.0, 0
    stream = torch.cuda.current_stream()
    for grid in (4 * cus, 8 * cus, 16 * cus, 32 * cus):
        pkv.probe_stream_read(buf, sink, grid)
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.probe_stream_read(buf, sink, grid)
            e1.record(stream)
            e1.synchronize()
            gbps = buf.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbps > best:
                best, best_grid = gbps, grid
    del buf
    torch.cuda.empty_cache()
    return {"gbps": round(best, 1), "grid": best_grid, "bytes": gib << 30,
            "kernel": "pa_probe_stream_read (16-byte non-temporal loads, 8 KB contiguous runs per wave, 8 in flight per lane)"}


class Relaid:
    """The decode batch of a loaded workload laid out again: the same sequences
    and K/V values in a new pool of another block size and/or placement,
    optionally only the first kv_heads KV heads (and their query heads). Set
    up through the library: its block allocator gives the slots (distinct
    token ids per sequence, so no block is shared by the prefix hash) and
    pa_cache_write stores the rows."""

    def __init__(self, ld, block_size, placement="random", kv_heads=None, replicas=2, seed=7):
        import math
        import numpy as np
        import torch
        import paged_kv_cache_316_amd as pkv
        wl = ld.wl
        self.wl, self.block_size, self.placement = wl, block_size, placement
        B = block_size
        lens = ld.lens.astype(np.int64)
        S = len(lens)
        Hkv = kv_heads or wl.num_kv_heads
        G = wl.num_q_heads // wl.num_kv_heads
        self.num_kv_heads, self.num_q_heads = Hkv, Hkv * G
        need = int(sum(-(-int(L) // B) for L in lens))
        if placement == "contiguous":  # FIFO from 0, 1, 2, ...: each sequence's blocks in order
            num_blocks, order = need, np.arange(need, dtype=np.int32)
        else:
            num_blocks = int(math.ceil(1.1 * need))
            order = np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)
        alloc = pkv.BlockAllocator(num_blocks, B, order)
        slots, rows = [], []
        for i, seq in enumerate(wl.decode_seqs):
            L = int(lens[i])
            _, sl = alloc.allocate(i, (np.arange(L) + (i << 16)).astype(np.int32))
            slots.append(sl)
            rows.append(np.asarray(wl.hist[seq][:L]))
        slots, rows = np.concatenate(slots), np.concatenate(rows)
        pool_dt = {"f32": torch.float32, "bf16": torch.bfloat16,
                   "fp8_e4m3": torch.float8_e4m3fn}[wl.pool_dtype]
        pool = pkv.KVPool.empty(num_blocks, Hkv, B, wl.head_dim, pool_dt,
                                k_scale=wl.k_scale, v_scale=wl.v_scale)
        for a in range(0, len(slots), 1 << 15):
            r = rows[a:a + (1 << 15)]
            k = np.ascontiguousarray(wl.rows_k[r][:, :Hkv])
            v = np.ascontiguousarray(wl.rows_v[r][:, :Hkv])
            dev = (lambda x: torch.from_numpy(x).cuda()) if wl.dtype == "f32" else \
                  (lambda x: torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16))
            pkv.cache_write(pool, dev(k), dev(v), torch.from_numpy(slots[a:a + (1 << 15)]).cuda())
        self.pools = [pool] + [pkv.KVPool(pool.k.clone(), pool.v.clone(), wl.k_scale, wl.v_scale)
                               for _ in range(replicas - 1)]
        tables, lens32 = alloc.batch_tables(list(range(S)))
        self.lens = lens32
        self.tables_d = torch.from_numpy(tables).cuda()
        self.lens_d = torch.from_numpy(lens32).cuda()
        self.q = ld.q[:, :self.num_q_heads].contiguous()
        self.per_tok = 2 * Hkv * wl.head_dim * wl.elt_bytes
        self.kv_bytes = float(lens.sum()) * self.per_tok
        self.waste_bytes = float(sum(-(-int(L) // B) * B - int(L) for L in lens)) * self.per_tok
        self.pool_bytes = float(num_blocks) * B * self.per_tok
        torch.cuda.synchronize()

    def decode_time(self, steps, warmup, workers):
        import torch
        import paged_kv_cache_316_amd as pkv
        S = len(self.lens)
        plans = [pkv.DecodePlan(p, S, self.num_q_heads, workers) for p in self.pools]
        stream = torch.cuda.current_stream()

        def step(i, ev):
            j = i % len(self.pools)
            if ev is not None:
                ev[0].record(stream)
                ev[1].record(stream)
            pkv.decode(self.q, self.pools[j], self.tables_d, self.lens_d, self.wl.scale, workers,
                       plan=plans[j])
            if ev is not None:
                ev[2].record(stream)
        ms_step, _, d_ms = time_steps(step, steps, warmup)
        return ms_step, d_ms, plans[0].out


def layout_rows(ld, steps, warmup, workers):
    """The pages' two kernel claims on the LLaMA-13B-shaped batch: paged access
    costs little against contiguous storage ("LLM inference engine internals",
    section 2.4, closing paragraph), and small blocks read less efficiently
    while large ones waste the unused part of each sequence's last block
    ("vLLM PagedAttention explained", section 8.1). The same sequences and
    values are laid out with 8-, 16-, 32- and 64-token blocks at random
    placement, and with 16-token blocks in order (each sequence's blocks
    consecutive in the pool)."""
    import gc
    import torch
    rows, base_out, times = {}, None, {}
    for B, placement in ((16, "random"), (16, "contiguous"), (8, "random"), (32, "random"),
                         (64, "random")):
        r = Relaid(ld, B, placement)
        ms_step, d_ms, out = r.decode_time(steps, warmup, workers)
        t = float(d_ms.mean()) * 1e-3
        times[(B, placement)] = t
        out = out.clone()
        if base_out is None:
            base_out = out
        gbps = r.kv_bytes / t / 1e9
        name = ("decode_llama13b_contiguous" if placement == "contiguous"
                else f"decode_llama13b_B{B}")
        rows[name] = {
            "block_size": B, "placement": placement, "decode_us": _stats_us(d_ms),
            "kv_bytes": int(r.kv_bytes), "decode_kv_gbps": round(gbps, 2),
            "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "last_block_waste_bytes": int(r.waste_bytes),
            "last_block_waste_pct_of_pool_use": round(100 * r.waste_bytes /
                                                      (r.kv_bytes + r.waste_bytes), 3),
            "pool_bytes": int(r.pool_bytes),
            # the kernels' arithmetic depends only on logical positions (16-token
            # tiles), so every layout gives the same bits
            "output_bitwise_equal_to_B16_random": bool(torch.equal(out.view(torch.int16),
                                                                   base_out.view(torch.int16)))}
        del r
        gc.collect()
        torch.cuda.empty_cache()
    t_rand, t_cont = times[(16, "random")], times[(16, "contiguous")]
    rows["decode_llama13b_contiguous"]["paged_random_vs_contiguous_overhead_pct"] = \
        round(100 * (t_rand / t_cont - 1), 2)
    return rows


def tp_shard_row(ld, steps, warmup, workers):
    """One GPU's share of the Llama-2-70B-shaped layer under 4-way tensor
    parallelism as the pages describe it ("vLLM PagedAttention explained",
    section 6: every GPU holds the same block tables and its own heads' KV):
    16 query and 2 KV heads, the same sequences and tables."""
    r = Relaid(ld, ld.wl.block_size, "random", kv_heads=ld.wl.num_kv_heads // 4)
    ms_step, d_ms, _ = r.decode_time(steps, warmup, workers)
    t = float(d_ms.mean()) * 1e-3
    gbps = r.kv_bytes / t / 1e9
    return {"workload": "Llama-2-70B-shaped layer, one of 4 tensor-parallel shards: 256 seqs, "
                        "16 q / 2 KV heads x 128, bf16, block 16, lengths log-uniform [128,8192]",
            "num_q_heads": r.num_q_heads, "num_kv_heads": r.num_kv_heads,
            "decode_us": _stats_us(d_ms), "kv_bytes": int(r.kv_bytes),
            "decode_kv_gbps": round(gbps, 2), "tokens_per_s": round(len(r.lens) / t, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}}


def decode_row(ld, steps, warmup, workers, path="plain"):
    step = (decode_step_fn(ld, workers) if path == "plain"
            else shared_prefix_step_fn(ld, workers, shared_prefix_blocks(ld)))
    ms_step, w_ms, d_ms = time_steps(step, steps, warmup)
    S = len(ld.wl.decode_seqs)
    t = float(d_ms.mean()) * 1e-3
    # the shared-prefix call reads the common blocks once: its roofline is
    # taken on those unique bytes (the logical rate is reported beside it)
    algo_bytes = ld.kv_bytes if path == "plain" else unique_kv_bytes(ld)
    achieved = algo_bytes / t / 1e9
    extra = {} if path == "plain" else {"unique_kv_bytes": int(algo_bytes),
                                        "logical_kv_gbps": round(ld.kv_bytes / t / 1e9, 2)}
    return {**extra, "ms_per_step": round(ms_step, 5),
            "kv_gbps_step": round(ld.kv_bytes / (ms_step * 1e-3) / 1e9, 2),
            "tokens_per_s": round(S / (ms_step * 1e-3), 1),
            "decode_kv_gbps": round(achieved, 2),
            "decode_us": _stats_us(d_ms), "cache_write_us": round(float(w_ms.mean()) * 1e3, 2),
            "kv_bytes_per_step": int(ld.kv_bytes), "tokens": int(ld.lens.sum()),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "traffic": (load_traffic(ld.name) if path == "plain"
                                     else load_traffic(ld.name, "prefix_shared")),
                         "kernel": "pa_decode (balanced split kernel + LSE combine kernel)"
                                   if path == "plain" else
                                   "pa_decode_shared_prefix (tail decode + prefix pass + merge), "
                                   "unique bytes over the whole call"}}


def prefill_row(ld, steps, warmup):
    ms_step, w_ms, p_ms = time_steps(prefill_step_fn(ld), steps, warmup)
    wl = ld.wl
    flops = 4.0 * wl.head_dim * wl.num_q_heads * ld.p_keys
    tflops = flops / (float(p_ms.mean()) * 1e-3) / 1e12
    rows = len(wl.prefill_seqs) * wl.prefill_len
    return {"chunks": len(wl.prefill_seqs), "rows_per_chunk": wl.prefill_len,
            "ms_per_step": round(ms_step, 5), "prefill_us": _stats_us(p_ms),
            "cache_write_us": round(float(w_ms.mean()) * 1e3, 2),
            "flops_per_call": flops, "prefill_tokens_per_s": round(rows / (ms_step * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": load_traffic(ld.name, "prefill"),
                         "kernel": "pa_prefill_chunk (bf16 MFMA 32x32x16)"}}


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
    ap.add_argument("--no-extra-rows", action="store_true",
                    help="skip the Llama-2-70B-shaped GQA decode, chunked-prefill, mixed-step, "
                         "speculative-verification, FP8-KV decode, block-swap, block-layout, "
                         "tensor-parallel-shard, shared-block and shared-prefix decode rows")
    ap.add_argument("--rows", default="",
                    help="comma-separated extra rows to run (default: all), e.g. "
                         "prefill_llama70b,swap_llama13b")
    ap.add_argument("--decode-path", default="plain", choices=("plain", "shared-prefix"),
                    help="entry point the main row times: pa_decode, or pa_decode_shared_prefix "
                         "(prefix workload only)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(decode shards by sequences or heads with no exchange inside attention).",
              file=sys.stderr)
        sys.exit(2)

    import gc

    import torch

    torch.cuda.set_device(0)
    ld = Loaded(args.workload, args.replicas)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.decode_path == "shared-prefix" and args.workload != "prefix":
        print("--decode-path shared-prefix needs --workload prefix", file=sys.stderr)
        sys.exit(2)
    row = decode_row(ld, args.steps, args.warmup, args.workers, args.decode_path)
    ceiling = stream_read_ceiling()
    wl = ld.wl
    S = len(wl.decode_seqs)
    result = {
        "metric": "paged decode attention: KV GB/s read (% of HBM peak) and decode tokens/s",
        "value": row["kv_gbps_step"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": row["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "num_seqs": S,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "tokens": row["tokens"],
                   "kv_bytes_per_step": row["kv_bytes_per_step"], "pool_replicas": args.replicas,
                   "accumulation": "fp32", "decode_workers": args.workers or "default (8 per CU)",
                   "decode_path": args.decode_path},
        "pct_hbm_peak": round(100 * row["kv_gbps_step"] / HBM_PEAK_GBPS, 2),
        "tokens_per_s": row["tokens_per_s"],
        "tokens_per_s_model_equiv": {"layers": MODEL_LAYERS[args.workload],
                                     "value": round(row["tokens_per_s"] / MODEL_LAYERS[args.workload], 1),
                                     "note": "attention-only: one layer's step time x layers"},
        "decode_kv_gbps": row["decode_kv_gbps"],
        "decode_us": row["decode_us"],
        "cache_write_us": row["cache_write_us"],
        "roofline": row["roofline"],
        "kernel_source_hash": kernel_source_hash(),
        "stream_read_ceiling": ceiling,
        "pct_of_stream_ceiling": round(100 * row["decode_kv_gbps"] / ceiling["gbps"], 2),
        "prefill_source_hash": kernel_source_hash("prefill"),
        "cache_ops_source_hash": kernel_source_hash("cache_ops"),
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    if not args.no_extra_rows:
        wanted = set(args.rows.split(",")) if args.rows else None
        rows = {}

        def want(name):
            return wanted is None or name in wanted

        def switch(name, replicas=args.replicas):
            nonlocal ld
            if ld is not None and ld.name == name:
                return
            ld = None
            gc.collect()
            torch.cuda.empty_cache()
            ld = Loaded(name, replicas)

        global _warm_s
        _warm_s = EXTRA_ROW_WARM_S
        short = max(20, args.steps // 4)
        if want("swap_llama13b"):
            switch("llama13b", 1)
            rows["swap_llama13b"] = swap_row(ld)
            rows["swap_llama13b"]["workload"] = (
                "preemption by swapping: the longest sequences' blocks of the LLaMA-13B-shaped "
                "batch, up to 1024 blocks of 16 tokens x 40 heads x 128, bf16")
        if want("decode_llama70b_gqa") and args.workload != "llama70b":
            switch("llama70b")
            g = rows["decode_llama70b_gqa"] = decode_row(ld, short, args.warmup, args.workers)
            g["tokens_per_s_model_equiv"] = round(g["tokens_per_s"] / MODEL_LAYERS["llama70b"], 1)
            g["pct_of_stream_ceiling"] = round(100 * g["decode_kv_gbps"] / ceiling["gbps"], 2)
        if want("prefill_llama70b"):
            switch("llama70b")
            rows["prefill_llama70b"] = prefill_row(ld, max(10, args.steps // 10),
                                                   min(args.warmup, 5))
            rows["workload_llama70b"] = (WORKLOAD_TEXT["llama70b"] +
                                         "; prefill: 8 x 512-row causal chunks")
        if want("mixed_llama70b_step"):
            switch("llama70b")
            rows["mixed_llama70b_step"] = mixed_row(ld, max(10, args.steps // 10),
                                                    min(args.warmup, 5), args.workers)
        if want("spec_verify_llama70b"):
            switch("llama70b")
            rows["spec_verify_llama70b"] = spec_verify_row(ld, short, min(args.warmup, 5),
                                                           args.workers)
        if want("spec_verify_llama70b_fp8"):
            switch("llama70b_fp8")
            rows["spec_verify_llama70b_fp8"] = spec_verify_row(ld, short, min(args.warmup, 5),
                                                               args.workers)
        if want("decode_llama13b_fp8") and args.workload != "llama13b_fp8":
            switch("llama13b_fp8")
            f = rows["decode_llama13b_fp8"] = decode_row(ld, short, args.warmup, args.workers)
            f["tokens_per_s_model_equiv"] = round(f["tokens_per_s"] / MODEL_LAYERS["llama13b_fp8"], 1)
            f["pct_of_stream_ceiling"] = round(100 * f["decode_kv_gbps"] / ceiling["gbps"], 2)
            f["workload"] = WORKLOAD_TEXT["llama13b_fp8"]
        if any(want(n) for n in ("decode_llama13b_contiguous", "decode_llama13b_B8",
                                 "decode_llama13b_B16", "decode_llama13b_B32",
                                 "decode_llama13b_B64", "layouts")):
            switch("llama13b", 1)
            rows.update(layout_rows(ld, short, args.warmup, args.workers))
        if want("decode_llama70b_tp4_shard"):
            switch("llama70b", 1)
            rows["decode_llama70b_tp4_shard"] = tp_shard_row(ld, short, args.warmup, args.workers)
        for name in ("cow", "cow504", "beam"):  # shared blocks, plain decode
            if want(f"decode_{name}"):
                switch(name)
                rows[f"decode_{name}"] = shared_block_row(ld, short, args.warmup, args.workers)
        if want("decode_prefix_shared"):
            switch("prefix")
            rows["decode_prefix_shared"] = shared_prefix_row(ld, short, args.warmup, args.workers)
        result["rows"] = rows
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
