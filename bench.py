#!/usr/bin/env python3
"""Paged attention throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM: for the decode workloads one ``paged_attn_decode``
call per layer (block-table walk, K/V gather, QK, online softmax, PV,
partition merge), for the multi-token workloads one ``paged_attn_multiq`` call.
Several replicas of the K/V pool are rotated between steps so that the 256 MB
Infinity Cache cannot serve a step from the previous one's reads.

Prints ONE JSON line: throughput on algorithmic KV bytes (every visible token's
K and V read once: sum_s L_s * 2 * Hk * D * elem), tokens/s, the roofline of
the dominant launch (timed live with HIP events on the launch stream) and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (KV bytes) + % of peak; tokens/s"
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
DECODE = ("llama3_8b_decode", "llama3_70b_decode", "shared_prefix_mix", "tiny_fp32")
MULTIQ = ("spec_verify", "chunked_prefill")
APPEND = ("kv_append",)
APPEND_METRIC = "paged KV append: achieved HBM GB/s (new K/V read + written)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="llama3_8b_decode", choices=DECODE + MULTIQ + APPEND)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=None,
                    help="K/V pool replicas rotated between steps (default: >= 2 GiB in total)")
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library's)")
    ap.add_argument("--layers", type=int, default=None, help="override layer count (70B workload)")
    ap.add_argument("--kv-dtype", default=None, choices=("fp8",),
                    help="decode workloads: keep the K/V pools as 8-bit E4M3 codes "
                         "(paged_attn_decode_fp8kv, unit scales) instead of bf16")
    ap.add_argument("--cascade", action="store_true",
                    help="shared_prefix_mix: attend the shared prefix once for all sequences "
                         "(paged_attn_decode_shared_prefix) instead of per sequence")
    ap.add_argument("--block-size", type=int, default=None,
                    help="tokens per block for the Llama-3-8B decode workload (default 16)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM counters) and exit")
    ap.add_argument("--hbm-read", type=float, default=None, metavar="GIB",
                    help="only time plain streaming reads of a GIB-GiB buffer (the device's "
                         "HBM read ceiling, paged_hbm_read) and exit")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workload set-up
# ---------------------------------------------------------------------------

def make_structure(name, seed, layers, block_size=None):
    from paged_kv_cache_289_amd import workloads as W
    if block_size is not None:
        if name != "llama3_8b_decode":
            raise SystemExit("--block-size applies to the llama3_8b_decode workload only")
        return W.llama3_8b_decode(seed, block_size=block_size)
    if name == "llama3_70b_decode":
        return W.llama3_70b_decode(seed, layers=layers or 80)
    return W.NAMED[name](seed)


def kv_bytes_of(st) -> int:
    """Algorithmic KV bytes of one call: every visible token's K and V, once."""
    return int(st.context_lens.astype(np.int64).sum()) * 2 * st.num_kv_heads * st.head_dim * \
        st.elem_bytes


def unique_kv_bytes_of(st) -> int:
    """Bytes of distinct (block, slot) pairs the call touches (shared prefixes count once)."""
    seen = set()
    B = st.block_size
    for s in range(st.num_seqs):
        L = int(st.context_lens[s])
        for j in range(-(-L // B)):
            seen.add((int(st.block_tables[s, j]), min(B, L - j * B)))
    tokens = 0
    per_block = {}
    for b, n in seen:
        per_block[b] = max(per_block.get(b, 0), n)
    tokens = sum(per_block.values())
    return tokens * 2 * st.num_kv_heads * st.head_dim * st.elem_bytes


def flops_of(st, causal=True) -> int:
    """QK and PV multiply-adds (2 flops each) over every visible (row, head, key)."""
    tot = 0
    for s in range(st.num_seqs):
        n, L = int(st.q_lens[s]), int(st.context_lens[s])
        vis = sum((L - n + i + 1) if causal else L for i in range(n))
        tot += vis
    return 4 * st.head_dim * st.num_heads * tot


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_289_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, src_hash: str):
    """HBM bytes per launch of the main kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    1 GiB copy), or None when there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# ---------------------------------------------------------------------------

def host_cores() -> int:
    """CPU threads this process may run: its affinity set, capped by a cgroup CPU quota
    when one is set."""
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    return n


def cpu_baseline(st, dv, budget_s, is_multiq, kv_fp8=False):
    """The fp64 oracle, as it stands, on whole sequences of the same workload for about
    ``budget_s`` seconds at one thread and again at every host core (BLAS threads set
    with threadpoolctl); GB/s on the same KV-byte rule as the GPU figure."""
    import oracle.paged_attention as OP
    from paged_kv_cache_289_amd import workloads as W
    from threadpoolctl import threadpool_limits
    vals = {k: W.torch_to_host(v, st.dtype) for k, v in dv.items()}
    per_tok = 2 * st.num_kv_heads * st.head_dim * (1 if kv_fp8 else st.elem_bytes)
    order = list(np.argsort(-st.context_lens))[::max(1, st.num_seqs // 16)] or [0]
    order = list(order) + [s for s in range(st.num_seqs) if s not in order]

    def one(s):
        if is_multiq:
            OP.paged_multiq(vals["q"], vals["k_cache"], vals["v_cache"], st.block_tables,
                            st.context_lens, st.q_offsets, st.block_size, st.scale, st.dtype,
                            seqs=[int(s)])
        elif kv_fp8:
            OP.paged_decode_quant_kv(vals["q"], st.dtype, vals["k_cache"], vals["v_cache"],
                                     "fp8e4m3", 1.0, 1.0, st.block_tables, st.context_lens,
                                     st.block_size, st.scale, seqs=[int(s)])
        else:
            OP.paged_decode(vals["q"], vals["k_cache"], vals["v_cache"], st.block_tables,
                            st.context_lens, st.block_size, st.scale, st.dtype, seqs=[int(s)])

    def timed(threads, budget):
        done, spent, used, passes = 0, 0.0, [], 0
        with threadpool_limits(limits=threads):
            # whole passes over the sequences (the last may stop early) until the budget is spent
            while spent < budget and passes < 50:
                passes += 1
                for s in order:
                    if spent >= budget:
                        break
                    t0 = time.perf_counter()
                    one(s)
                    spent += time.perf_counter() - t0
                    done += int(st.context_lens[s]) * per_tok
                    used.append(int(s))
        gbps = done / spent / 1e9 if spent > 0 else None
        return {"value": round(gbps, 4) if gbps else None, "unit": "GB/s", "cores": threads,
                "kind": "oracle",
                "sample": f"{len(set(used))} of {st.num_seqs} sequences of one layer, "
                          f"{len(used)} sequence calls over {passes} pass(es) "
                          f"({done / 2**20:.1f} MiB of KV) in {spent:.1f} s, fp64 NumPy, "
                          f"{threads} BLAS thread(s)"}

    cores = host_cores()
    single = timed(1, budget_s / 2)
    res = timed(cores, budget_s / 2)
    res["single_thread"] = {k: single[k] for k in ("value", "unit", "cores", "sample")}
    return res


# ---------------------------------------------------------------------------
# KV append (prefill chunks written into their slots)
# ---------------------------------------------------------------------------

def append_bench(a, st):
    """One step = one paged_kv_append call writing every sequence's new chunk.  The
    new rows are rotated among replicas so that the Infinity Cache cannot serve
    a step's reads from the previous one."""
    import torch
    import oracle.kv_cache as OK
    from paged_kv_cache_289_amd import ops, workloads as W
    dev = torch.device("cuda:0")
    T, Hk, D, B = st.total_q, st.num_kv_heads, st.head_dim, st.block_size
    tables = torch.from_numpy(st.block_tables).to(dev)
    lens = torch.from_numpy(st.context_lens).to(dev)
    qoff = torch.from_numpy(st.q_offsets).to(dev)
    dv = W.device_values(st, dev)
    kc, vc = dv["k_cache"], dv["v_cache"]
    new_bytes = 2 * T * Hk * D * st.elem_bytes          # K and V rows of the new tokens
    reps = a.replicas or min(8, max(2, math.ceil(512 * 2**20 / new_bytes)))
    g = torch.Generator(device=dev)
    g.manual_seed(a.seed * 7919 + 11)
    news = [tuple(torch.randn((T, Hk, D), generator=g, device=dev).to(kc.dtype)
                  for _ in range(2)) for _ in range(reps)]
    steps = a.steps if a.steps is not None else 100
    warm = a.warmup if a.warmup is not None else 10
    stream = torch.cuda.current_stream()
    fn = ops.LIB.paged_kv_append
    args = [ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()), None, None,
            ctypes.c_void_p(tables.data_ptr()), ctypes.c_void_p(lens.data_ptr()),
            ctypes.c_void_p(qoff.data_ptr()), st.num_seqs, T, Hk, D, B, st.num_blocks,
            st.block_tables.shape[1], st.max_context_len, ops._dtype(kc),
            ctypes.c_void_p(int(stream.cuda_stream))]
    ptrs = [(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr())) for k, v in news]

    def call(i):
        args[2], args[3] = ptrs[i % reps]
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"paged_kv_append returned {rc}")

    for i in range(warm):
        call(i)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in kev:
        e0.record(stream)
        e1.record(stream)
    kev_ptrs = [(ctypes.c_void_p(e0.cuda_event), ctypes.c_void_p(e1.cuda_event)) for e0, e1 in kev]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):        # the metric: whole calls back to back
        call(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for i in range(steps):        # the roofline: each kernel between dispatch-stamped events
        ops.LIB.paged_attn_set_kernel_events(*kev_ptrs[i])
        call(i)
    torch.cuda.synchronize()
    ops.set_kernel_events(None, None)
    ms_per_step = t0.elapsed_time(t1) / steps
    kernel_ms = np.array([e0.elapsed_time(e1) for e0, e1 in kev])
    algo = 2 * new_bytes                                  # read once, written once
    value = algo / (ms_per_step * 1e-3) / 1e9
    kern = float(kernel_ms.mean())
    ach = algo / (kern * 1e-3) / 1e9
    res = {
        "metric": APPEND_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": st.dtype,
        "data": "synthetic",
        "config": {"workload": st.name, "num_seqs": st.num_seqs, "new_tokens": T,
                   "num_kv_heads": Hk, "head_dim": D, "block_size": B,
                   "pool_blocks": st.num_blocks, "new_row_replicas": reps, "seed": a.seed},
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "kernel_ms": {"mean": round(kern, 5), "p50": round(float(np.median(kernel_ms)), 5)},
        "wall_s_timed": round(wall, 3), "source_hash": source_hash(),
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(st.name, source_hash()),
                     "kernel": "append kernel", "algorithmic_bytes_per_launch": int(algo)},
    }
    if a.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on the whole workload")
        host = {k: W.torch_to_host(v, st.dtype) for k, v in
                (("k", kc), ("v", vc), ("kn", news[0][0]), ("vn", news[0][1]))}
        c0 = time.perf_counter()
        OK.append_kv(host["k"], host["v"], host["kn"], host["vn"], st.block_tables,
                     st.context_lens, st.q_offsets, B)
        spent = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": round(algo / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the whole workload ({T} new tokens) in {spent:.1f} s, "
                                         f"NumPy, one thread (the oracle copies both pools first)"}
    else:
        res["cpu_baseline"] = None
    line = json.dumps(res)
    print(line, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(line + "\n")


# ---------------------------------------------------------------------------
# HBM read ceiling
# ---------------------------------------------------------------------------

def hbm_read_bench(a, dev):
    """K back-to-back plain streaming reads of one buffer (grid-stride cached and
    non-temporal loads, and per-wave runs through direct-to-LDS loads), bracketed
    by events: the read rate this device sustains."""
    import torch
    from paged_kv_cache_289_amd import ops
    n = int(a.hbm_read * 2**30) // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.view(torch.int32).random_(generator=torch.Generator(device=dev).manual_seed(a.seed))
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    steps = a.steps if a.steps is not None else 20
    warm = a.warmup if a.warmup is not None else 3
    stream = torch.cuda.current_stream()
    res = {"metric": "HBM streaming read GB/s (paged_hbm_read)", "unit": "GB/s", "n_gpus": 1,
           "steps": steps, "warmup": warm, "bytes_per_read": n, "peak": PEAK_HBM_GBPS}
    keys = ("cached", "nontemporal", "wave_runs_lds")
    for mode, key in enumerate(keys):
        for _ in range(warm):
            ops.hbm_read(buf, sink, mode=mode, stream=stream)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(steps):
            ops.hbm_read(buf, sink, mode=mode, stream=stream)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        res[key] = {"ms_per_read": round(ms, 4), "GBps": round(n / (ms * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    res["value"] = max(res[k]["GBps"] for k in keys)
    line = json.dumps(res)
    print(line, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(line + "\n")


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the attention "
              f"path shards by KV head or by sequence with no exchange, so one GPU's share "
              f"is the kernel at its real shape).", file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_kv_cache_289_amd import ops, workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if a.copy_calibration:
        n = 1 << 30
        x = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    if a.hbm_read is not None:
        return hbm_read_bench(a, dev)

    is_multiq = a.workload in MULTIQ
    st = make_structure(a.workload, a.seed, a.layers, a.block_size)
    if a.workload in APPEND:
        log(f"[bench] {st.name}: {json.dumps(st.summary())}")
        return append_bench(a, st)
    layers = st.layers
    kv_fp8 = a.kv_dtype == "fp8"
    if kv_fp8 and a.workload not in ("llama3_8b_decode", "llama3_70b_decode"):
        raise SystemExit("--kv-dtype fp8 applies to the decode workloads only")
    kv_call = kv_bytes_of(st) // (st.elem_bytes if kv_fp8 else 1)
    steps = a.steps if a.steps is not None else (10 if layers > 1 else 100)
    warm = a.warmup if a.warmup is not None else (2 if layers > 1 else 10)
    log(f"[bench] {st.name}: {json.dumps(st.summary())}")

    # inputs resident in HBM: q, tables, lens; K/V pool replicas (one per layer for the
    # 80-layer workload, which already spans 80 GiB)
    tables = torch.from_numpy(st.block_tables).to(dev)
    lens = torch.from_numpy(st.context_lens).to(dev)
    qoff = torch.from_numpy(st.q_offsets).to(dev)
    dv = W.device_values(st, dev)

    def fp8(t):   # the same values rounded to 8-bit E4M3 codes (input data only)
        return t.to(torch.float8_e4m3fn).view(torch.uint8) if kv_fp8 else t

    dv["k_cache"], dv["v_cache"] = fp8(dv["k_cache"]), fp8(dv["v_cache"])
    pool_bytes = 2 * dv["k_cache"].numel() * dv["k_cache"].element_size()
    if layers > 1:
        pools = [(dv["k_cache"], dv["v_cache"])]
        for l in range(1, layers):
            d = W.device_values(st, dev, layer=l)
            pools.append((fp8(d["k_cache"]), fp8(d["v_cache"])))
            del d
            if l % 10 == 0:
                log(f"[bench] generated {l + 1}/{layers} layers")
        reps = 1
    else:
        reps = a.replicas or max(1, math.ceil(2 * 2**30 / max(pool_bytes, 1)))
        reps = min(reps, 16)
        pools = [(dv["k_cache"], dv["v_cache"])] + [
            (dv["k_cache"].clone(), dv["v_cache"].clone()) for _ in range(reps - 1)]
    q = dv["q"]
    out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    H, D = st.num_heads, st.head_dim
    # 0 = the library's choice: balanced split for decode and for multi-token
    # calls with few rows per KV head, else a partition size (reported below)
    part = a.partition
    if is_multiq and ops.multiq_uses_split(st.num_seqs, st.max_q_len, st.num_heads,
                                           st.num_kv_heads, st.head_dim, q.dtype, part):
        part_used = "balanced split"
    else:
        part_used = part or (ops.default_partition(st.num_seqs, st.num_heads, st.num_kv_heads,
                                                   st.block_size, st.max_context_len,
                                                   st.max_q_len)
                             if is_multiq else "balanced split")
    wsb = ops.workspace_size(st.num_seqs, st.total_q, st.max_q_len, H, st.num_kv_heads, D,
                             st.block_size, st.max_context_len, part)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    if is_multiq:
        prepared = ops.prepare_multiq(q, pools[0][0], pools[0][1], tables, lens, qoff, st.scale,
                                      st.max_context_len, st.max_q_len, out,
                                      partition_tokens=part, workspace=ws, stream=stream)
    else:
        prepared = None
    if kv_fp8:
        prepared = ops.prepare_decode_fp8kv(q, pools[0][0], pools[0][1], tables, lens, st.scale,
                                            1.0, 1.0, st.max_context_len, out, stream=stream)
        part_used = "balanced split"
    elif a.cascade:
        if a.workload != "shared_prefix_mix":
            raise SystemExit("--cascade applies to the shared_prefix_mix workload only")
        # leading table columns that every sequence shares (host-side structure)
        nb = -(-st.context_lens.astype(np.int64) // st.block_size)
        P = 0
        while P < nb.min() and np.all(st.block_tables[:, P] == st.block_tables[0, P]):
            P += 1
        prepared = ops.prepare_decode_shared_prefix(q, pools[0][0], pools[0][1], tables, lens,
                                                    st.scale, st.max_context_len, P, out,
                                                    stream=stream)
        part_used = f"shared-prefix cascade over {P} blocks"
    elif not is_multiq:
        prepared = ops.prepare_decode(q, pools[0][0], pools[0][1], tables, lens, st.scale,
                                      st.max_context_len, out, partition_tokens=part,
                                      workspace=ws, stream=stream)
    call = prepared.run

    calls_per_step = layers
    npools = len(pools)
    for i in range(warm * calls_per_step):
        call(*pools[i % npools])
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps * calls_per_step, 64))]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps * calls_per_step)]
    for e0, e1 in kev:            # materialize the events before the timed regions
        e0.record(stream)
        e1.record(stream)
    kev_ptrs = [(ctypes.c_void_p(e0.cuda_event), ctypes.c_void_p(e1.cuda_event)) for e0, e1 in kev]
    set_events = ops.LIB.paged_attn_set_kernel_events

    def pool_of(step, c):
        return pools[(step * calls_per_step + c) % npools] if layers == 1 else pools[c]

    # Timed region 1 (the metric): K whole steps back to back, with nothing
    # between the calls.
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for step in range(steps):
        for c in range(calls_per_step):
            call(*pool_of(step, c))
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # Timed region 2 (the roofline): the same K steps, each call's main kernel
    # bracketed by HIP events that the library hands to hipExtLaunchKernel on
    # the launch stream, which stamps them with the dispatch's own start and
    # end.  Kept out of region 1: launching through them costs a few
    # microseconds per call.
    kernel_ms = None
    if not a.cascade:   # (the cascade's several kernels take no events: whole calls are timed)
        torch.cuda.synchronize()
        k = 0
        for step in range(steps):
            for c in range(calls_per_step):
                set_events(*kev_ptrs[k])
                call(*pool_of(step, c))
                k += 1
        torch.cuda.synchronize()
        ops.set_kernel_events(None, None)
        kernel_ms = np.array([s.elapsed_time(e) for s, e in kev])
    for k, (e0, e1) in enumerate(ev):     # informational: one call between two events
        kc, vc = pools[k % npools] if layers == 1 else pools[k % calls_per_step]
        e0.record(stream)
        call(kc, vc)
        e1.record(stream)
    torch.cuda.synchronize()
    per_call_ms = np.array([s.elapsed_time(e) for s, e in ev])
    ms_per_step = total_ms / steps
    call_ms = float(per_call_ms.mean())

    kv_step = kv_call * calls_per_step
    value = kv_step / (ms_per_step * 1e-3) / 1e9
    tokens_step = st.total_q
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 K/V, bf16 q" if kv_fp8 else st.dtype, "data": "synthetic",
        "config": {
            "workload": st.name, "num_seqs": st.num_seqs, "num_heads": H,
            "num_kv_heads": st.num_kv_heads, "head_dim": D, "block_size": st.block_size,
            "sum_context": int(st.context_lens.sum()), "max_context": st.max_context_len,
            "query_tokens": st.total_q, "layers": layers, "partition_tokens": part_used,
            "pool_replicas": reps if layers == 1 else layers, "seed": a.seed,
            "pool_blocks": st.num_blocks,
        },
        "frac_of_peak_hbm": round(value / PEAK_HBM_GBPS, 4),
        "tokens_per_s": round(tokens_step / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_step,
        "call_ms": {"mean": round(call_ms, 5), "p10": round(float(np.percentile(per_call_ms, 10)), 5),
                    "p50": round(float(np.median(per_call_ms)), 5),
                    "p90": round(float(np.percentile(per_call_ms, 90)), 5)},
        "wall_s_timed": round(wall, 3),
        "source_hash": source_hash(),
    }
    if a.workload == "shared_prefix_mix":
        ub = unique_kv_bytes_of(st)
        res["unique_kv_bytes_per_step"] = ub
        res["unique_GBps"] = round(ub / (ms_per_step * 1e-3) / 1e9, 2)

    # roofline of the dominant kernel (the call's main kernel, bracketed by HIP events that
    # the library records on the launch stream); for the shared-prefix cascade, whose
    # several kernels share the work, the whole call
    if kernel_ms is None:
        kernel_ms = per_call_ms
    kern_ms = float(kernel_ms.mean())
    res["kernel_ms"] = {"mean": round(kern_ms, 5), "p50": round(float(np.median(kernel_ms)), 5)}
    if is_multiq and a.workload == "chunked_prefill":
        fl = flops_of(st)
        ach = fl / (kern_ms * 1e-3) / 1e12
        basis = None
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        basis = res.get("unique_kv_bytes_per_step", kv_step) // calls_per_step
        ach = basis / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4)}
    roof["traffic"] = measured_traffic(st.name + ("_cascade" if a.cascade else "") +
                                       ("_fp8kv" if kv_fp8 else ""),
                                       res["source_hash"])
    roof["kernel"] = ("shared-prefix decode, whole call (prefix multi-query pass, tails' decode, "
                      "fold)" if a.cascade else
                      "multi-query main kernel" if is_multiq else "decode main kernel (balanced split)")
    roof["algorithmic_bytes_per_launch"] = int(basis) if basis is not None else None
    if is_multiq:
        res["tflops"] = round(flops_of(st) / (call_ms * 1e-3) / 1e12, 2)
    res["roofline"] = roof

    if a.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(st, {"q": dv["q"], "k_cache": pools[0][0],
                                                "v_cache": pools[0][1]},
                                           a.cpu_seconds, is_multiq, kv_fp8)
    else:
        res["cpu_baseline"] = None

    line = json.dumps(res)
    print(line, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
