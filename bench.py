#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Default workload: single-layer paged decode at Qwen3-0.6B shape (16 query heads, 8 KV
heads, head_dim 128, bf16), batch 64, context lengths uniform in [512, 4096], block
size 16, physical blocks shuffled over a pool of need + 10 %.  One step is the hot
path of one layer: pa_write_kv of the 64 new tokens, then the decode as its two passes
(pa_decode_partials, pa_decode_merge), all inputs resident in HBM.

Prints one JSON line.  ``value`` is the whole-step throughput in GB/s of algorithmic
HBM traffic (wall clock per step); ``roofline`` describes the dominant kernel — the
decode's first pass, which reads every K/V byte — timed with HIP events on the stream it
runs on, with the whole decode call reported beside it; ``cpu_baseline`` is the CPU
oracle timed on the host on the same inputs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published

WORKLOADS = ("qwen3_decode_b64", "long_decode_b8", "shared_prefix_decode_b128",
             "gqa8_decode_b64", "chunked_prefill_r16", "prompt_chunk_7680_512")
# prefill workloads timed through pa_prefill_varlen_splitk (key splitting) rather than
# pa_prefill_varlen: one 512-token chunk of a long prompt after 7680 cached tokens, a batch
# with far fewer jobs than the GPU has workgroup slots
SPLIT_WORKLOADS = ("prompt_chunk_7680_512",)


def make_workload(name: str, seed: int):
    from paged_kv_cache_73_amd import workloads as W
    return {"qwen3_decode_b64": W.qwen3_decode, "long_decode_b8": W.long_decode,
            "shared_prefix_decode_b128": W.shared_prefix_decode,
            "gqa8_decode_b64": W.gqa8_decode,
            "chunked_prefill_r16": W.chunked_prefill,
            "prompt_chunk_7680_512": lambda seed: W.prefill_workload(
                [7680], [512], seed=seed, name="prompt_chunk_7680_512")}[name](seed=seed)


def decode_bytes(w, plan) -> int:
    """Algorithmic HBM bytes of one pa_decode: K and V of every key read once
    (2*Hkv*d*elem per sequence-token), q read and out written (Hq*d*elem each per
    sequence), and one 4-byte table entry per page."""
    e = w.elem_bytes
    keys = sum(plan.seqlens_k)
    pages = sum(-(-n // w.block_size) for n in plan.seqlens_k)
    return keys * 2 * w.kv_dim * e + w.batch * 2 * w.num_heads * w.head_dim * e + pages * 4


def decode_unique_bytes(w, plan) -> int:
    """decode_bytes with every physical block counted once: a block that several tables
    share (a shared prefix) is read from HBM once at best.  The rows of a block that count
    are the most any of its sequences uses."""
    e = w.elem_bytes
    B = w.block_size
    rows = {}
    for row, n in zip(plan.tables, plan.seqlens_k):
        for j in range(-(-n // B)):
            blk = row[j]
            rows[blk] = max(rows.get(blk, 0), min(B, n - j * B))
    pages = sum(-(-n // B) for n in plan.seqlens_k)
    return (sum(rows.values()) * 2 * w.kv_dim * e
            + w.batch * 2 * w.num_heads * w.head_dim * e + pages * 4)


def write_bytes(w, plan) -> int:
    """pa_write_kv reads each new K and V row and writes it once; copy-on-write
    copies read and write whole blocks of K and V."""
    e = w.elem_bytes
    rows = len(plan.new_slots)
    blk = w.block_size * w.kv_dim * e
    return rows * 4 * w.kv_dim * e + len(plan.copies) * 4 * blk


def prefill_flops(w, plan) -> float:
    """4*d*Hq per visible (query, key) pair.  Request i with q_i queries after c_i cached
    keys has q_i*c_i + q_i(q_i+1)/2 causal pairs, q_i*(c_i + q_i) without the mask."""
    tot = 0
    for qn, c in zip(w.new, w.cached):
        tot += qn * c + (qn * (qn + 1) // 2 if w.causal else qn * qn)
    return 4.0 * w.head_dim * w.num_heads * tot


def source_hash(paths) -> str:
    """First 16 hex digits of the SHA-256 of the files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_files, workload: str):
    """HBM traffic per launch from a committed rocprofv3 counter summary, if it was
    taken on the current source of the kernel (and of its launch code); otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(kernel_files):
        return None
    return rec.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# The oracle's inputs for the CPU baseline, set in the parent before its worker processes
# are forked (they inherit them; nothing is pickled).  The GPU is not touched before then.
_ORACLE = {}


def _one_thread() -> None:
    from threadpoolctl import threadpool_limits
    _ORACLE["limit"] = threadpool_limits(limits=1)


def _oracle_item(item) -> float:
    """One unit of oracle work, and its algorithmic count: ("d", b) the decode of sequence
    b (bytes); ("p", i, t0, t1) query rows t0..t1-1 of request i (flops).  Rows of a
    request are computed as a request of their own whose keys end at the last row's causal
    limit, which the oracle's pins show equal to the one-shot rows."""
    from oracle import attention as OA
    o = _ORACLE
    w = o["w"]
    if item[0] == "d":
        b = item[1]
        OA.decode(o["q"][b:b + 1], o["k"], o["v"], o["table"][b:b + 1], [o["seqlens"][b]],
                  w.scale, w.dtype)
        return o["unit"][item]
    _, i, t0, t1 = item
    q_len, k_len = o["q_lens"][i], o["k_lens"][i]
    ks = k_len - (q_len - t1) if w.causal else k_len
    rows = slice(o["cu_q"][i] + t0, o["cu_q"][i] + t1)
    OA.prefill_varlen(o["q"][rows], o["k"], o["v"], [0, t1 - t0], [0, ks], o["table"][i:i + 1],
                      w.scale, w.causal, w.dtype)
    return o["unit"][item]


def cpu_baseline(w, seconds: float) -> dict:
    """The CPU oracle (gather + two-pass softmax in float64) on the same inputs, timed on
    one core and on all the host cores this process may use (a process pool, one BLAS
    thread each, over sequences or over 64-row blocks of requests), each the median of
    three runs of about ``seconds``.  Value: GB/s of the decode's algorithmic bytes, or
    TFLOP/s of the prefill's algorithmic flops."""
    import multiprocessing as mp
    import statistics

    import numpy as np

    from tests.harness import oracle_run, storage

    o = oracle_run(w, attention=False)
    plan = o.plan
    e = w.elem_bytes
    _ORACLE.update(w=w, q=storage(w.q, w.dtype), k=o.k_pool, v=o.v_pool,
                   table=np.asarray(plan.tables), seqlens=plan.seqlens_k, cu_q=plan.cu_q,
                   q_lens=list(w.new), k_lens=plan.seqlens_k, unit={})
    unit = _ORACLE["unit"]
    if w.kind == "decode":
        items = [("d", b) for b in range(w.batch)]
        for it in items:
            unit[it] = plan.seqlens_k[it[1]] * 2 * w.kv_dim * e + 2 * w.num_heads * w.head_dim * e
        per, scale, name = 1e9, "GB/s", "sequences"
    else:
        items = []
        for i, (qn, c) in enumerate(zip(w.new, w.cached)):
            for t0 in range(0, qn, 64):
                t1 = min(qn, t0 + 64)
                it = ("p", i, t0, t1)
                items.append(it)
                pairs = sum((c + t + 1) if w.causal else (c + qn) for t in range(t0, t1))
                unit[it] = 4.0 * w.head_dim * w.num_heads * pairs
        per, scale, name = 1e12, "TFLOP/s", "64-row blocks"
    items.sort(key=lambda it: -unit[it])   # longest first: the pool balances better

    # one core: items in order, cycling, until `seconds` have passed; median of 3 runs
    _one_thread()
    one = []
    done_items = 0
    for _ in range(3):
        work, n, t0 = 0.0, 0, time.perf_counter()
        while True:
            work += _oracle_item(items[n % len(items)])
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        one.append(work / el / per)
        done_items = n
    rate1 = statistics.median(one)

    # all cores: a forked pool (the parent has not touched the GPU), at most 16 workers
    # (the host share of one GPU); each run covers the items enough times to last about
    # `seconds` at the measured one-core rate times the worker count
    nproc = os.cpu_count() or 1
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    workers = max(1, min(16, avail))
    total = sum(unit[it] for it in items)
    reps = max(1, round(seconds * workers * rate1 * per / total))
    runs = []
    with mp.get_context("fork").Pool(workers, initializer=_one_thread) as pool:
        pool.map(_oracle_item, items[:workers], chunksize=1)   # workers up
        for _ in range(3):
            t0 = time.perf_counter()
            work = sum(pool.imap_unordered(_oracle_item, items * reps, chunksize=1))
            runs.append(work / (time.perf_counter() - t0) / per)
    rate_all = statistics.median(runs)
    _ORACLE.clear()
    out = {"value": rate_all, "unit": scale, "cores": workers, "kind": "oracle",
           "value_all_cores": rate_all, "cores_all": workers, "value_1core": rate1,
           "runs_all_cores": runs, "runs_1core": one, "nproc": nproc, "cpus_allowed": avail,
           "cpu_model": _cpu_model(),
           "sample": (f"all {len(items)} {name} x {reps} per all-core run; one core: "
                      f"{done_items} {name} per run (about {seconds:.0f} s); median of 3 runs "
                      f"each; float64 gather + two-pass softmax, one BLAS thread per process")}
    if w.kind == "decode":
        keys = sum(plan.seqlens_k)
        out["seq_tokens_per_s_all_cores"] = rate_all * per * keys / total
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="qwen3_decode_b64", choices=WORKLOADS)
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=2.5,
                    help="length of each of the three one-core and all-core oracle runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="decode launches timed after flushing the caches (reported apart)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) "
              "is not supported: there is no multi-GPU path to measure.", file=sys.stderr)
        return 2

    import torch

    w = make_workload(args.workload, args.seed)
    # the CPU oracle first: its worker processes are forked before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)

    from paged_kv_cache_73_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        from paged_kv_cache_73_amd import build as B
        B.build()
    from paged_kv_cache_73_amd import runner as R

    dev = "cuda:0"
    torch.cuda.set_device(0)
    r = R.setup(w, dev)
    P = args.partition_tokens
    if w.kind == "decode":
        R.ensure_workspace(w, r, P)
    torch.cuda.synchronize()

    split = w.name in SPLIT_WORKLOADS

    def attend():
        if split:
            R.attend_splitk(w, r)
        else:
            R.attend(w, r, P)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        R.write(w, r)
        attend()
    torch.cuda.synchronize()

    # The timed region: exactly args.steps steps (the write of the step's new rows, then
    # the attention call) and nothing else on the stream, between two synchronizes.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        R.write(w, r)
        attend()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Then the same steps again with events on the kernels' stream around exactly one
    # library call each (an event between two launches delays the second, so these are
    # kept out of the timed region): the whole attention call of the step (pa_decode: both
    # passes and the gap between them; pa_prefill_varlen: one kernel), then, for decode,
    # its first pass alone (the kernel that reads every K/V byte, which the roofline line
    # is about).  The write of the step's new rows runs before each, outside the events.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        R.write(w, r)
        a.record(stream)
        attend()
        b.record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in ev]

    def pass1():
        if w.kind == "decode":
            R.attend_partials(w, r, P)
        else:
            attend()

    if w.kind == "decode":
        for a, b in ev:
            R.write(w, r)
            a.record(stream)
            pass1()
            b.record(stream)
        torch.cuda.synchronize()
        attn_ms = sorted(a.elapsed_time(b) for a, b in ev)
    else:
        attn_ms = sorted(call_ms)
    attn_mean_ms = sum(attn_ms) / len(attn_ms)
    attn_median_ms = attn_ms[len(attn_ms) // 2]

    # the same calls after evicting L2 and the MALL by reading 1 GiB (a read leaves clean
    # lines, so the timed call pays no write-backs)
    flush = torch.ones(1 << 29, dtype=torch.float32, device=dev)

    def cold_times(fn):
        out = []
        for _ in range(args.cold_reps):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return out

    cold_call = cold_times(attend)
    cold = cold_times(pass1) if w.kind == "decode" else cold_call
    # attainable read bandwidth: plain streaming read of 2 GiB (best of a few grids)
    import paged_kv_cache_73_amd as pa
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    attainable = 0.0
    for grid in (4096, 8192):
        pa.pa_probe_stream_read(flush, sink, grid)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            pa.pa_probe_stream_read(flush, sink, grid)
        b.record(stream)
        torch.cuda.synchronize()
        attainable = max(attainable, 5 * flush.numel() * 4 / (a.elapsed_time(b) * 1e-3) / 1e9)
    del flush
    if args.calibrate_copy:
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cold_median_ms = sorted(cold)[len(cold) // 2] if cold else None
    cold_call_median_ms = sorted(cold_call)[len(cold_call) // 2] if cold_call else None

    # copy-on-write copies of the step (pa_copy_blocks) timed on their own
    cow = None
    if r.copy_src.numel():
        import paged_kv_cache_73_amd as pa
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in cev:
            a.record(stream)
            pa.pa_copy_blocks(r.pool, r.copy_src, r.copy_dst)
            b.record(stream)
        torch.cuda.synchronize()
        cus = sorted(1e3 * a.elapsed_time(b) for a, b in cev)
        cbytes = 4 * len(r.plan.copies) * w.block_size * w.kv_dim * w.elem_bytes
        cow = {"pairs": len(r.plan.copies), "bytes": cbytes,
               "us_mean": sum(cus) / len(cus), "us_median": cus[len(cus) // 2],
               "achieved_GBps": cbytes / (sum(cus) / len(cus) * 1e-6) / 1e9}

    # the same step with the KV write fused into the decode launch (pa_decode_append)
    fused = None
    if w.kind == "decode":
        for _ in range(args.warmup):
            R.step(w, r, P, fused=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            R.step(w, r, P, fused=True)
        torch.cuda.synchronize()
        fwall = time.perf_counter() - t1
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in fev:
            a.record(stream)
            R.step(w, r, P, fused=True)
            b.record(stream)
        torch.cuda.synchronize()
        fms = sorted(a.elapsed_time(b) for a, b in fev)
        fused = {"ms_per_step": fwall * 1e3 / args.steps,
                 "launch_us_mean": 1e3 * sum(fms) / len(fms),
                 "launch_us_median": 1e3 * fms[len(fms) // 2]}

    # the same prefill over contiguous K/V (no block table): the cost of paging
    contiguous = None
    if w.kind == "prefill" and w.groups is None:
        from paged_kv_cache_73_amd import workloads as W
        kc, vc = (t.to(dev) for t in W.contiguous_kv(w))
        for _ in range(args.warmup):
            R.attend_contiguous(w, r, kc, vc)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in cev:
            a.record(stream)
            R.attend_contiguous(w, r, kc, vc)
            b.record(stream)
        torch.cuda.synchronize()
        cms = sorted(a.elapsed_time(b) for a, b in cev)
        contiguous = {"launch_us_mean": 1e3 * sum(cms) / len(cms),
                      "launch_us_median": 1e3 * cms[len(cms) // 2]}
        del kc, vc

    # a split workload: the same prefill through the unsplit call, for comparison
    unsplit = None
    if split:
        for _ in range(args.warmup):
            R.attend(w, r, P)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in pev:
            a.record(stream)
            R.attend(w, r, P)
            b.record(stream)
        torch.cuda.synchronize()
        pms = sorted(a.elapsed_time(b) for a, b in pev)
        unsplit = {"call": "pa_prefill_varlen", "launch_us_mean": 1e3 * sum(pms) / len(pms),
                   "launch_us_median": 1e3 * pms[len(pms) // 2]}

    plan = r.plan
    csrc = os.path.join(ROOT, "paged_kv_cache_73_amd", "csrc")
    # bf16 decode with 5-8, 16 or 32 query heads per KV head at head_dim 64/128 and block
    # size 16/32 runs on the prefill kernel (the library's routing rule)
    group = w.num_heads // w.num_kv_heads
    on_mc = (w.kind == "decode" and w.dtype == "bf16" and w.head_dim in (64, 128)
             and w.block_size in (16, 32) and (5 <= group <= 8 or group in (16, 32)))
    kernel_src = ([os.path.join(csrc, "decode_kernel.h"), os.path.join(csrc, "decode.hip")]
                  if w.kind == "decode" and not on_mc else
                  [os.path.join(csrc, f) for f in ("prefill_kernel.h", "prefill_launch.h", "prefill.hip")])
    cfg = {"workload": w.name, "batch": w.batch, "num_heads": w.num_heads,
           "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
           "num_blocks": w.num_blocks, "seed": args.seed}
    if w.kind == "decode":
        dbytes = decode_bytes(w, plan)
        # shared pages: the roofline numerator counts each physical block once (the
        # logical count, every sequence's keys, is reported beside it)
        ubytes = decode_unique_bytes(w, plan)
        shared = ubytes != dbytes
        step_bytes = ubytes + write_bytes(w, plan)
        keys = sum(plan.seqlens_k)
        achieved = dbytes / (attn_mean_ms * 1e-3) / 1e9
        cfg.update({"context_min": min(plan.seqlens_k), "context_max": max(plan.seqlens_k),
                    "sum_context": keys, "partition_tokens": P or "auto"})
        if fused is not None:
            fused["value"] = step_bytes / (fused["ms_per_step"] * 1e-3) / 1e9
            fused["unit"] = "GB/s"
        line = {
            "metric": "decode-attn HBM GB/s (% of peak) + seq-tokens/s, Qwen3-0.6B shape B=64",
            "value": step_bytes / (ms_per_step * 1e-3) / 1e9,
            "unit": "GB/s",
            "pct_of_hbm_peak": 100.0 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "seq_tokens_per_s": keys / (ms_per_step * 1e-3),
            "fused_append_step": fused,
        }
        call_mean_ms = sum(call_ms) / len(call_ms)
        if shared:
            achieved = ubytes / (attn_mean_ms * 1e-3) / 1e9
            line["logical_bytes_per_launch"] = dbytes
            line["logical_GBps_pass1"] = dbytes / (attn_mean_ms * 1e-3) / 1e9
        rbytes = ubytes
        line["headline"] = {
            "what": ("whole pa_decode call (pass 1, merge and the gap between them), "
                     "L2 and MALL evicted before each call"),
            "us_median": None if cold_call_median_ms is None else cold_call_median_ms * 1e3,
            "GBps": None if not cold_call_median_ms else rbytes / (cold_call_median_ms * 1e-3) / 1e9,
            "frac_of_peak": None if not cold_call_median_ms else
            rbytes / (cold_call_median_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "warm_us_mean": call_mean_ms * 1e3,
            "warm_GBps": rbytes / (call_mean_ms * 1e-3) / 1e9,
            "warm_frac_of_peak": rbytes / (call_mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        if cow is not None:
            line["copy_on_write"] = cow
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(kernel_src, w.name),
                "kernel": ("prefill_kernel key ranges (pa_decode_partials, pass 1 of pa_decode, "
                           "matrix-core route)" if on_mc else
                           "decode_partial_kernel (pa_decode_partials, pass 1 of pa_decode)"),
                "algorithmic_bytes_per_launch": rbytes,
                "bytes_counted": "each physical block once" if shared else "every sequence's keys",
                "launch_us_mean": attn_mean_ms * 1e3, "launch_us_median": attn_median_ms * 1e3,
                "pa_decode_call_us_mean": call_mean_ms * 1e3,
                "pa_decode_call_achieved": rbytes / (call_mean_ms * 1e-3) / 1e9,
                "pa_decode_call_frac": rbytes / (call_mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "cold_launch_us_median": None if cold_median_ms is None else cold_median_ms * 1e3,
                "cold_achieved": None if not cold_median_ms else rbytes / (cold_median_ms * 1e-3) / 1e9,
                "cold_call_us_median": None if cold_call_median_ms is None else cold_call_median_ms * 1e3,
                "attainable_stream_read": attainable,
                "frac_of_attainable": achieved / attainable if attainable else None}
    else:
        fl = prefill_flops(w, plan)
        achieved = fl / (attn_mean_ms * 1e-3) / 1e12
        cfg.update({"sum_q": sum(w.new), "sum_k": sum(plan.seqlens_k), "causal": w.causal})
        line = {"metric": "varlen paged prefill TFLOP/s (% of bf16 MFMA peak)",
                "value": fl / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s"}
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                "traffic": load_traffic(kernel_src, w.name),
                "kernel": ("pa_prefill_varlen_splitk (prefill_kernel key ranges + prefill_merge_kernel)"
                           if split else "pa_prefill_varlen"),
                "algorithmic_flops_per_launch": fl, "launch_us_mean": attn_mean_ms * 1e3,
                "launch_us_median": attn_median_ms * 1e3,
                "cold_launch_us_median": None if cold_median_ms is None else cold_median_ms * 1e3,
                "cold_achieved": None if not cold_median_ms else fl / (cold_median_ms * 1e-3) / 1e12,
                "contiguous_kv": contiguous}
        line["headline"] = {
            "what": "pa_prefill_varlen call, L2 and MALL evicted before each call",
            "us_median": None if cold_median_ms is None else cold_median_ms * 1e3,
            "TFLOPs": None if not cold_median_ms else fl / (cold_median_ms * 1e-3) / 1e12,
            "frac_of_peak": None if not cold_median_ms else
            fl / (cold_median_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "warm_us_mean": attn_mean_ms * 1e3, "warm_frac_of_peak": achieved / BF16_MFMA_PEAK_TFLOPS}
        if contiguous:
            contiguous["achieved"] = fl / (contiguous["launch_us_mean"] * 1e-6) / 1e12
        if unsplit:
            unsplit["achieved"] = fl / (unsplit["launch_us_mean"] * 1e-6) / 1e12
            roof["unsplit"] = unsplit
    line.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                 "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
                 "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
                 "config": cfg, "roofline": roof})
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
