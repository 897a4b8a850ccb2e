#!/usr/bin/env python3
"""Paged-KV decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: copy-on-write block
copies (when the workload has any), reshape_and_cache of the step's new tokens
and paged_attention_decode (main pass + merge pass of split sequences).  The
default workload is the Llama-3-70B-layer-shaped mixed-length batch (256
sequences, lognormal lengths with median 300 clipped to [16, 8192], 64 query /
8 KV heads, head_dim 128, bf16).  Inputs are resident in HBM before timing.
Several independent copies of the KV pool (same tables) are used round-robin
so that reads come from HBM, not from the 256 MB last-level cache.

Prints one JSON line.  `value` is the step's algorithmic bytes over its wall
time (GB/s); `roofline` is the decode main pass alone, timed with HIP events
on its own stream in a second pass of the same steps; `cpu_baseline` is the
oracle on a bounded sample of the same batch on the host cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode achieved HBM GB/s (% of peak); attended KV tokens/s"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
CSRC = os.path.join(ROOT, "paged_kv_cache_06_amd", "csrc")
# main-pass kernels of a decode call (matrix-core items kernels, VALU path) and
# the sources each is built from
_DECODE_SOURCES = ("pa_decode.hip", "pa_decode_common.h", "pa_decode_int8.h", "pa_cache_write.h",
                   "pa_common.h")
DECODE_KERNELS = {
    "decode_items_kernel": _DECODE_SOURCES,
    "decode_generic_kernel": _DECODE_SOURCES,
    "decode_items_i8_kernel": _DECODE_SOURCES,
}
# kernels with counter-measured traffic files and every source each is built from
KERNEL_SOURCES = dict(DECODE_KERNELS,
                      prefill_kernel=("pa_prefill.hip", "pa_decode_common.h", "pa_common.h"))


def traffic_file(kernel):
    if kernel == "decode_items_kernel":
        return TRAFFIC_FILE
    if kernel == "prefill_kernel":
        return os.path.join(ROOT, "profiles", "prefill_traffic.json")
    return os.path.join(ROOT, "profiles", f"decode_traffic_{kernel}.json")


def unique_kv_tokens(lens, rows):
    """Cached positions of distinct physical blocks that one decode call reads:
    a block shared by several tables counts once, with the most positions any
    of them attends in it (shared prefixes are read from HBM once)."""
    import numpy as np
    used = {}
    for s, n in enumerate(np.asarray(lens, dtype=np.int64)):
        for i in range(int(-(-n // 16))):
            b = int(rows[s][i])
            used[b] = max(used.get(b, 0), int(min(16, n - 16 * i)))
    return sum(used.values())


def decode_bytes(w, int8=False, rows=None):
    """Algorithmic bytes of one decode call: every cached K and V element of every
    (sequence, KV head) once -- with `rows` (the block tables), every element of
    every distinct physical block once, so that shared prefix blocks count once
    -- q and out once, table entries in use and lengths (INT8 cache: 1-byte
    elements plus the two [Hkv, D] fp32 scale arrays)."""
    import numpy as np
    lens = np.asarray(w.context_lens, dtype=np.int64)
    e = w.elem_bytes
    kv_tokens = int(lens.sum()) if rows is None else unique_kv_tokens(lens, rows)
    kv = kv_tokens * 2 * w.num_kv_heads * w.head_dim * (1 if int8 else e)
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * e
    tables = 4 * int((-(-lens // 16)).sum())
    scales = 2 * w.num_kv_heads * w.head_dim * 4 if int8 else 0
    return kv + qo + tables + 4 * w.num_seqs + scales


def step_bytes(w, db, int8=False):
    """decode bytes (shared blocks once) + the step's token writes (read + write
    + slots) + block copies."""
    B = db.phases[2]
    e = w.elem_bytes
    ec = 1 if int8 else e
    t = B.slots.shape[0]
    writes = 2 * t * w.num_kv_heads * w.head_dim * (e + ec) + 8 * t
    if int8:
        writes += 2 * w.num_kv_heads * w.head_dim * 4
    block = w.num_kv_heads * 16 * w.head_dim * ec
    copies = B.pairs.shape[0] * 2 * (2 * block) + 16 * B.pairs.shape[0]
    return decode_bytes(w, int8, db.bm.rows) + writes + copies


def kv_memory(w, db):
    """The pages' memory figures for this batch, from the library's block pool:
    slots the paged cache holds against the tokens it stores, against a
    contiguous reservation of the batch's longest context per sequence, and
    (shared prompts) blocks held against the same prompts with one sample each
    and against every sample holding its own copy."""
    import numpy as np
    import paged_kv_cache_06_amd as pa
    lens = np.asarray(w.context_lens, dtype=np.int64)
    used = db.bm.pool.stats()["used"]
    tokens = unique_kv_tokens(lens, db.bm.rows)  # distinct cached positions
    paged_slots = used * 16
    reserved = int(lens.max()) * w.num_seqs
    out = {"tokens": int(tokens), "blocks_held": int(used), "paged_slots": int(paged_slots),
           "paged_waste_pct": round(100.0 * (paged_slots - tokens) / paged_slots, 3),
           "contiguous_reserved_slots": int(reserved),
           "contiguous_waste_pct": round(100.0 * (reserved - lens.sum()) / reserved, 3)}
    prompts = np.asarray(w.prompt_of)
    if (prompts >= 0).any():
        first = [int(np.flatnonzero(prompts == p)[0]) for p in range(len(w.prompt_lens))]
        pool = pa.Pool(w.num_blocks)
        bm = pa.BlockManager(pool, len(first), db.bm.rows.shape[1])
        for i, s in enumerate(first):
            bm.append(i, int(w.prompt_lens[prompts[s]]))
            bm.append(i, int(w.private_lens[s]))
        out.update(samples_per_prompt=round(w.num_seqs / len(first), 3),
                   blocks_one_sample_per_prompt=int(pool.stats()["used"]),
                   blocks_every_sample_unshared=int((-(-lens // 16)).sum()))
        out["shared_vs_one_sample"] = round(used / out["blocks_one_sample_per_prompt"], 4)
    return out


def source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def launch_percentiles(kind):
    """p10, median and p90 of the launch times (ms, HIP events) of one kernel
    kind over the timed pass just ended."""
    import numpy as np
    import paged_kv_cache_06_amd as pa
    ms = pa.timing_launches(kind)
    if not ms:
        return None
    return [round(float(v), 5) for v in np.percentile(np.asarray(ms), [10, 50, 90])]


def load_traffic(workload, kernel):
    """Counter-measured HBM bytes per launch of `kernel`, if taken on its current source."""
    try:
        with open(traffic_file(kernel)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel") != kernel or t.get("source_sha256_16") != source_hash(kernel)
            or t.get("workload") != workload):
        return None
    return t.get("bytes_per_launch")


def pmc_summary(fetch_dir, write_dir, workload, kernel, out_path=None):
    """HBM bytes per decode launch from two rocprofv3 --pmc runs of this bench
    (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch), each scaled by
    what the same counter reads for the run's plain 1 GiB device copy."""
    import csv
    import glob
    import statistics

    def rows(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                out += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        if not out:
            raise SystemExit(f"no {counter} rows under {d}")
        return out

    result = {"workload": workload, "kernel": kernel, "source_sha256_16": source_hash(kernel)}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rs = rows(d, counter)
        copies = [r for r in rs if "copyBuffer" in r["Kernel_Name"]]
        big = max(int(r["Grid_Size"]) for r in copies)
        cal = statistics.median(float(r["Counter_Value"]) for r in copies
                                if int(r["Grid_Size"]) == big)
        factor = (1 << 30) / 1024.0 / cal  # the copy moves 1 GiB each way
        dec = [float(r["Counter_Value"]) for r in rs if kernel in r["Kernel_Name"]]
        kib = statistics.median(dec)
        result[counter] = {"kib_per_dispatch_raw": kib, "calibration_factor": round(factor, 4),
                           "bytes_per_launch": int(kib * 1024 * factor),
                           "dispatches": len(dec)}
    result["bytes_per_launch"] = (result["FETCH_SIZE"]["bytes_per_launch"]
                                  + result["WRITE_SIZE"]["bytes_per_launch"])
    out_path = out_path or traffic_file(kernel)
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(result, f, indent=1)
    print(json.dumps(result))


def host_cpu():
    """The host's CPU model and the logical CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "usable_cpus": usable}


# Oracle state the CPU baseline's worker processes share: set in the parent
# before the pool forks, read (never written) by the children.
_ORACLE_STATE = {}


def _oracle_cache(w, int8):
    """The oracle's own pool, tables and paged cache of the batch after its
    step (not timed)."""
    import numpy as np
    from oracle import cache_ops, quant, step
    pl = step.plan(w)
    if int8:
        sk, sv = w.int8_scales()
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        kc = np.full(shape, 127, np.int8)
        vc = kc.copy()
        for ph in pl.phases:
            cache_ops.copy_blocks(kc, vc, ph.pairs)
            quant.reshape_and_cache(ph.key, ph.value, w.dtype, kc, vc, ph.slots, sk, sv)
        return pl.tables, kc, vc, sk, sv
    kc, vc = step.empty_cache(w, 0)
    for ph in pl.phases:
        step.apply_phase(ph, kc, vc)
    return pl.tables, kc, vc, None, None


def _oracle_decode(seqs):
    """The oracle's paged decode (gather through its table, fp64 attention) of
    the given sequences, BLAS on one thread; returns (tokens, bytes)."""
    from oracle import attention, quant
    from threadpoolctl import threadpool_limits
    w, int8 = _ORACLE_STATE["w"], _ORACLE_STATE["int8"]
    tables, kc, vc, sk, sv = _ORACLE_STATE["cache"]
    lens = w.context_lens
    ec = 1 if int8 else w.elem_bytes
    tokens = nbytes = 0
    with threadpool_limits(1):
        for s in seqs:
            if int8:
                quant.paged_decode(w.q[s:s + 1], kc, vc, sk, sv, [tables[s]], lens[s:s + 1],
                                   w.scale, w.dtype)
            else:
                attention.paged_decode(w.q[s:s + 1], kc, vc, [tables[s]], lens[s:s + 1],
                                       w.scale, w.dtype)
            n = int(lens[s])
            tokens += n
            nbytes += n * 2 * w.num_kv_heads * w.head_dim * ec + 2 * w.num_q_heads * w.head_dim * w.elem_bytes
    return tokens, nbytes


def cpu_baseline(w, budget_s, int8=False):
    """The oracle's decode of the batch on the host cores, ~budget_s of work per
    run: once on one core (sequences in order, whole passes or a prefix), then
    on all usable cores (a pool of forked worker processes, one BLAS thread
    each, over about as many whole passes as fit the budget at the one-core
    rate times the workers).  Runs before the GPU is touched, so no worker
    inherits device state.  INT8 cache: attention over the oracle's code *
    scale values."""
    import multiprocessing

    _ORACLE_STATE.update(w=w, int8=int8, cache=_oracle_cache(w, int8))
    order = list(range(w.num_seqs))
    # one core
    tok1 = by1 = seqs1 = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for s in order:
            t, b = _oracle_decode([s])
            tok1, by1, seqs1 = tok1 + t, by1 + b, seqs1 + 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt1 = time.perf_counter() - t0
    # all usable cores (at most 16 processes)
    workers = max(1, min(16, host_cpu()["usable_cpus"] or 1))
    passes = max(1, int(round(seqs1 / dt1 * workers * budget_s / w.num_seqs)))
    work = [[s] for _ in range(passes) for s in order]
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_decode, [[0]] * workers)  # workers started and warm
        t0 = time.perf_counter()
        res = pool.map(_oracle_decode, work, chunksize=4)
        dtn = time.perf_counter() - t0
    _ORACLE_STATE.clear()
    tokn = sum(t for t, _ in res)
    byn = sum(b for _, b in res)
    what = ("fp64 NumPy attention over the oracle's INT8 codes x scales, gathered through its "
            "tables" if int8 else "fp64 NumPy attention, K/V gathered through the oracle's own "
            "block tables from its paged cache")
    return {"value": round(byn / dtn / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "tokens_per_s": round(tokn / dtn, 1),
            "single_core": {"value": round(by1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "tokens_per_s": round(tok1 / dt1, 1)},
            "host": host_cpu(),
            "sample": f"oracle paged decode ({what}) of the {w.num_seqs}-sequence batch: on 1 "
                      f"core {seqs1} sequence decodes ({tok1} attended tokens) in {dt1:.1f} s; "
                      f"on {workers} worker processes (1 BLAS thread each) {passes} whole "
                      f"pass(es) ({len(work)} sequence decodes, {tokn} attended tokens) in "
                      f"{dtn:.1f} s"}


HOST_LINK_PEAK_GBS = 63.0  # PCIe 5.0 x16 per direction: 32 GT/s x 16 lanes x 128/130


def swap_bench(args):
    """Move every block of the batch to a pinned host pool and back, K times:
    pool bookkeeping (pa_swap_blocks) on the host, one pa_transfer_blocks per
    direction on the device.  Prints one JSON line."""
    import numpy as np
    import torch
    import paged_kv_cache_06_amd as pa
    import workloads
    from paged_kv_cache_06_amd import runner
    w = workloads.make(args.config)
    int8 = args.kv == "int8"
    db = runner.DeviceBatch(w, int8=int8)
    db.prefill()
    torch.cuda.synchronize()
    kd, vd = db.caches[0]
    host = pa.Pool(w.num_blocks)
    kh, vh = pa.new_host_kv_cache(w.num_blocks, w.num_kv_heads, w.head_dim, kd.dtype)
    nb = [int(n) for n in db.bm.nblocks]
    ec = 1 if int8 else w.elem_bytes
    block_bytes = 2 * w.num_kv_heads * 16 * w.head_dim * ec
    t_out = t_in = t_host = 0.0
    moved = 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for it in range(args.warmup + args.steps):
        h0 = time.perf_counter()
        out_pairs = [pa.swap_blocks(db.bm.pool, host, db.bm.rows[s, :nb[s]])
                     for s in range(w.num_seqs)]
        h1 = time.perf_counter()
        po = torch.from_numpy(np.concatenate(out_pairs)).cuda()
        ev[0].record()
        pa.transfer_blocks(kd, vd, kh, vh, po)
        ev[1].record()
        h2 = time.perf_counter()
        in_pairs = [pa.swap_blocks(host, db.bm.pool, p[:, 1]) for p in out_pairs]
        h3 = time.perf_counter()
        for s, p in enumerate(in_pairs):
            db.bm.rows[s, :nb[s]] = p[:, 1]
        pi = torch.from_numpy(np.concatenate(in_pairs)).cuda()
        ev[2].record()
        pa.transfer_blocks(kh, vh, kd, vd, pi)
        ev[3].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            t_out += ev[0].elapsed_time(ev[1])
            t_in += ev[2].elapsed_time(ev[3])
            t_host += (h1 - h0) + (h3 - h2)
            moved += po.shape[0]
    n = max(1, args.steps)
    per_dir = moved / n * block_bytes
    out_gbs = per_dir / (t_out / n * 1e-3) / 1e9
    in_gbs = per_dir / (t_in / n * 1e-3) / 1e9
    value = 2 * per_dir / ((t_out + t_in) / n * 1e-3) / 1e9
    print(json.dumps({
        "metric": "block swap device <-> pinned host GB/s", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t_out + t_in) / n, 4), "higher_is_better": True,
        "dtype": "i8" if int8 else w.dtype, "data": "synthetic",
        "config": {"workload": w.name + ("-int8kv" if int8 else ""), "blocks_per_direction":
                   int(moved / n), "block_bytes": block_bytes},
        "swap_out_gbs": round(out_gbs, 2), "swap_in_gbs": round(in_gbs, 2),
        "host_bookkeeping_ms_per_step": round(t_host / n * 1e3, 3),
        "roofline": {"bound": "host-link", "kernel": "transfer_blocks_kernel",
                     "achieved": round(value, 2), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HOST_LINK_PEAK_GBS, 4), "traffic": None},
    }), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak


def prefill_flops(w):
    """QK and PV of every chunk query against every position up to its own,
    2 flops per multiply-add: sum over queries of (p + 1) * 4 * Hq * D."""
    import numpy as np
    lens = np.asarray(w.context_lens, dtype=np.int64)
    n = np.asarray(w.step_lens, dtype=np.int64)
    # positions p = len - n + i, i < n: sum of (p + 1) = n * (len - n) + n (n + 1) / 2
    pairs = int((n * (lens - n) + n * (n + 1) // 2).sum())
    return pairs * 4 * w.num_q_heads * w.head_dim, pairs


def prefill_bench(args):
    """Chunked prefill: the step writes every chunk's K/V and attends its
    queries causally; K steps.  Prints one JSON line."""
    import numpy as np
    import torch
    import paged_kv_cache_06_amd as pa
    import workloads
    from paged_kv_cache_06_amd import runner
    w = workloads.make("prefill")
    db = runner.DeviceBatch(w)
    db.prefill()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        db._apply(db.dev_phases[2], db.caches[0])
        db.attend_chunks()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        db._apply(db.dev_phases[2], db.caches[0])
        db.attend_chunks()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pa.timing_begin(4 * args.steps + 16)
    for _ in range(args.steps):
        db._apply(db.dev_phases[2], db.caches[0])
        db.attend_chunks()
    torch.cuda.synchronize()
    kt = pa.timing_end()
    flops, pairs = prefill_flops(w)
    ms_step = (t1 - t0) * 1e3 / args.steps
    k = kt["prefill"]
    k_ms = k["ms"] / max(1, k["launches"])
    achieved = flops / (k_ms * 1e-3) / 1e12
    tokens = int(np.sum(w.step_lens))
    result = {
        "metric": "chunked-prefill paged attention TFLOP/s; prefill tokens/s",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "chunk_tokens": tokens,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "attended_pairs": pairs},
        "prefill_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "kernels_ms_per_step": {kk: round(v["ms"] / max(1, v["launches"]), 5)
                                for kk, v in kt.items() if v["launches"]},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": flops,
                     "avg_launch_ms": round(k_ms, 5),
                     "launch_ms_p10_p50_p90": launch_percentiles("prefill"),
                     "traffic": load_traffic(w.name, "prefill_kernel")},
    }
    if args.calibrate_copy > 0:
        calibration_copies(args.calibrate_copy)
        result["calibration_copy_bytes"] = args.calibrate_copy << 20
    print(json.dumps(result), flush=True)


def calibration_copies(mib):
    """Three plain device copies of `mib` MiB: a known-size reference for the
    HBM byte counters."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def measured_copy_gbs(mib=1024, reps=10):
    """HBM rate of a plain 1 GiB device-to-device copy on this machine (bytes read
    plus bytes written per second, HIP events on the copy's stream): the
    measured streaming reference beside the 8 TB/s specification."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    stop.synchronize()
    ms = start.elapsed_time(stop) / reps
    del src, dst
    return round(2 * (mib << 20) / (ms * 1e-3) / 1e9, 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="3", help="workload 1..5 or 4b (default 3)")
    ap.add_argument("--copies", type=int, default=0,
                    help="KV pool copies used round-robin (default: enough for >= 1.5 GB)")
    ap.add_argument("--partition", type=int, default=-1, help="-1 auto, 0 none, else tokens")
    ap.add_argument("--kv", choices=("native", "int8"), default="native",
                    help="KV cache storage: the workload's dtype, or INT8 codes with "
                         "per-channel scales")
    ap.add_argument("--no-shared", action="store_true",
                    help="workloads with shared prompts: decode every sequence's blocks through "
                         "its own table instead of reading each shared prefix once")
    ap.add_argument("--swap", action="store_true",
                    help="instead of decode steps: move every block of the batch to a pinned "
                         "host pool and back (host-tier swap bandwidth)")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of decode steps: the chunked-prefill workload (16 sequences, "
                         "512-token chunks after U{0..3584} cached tokens, 32/8 heads, D 128)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of oracle work per CPU-baseline run (one core, all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run 3 plain device copies of MIB MiB (a known-size "
                         "reference for HBM byte counters)")
    ap.add_argument("--kernel", default="decode_items_kernel", choices=sorted(KERNEL_SOURCES),
                    help="kernel the --pmc-summary counters belong to")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench, taken with --calibrate-copy 1024, into profiles/ "
                         "(decode_traffic.json for the items kernel, "
                         "decode_traffic_<kernel>.json otherwise)")
    args = ap.parse_args()

    if args.pmc_summary:
        import workloads
        if args.prefill:
            name = workloads.CONFIG_NAMES["prefill"]
        else:
            name = workloads.CONFIG_NAMES[int(args.config) if args.config.isdigit() else args.config]
            name += "-int8kv" if args.kv == "int8" else ""
        pmc_summary(*args.pmc_summary, name, args.kernel)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    cpu = None
    if not (args.swap or args.prefill or args.no_cpu_baseline):
        # the oracle on the host cores first, before anything touches the GPU
        import workloads
        cpu = cpu_baseline(workloads.make(args.config), args.cpu_seconds, args.kv == "int8")
        print(f"# cpu baseline: {cpu['tokens_per_s']:.0f} tokens/s on {cpu['cores']} "
              f"processes, {cpu['single_core']['tokens_per_s']:.0f} on one", file=sys.stderr,
              flush=True)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.swap:
        swap_bench(args)
        return
    if args.prefill:
        prefill_bench(args)
        return
    import paged_kv_cache_06_amd as pa
    if not os.path.exists(pa.lib_path()):
        from paged_kv_cache_06_amd import _build
        _build.build()
    import workloads
    from paged_kv_cache_06_amd import runner

    t_setup = time.perf_counter()
    w = workloads.make(args.config)
    int8 = args.kv == "int8"
    if int8 and (w.dtype == "f32" or w.head_dim not in (64, 128)):
        print("the INT8 cache serves fp16/bf16 queries at head_dim 64 or 128", file=sys.stderr)
        sys.exit(2)
    ec = 1 if int8 else w.elem_bytes
    pool_bytes = 2 * (w.num_blocks + 1) * w.num_kv_heads * 16 * w.head_dim * ec
    copies = args.copies or max(1, int(np.ceil(1.5e9 / pool_bytes)))
    shared = not args.no_shared and bool(np.any(np.asarray(w.prompt_of) >= 0))
    db = runner.DeviceBatch(w, copies=copies, int8=int8, shared_prefix=shared)
    db.prefill()
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f} s: workload {w.name}, "
          f"{int(np.sum(w.context_lens))} tokens, {copies} pool copies", file=sys.stderr,
          flush=True)

    for i in range(args.warmup):
        db.step(copy=i % copies, partition_size=args.partition)
    torch.cuda.synchronize()

    # timed region: K steps, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        db.step(copy=i % copies, partition_size=args.partition)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the same K steps again with HIP events around every library kernel, on
    # the stream it runs on (events add a few microseconds per launch, so they
    # stay out of the region above)
    pa.timing_begin(8 * args.steps + 16)
    for i in range(args.steps):
        db.step(copy=i % copies, partition_size=args.partition)
    torch.cuda.synchronize()
    kt = pa.timing_end()

    ms_step = (t1 - t0) * 1e3 / args.steps
    sbytes = step_bytes(w, db, int8)
    dbytes = decode_bytes(w, int8, db.bm.rows)      # shared blocks once: the roofline's bytes
    logical = decode_bytes(w, int8)                 # every sequence's blocks, shared or not
    tokens = int(np.sum(w.context_lens))
    dec = kt["decode"]
    dec_ms = dec["ms"] / max(1, dec["launches"])
    achieved = dbytes / (dec_ms * 1e-3) / 1e9
    # the partition the plan used: the automatic one may be doubled, for shared
    # prefixes on the host and for an even batch by the plan itself
    ps = pa.last_plan_partition()
    if int8:
        main_kernel = "decode_items_i8_kernel"
    elif w.dtype != "f32" and w.head_dim in (64, 128):
        main_kernel = "decode_items_kernel"
    else:
        main_kernel = "decode_generic_kernel"
    workload_name = w.name + ("-int8kv" if int8 else "")
    traffic = load_traffic(workload_name, main_kernel)
    result = {
        "metric": METRIC,
        "value": round(sbytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"i8kv+{w.dtype}" if int8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": workload_name, "kv_cache": "int8 per-channel" if int8 else w.dtype,
                   "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": 16,
                   "attended_tokens": tokens, "max_context_len": db.max_context_len,
                   "partition_size": ps, "kv_pool_copies": copies, "parallelism": "none",
                   "shared_prefix_groups": int(db.shared[2].numel()) if db.shared else 0},
        "pct_of_hbm_peak": round(100 * sbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "attended_kv_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "kernels_ms_per_step": {k: round(v["ms"] / max(1, v["launches"]), 5)
                                for k, v in kt.items() if v["launches"]},
        "roofline": {"bound": "hbm", "kernel": main_kernel,
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": dbytes,
                     "avg_launch_ms": round(dec_ms, 5),
                     "launch_ms_p10_p50_p90": launch_percentiles("decode"),
                     "traffic": traffic},
    }
    copy_gbs = measured_copy_gbs()
    result["roofline"]["measured_copy_gbs"] = copy_gbs
    result["roofline"]["frac_of_measured_copy"] = round(achieved / copy_gbs, 4)
    result["kv_memory"] = kv_memory(w, db)
    if logical != dbytes:  # shared prefixes: also the per-sequence (logical) figure
        result["logical_bytes_per_launch"] = logical
        result["logical_gb_per_s"] = round(logical / (dec_ms * 1e-3) / 1e9, 2)
    if args.calibrate_copy > 0:
        calibration_copies(args.calibrate_copy)
        result["calibration_copy_bytes"] = args.calibrate_copy << 20
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
