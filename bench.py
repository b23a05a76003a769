"""Benchmark of the paged decode hot path on one MI355X.

One step = one pass of the whole path over one batch: the step's copy-on-write
block copies (if the workload has any), the paged append of each sequence's
newest token and decode attention over every cached token -- the append is
fused into the decode launch when the workload appends.  Default workload:
``llama13b_long`` (32 sequences, 40 MHA heads of 128, 16-token blocks,
lognormal lengths with median 4096 clipped to [1024, 16384], bf16).

Prints ONE JSON line: achieved HBM GB/s on the KV bytes the step reads
(``value``), sequence-steps per second, the decode kernel's roofline entry
(HIP-event timing, on the stream it runs on, of the attention launches of at
least ten timed steps) and the CPU oracle's throughput on a bounded sample of the
same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (KV read) & % of peak; seq-steps/sec"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, vendor specification
EVENT_SAMPLES = 10             # attention launches event-timed per run (at least)
# Sources that define each attention kernel and what runs with it in a step
# (the merge kernels live in decode_kernel.hip): a counter summary stays
# valid while these are unchanged.
_CSRC = os.path.join(ROOT, "paged_kv_cache_310_amd", "csrc")
KERNEL_SOURCES = {
    name: [os.path.join(_CSRC, f) for f in files + ("decode_common.h", "pa_internal.h")]
    for name, files in (("decode_valu_kernel", ("decode_kernel.hip",)),
                        ("decode_gqa_kernel", ("gqa_kernel.hip", "gqa_body.h", "merge_body.h",
                                               "decode_kernel.hip")),
                        ("decode_shared_kernel", ("shared_kernel.hip", "gqa_body.h",
                                                  "merge_body.h")),
                        ("prefill_kernel", ("prefill_kernel.hip",)))
}


def event_every(steps: int) -> int:
    """Timed steps per step whose attention kernel is event-timed: every
    step up to EVENT_SAMPLES steps, then spaced so that at least
    EVENT_SAMPLES launches are timed."""
    return max(1, steps // EVENT_SAMPLES)


def attention_kernel_name(w, shared: bool = False) -> str:
    """The attention kernel the step launches for this workload: with the
    groups (pa_decode_shared) the shared-prefix kernel for bf16 head_dim 128
    and 1..16 query heads per KV head; pa_decode's matrix-core kernel for
    bf16 head_dim 128 with 2..16 query heads per KV head; else the vector
    kernel."""
    group = w.num_q_heads // w.num_kv_heads
    if shared and w.dtype == "bf16" and w.head_dim == 128 and 1 <= group <= 16:
        return "decode_shared_kernel"
    if w.dtype == "bf16" and w.head_dim == 128 and 2 <= group <= 16:
        return "decode_gqa_kernel"
    return "decode_valu_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle-s", type=float, default=0.3,
                   help="untimed steps for this many seconds before the warm-up steps")
    p.add_argument("--workload", default="llama13b_long")
    p.add_argument("--workers", type=int, default=0, help="decode workers (0 = library default)")
    p.add_argument("--plain", action="store_true",
                   help="time pa_decode even when the workload has groups sharing a prefix "
                        "(default for such workloads: pa_decode_shared)")
    p.add_argument("--cold-steps", type=int, default=20,
                   help="extra steps, each after a 512 MiB write that evicts the MALL")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU oracle time budget for the baseline sample (0 = skip)")
    p.add_argument("--prefill-workload", default=None,
                   help="measure multi-token (prefill) attention on this workload instead "
                        "(llama13b_prefill, gqa_chunked_prefill or gqa_single_chunk_32k)")
    p.add_argument("--probe", type=int, default=1,
                   help="also measure the read ceiling of the same pools with pa_read_probe "
                        "(0 = skip)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[kernel]:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, kernel: str, kind: str = "decode"):
    """HBM bytes per attention launch (``kind`` decode or prefill) from the
    committed rocprofv3 counter summary of this workload, or None when absent
    or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source sha256\[:16\]: `([0-9a-f]+)`", text)
    t = re.search(r"hbm bytes per launch \(calibrated\): `([0-9.e+]+)`", text)
    if not m or not t or m.group(1) != kernel_source_hash(kernel):
        return None
    return float(t.group(1))


def decode_tile_order(w, shared: bool = False) -> np.ndarray:
    """Tile ids (16-token tiles of a pool, in address order) in the order the
    decode kernels walk them: KV head by KV head, each sequence's cached
    tokens in logical order through its block table.  ``shared``: each
    group's shared chunks once (through its first member's table), then every
    sequence's remaining chunks."""
    cpb = w.block_size // 16
    per_head = []

    def tiles(s, c):
        blocks = w.block_tables[s, c // cpb].astype(np.int64)
        return blocks * w.num_kv_heads * cpb + c % cpb

    start = np.zeros(w.num_seqs, np.int64)
    if shared:
        lens = w.context_lens.astype(np.int64)
        start = np.minimum(np.maximum(w.prefix_lens.astype(np.int64), 0), lens) // 16
        for g in range(len(w.group_start) - 1):
            lo, hi = int(w.group_start[g]), int(w.group_start[g + 1])
            if hi > lo:
                per_head.append(tiles(lo, np.arange(start[lo])))
    for s in range(w.num_seqs):
        n = -(-int(w.context_lens[s]) // 16)
        per_head.append(tiles(s, np.arange(start[s], n)))
    base = np.concatenate(per_head) if per_head else np.zeros(0, np.int64)
    return np.concatenate([base + h * cpb for h in range(w.num_kv_heads)]).astype(np.int32)


def read_ceiling(pa, k, v, w, workers: int, reps: int = 5, shared: bool = False):
    """Bandwidth of the decode kernels' access pattern without their
    arithmetic, measured on the same pools in the same run with
    pa_read_probe (K plain, V non-temporal, as the attention kernels load
    them): the tiles the step reads in the decode kernels' own order, every
    16-token tile of both pools in a random order, and the K pool in address
    order.  Medians of `reps` timed passes after one untimed."""
    import torch
    tile = 16 * w.head_dim * (2 if w.dtype == "bf16" else 4)
    if tile not in (4096, 8192):
        return None
    gen = torch.Generator(device="cpu").manual_seed(3199)
    ntiles = k.numel() * k.element_size() // tile
    ids_dec = torch.from_numpy(decode_tile_order(w, shared)).to(k.device)
    ids_k = torch.randperm(ntiles, generator=gen).to(torch.int32).to(k.device)
    ids_v = torch.randperm(ntiles, generator=gen).to(torch.int32).to(k.device)

    def timed(fn):
        fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(out))

    dec = 2 * ids_dec.numel() * tile
    t_dec = timed(lambda: (pa.pa_read_probe(k, ids_dec, tile, False, num_workers=workers),
                           pa.pa_read_probe(v, ids_dec, tile, True, num_workers=workers)))
    both = 2 * ntiles * tile
    t_rand = timed(lambda: (pa.pa_read_probe(k, ids_k, tile, False, num_workers=workers),
                            pa.pa_read_probe(v, ids_v, tile, True, num_workers=workers)))
    t_seq = timed(lambda: pa.pa_read_probe(k, None, tile, False, num_workers=workers))
    return {"what": f"pa_read_probe, {tile} B tiles, K plain and V non-temporal: the step's "
                    "tiles in the decode kernels' order; every tile of both pools in random "
                    f"order; the K pool in address order. {reps} passes, median",
            "bytes_decode_order": dec, "decode_order_gbps": round(dec / t_dec / 1e9, 1),
            "bytes_random": both, "random_tiles_gbps": round(both / t_rand / 1e9, 1),
            "sequential_gbps": round(ntiles * tile / t_seq / 1e9, 1)}


def cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle on whole sequences (all heads) of the workload,
    in a fixed seeded order, until the time budget is used."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    k, v = w.k_cache, w.v_cache
    if w.slot_mapping is not None:
        k, v = oracle.append_kv(k, v, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    order = np.random.default_rng(0).permutation(w.num_seqs)
    done_bytes, seqs = 0, 0
    per_tok = 2 * w.num_kv_heads * w.head_dim * (2 if w.dtype == "bf16" else 4)
    t0 = time.perf_counter()
    for s in order:
        rows = [(int(s), h) for h in range(w.num_q_heads)]
        oracle.decode(w.q, k, v, w.block_tables, w.context_lens, w.scale, w.dtype, w.block_size,
                      rows=rows)
        done_bytes += int(w.context_lens[s]) * per_tok
        seqs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{seqs} of {w.num_seqs} sequences (all {w.num_q_heads} heads, "
                  f"{done_bytes / 1e9:.3f} GB of KV) in {dt:.1f} s, fp64 numpy, "
                  f"seq-steps/s {seqs / dt:.3f}; cpu '{cpu}', "
                  f"os.cpu_count {os.cpu_count()}, affinity {len(os.sched_getaffinity(0))}",
    }


def prefill_cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle's multi-token attention on query tokens of the
    workload (all heads of each), in a fixed seeded order, in batches of 16
    tokens until the time budget is used; rate in flop/s of the same
    algorithmic count the GPU figure uses."""
    import oracle
    k, v = oracle.append_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    starts = w.query_start.astype(np.int64)
    seq_of = np.searchsorted(starts, np.arange(w.num_query_tokens), side="right") - 1
    order = np.random.default_rng(0).permutation(w.num_query_tokens)
    flops, tokens = 0, 0
    t0 = time.perf_counter()
    for first in range(0, len(order), 16):
        batch = order[first:first + 16]
        rows = [(int(t), h) for t in batch for h in range(w.num_q_heads)]
        oracle.prefill(w.q, k, v, w.block_tables, w.context_lens, w.query_start, w.scale,
                       w.dtype, w.block_size, rows=rows)
        for t in batch:
            s = int(seq_of[t])
            pos = int(w.context_lens[s]) - int(starts[s + 1] - starts[s]) + int(t - starts[s])
            flops += 4 * w.head_dim * (pos + 1) * w.num_q_heads
        tokens += len(batch)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{tokens} of {w.num_query_tokens} query tokens (all {w.num_q_heads} heads) "
                      f"in {dt:.1f} s, fp64 numpy"}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def run_prefill(args):
    """One JSON line for multi-token attention (``pa_prefill``) on a prefill
    workload: TFLOP/s against the dense bf16 MFMA peak, the oracle beside it."""
    from paged_kv_cache_310_amd import prefill_bench
    from paged_kv_cache_310_amd import workloads as wl
    r = prefill_bench.run(args.prefill_workload, max(args.steps, 1), 0.6)
    line = {
        "metric": r["metric"], "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": max(args.steps, 1), "warmup": "0.6 s", "ms_per_step": round(r["us_per_call"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"], "num_seqs": r["num_seqs"],
                   "query_tokens": r["query_tokens"], "cached_tokens": r["cached_tokens"],
                   "heads": r["heads"], "head_dim": 128, "block_size": 16,
                   "context_splits": r["context_splits"]},
        "roofline": {"bound": "mfma", "achieved": r["tflops"], "peak": prefill_bench.PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": r["frac"],
                     "traffic": counter_traffic(r["workload"], "prefill_kernel", "prefill"),
                     "kernel": "prefill_kernel",
                     "kernel_source_sha256_16": kernel_source_hash("prefill_kernel")},
    }
    if args.cpu_seconds > 0:
        w = wl.make_prefill_workload(args.prefill_workload, poison=False)
        line["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path runs without collectives or sharding; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_310_amd as pa
    from paged_kv_cache_310_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.prefill_workload:
        run_prefill(args)
        return

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 3}))
        return

    t0 = time.perf_counter()
    w = wl.make_workload(args.workload, poison=False)
    log(f"workload {w.name}: {w.num_seqs} seqs, {int(w.context_lens.sum())} tokens, "
        f"{w.kv_bytes / 1e9:.3f} GB KV, generated in {time.perf_counter() - t0:.1f} s")

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k, v = to_dev(w.q), to_dev(w.k_cache), to_dev(w.v_cache)
    tables, lens = to_dev(w.block_tables), to_dev(w.context_lens)
    k_new, v_new, slots, pairs = to_dev(w.k_new), to_dev(w.v_new), to_dev(w.slot_mapping), \
        to_dev(w.block_mapping)
    out = torch.empty_like(q)
    shared = w.group_start is not None and not args.plain
    size_fn = pa.pa_decode_shared_workspace_size if shared else pa.pa_decode_workspace_size
    ws_bytes = size_fn(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, args.workers)
    workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    gstart, plens = (to_dev(w.group_start), to_dev(w.prefix_lens)) if shared else (None, None)

    def step(ev=None):
        if pairs is not None:
            pa.pa_copy_blocks(k, v, pairs)
        if ev is not None:
            # the library passes these as the attention launch's own events
            pa.pa_set_decode_events(ev[0], ev[1])
        if shared:
            pa.pa_decode_shared(q, k, v, tables, lens, float(w.scale), gstart, plens, out=out,
                                k_new=k_new, v_new=v_new, slot_mapping=slots,
                                workspace=workspace, num_workers=args.workers)
        else:
            pa.pa_decode(q, k, v, tables, lens, float(w.scale), out=out, k_new=k_new,
                         v_new=v_new, slot_mapping=slots, workspace=workspace,
                         num_workers=args.workers)
        if ev is not None:
            pa.pa_set_decode_events(None, None)

    # Settle: after a process starts issuing work, the first few dozen decode
    # launches run 5-20% slower than the rest (a transient of the device's
    # clocks under the new load, a few milliseconds long; it shows in every
    # kernel trace), so the run first steps untimed for settle_s seconds and
    # a short run's few warm-up steps still lead into the steady state.
    t_settle = time.perf_counter() + max(args.settle_s, 0.0)
    while time.perf_counter() < t_settle:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The attention kernel of every event_every(steps)-th timed step is
    # bracketed by HIP events (at least EVENT_SAMPLES launches); recording
    # them costs ~15 us of queue time per step, so doing it on every step of a
    # long run would time the probe as much as the path.
    sampled = list(range(0, args.steps, event_every(args.steps)))
    events = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for i in sampled}
    for pair in events.values():      # torch creates an event on its first record:
        for e in pair:                # do that here, outside the timed region
            e.record()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    kernel_ms = np.array([a.elapsed_time(b) for a, b in events.values()])
    ms_per_step = wall * 1e3 / args.steps

    # Steps after evicting the 256 MiB MALL (outside any timed region), two
    # ways: reading a 512 MiB buffer leaves the cache holding clean lines, so
    # the step pays only for the misses; writing it leaves dirty lines whose
    # write-back to HBM then overlaps the step.
    cold_ms = cold_write_ms = None
    if args.cold_steps:
        sweep = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        cold, cold_write = [], []
        for _ in range(args.cold_steps):
            for kind, acc in (("read", cold), ("write", cold_write)):
                if kind == "read":
                    sweep.sum()
                else:
                    sweep.fill_(1.0)
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                step(ev)
                torch.cuda.synchronize()
                acc.append(ev[0].elapsed_time(ev[1]))
        cold_ms = float(np.median(cold))
        cold_write_ms = float(np.median(cold_write))
        del sweep

    probe = read_ceiling(pa, k, v, w, args.workers, shared=shared) if args.probe else None

    # Bytes the step must read: every cached token's K and V rows for every
    # KV head -- with the groups, each group's shared tokens once.
    kv = w.kv_shared_read_bytes if shared else w.kv_bytes
    avg_kernel_s = float(kernel_ms.mean()) / 1e3
    achieved = kv / avg_kernel_s / 1e9
    value = kv / (ms_per_step / 1e3) / 1e9
    kernel = attention_kernel_name(w, shared)
    traffic = counter_traffic(w.name + ("" if shared or w.group_start is None else "_plain"),
                              kernel)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_s,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
            "context_tokens": int(w.context_lens.sum()), "kv_bytes_per_step": kv,
            "logical_kv_bytes_per_step": w.kv_bytes,
            "step": ("copy + " if pairs is not None else "")
                    + ("fused append + " if slots is not None else "")
                    + ("decode with shared prefixes read once per group" if shared else "decode"),
            "groups": None if w.group_start is None else int(len(w.group_start) - 1),
            "workers": args.workers or "default",
        },
        "logical_kv_gbps": round(w.kv_bytes / (ms_per_step / 1e3) / 1e9, 2),
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_per_step / 1e3), 1),
        "decode_kernel_ms": {"launches_timed": len(kernel_ms),
                             "mean": round(float(kernel_ms.mean()), 5),
                             "median": round(float(np.median(kernel_ms)), 5),
                             "p10": round(float(np.percentile(kernel_ms, 10)), 5),
                             "p90": round(float(np.percentile(kernel_ms, 90)), 5),
                             "cold_median_after_mall_read_sweep":
                                 None if cold_ms is None else round(cold_ms, 5),
                             "cold_median_after_mall_write_sweep":
                                 None if cold_write_ms is None else round(cold_write_ms, 5)},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "kernel_source_sha256_16": kernel_source_hash(kernel),
        },
        "device": torch.cuda.get_device_name(dev),
        "host": platform.node(),
    }
    if probe is not None:
        probe["attention_kernel_frac_of_decode_order"] = round(
            achieved / probe["decode_order_gbps"], 4)
        result["read_ceiling_probe"] = probe
    if args.cpu_seconds > 0:
        log("timing the CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
