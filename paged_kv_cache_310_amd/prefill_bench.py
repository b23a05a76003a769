"""Multi-token (prefill) attention timing: ``python -m
paged_kv_cache_310_amd.prefill_bench [--workload NAME]`` prints one JSON line
per workload.

The timed call is ``pa_prefill`` alone (the chunk's append runs once before
timing) with the library's automatic context split (``num_splits=0``: no
split unless the batch's row tiles leave the device underfilled; then the
split kernel and the merge of the split rows are both timed); inputs are
resident in HBM.  Device time comes from HIP events on
the stream the call uses, averaged over ``--iters`` calls after at least
``--warmup-s`` seconds of untimed calls.  Algorithmic work: every query row
(query token x query head) at position p costs 4 * head_dim * (p + 1) flops
-- a multiply and an add per element of q.K over its p + 1 visible keys and
of P.V -- so ``tflops`` is against the dense bf16 matrix-core peak of
2.5 PFLOP/s; ``kv_gbps`` counts the K and V bytes of every cached token once
per (sequence, KV head) (the HBM floor).
"""

from __future__ import annotations

import argparse
import json
import time

import numpy as np
import torch

from . import workloads as wl

PEAK_TFLOPS = 2500.0
PEAK_GBPS = 8000.0


def algorithmic_flops(w: wl.PrefillWorkload) -> int:
    total = 0
    for s in range(w.num_seqs):
        L, n = int(w.context_lens[s]), int(w.query_lens[s])
        # positions L-n .. L-1 see L-n+1 .. L keys
        total += (n * (L - n + 1) + n * (n - 1) // 2) * w.num_q_heads
    return 4 * w.head_dim * total


def run(name: str, iters: int, warmup_s: float) -> dict:
    import paged_kv_cache_310_amd as pa
    w = wl.make_prefill_workload(name, poison=False)
    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    k, v = to_dev(w.k_cache), to_dev(w.v_cache)
    pa.pa_append_kv(k, v, to_dev(w.k_new), to_dev(w.v_new), to_dev(w.slot_mapping))
    q, tab = to_dev(w.q), to_dev(w.block_tables)
    lens, qs = to_dev(w.context_lens), to_dev(w.query_start)
    out = torch.empty_like(q)
    mq = w.max_query_len
    splits, nbytes = pa.pa_prefill_split_plan(w.num_seqs, mq, w.num_query_tokens, w.num_q_heads,
                                              w.num_kv_heads, w.head_dim, w.block_size,
                                              w.block_tables.shape[1], 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def call():
        pa.pa_prefill(q, k, v, tab, lens, qs, float(w.scale), max_query_len=mq, out=out,
                      num_splits=0, workspace=ws)

    t_end = time.perf_counter() + warmup_s
    while time.perf_counter() < t_end:
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        call()
    e1.record()
    e1.synchronize()
    us = e0.elapsed_time(e1) / iters * 1e3
    flops = algorithmic_flops(w)
    kv = int(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim * 2
    tflops = flops / us / 1e6
    return {
        "metric": "paged prefill attention: achieved TFLOP/s (bf16 matrix cores)",
        "workload": name, "num_seqs": w.num_seqs, "query_tokens": w.num_query_tokens,
        "cached_tokens": int(w.context_lens.sum()), "heads": [w.num_q_heads, w.num_kv_heads],
        "context_splits": splits, "us_per_call": round(us, 2), "algorithmic_flops": flops,
        "tflops": round(tflops, 1), "peak_tflops": PEAK_TFLOPS,
        "frac": round(tflops / PEAK_TFLOPS, 4),
        "kv_gbps": round(kv / us / 1e3, 1),
        "query_tokens_per_s": round(w.num_query_tokens / us * 1e6, 0),
    }


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--workload", choices=wl.PREFILL_WORKLOADS, action="append")
    p.add_argument("--iters", type=int, default=50)
    p.add_argument("--warmup-s", type=float, default=0.6)
    a = p.parse_args()
    for name in a.workload or wl.PREFILL_WORKLOADS:
        print(json.dumps(run(name, a.iters, a.warmup_s)), flush=True)


if __name__ == "__main__":
    main()
