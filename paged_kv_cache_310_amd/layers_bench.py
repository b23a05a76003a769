"""Whole-model append and copy: per-layer calls against one layer-batched call.

``python -m paged_kv_cache_310_amd.layers_bench [--layers 40]`` prints one
JSON line.  Workload: the LLaMA-13B-shaped shared-prefix decode step (40 KV
heads, head_dim 128, bf16, 16-token blocks, 128 sequences = 16 prompt groups x
8 samples) repeated over every layer of the model: each step appends one token
per sequence (128 distinct random slots of a 2700-block pool per layer) and
copies 16 shared tail blocks to fresh blocks (copy-on-write), in every
layer's pools.  Times come from HIP events on the stream the calls use,
averaged over ``--iters`` steps after a warm-up; ``gbps`` counts algorithmic
bytes (each copied or appended byte read once and written once).
"""

from __future__ import annotations

import argparse
import json
import time

import numpy as np
import torch


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--layers", type=int, default=40)
    p.add_argument("--seqs", type=int, default=128)
    p.add_argument("--copies", type=int, default=16)
    p.add_argument("--blocks", type=int, default=2700)
    p.add_argument("--iters", type=int, default=200)
    p.add_argument("--warmup-s", type=float, default=0.6)
    return p.parse_args()


def main():
    a = _args()
    import paged_kv_cache_310_amd as pa
    dev = torch.device("cuda:0")
    hkv, bs, d = 40, 16, 128
    rng = np.random.default_rng(0)
    ks = [torch.zeros(a.blocks, hkv, bs, d, dtype=torch.bfloat16, device=dev)
          for _ in range(a.layers)]
    vs = [torch.zeros_like(k) for k in ks]
    kn = [torch.randn(a.seqs, hkv, d, device=dev).bfloat16() for _ in range(a.layers)]
    vn = [torch.randn(a.seqs, hkv, d, device=dev).bfloat16() for _ in range(a.layers)]
    slots = torch.from_numpy(rng.choice(a.blocks * bs, a.seqs, replace=False).astype(np.int64))
    perm = rng.permutation(a.blocks)
    pairs = np.stack([perm[: a.copies], perm[a.copies: 2 * a.copies]], axis=1).astype(np.int64)
    slots, pairs = slots.to(dev), torch.from_numpy(pairs).to(dev)

    def per_layer():
        for l in range(a.layers):
            pa.pa_copy_blocks(ks[l], vs[l], pairs)
            pa.pa_append_kv(ks[l], vs[l], kn[l], vn[l], slots)

    def batched():
        pa.pa_copy_blocks_layers(ks, vs, pairs)
        pa.pa_append_kv_layers(ks, vs, kn, vn, slots)

    def measure(fn):
        t_end = time.perf_counter() + a.warmup_s
        while time.perf_counter() < t_end:
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for _ in range(a.iters):
            fn()
        e1.record()
        e1.synchronize()
        host = (time.perf_counter() - h0) / a.iters
        return e0.elapsed_time(e1) / a.iters * 1e3, host * 1e6

    block_bytes = hkv * bs * d * 2
    algo = a.layers * 2 * (2 * a.copies * block_bytes + 2 * a.seqs * hkv * d * 2)
    # interleave the two forms so neither is favoured by clocks settling
    res = {"per_layer": [], "batched": []}
    for _ in range(3):
        res["per_layer"].append(measure(per_layer))
        res["batched"].append(measure(batched))
    out = {}
    for k, v in res.items():
        gpu_us = float(np.median([x[0] for x in v]))
        host_us = float(np.median([x[1] for x in v]))
        out[k] = {"gpu_us_per_step": round(gpu_us, 2), "host_us_per_step": round(host_us, 2),
                  "gbps": round(algo / gpu_us / 1e3, 1)}
    print(json.dumps({
        "metric": "multi-layer append + copy-on-write copy, microseconds per model step",
        "workload": "llama13b shared-prefix step x layers",
        "layers": a.layers, "seqs": a.seqs, "copies": a.copies, "pool_blocks": a.blocks,
        "algorithmic_bytes_per_step": algo, "launches_per_step":
            {"per_layer": 2 * a.layers, "batched": 2 * ((a.layers + 31) // 32)},
        **out,
        "speedup_gpu": round(out["per_layer"]["gpu_us_per_step"]
                             / out["batched"]["gpu_us_per_step"], 2),
        "peak_gbps": 8000.0,
    }))


if __name__ == "__main__":
    main()
