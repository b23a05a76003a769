"""Beam-search churn, timed end to end on one layer.

``python -m paged_kv_cache_310_amd.beam_bench`` prints one JSON line.
Workload (LLaMA-13B-shaped heads: 40 KV heads, head_dim 128, bf16, 16-token
blocks): 16 requests, each a 1000-token prompt (so its last prompt block is
partly filled) searched with 8 beams.  Every step keeps 2 seeded survivors per
request, forks each back to 8 beams (one batched free and one batched fork
call for all requests), asks the host block manager (libpabm.so) for the
slots, the copy-on-write pairs and what each request's beams share
(pa_bm_shared_prefix), and runs pa_copy_blocks and a fused append +
pa_decode_shared for all 128 beams, each request's beams one group
(``--plain``: pa_decode).

Reported per step: wall-clock time of the whole step (host manager + uploads
+ device work), the host's shares (the manager with the survivor choice, the
uploads -- synchronous copies from pageable memory, which wait for the step
before -- and the launches), device time of the copy and of the
decode (HIP events on the stream the calls use, sampled every 10th step so the
events do not slow the loop), copies per step, and the decode's KV read rate
in algorithmic bytes (every cached token's K and V rows of every beam, shared
blocks counted once per beam that reads them -- the logical bytes).
"""

from __future__ import annotations

import argparse
import json
import time

import numpy as np
import torch


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--requests", type=int, default=16)
    p.add_argument("--width", type=int, default=8)
    p.add_argument("--keep", type=int, default=2)
    p.add_argument("--prompt", type=int, default=1000)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--plain", dest="shared", action="store_false",
                   help="decode with pa_decode instead of pa_decode_shared (each request's "
                        "beams as one group)")
    return p.parse_args()


def main():
    a = _args()
    import paged_kv_cache_310_amd as pa
    from paged_kv_cache_310_amd.kv_block_manager import KVBlockManager
    dev = torch.device("cuda:0")
    hkv, hq, bs, d = 40, 40, 16, 128
    steps_total = a.warmup + a.steps
    per_req = -(-a.prompt // bs) + a.width * (-(-steps_total // bs) + 2)
    nb = a.requests * per_req + 64
    rng = np.random.default_rng(0)
    k = torch.randn(nb, hkv, bs, d, device=dev).bfloat16()
    v = torch.randn(nb, hkv, bs, d, device=dev).bfloat16()
    b = a.requests * a.width
    q = torch.randn(b, hq, d, device=dev).bfloat16()
    kn = torch.randn(b, hkv, d, device=dev).bfloat16()
    vn = torch.randn(b, hkv, d, device=dev).bfloat16()
    out = torch.empty_like(q)
    ws = pa.decode_workspace(dev, pa.pa_decode_shared_workspace_size(b, hq, hkv, d))
    # Each request's beams are one group: they share the prompt's blocks.
    starts = np.arange(0, b + 1, a.width, dtype=np.int64)
    starts_d = torch.from_numpy(starts.astype(np.int32)).to(dev)
    scale = 1.0 / np.sqrt(d)

    mgr = KVBlockManager(nb, bs, free_order=rng.permutation(nb))
    beams, next_id = [], 0
    for r in range(a.requests):
        root = next_id
        mgr.add_sequence(root, a.prompt)
        group = [root]
        next_id += 1
        for _ in range(a.width - 1):
            mgr.fork(root, next_id)
            group.append(next_id)
            next_id += 1
        beams.append(group)
    max_blocks = -(-(a.prompt + steps_total) // bs)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    rec = {"wall": [], "mgr": [], "upload": [], "launch": [], "copy": [], "decode": [],
           "copies": [], "kv": []}

    def step(sample: bool, timed: bool):
        nonlocal next_id
        t0 = time.perf_counter()
        live, dead, parents, children = [], [], [], []
        for r in range(a.requests):
            group = beams[r]
            survivors = sorted(rng.choice(group, size=a.keep, replace=False).tolist())
            dead.extend(s for s in group if s not in survivors)
            group = []
            for s in survivors:
                group.append(s)
                for _ in range(a.width // a.keep - 1):
                    parents.append(s)
                    children.append(next_id)
                    group.append(next_id)
                    next_id += 1
            beams[r] = group
            live.extend(group)
        mgr.free_many(dead)
        mgr.fork_many(parents, children)
        slots, copies = mgr.append_slots(live)
        tables, lens = mgr.block_tables(live, max_blocks=max_blocks)
        prefix = mgr.shared_prefix(live, starts) if a.shared else None
        t1 = time.perf_counter()
        slots_d = torch.from_numpy(slots).to(dev)
        tables_d = torch.from_numpy(tables).to(dev)
        lens_d = torch.from_numpy(lens).to(dev)
        copies_d = torch.from_numpy(copies).to(dev) if len(copies) else None
        prefix_d = torch.from_numpy(prefix).to(dev) if a.shared else None
        t2 = time.perf_counter()
        if sample:
            ev[0].record()
        if copies_d is not None:
            pa.pa_copy_blocks(k, v, copies_d)
        if sample:
            ev[1].record()
        if a.shared:
            pa.pa_decode_shared(q, k, v, tables_d, lens_d, float(scale), starts_d,
                                prefix_d, out=out, k_new=kn, v_new=vn,
                                slot_mapping=slots_d, workspace=ws)
        else:
            pa.pa_decode(q, k, v, tables_d, lens_d, float(scale), out=out, k_new=kn, v_new=vn,
                         slot_mapping=slots_d, workspace=ws)
        if sample:
            ev[2].record()
            ev[2].synchronize()
            rec["copy"].append(ev[0].elapsed_time(ev[1]) * 1e3)
            rec["decode"].append(ev[1].elapsed_time(ev[2]) * 1e3)
            rec["kv"].append(int(lens.astype(np.int64).sum()) * 2 * hkv * d * 2)
        if timed:
            t3 = time.perf_counter()
            rec["mgr"].append((t1 - t0) * 1e6)
            rec["upload"].append((t2 - t1) * 1e6)
            rec["launch"].append((t3 - t2) * 1e6)
            rec["copies"].append(len(copies))

    for _ in range(a.warmup):
        step(False, False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(a.steps):
        step(i % 10 == 9, True)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) / a.steps * 1e6
    mgr.check()
    decode_us = float(np.median(rec["decode"]))
    kv = float(np.median(rec["kv"]))
    print(json.dumps({
        "metric": "beam-search churn step, microseconds (lower is better)",
        "workload": f"llama13b heads, {a.requests} requests x {a.width} beams, prompt "
                    f"{a.prompt}, keep {a.keep}",
        "decode": "pa_decode_shared (each request's beams one group)" if a.shared
                  else "pa_decode",
        "steps": a.steps, "pool_blocks": nb,
        "step_us_wall": round(wall, 1),
        "manager_us": round(float(np.median(rec["mgr"])), 1),
        "upload_us": round(float(np.median(rec["upload"])), 1),
        "launch_us": round(float(np.median(rec["launch"])), 1),
        "copy_gpu_us": round(float(np.median(rec["copy"])), 1),
        "decode_gpu_us": round(decode_us, 1),
        "copies_per_step": round(float(np.mean(rec["copies"])), 1),
        "decode_kv_gbps": round(kv / decode_us / 1e3, 1),
        "peak_gbps": 8000.0,
    }))


if __name__ == "__main__":
    main()
