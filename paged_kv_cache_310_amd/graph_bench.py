"""Decode step launched eagerly against the same step replayed from a HIP graph.

``python -m paged_kv_cache_310_amd.graph_bench [--workloads tiny_fp32,...]``
prints one JSON line per workload. The step is the one bench.py times:
* ``pa_copy_blocks``, when the workload has copy pairs;
* ``pa_decode`` with the newest token appended in the same launch, when the
  workload appends;
* decode attention and the merge of split segments.

Eager: the calls are enqueued one by one. Graph: one step is captured with
``torch.cuda.graph`` (workspace and outputs allocated beforehand) and replayed.
The two forms run interleaved: 7 rounds of ``--iters`` steps each, after a
warm-up. Times are HIP events on the stream the steps use, median per form.
A replayed graph must give the eager result bit for bit, checked before timing.
"""

from __future__ import annotations

import argparse
import json
import time

import numpy as np
import torch


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--workloads", default="tiny_fp32,gqa_pareto_bs16,llama13b_long")
    p.add_argument("--iters", type=int, default=50)
    p.add_argument("--warmup-s", type=float, default=0.3)
    return p.parse_args()


def _to_dev(a, dev):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def run(name: str, iters: int, warmup_s: float) -> dict:
    import paged_kv_cache_310_amd as pa
    from . import workloads as wl
    dev = torch.device("cuda:0")
    w = wl.make_workload(name, poison=False)
    q, k, v = _to_dev(w.q, dev), _to_dev(w.k_cache, dev), _to_dev(w.v_cache, dev)
    tab, lens = _to_dev(w.block_tables, dev), _to_dev(w.context_lens, dev)
    kn, vn = _to_dev(w.k_new, dev), _to_dev(w.v_new, dev)
    slots, pairs = _to_dev(w.slot_mapping, dev), _to_dev(w.block_mapping, dev)
    ws = torch.zeros(pa.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def step():
        if pairs is not None:
            pa.pa_copy_blocks(k, v, pairs)
        pa.pa_decode(q, k, v, tab, lens, float(w.scale), out=out, k_new=kn, v_new=vn,
                     slot_mapping=slots, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out.view(torch.uint8), ref.view(torch.uint8)):
        raise RuntimeError(f"{name}: graph replay differs from the eager step")

    forms = {"eager": step, "graph": g.replay}
    t_end = time.perf_counter() + warmup_s
    while time.perf_counter() < t_end:
        for fn in forms.values():
            fn()
        torch.cuda.synchronize()
    times = {f: [] for f in forms}
    for _ in range(7):
        for f, fn in forms.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            e1.synchronize()
            times[f].append(e0.elapsed_time(e1) * 1e3 / iters)
    res = {f: round(float(np.median(t)), 2) for f, t in times.items()}
    return {"metric": "decode step, microseconds: eager launches vs HIP graph replay",
            "workload": name, "kv_bytes_per_step": w.kv_bytes,
            "step": ("copy + " if pairs is not None else "")
                    + ("fused append + decode" if slots is not None else "decode"),
            "eager_us": res["eager"], "graph_us": res["graph"],
            "eager_gbps": round(w.kv_bytes / res["eager"] / 1e3, 1),
            "graph_gbps": round(w.kv_bytes / res["graph"] / 1e3, 1),
            "graph_speedup": round(res["eager"] / res["graph"], 3)}


def main():
    a = _args()
    torch.cuda.set_device(0)
    for name in a.workloads.split(","):
        print(json.dumps(run(name, a.iters, a.warmup_s)), flush=True)


if __name__ == "__main__":
    main()
