"""Timing of the host block manager (libpabm.so) on the operations a serving
step makes; prints one JSON line.  ``python -m paged_kv_cache_310_amd.bm_bench``.

* decode step: one slot per sequence for 256 sequences (one
  ``append_slots`` call), repeated over 512 steps from lengths 1..2048;
* prefix admission: 64 sequences that share a 1024-token prompt prefix, each
  registered with its token ids (the first allocates, the rest reuse);
* beam churn: 32 beams per request, each step forks the 8 best beams 4 ways,
  frees the rest (one batched free and one batched fork call) and appends one
  token to every beam (copy-on-write of the shared tail blocks).
Times are host wall clock, median of repeats, in microseconds.
"""

from __future__ import annotations

import json
import platform
import time

import numpy as np

from .kv_block_manager import KVBlockManager


def _median_us(fn, repeats: int = 5) -> float:
    t = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        fn()
        t.append(time.perf_counter() - t0)
    return float(np.median(t)) * 1e6


def decode_steps(num_seqs: int = 256, steps: int = 512, bs: int = 16) -> float:
    rng = np.random.default_rng(0)
    lens = rng.integers(1, 2049, size=num_seqs)
    blocks = int(sum(-(-(int(n) + steps) // bs) for n in lens)) + 16

    def run():
        m = KVBlockManager(blocks, bs)
        for s, n in enumerate(lens):
            m.add_sequence(s, int(n))
        seqs = np.arange(num_seqs)
        t0 = time.perf_counter()
        for _ in range(steps):
            m.append_slots(seqs)
        run.elapsed = time.perf_counter() - t0

    run()
    best = []
    for _ in range(3):
        run()
        best.append(run.elapsed)
    return float(np.median(best)) / steps * 1e6


def prefix_admission(n: int = 64, prefix: int = 1024, tail: int = 64, bs: int = 16) -> float:
    rng = np.random.default_rng(1)
    shared = rng.integers(0, 32000, size=prefix).astype(np.int32)
    prompts = [np.concatenate([shared, rng.integers(0, 32000, size=tail).astype(np.int32)])
               for _ in range(n)]

    def run():
        m = KVBlockManager(n * (prefix + tail) // bs + 64, bs, prefix_cache=True)
        for s, p in enumerate(prompts):
            m.add_sequence(s, tokens=p)
        assert m.stats()["prefix_hit_blocks"] == (n - 1) * (prefix // bs)

    return _median_us(run) / n


def beam_churn(beams: int = 32, keep: int = 8, steps: int = 64, prompt: int = 500,
               bs: int = 16) -> float:
    def run():
        m = KVBlockManager(4096, bs)
        m.add_sequence(0, prompt)
        live = [0]
        nxt = 1
        for b in range(1, beams):
            m.fork(0, nxt)
            live.append(nxt)
            nxt += 1
        t0 = time.perf_counter()
        for _ in range(steps):
            survivors, dead = live[:keep], live[keep:]
            m.free_many(dead)
            live, parents, children = [], [], []
            for s in survivors:
                live.append(s)
                for _ in range(beams // keep - 1):
                    parents.append(s)
                    children.append(nxt)
                    live.append(nxt)
                    nxt += 1
            m.fork_many(parents, children)
            m.append_slots(live)
        run.elapsed = time.perf_counter() - t0

    run()
    best = []
    for _ in range(3):
        run()
        best.append(run.elapsed)
    return float(np.median(best)) / steps * 1e6


def main():
    result = {
        "metric": "host block manager: microseconds per operation (lower is better)",
        "decode_step_256_seqs_us": round(decode_steps(), 2),
        "prefix_admission_per_seq_us": round(prefix_admission(), 2),
        "beam_churn_step_32_beams_us": round(beam_churn(), 2),
        "host": platform.node(),
        "cpu": platform.processor() or platform.machine(),
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
