"""Multi-token (prefill) attention on the GPU against the oracle.

The chunk's keys/values are appended with pa_append_kv first (pools start
poisoned with NaN at those slots and at every slot no sequence holds), then
pa_prefill runs; every output row is compared with ``oracle.prefill`` on
small ragged cases, sampled rows on the full-size workloads, within the bf16
tolerance (max-abs 2e-2, row max-rel 1e-2)."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import assert_attention_close, out_f64, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_device(w, max_query_len=None):
    import paged_kv_cache_310_amd as pa
    k, v = to_dev(w.k_cache), to_dev(w.v_cache)
    if w.num_query_tokens:
        pa.pa_append_kv(k, v, to_dev(w.k_new), to_dev(w.v_new), to_dev(w.slot_mapping))
    out = pa.pa_prefill(to_dev(w.q), k, v, to_dev(w.block_tables), to_dev(w.context_lens),
                        to_dev(w.query_start), float(w.scale),
                        max_query_len=w.max_query_len if max_query_len is None else max_query_len)
    torch.cuda.synchronize()
    return out


def oracle_rows(w, rows=None):
    import oracle
    k, v = oracle.append_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    return oracle.prefill(w.q, k, v, w.block_tables, w.context_lens, w.query_start, w.scale,
                          w.dtype, w.block_size, rows=rows)


# (context length, chunk length) per sequence: fresh prompts across the
# 32-key step and 128-row tile edges, chunks on top of earlier context, a
# one-token chunk (a decode step) and an empty chunk.
RAGGED = [(1, 1), (15, 15), (16, 16), (17, 17), (33, 33), (100, 100), (200, 200),
          (300, 64), (1000, 1), (513, 130), (77, 0), (64, 33)]
SHAPES = [(40, 40, 16), (4, 4, 32), (8, 2, 16), (16, 2, 32), (64, 8, 16), (6, 2, 16),
          (32, 2, 16)]


@pytest.mark.parametrize("hq,hkv,bs", SHAPES)
def test_small_ragged(hq, hkv, bs):
    say("prefill small", hq, hkv, bs)
    ctx = [c for c, _ in RAGGED]
    nq = [n for _, n in RAGGED]
    w = wl.make_prefill("small", 600 + hq + bs, wl.BF16, hq, hkv, 128, bs, ctx, nq)
    got = out_f64(run_device(w))
    ref = oracle_rows(w)
    err = assert_attention_close(got, ref, wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("nseq", [64, 65, 130])
def test_many_sequences(nseq):
    """Batches of up to 64 sequences take each sequence's chunk bounds from
    the lanes that summed the batch; larger ones read them again: both sides
    of that edge, ragged fresh prompts and chunks."""
    say("prefill many sequences", nseq)
    rng = np.random.default_rng(700 + nseq)
    ctx = [int(x) for x in rng.integers(1, 90, nseq)]
    nq = [int(rng.integers(0, c + 1)) if i % 3 else c for i, c in enumerate(ctx)]
    w = wl.make_prefill("many", 710 + nseq, wl.BF16, 8, 2, 128, 16, ctx, nq)
    got = out_f64(run_device(w))
    ref = oracle_rows(w)
    err = assert_attention_close(got, ref, wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("bs", [16, 32])
def test_long_context_crosses_table_windows(bs):
    """Contexts past 1024 table entries: the kernel restages its LDS copy of
    the block table while walking the keys."""
    say("prefill long", bs)
    w = wl.make_prefill("long", 620 + bs, wl.BF16, 4, 2, 128, bs, [40000, 20000, 33000],
                        [64, 1, 5])
    got = out_f64(run_device(w))
    ref = oracle_rows(w)
    err = assert_attention_close(got, ref, wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_any_scale(scale):
    """A negative scale (the kernel flips q's sign), zero (uniform weights
    over the visible keys) and a large one (peaked weights)."""
    w = wl.make_prefill("scale", 630, wl.BF16, 8, 2, 128, 16, [70, 33, 200], [70, 5, 64])
    w = wl.PrefillWorkload(**{**w.__dict__, "scale": np.float32(scale)})
    got = out_f64(run_device(w))
    assert_attention_close(got, oracle_rows(w), wl.BF16)


def test_max_query_len_larger_than_needed_changes_nothing():
    w = wl.make_prefill("slack", 611, wl.BF16, 8, 2, 128, 16, [90, 40, 7], [90, 12, 7])
    a = run_device(w)
    b = run_device(w, max_query_len=700)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_physical_permutation_gives_bitwise_identical_output():
    w = wl.make_prefill("perm", 612, wl.BF16, 16, 4, 128, 16, [300, 45, 129], [200, 45, 1])
    a = run_device(w)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.num_blocks)              # new physical id of each block
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1)
    slots = perm[w.slot_mapping // w.block_size] * w.block_size + w.slot_mapping % w.block_size
    w2 = wl.PrefillWorkload(**{**w.__dict__, "k_cache": k, "v_cache": v,
                               "block_tables": tables.astype(np.int32),
                               "slot_mapping": slots.astype(np.int64)})
    b = run_device(w2)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_one_chunk_equals_two_chunks():
    """A prompt run as one chunk and as two (the second on top of the first)
    agree within rounding, and each agrees with the oracle."""
    import paged_kv_cache_310_amd as pa
    L, first = 700, 260
    w = wl.make_prefill("whole", 613, wl.BF16, 8, 8, 128, 16, [L], [L])
    whole = out_f64(run_device(w))
    k, v = to_dev(w.k_cache), to_dev(w.v_cache)
    pa.pa_append_kv(k, v, to_dev(w.k_new), to_dev(w.v_new), to_dev(w.slot_mapping))
    tab = to_dev(w.block_tables)
    q = to_dev(w.q)
    a = pa.pa_prefill(q[:first].contiguous(), k, v, tab, to_dev(np.asarray([first], np.int32)),
                      to_dev(np.asarray([0, first], np.int32)), float(w.scale))
    b = pa.pa_prefill(q[first:].contiguous(), k, v, tab, to_dev(np.asarray([L], np.int32)),
                      to_dev(np.asarray([0, L - first], np.int32)), float(w.scale))
    torch.cuda.synchronize()
    split = np.concatenate([out_f64(a), out_f64(b)])
    ref = oracle_rows(w)
    assert_attention_close(whole, ref, wl.BF16)
    assert_attention_close(split, ref, wl.BF16)


def test_rejects_unsupported_and_checks_contract():
    code = r"""
import torch
import paged_kv_cache_310_amd as pa
from paged_kv_cache_310_amd._binding import PAError
d = 'cuda:0'
k = torch.zeros(8, 2, 16, 128, device=d, dtype=torch.bfloat16); v = torch.zeros_like(k)
q = torch.zeros(5, 4, 128, device=d, dtype=torch.bfloat16)
tab = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device=d)
i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=d)
def status(f):
    try:
        f(); torch.cuda.synchronize(); return 0
    except PAError as e:
        return e.status
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([0, 2, 5]), 0.1)))   # valid
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 2]), i32([0, 2, 5]), 0.1)))   # chunk 3 > ctx 2
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([1, 2, 5]), 0.1)))   # start != 0
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([0, 2, 4]), 0.1)))   # end != tokens
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([40, 3]), i32([0, 2, 5]), 0.1)))   # ctx > table
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([0, 2, 5]), 0.1, max_query_len=2)))
kf = torch.zeros(8, 2, 16, 128, device=d); qf = torch.zeros(5, 4, 128, device=d)
print(status(lambda: pa.pa_prefill(qf, kf, kf, tab, i32([20, 3]), i32([0, 2, 5]), 0.1)))
"""
    env = dict(os.environ, PA_CHECK="1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120, cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert res.returncode == 0, res.stderr
    assert res.stdout.split() == ["0", "5", "5", "5", "5", "5", "2"], res.stdout


def _sample_rows(w, seed=0, per_seq=6):
    """(query token, head) pairs per sequence: first and last chunk token and
    seeded middle ones, with the first, last and a seeded head."""
    rng = np.random.default_rng(seed)
    rows = []
    for s in range(w.num_seqs):
        a, b = int(w.query_start[s]), int(w.query_start[s + 1])
        if a == b:
            continue
        toks = {a, b - 1, *rng.integers(a, b, per_seq - 2).tolist()}
        for t in sorted(toks):
            heads = {0, w.num_q_heads - 1, int(rng.integers(0, w.num_q_heads))}
            rows.extend((t, h) for h in sorted(heads))
    return rows


@pytest.mark.parametrize("name", wl.PREFILL_WORKLOADS)
def test_full_size_workload(name):
    say("generating", name)
    w = wl.make_prefill_workload(name)
    say("device", name, "tokens", w.num_query_tokens)
    got = out_f64(run_device(w))
    assert np.all(np.isfinite(got))
    rows = _sample_rows(w)
    say("oracle rows", len(rows))
    ref = oracle_rows(w, rows=rows)
    err = assert_attention_close(got, ref, wl.BF16, rows=rows)
    say(name, "max-abs %.3e row-rel %.3e" % err)
