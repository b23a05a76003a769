"""Prefill with the context split over several workgroups per row tile
(pa_prefill_split) on the GPU against the oracle.

The split changes only the fp32 summation order, so every case is held to
the same bf16 tolerance as pa_prefill (max-abs 2e-2, row max-rel 1e-2):
* forced split counts on ragged batches, where short contexts leave later
  splits with no key at all and rows see no key in some splits;
* contexts past one LDS table window, so splits start inside a window and
  cross into the next;
* a zero and a negative scale;
* the automatic choice on single long sequences with short chunks (the case
  splitting is for), on sampled rows;
* repeat calls give identical bytes, and a workspace serves a smaller call;
* PA_CHECK=1 rejects broken index arrays, and split counts past 32 are
  rejected.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import assert_attention_close, out_f64, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def device_inputs(w):
    import paged_kv_cache_310_amd as pa
    k, v = to_dev(w.k_cache), to_dev(w.v_cache)
    if w.num_query_tokens:
        pa.pa_append_kv(k, v, to_dev(w.k_new), to_dev(w.v_new), to_dev(w.slot_mapping))
    return dict(q=to_dev(w.q), k_cache=k, v_cache=v, block_tables=to_dev(w.block_tables),
                context_lens=to_dev(w.context_lens), query_start=to_dev(w.query_start),
                scale=float(w.scale), max_query_len=w.max_query_len)


def run_split(w, splits, workspace=None, inputs=None):
    import paged_kv_cache_310_amd as pa
    d = device_inputs(w) if inputs is None else inputs
    out = pa.pa_prefill(**d, num_splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return out


def oracle_rows(w, rows=None):
    import oracle
    k, v = oracle.append_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    return oracle.prefill(w.q, k, v, w.block_tables, w.context_lens, w.query_start, w.scale,
                          w.dtype, w.block_size, rows=rows)


# (context length, chunk length): one-step contexts (later splits get no
# step), chunks on long earlier contexts (rows see no key in some splits),
# fresh prompts across the 128-row tile edge, an empty chunk.
RAGGED = [(1, 1), (17, 17), (100, 100), (200, 200), (2000, 40), (1000, 1), (513, 130),
          (77, 0), (3000, 3)]


@pytest.mark.parametrize("splits", [2, 3, 5, 16, 32])
@pytest.mark.parametrize("hq,hkv,bs", [(8, 2, 16), (40, 40, 16), (16, 2, 32)])
def test_forced_splits_ragged(hq, hkv, bs, splits):
    say("prefill split ragged", hq, hkv, bs, splits)
    w = wl.make_prefill("split", 700 + hq + bs, wl.BF16, hq, hkv, 128, bs,
                        [c for c, _ in RAGGED], [n for _, n in RAGGED])
    err = assert_attention_close(out_f64(run_split(w, splits)), oracle_rows(w), wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("splits", [3, 7, 16, 32])
@pytest.mark.parametrize("bs", [16, 32])
def test_splits_cross_table_windows(bs, splits):
    """Contexts of 20k-40k keys span several 1024-entry table windows: split
    boundaries fall inside windows."""
    say("prefill split long", bs, splits)
    w = wl.make_prefill("splitlong", 720 + bs, wl.BF16, 4, 2, 128, bs, [40000, 20000, 33000],
                        [64, 1, 5])
    err = assert_attention_close(out_f64(run_split(w, splits)), oracle_rows(w), wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


# (block size, context, splits) whose split of one query token starts one
# step before, two steps before, or on the first step of a block-table window
# (512 steps of 32 keys at 16-token blocks, 1,024 at 32): split 7 of 8 over
# 580 steps starts at step 511, split 6 of 7 over 590 at 510, split 8 of 9
# over 570 at 512, and split 3 of 4 over 1,362 at 1,023.
WINDOW_EDGES = [(16, 18560, 8), (16, 18880, 7), (16, 18240, 9), (32, 43584, 4)]


@pytest.mark.parametrize("bs,ctx,splits", WINDOW_EDGES)
def test_split_starts_at_table_window_edges(bs, ctx, splits):
    """A split's first step reads its table entries directly and later ones
    through the staged window, restaged a step ahead of each boundary: a
    split that starts just before, or on, a window boundary still reads every
    block through the right window."""
    say("prefill split window edge", bs, ctx, splits)
    w = wl.make_prefill("splitedge", 760 + splits, wl.BF16, 4, 2, 128, bs, [ctx], [1])
    err = assert_attention_close(out_f64(run_split(w, splits)), oracle_rows(w), wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_split_any_scale(scale):
    w = wl.make_prefill("splitscale", 730, wl.BF16, 8, 2, 128, 16, [70, 600, 2000],
                        [70, 5, 64])
    w = wl.PrefillWorkload(**{**w.__dict__, "scale": np.float32(scale)})
    assert_attention_close(out_f64(run_split(w, 4)), oracle_rows(w), wl.BF16)


def test_repeat_is_bitwise_and_workspace_serves_smaller_calls():
    import paged_kv_cache_310_amd as pa
    w = wl.make_prefill("splitrep", 740, wl.BF16, 16, 2, 128, 16, [5000, 3000], [200, 64])
    small = wl.make_prefill("splitrep2", 741, wl.BF16, 16, 2, 128, 16, [2500], [33])
    _, nbytes = pa.pa_prefill_split_plan(2, w.max_query_len, w.num_query_tokens, 16, 2, 128, 16,
                                         w.block_tables.shape[1], 6)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")   # NaN-filled
    d = device_inputs(w)
    a = run_split(w, 6, ws, d)
    b = run_split(w, 6, ws, d)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_attention_close(out_f64(a), oracle_rows(w), wl.BF16)
    got = run_split(small, 6, ws)
    assert_attention_close(out_f64(got), oracle_rows(small), wl.BF16)


def _sample(w, n_tokens, heads, seed):
    rng = np.random.default_rng(seed)
    t = w.num_query_tokens
    toks = sorted(set([0, t - 1] + list(rng.integers(0, t, n_tokens))))
    return [(tok, int(h)) for tok in toks for h in rng.choice(w.num_q_heads, heads, False)]


@pytest.mark.parametrize("ctx,nq", [(32768, 64), (8192, 16), (4096, 512)])
def test_auto_split_single_long_sequence(ctx, nq):
    """One sequence of 64 query / 8 KV heads: the automatic choice splits
    (the row tiles alone would occupy a few dozen workgroups)."""
    import paged_kv_cache_310_amd as pa
    w = wl.make_prefill("splitauto", 750, wl.BF16, 64, 8, 128, 16, [ctx], [nq])
    splits, nbytes = pa.pa_prefill_split_plan(1, nq, nq, 64, 8, 128, 16,
                                              w.block_tables.shape[1], 0)
    say("auto split", ctx, nq, "->", splits, "splits", nbytes, "bytes")
    assert splits > 1
    got = out_f64(run_split(w, 0))
    assert np.all(np.isfinite(got))
    rows = _sample(w, 6, 8, 751)
    err = assert_attention_close(got, oracle_rows(w, rows=rows), wl.BF16, rows=rows)
    say("max-abs %.3e row-rel %.3e" % err)


def test_split_checks_contract_under_pa_check():
    """PA_CHECK=1 validates the index arrays of pa_prefill_split as it does
    pa_prefill's, before launching; split counts past 32 are rejected."""
    import os
    import subprocess
    import sys
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
S = dict(num_splits=3)
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([0, 2, 5]), 0.1, **S)))
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 2]), i32([0, 2, 5]), 0.1, **S)))
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([1, 2, 5]), 0.1, **S)))
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([40, 3]), i32([0, 2, 5]), 0.1, **S)))
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([0, 2, 5]), 0.1, num_splits=33)))
print(status(lambda: pa.pa_prefill(q, k, v, tab, i32([20, 3]), i32([0, 2, 5]), 0.1, num_splits=0)))
"""
    env = dict(os.environ, PA_CHECK="1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120, cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert res.returncode == 0, res.stderr
    assert res.stdout.split() == ["0", "5", "5", "5", "1", "0"], res.stdout
