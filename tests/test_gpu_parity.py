"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Data movement (append, copy) must be bit-exact on the whole pool; attention
must meet the tolerance in ``_gpu_util.assert_attention_close``.  Small
ragged cases compare every output; the full-size workloads (the shapes and
launch configuration the benchmark times) compare the whole pools and a
sample of outputs that covers every sequence.
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import (DeviceWorkload, assert_attention_close, oracle_decode, oracle_pools,
                       out_f64, sample_rows, to_dev, to_host)

pytestmark = pytest.mark.gpu

RAGGED = [1, 15, 16, 17, 33, 100, 255, 300, 513, 2, 64, 1000]


def small(dtype, d, bs, hq, hkv, lens=RAGGED, append=True, seed=5, poison=True, num_blocks=None):
    return wl.make_simple("small", seed, dtype, hq, hkv, d, bs, lens, append=append, poison=poison,
                          num_blocks=num_blocks)


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available()
    import paged_kv_cache_310_amd as pa
    from paged_kv_cache_310_amd import _binding
    assert os.path.exists(_binding.library_path()), "libpa.so is not built"
    say("default workers", pa.pa_decode_default_workers(), torch.cuda.get_device_name(0))
    yield


# ----------------------------------------------------------------- small cases
SHAPES = [(wl.BF16, 128, 16, 8, 8), (wl.BF16, 128, 32, 8, 8), (wl.BF16, 64, 16, 4, 4),
          (wl.BF16, 64, 32, 4, 4), (wl.FP32, 64, 16, 4, 4), (wl.FP32, 64, 32, 4, 4),
          (wl.FP32, 128, 16, 4, 4), (wl.FP32, 128, 32, 2, 2), (wl.BF16, 128, 16, 16, 2),
          (wl.BF16, 128, 32, 8, 1), (wl.FP32, 64, 16, 8, 2),
          # grouped queries on the matrix-core kernel: groups 2, 3, 4, 16
          (wl.BF16, 128, 16, 4, 2), (wl.BF16, 128, 32, 6, 2), (wl.BF16, 128, 16, 16, 4),
          (wl.BF16, 128, 32, 32, 2)]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("dtype,d,bs,hq,hkv", SHAPES)
def test_small_ragged(dtype, d, bs, hq, hkv, fused):
    say("small", dtype, d, bs, hq, hkv, fused)
    w = small(dtype, d, bs, hq, hkv)
    dw = DeviceWorkload(w)
    out = dw.step(fused=fused)
    k_ref, v_ref = oracle_pools(w)
    assert np.array_equal(to_host(dw.k).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(to_host(dw.v).view(np.uint8), v_ref.view(np.uint8))
    assert_attention_close(out_f64(out), oracle_decode(w, k_ref, v_ref), dtype)


@pytest.mark.parametrize("group", [1, 8])
@pytest.mark.parametrize("workers", [1, 2, 3, 7, 8, 64, 257, 4096, 100000])
def test_worker_counts(workers, group):
    say("workers", workers, "group", group)
    w = small(wl.BF16, 128, 16, 4 * group, 4, seed=11)
    ref = oracle_decode(w, *oracle_pools(w))
    dw = DeviceWorkload(w)
    out = dw.step(fused=True, num_workers=workers)
    assert_attention_close(out_f64(out), ref, wl.BF16)


@pytest.mark.parametrize("dtype,d,hq,hkv", [(wl.FP32, 64, 4, 4), (wl.FP32, 128, 4, 4),
                                             (wl.BF16, 64, 4, 4), (wl.BF16, 128, 16, 2)])
@pytest.mark.parametrize("per_segment", [15, 16, 64, 96, 160])
def test_merge_of_many_pieces(dtype, d, hq, hkv, per_segment):
    """One long and one short sequence with many workers per segment: from 16
    per segment on, segments are merged by a workgroup each (every wave folds a
    quarter of the pieces, in rounds of 16 past 64 pieces); 15 stays on the
    one-wave merge.  96 and 160 per segment are what the default worker count
    gives one sequence at 32k with 8 and 4 KV heads."""
    say("many pieces", dtype, d, hq, hkv, per_segment)
    w = small(dtype, d, 16, hq, hkv, lens=[3000, 40], seed=13)
    segments = 2 * (hkv if hq != hkv and dtype == wl.BF16 and d == 128 else hq)
    ref = oracle_decode(w, *oracle_pools(w))
    dw = DeviceWorkload(w)
    out = dw.step(fused=True, num_workers=per_segment * segments)
    assert_attention_close(out_f64(out), ref, dtype)


def test_repeat_runs_are_bitwise_identical():
    w = small(wl.BF16, 128, 16, 8, 8, seed=12)
    dw = DeviceWorkload(w)
    a = dw.step(fused=True).clone()
    b = dw.step(fused=True).clone()     # the append rewrites the same values
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fused_append_equals_separate_append():
    # Same pools bit for bit; outputs agree to the tolerance (the fused path
    # adds the newest token in a different fp32 summation order).
    w = small(wl.BF16, 128, 16, 8, 8, seed=13)
    d1, d2 = DeviceWorkload(w), DeviceWorkload(w)
    a = d1.step(fused=True)
    b = d2.step(fused=False)
    assert_attention_close(out_f64(a), out_f64(b), wl.BF16)
    assert torch.equal(d1.k.view(torch.int16), d2.k.view(torch.int16))
    assert torch.equal(d1.v.view(torch.int16), d2.v.view(torch.int16))


def test_workspace_reuse_across_shapes():
    """One workspace, calls of different shapes and worker counts in a row:
    counters left by one call must never be misread by the next."""
    import paged_kv_cache_310_amd as pa
    cases = [small(wl.BF16, 128, 16, 2, 2, seed=31), small(wl.BF16, 128, 16, 40, 40, seed=32),
             small(wl.BF16, 128, 16, 64, 8, seed=33), small(wl.FP32, 64, 16, 2, 2, seed=34)]
    workers = [4096, 97, 1000, 64]
    need = max(pa.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, n)
               for w, n in zip(cases, workers))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for round_ in range(2):
        for i, w in enumerate(cases):
            dw = DeviceWorkload(w)
            out = pa.pa_decode(dw.q, dw.k, dw.v, dw.tables, dw.lens, float(w.scale),
                               k_new=dw.k_new, v_new=dw.v_new, slot_mapping=dw.slots,
                               workspace=ws, num_workers=workers[i])
            torch.cuda.synchronize()
            assert_attention_close(out_f64(out), oracle_decode(w, *oracle_pools(w)), w.dtype)


def test_decode_event_hook_times_the_attention_kernel():
    import paged_kv_cache_310_amd as pa
    w = small(wl.BF16, 128, 16, 8, 8, append=False, seed=35)
    dw = DeviceWorkload(w)
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    inner = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    outer[0].record()
    pa.pa_set_decode_events(inner[0], inner[1])
    try:
        out = pa.pa_decode(dw.q, dw.k, dw.v, dw.tables, dw.lens, float(w.scale), num_workers=64)
    finally:
        pa.pa_set_decode_events(None, None)
    outer[1].record()
    torch.cuda.synchronize()
    t_in, t_out = inner[0].elapsed_time(inner[1]), outer[0].elapsed_time(outer[1])
    assert 0 < t_in <= t_out
    assert_attention_close(out_f64(out), oracle_decode(w, w.k_cache, w.v_cache), wl.BF16)


def test_empty_sequences_give_zero_rows():
    lens = [0, 5, 0, 0, 40, 0]
    w = small(wl.BF16, 128, 16, 8, 8, lens=lens, append=False, seed=14)
    dw = DeviceWorkload(w)
    out = dw.step()
    got = out_f64(out)
    assert np.all(got[[0, 2, 3, 5]] == 0)
    assert_attention_close(got, oracle_decode(w, w.k_cache, w.v_cache), wl.BF16)
    w0 = small(wl.FP32, 64, 16, 4, 4, lens=[0, 0, 0], append=False, seed=15, num_blocks=4)
    out0 = DeviceWorkload(w0).step()
    assert torch.count_nonzero(out0).item() == 0


@pytest.mark.parametrize("hq,hkv,append", [(2, 2, True), (8, 1, True), (2, 2, False)],
                         ids=["mha-append", "gqa8-append", "mha-with-empty"])
def test_more_sequences_than_the_length_cache(hq, hkv, append):
    """5,000 sequences: the split caches 4,096 lengths in LDS and reads the
    rest from memory; ragged 0..40-token contexts, many segments per worker."""
    rng = np.random.default_rng(4242 + hq)
    lens = rng.integers(1 if append else 0, 41, 5000)
    say("many sequences", hq, hkv, append, int(lens.sum()), "tokens")
    w = small(wl.BF16, 128, 16, hq, hkv, lens=lens.tolist(), append=append, seed=21 + hq)
    out = DeviceWorkload(w).step()
    got = out_f64(out)
    assert not np.isnan(got).any()
    if not append:
        assert np.all(got[lens == 0] == 0)
    rows = sample_rows(w, per_seq_heads=1, seed=3)
    k, v = oracle_pools(w)
    err = assert_attention_close(got, oracle_decode(w, k, v, rows=rows), wl.BF16, rows=rows)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.FP32])
def test_single_token_returns_its_value_exactly(dtype):
    w = small(dtype, 128 if dtype == wl.BF16 else 64, 16, 4, 4, lens=[1] * 9, append=True, seed=16)
    dw = DeviceWorkload(w)
    out = dw.step(fused=True)
    got = to_host(out)
    for s in range(w.num_seqs):
        for h in range(w.num_q_heads):
            assert np.array_equal(got[s, h], w.v_new[s, h])


def test_large_scores_stay_finite_and_accurate():
    w = small(wl.BF16, 128, 16, 8, 8, seed=17, poison=True)
    q = w.q.view(np.uint16)
    q32 = (q.astype(np.uint32) << 16).view(np.float32) * np.float32(30.0)
    w.q = wl.f32_to_bf16_bits(q32)
    dw = DeviceWorkload(w)
    out = dw.step(fused=True)
    assert_attention_close(out_f64(out), oracle_decode(w, *oracle_pools(w)), wl.BF16)


def _permute_physical(w, seed):
    """Same logical data, different physical blocks."""
    perm = np.random.default_rng(seed).permutation(w.num_blocks)
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    return k, v, tables


def test_physical_permutation_gives_bitwise_identical_output():
    w = small(wl.BF16, 128, 16, 8, 8, append=False, seed=18)
    base = DeviceWorkload(w).step()
    for seed in (1, 2):
        k, v, tables = _permute_physical(w, seed)
        w2 = wl.Workload(**{**w.__dict__, "k_cache": k, "v_cache": v, "block_tables": tables})
        out = DeviceWorkload(w2).step()
        assert torch.equal(base.view(torch.int16), out.view(torch.int16))


def test_shared_prefix_blocks_equal_private_copies():
    w = small(wl.BF16, 128, 16, 8, 8, lens=[100, 100, 100], append=False, seed=19,
              num_blocks=40)
    k, v, t = w.k_cache.copy(), w.v_cache.copy(), w.block_tables.copy()
    used = set(t[t >= 0].tolist())
    free = [b for b in range(w.num_blocks) if b not in used]
    # sequence 1 and 2 share sequence 0's first 4 blocks (aliased) ...
    shared = t.copy()
    shared[1, :4] = t[0, :4]
    shared[2, :4] = t[0, :4]
    # ... or hold private copies of them
    private = t.copy()
    for s in (1, 2):
        for j in range(4):
            b = free.pop()
            k[b] = k[t[0, j]]
            v[b] = v[t[0, j]]
            private[s, j] = b
    wa = wl.Workload(**{**w.__dict__, "k_cache": k, "v_cache": v, "block_tables": shared})
    wb = wl.Workload(**{**w.__dict__, "k_cache": k, "v_cache": v, "block_tables": private})
    a = DeviceWorkload(wa).step()
    b = DeviceWorkload(wb).step()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_attention_close(out_f64(a), oracle_decode(wa, k, v), wl.BF16)


def test_copy_blocks_bit_exact_and_source_untouched():
    w = small(wl.BF16, 128, 32, 8, 8, lens=[40, 70, 9], append=False, seed=20, num_blocks=16)
    used = sorted(set(w.block_tables[w.block_tables >= 0].tolist()))
    free = [b for b in range(w.num_blocks) if b not in used]
    pairs = np.asarray([[used[0], free[0]], [used[1], free[1]], [used[2], free[2]]], np.int64)
    import paged_kv_cache_310_amd as pa
    import oracle
    k, v = to_dev(w.k_cache), to_dev(w.v_cache)
    pa.pa_copy_blocks(k, v, to_dev(pairs))
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.copy_blocks(w.k_cache, w.v_cache, pairs)
    assert np.array_equal(to_host(k), k_ref) and np.array_equal(to_host(v), v_ref)


def test_pa_check_rejects_contract_violations():
    code = r"""
import torch, numpy as np
import paged_kv_cache_310_amd as pa
from paged_kv_cache_310_amd._binding import PAError
d = 'cuda:0'
k = torch.zeros(8, 2, 16, 64, device=d); v = torch.zeros_like(k)
kn = torch.zeros(2, 2, 64, device=d); vn = torch.zeros_like(kn)
def status(f):
    try:
        f(); torch.cuda.synchronize(); return 0
    except PAError as e:
        return e.status
print(status(lambda: pa.pa_append_kv(k, v, kn, vn, torch.tensor([3, 8 * 16], device=d))))
print(status(lambda: pa.pa_append_kv(k, v, kn, vn, torch.tensor([3, 3], device=d))))
print(status(lambda: pa.pa_copy_blocks(k, v, torch.tensor([[1, 2], [2, 3]], device=d))))
q = torch.zeros(2, 2, 64, device=d)
tab = torch.tensor([[0, 1], [2, 9]], dtype=torch.int32, device=d)
print(status(lambda: pa.pa_decode(q, k, v, tab, torch.tensor([20, 20], dtype=torch.int32, device=d), 0.125)))
print(status(lambda: pa.pa_decode(q, k, v, tab, torch.tensor([20, 40], dtype=torch.int32, device=d), 0.125)))
print(status(lambda: pa.pa_decode(q, k, v, tab, torch.tensor([20, 3], dtype=torch.int32, device=d), 0.125,
      k_new=kn, v_new=vn, slot_mapping=torch.tensor([1 * 16 + 3, 2 * 16 + 2], device=d))))
print(status(lambda: pa.pa_decode(q, k, v, tab, torch.tensor([20, 3], dtype=torch.int32, device=d), 0.125,
      k_new=kn, v_new=vn, slot_mapping=torch.tensor([1 * 16 + 3, -1], device=d))))
print(status(lambda: pa.pa_read_probe(k, torch.tensor([0, 16], dtype=torch.int32, device=d))))
print(status(lambda: pa.pa_read_probe(k, torch.tensor([0, 15], dtype=torch.int32, device=d))))
"""
    env = dict(os.environ, PA_CHECK="1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120, cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert res.returncode == 0, res.stderr
    assert res.stdout.split() == ["5", "5", "5", "5", "5", "0", "0", "5", "0"], res.stdout


def test_binding_rejects_strided_index_arrays_before_any_launch():
    """Strided views of the lengths, the slots or the workspace would make the
    kernels read raw memory past the data: the binding refuses them."""
    import paged_kv_cache_310_amd as pa
    w = small(wl.BF16, 128, 16, 8, 8, lens=[5, 17, 40, 64])
    d = DeviceWorkload(w)
    lens2 = torch.stack([d.lens, d.lens], 1).reshape(-1)[::2]
    slots2 = torch.stack([d.slots, d.slots], 1).reshape(-1)[::2]
    assert not lens2.is_contiguous() and not slots2.is_contiguous()
    with pytest.raises(ValueError):
        pa.pa_decode(d.q, d.k, d.v, d.tables, lens2, float(w.scale))
    with pytest.raises(ValueError):
        pa.pa_decode(d.q, d.k, d.v, d.tables, d.lens, float(w.scale), k_new=d.k_new,
                     v_new=d.v_new, slot_mapping=slots2)
    ws = torch.zeros(2 * pa.pa_decode_workspace_size(4, 8, 8, 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        pa.pa_decode(d.q, d.k, d.v, d.tables, d.lens, float(w.scale), workspace=ws[::2])
    with pytest.raises(ValueError):
        pa.pa_decode(d.q, d.k, d.v, d.tables, d.lens, float(w.scale), workspace=ws.cpu())


def test_streams_get_their_own_default_workspace():
    """Calls on two streams without an explicit workspace must not share one
    (they may run at once): outputs on each stream equal the single-stream
    result, for two shapes back to back."""
    import paged_kv_cache_310_amd as pa
    from paged_kv_cache_310_amd import _binding
    a = DeviceWorkload(small(wl.BF16, 128, 16, 8, 8, lens=[300, 1000, 17, 513], append=False))
    b = DeviceWorkload(small(wl.BF16, 128, 16, 16, 2, lens=[2000, 64, 700], append=False))
    ref_a = pa.pa_decode(a.q, a.k, a.v, a.tables, a.lens, float(a.w.scale))
    ref_b = pa.pa_decode(b.q, b.k, b.v, b.tables, b.lens, float(b.w.scale))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = pa.pa_decode(a.q, a.k, a.v, a.tables, a.lens, float(a.w.scale))
        with torch.cuda.stream(s2):
            ob = pa.pa_decode(b.q, b.k, b.v, b.tables, b.lens, float(b.w.scale))
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa.view(torch.int16), ref_a.view(torch.int16))
        assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16))
    keys = {k for k in _binding._workspaces if k[-1] in (s1.cuda_stream, s2.cuda_stream)}
    assert len(keys) == 2


# ---------------------------------------------------------- full-size workloads
@pytest.fixture(scope="module")
def cache():
    return {}


def _full(cache, name):
    if name not in cache:
        say("generating", name)
        cache[name] = wl.make_workload(name, poison=True)
    return cache[name]


def _check_full(w, fused=True, rows=None, compare_pools=True):
    say("device step", w.name, "fused" if fused else "separate")
    dw = DeviceWorkload(w)
    out = dw.step(fused=fused)
    k_ref, v_ref = oracle_pools(w)
    if compare_pools:
        say("comparing pools", w.name)
        assert np.array_equal(to_host(dw.k).view(np.uint8), k_ref.view(np.uint8))
        assert np.array_equal(to_host(dw.v).view(np.uint8), v_ref.view(np.uint8))
    rows = sample_rows(w) if rows is None else rows
    say("oracle rows", len(rows))
    ref = oracle_decode(w, k_ref, v_ref, rows=rows)
    err = assert_attention_close(out_f64(out), ref, w.dtype, rows=rows)
    say(w.name, "max-abs %.3e row-rel %.3e" % err)
    return out


def test_workload_tiny_fp32(cache):
    w = _full(cache, "tiny_fp32")
    all_rows = [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)]
    a = _check_full(w, fused=True, rows=all_rows)
    b = _check_full(w, fused=False, rows=all_rows)
    assert_attention_close(out_f64(a), out_f64(b), w.dtype)


def test_workload_opt13b_mha(cache):
    w = _full(cache, "opt13b_mha")
    all_rows = [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)]
    _check_full(w, rows=all_rows)


def test_workload_llama13b_long(cache):
    w = _full(cache, "llama13b_long")
    a = _check_full(w, fused=True)
    b = _check_full(w, fused=False, compare_pools=False)
    assert_attention_close(out_f64(a), out_f64(b), w.dtype)


def test_workload_shared_prefix_steady(cache):
    _check_full(_full(cache, "shared_prefix_steady"))


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
def test_workload_shared_prefix_fork(cache, fused):
    """The fork step as the benchmark times it (the 112 copy-on-write copies,
    then decode with the append fused), and with a separate append: whole
    pools bit-exact, outputs of every sequence."""
    _check_full(_full(cache, "shared_prefix_fork"), fused=fused)


@pytest.mark.parametrize("name", ["gqa_pareto_bs16", "gqa_pareto_bs32"])
def test_workload_gqa_pareto(cache, name):
    w = _full(cache, name)
    longest = np.argsort(w.context_lens)[-2:]
    rows = sample_rows(w) + [(int(s), h) for s in longest for h in range(w.num_q_heads)]
    _check_full(w, rows=sorted(set(rows)))


@pytest.mark.parametrize("name", ["gqa_single_4k", "gqa_single_32k"])
def test_workload_gqa_single_sequence(cache, name):
    """One sequence: each KV head's segment is split over many workers and
    merged (the default worker count is capped per segment)."""
    w = _full(cache, name)
    _check_full(w, rows=[(0, h) for h in range(w.num_q_heads)])


@pytest.mark.parametrize("hq,lens", [(40, [1024]), (40, [4096]), (40, [4096, 4096]),
                                     (32, [8192]), (8, [32768])],
                         ids=["40h-1k", "40h-4k", "40h-2x4k", "32h-8k", "8h-32k"])
def test_small_multi_head_batches(hq, lens):
    """Small batches on the vector kernel take 3 workers per CU by default,
    so each head's segment is split into many pieces (20 to 96 here): every
    output row against the oracle, pools bit-exact after the fused append."""
    w = wl.make_simple("mha_small", 11, wl.BF16, hq, hq, 128, 16, lens, append=True, poison=True)
    rows = [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)]
    _check_full(w, rows=rows)
