"""Pools larger than 4 GiB: every byte offset the kernels form is 64-bit.

The same logical data is placed in a small pool and above the 4.25 GiB mark
of a large one (every physical block id shifted by the same amount). Copy,
append, decode (vector and matrix-core kernels, append fused or separate) and
prefill must then give bitwise identical outputs and pools, and must leave
the large pool's lower part untouched. The small-pool outputs are also
checked against the oracle.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import (assert_attention_close, oracle_decode, oracle_pools, out_f64, to_dev)

pytestmark = pytest.mark.gpu

MARK = 17 << 28          # 4.25 GiB: every used block lies past this byte offset


def say(*a):
    print(*a, flush=True)


def lift(k_small, v_small):
    """Zeroed device pools whose block base + b holds small block b."""
    block_bytes = k_small[0].numel() * k_small.element_size()
    base = -(-MARK // block_bytes)
    shape = (base + k_small.shape[0],) + tuple(k_small.shape[1:])
    k = torch.zeros(shape, dtype=k_small.dtype, device=k_small.device)
    v = torch.zeros_like(k)
    k[base:] = k_small
    v[base:] = v_small
    return base, k, v


def shift_blocks(a, base):
    """Block ids (tables or copy pairs) moved up by base; -1 entries stay."""
    out = a.astype(np.int64) + base
    out[a < 0] = -1
    assert out.max() < 2**31
    return out.astype(a.dtype)


def shift_slots(slots, base, bs):
    out = slots.astype(np.int64) + base * bs
    out[slots < 0] = -1
    return out


def assert_same(a, b):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def assert_lower_untouched(pool, base):
    assert int(torch.count_nonzero(pool[:base].view(torch.int16))) == 0


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2)], ids=["mha", "gqa8"])
def test_decode_append_copy_past_4gib(hq, hkv, fused):
    import paged_kv_cache_310_amd as pa
    say("large pool decode", hq, hkv, "fused" if fused else "separate")
    w = wl.make_simple("big", 41 + hq, wl.BF16, hq, hkv, 128, 16, [1, 17, 300, 1000, 2049],
                       append=True, poison=True, random_copies=2)
    ks, vs = to_dev(w.k_cache), to_dev(w.v_cache)
    base, kb, vb = lift(ks, vs)
    say("base block", base, "pool bytes", kb.numel() * 2)
    q = to_dev(w.q)
    kn, vn, lens = to_dev(w.k_new), to_dev(w.v_new), to_dev(w.context_lens)
    runs = {}
    for name, k, v, tab, slots, pairs in (
            ("small", ks, vs, w.block_tables, w.slot_mapping, w.block_mapping),
            ("large", kb, vb, shift_blocks(w.block_tables, base),
             shift_slots(w.slot_mapping, base, 16), shift_blocks(w.block_mapping, base))):
        pa.pa_copy_blocks(k, v, to_dev(pairs))
        if not fused:
            pa.pa_append_kv(k, v, kn, vn, to_dev(slots))
        extra = dict(k_new=kn, v_new=vn, slot_mapping=to_dev(slots)) if fused else {}
        runs[name] = pa.pa_decode(q, k, v, to_dev(tab), lens, float(w.scale), **extra)
    torch.cuda.synchronize()
    assert_same(runs["small"], runs["large"])
    assert_same(ks, kb[base:])
    assert_same(vs, vb[base:])
    assert_lower_untouched(kb, base)
    assert_lower_untouched(vb, base)
    k_ref, v_ref = oracle_pools(w)
    err = assert_attention_close(out_f64(runs["small"]), oracle_decode(w, k_ref, v_ref), wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)
    del kb, vb
    torch.cuda.empty_cache()


def test_prefill_past_4gib():
    import oracle
    import paged_kv_cache_310_amd as pa
    say("large pool prefill")
    w = wl.make_prefill("bigpf", 47, wl.BF16, 16, 2, 128, 16, [300, 1000, 40, 2100],
                        [300, 200, 40, 33])
    ks, vs = to_dev(w.k_cache), to_dev(w.v_cache)
    base, kb, vb = lift(ks, vs)
    q, kn, vn = to_dev(w.q), to_dev(w.k_new), to_dev(w.v_new)
    lens, qs = to_dev(w.context_lens), to_dev(w.query_start)
    outs = {}
    for name, k, v, tab, slots in (
            ("small", ks, vs, w.block_tables, w.slot_mapping),
            ("large", kb, vb, shift_blocks(w.block_tables, base),
             shift_slots(w.slot_mapping, base, 16))):
        pa.pa_append_kv(k, v, kn, vn, to_dev(slots))
        outs[name] = pa.pa_prefill(q, k, v, to_dev(tab), lens, qs, float(w.scale),
                                   max_query_len=w.max_query_len)
    torch.cuda.synchronize()
    assert_same(outs["small"], outs["large"])
    assert_same(ks, kb[base:])
    assert_lower_untouched(kb, base)
    k_ref, v_ref = oracle.append_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping,
                                    w.block_size)
    ref = oracle.prefill(w.q, k_ref, v_ref, w.block_tables, w.context_lens, w.query_start,
                         w.scale, w.dtype, w.block_size)
    err = assert_attention_close(out_f64(outs["small"]), ref, wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)
    del kb, vb
    torch.cuda.empty_cache()
