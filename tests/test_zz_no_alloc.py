"""GPU test of pa_decode_noalloc: pa_decode with the library's static device
scratch array in place of a caller workspace.

Checked through the C ABI binding against pa_decode on the same inputs and
worker count (the same kernels and summation order, so bit-identical outputs
and pools), and against the CPU oracle at the attention tolerance, on two
calls in a row where the second is smaller (the array keeps the first call's
contents, which must not leak into the second).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import (DeviceWorkload, assert_attention_close, oracle_decode, oracle_pools,
                       out_f64, to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


CASES = [
    # (dtype, head_dim, block_size, q heads, kv heads, lengths of call 1, lengths of call 2)
    (wl.BF16, 128, 16, 40, 40, [3000, 17, 1025, 640, 2, 4096], [100, 33]),
    (wl.BF16, 128, 16, 64, 8, [9000, 1, 700, 5000, 257], [1500]),
    (wl.BF16, 128, 32, 32, 2, [20000, 64], [300, 16, 1]),
    (wl.FP32, 64, 16, 8, 8, [129, 64, 1000], [5]),
]


def _run_pair(w, workers):
    """pa_decode and pa_decode_noalloc on separate copies of the pools, both
    with the append fused; returns both outputs and pools."""
    import paged_kv_cache_310_amd as pa
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    ref = pa.pa_decode(a.q, a.k, a.v, a.tables, a.lens, float(w.scale), k_new=a.k_new,
                       v_new=a.v_new, slot_mapping=a.slots, num_workers=workers)
    got = pa.pa_decode_noalloc(b.q, b.k, b.v, b.tables, b.lens, float(w.scale), k_new=b.k_new,
                               v_new=b.v_new, slot_mapping=b.slots, num_workers=workers)
    torch.cuda.synchronize()
    return (ref, a), (got, b)


def _check(w, workers):
    (ref, a), (got, b) = _run_pair(w, workers)
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), "noalloc != pa_decode"
    assert torch.equal(b.k.view(torch.uint8), a.k.view(torch.uint8))
    assert torch.equal(b.v.view(torch.uint8), a.v.view(torch.uint8))
    k_ref, v_ref = oracle_pools(w)
    assert np.array_equal(to_host(b.k).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(to_host(b.v).view(np.uint8), v_ref.view(np.uint8))
    err = assert_attention_close(out_f64(got), oracle_decode(w, k_ref, v_ref), w.dtype)
    say(w.name, "workers", workers or "default", "max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("dtype,d,bs,hq,hkv,lens1,lens2", CASES)
@pytest.mark.parametrize("workers", [0, 37])
def test_noalloc_equals_pa_decode_on_two_calls(dtype, d, bs, hq, hkv, lens1, lens2, workers):
    say("noalloc", dtype, d, bs, hq, hkv, "workers", workers)
    _check(wl.make_simple("noalloc_first", 11, dtype, hq, hkv, d, bs, lens1, append=True,
                          poison=True), workers)
    _check(wl.make_simple("noalloc_second", 12, dtype, hq, hkv, d, bs, lens2, append=True,
                          poison=True), workers)


def test_noalloc_rejects_a_need_beyond_the_scratch_before_any_launch():
    """200,000 workers of a 64/8-head bf16 batch need 1.7 GB of partials, far
    past the array: PA_ERR_WORKSPACE, and nothing is written."""
    import paged_kv_cache_310_amd as pa
    w = wl.make_simple("noalloc_big", 13, wl.BF16, 64, 8, 128, 16, [100, 200], append=True,
                       poison=True)
    d = DeviceWorkload(w)
    out = torch.full_like(d.q, 7.0)
    k0 = d.k.clone()
    with pytest.raises(pa.PAError) as e:
        pa.pa_decode_noalloc(d.q, d.k, d.v, d.tables, d.lens, float(w.scale), out=out,
                             k_new=d.k_new, v_new=d.v_new, slot_mapping=d.slots,
                             num_workers=200000)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    assert torch.equal(d.k.view(torch.uint8), k0.view(torch.uint8))
