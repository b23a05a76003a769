"""Seeded random sweep of the GPU path against the oracle.

Every case draws its own shapes and lengths from its seed: dtype, head size,
block size, KV heads and query heads per KV head (vector and matrix-core
kernels), 1..12 sequences with ragged contexts (empty ones when nothing is
appended), fused or separate append, copy-on-write pairs, and the worker
count. Prefill cases draw (context, chunk) pairs and head groups; split
prefill cases also draw longer contexts and the split count (automatic
included). Pools must
match bit for bit and attention within the tolerance of every other parity
test.
"""

import numpy as np
import pytest

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import (DeviceWorkload, assert_attention_close, oracle_decode, oracle_pools,
                       out_f64, to_host)
from test_gpu_prefill import oracle_rows, run_device
from test_gpu_prefill_split import run_split

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def decode_case(seed):
    rng = np.random.default_rng(seed)
    c = dict(dtype=[wl.BF16, wl.FP32][int(rng.integers(2))], d=int(rng.choice([64, 128])),
             bs=int(rng.choice([16, 32])), hkv=int(rng.integers(1, 5)),
             group=int(rng.choice([1, 2, 3, 4, 8])), b=int(rng.integers(1, 13)),
             append=bool(rng.integers(2)), fused=bool(rng.integers(2)),
             copies=int(rng.integers(0, 3)), workers=int(rng.choice([0, 0, 1, 3, 64, 1000])))
    lo = 1 if c["append"] else 0
    lens = rng.integers(lo, 700, c["b"])
    short = rng.random(c["b"]) < 0.4
    lens[short] = rng.integers(lo, 20, int(short.sum()))
    c["lens"] = lens.tolist()
    return c


@pytest.mark.parametrize("seed", range(9100, 9140))
def test_random_decode(seed):
    c = decode_case(seed)
    say("decode case", seed, c)
    need = sum(wl.blocks_needed(x, c["bs"]) for x in c["lens"])
    w = wl.make_simple("rand", seed, c["dtype"], c["hkv"] * c["group"], c["hkv"], c["d"], c["bs"],
                       c["lens"], append=c["append"], poison=True,
                       num_blocks=max(int(np.ceil(need * 1.25)), need + 4),
                       random_copies=min(c["copies"], need))
    dw = DeviceWorkload(w)
    out = dw.step(fused=c["fused"], num_workers=c["workers"])
    k_ref, v_ref = oracle_pools(w)
    # bytes, so that the NaN poison of unused slots compares equal too
    assert np.array_equal(to_host(dw.k).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(to_host(dw.v).view(np.uint8), v_ref.view(np.uint8))
    err = assert_attention_close(out_f64(out), oracle_decode(w, k_ref, v_ref), c["dtype"])
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("seed", range(9200, 9216))
def test_random_prefill(seed):
    rng = np.random.default_rng(seed)
    hkv, group = int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8]))
    bs, b = int(rng.choice([16, 32])), int(rng.integers(1, 5))
    ctx = rng.integers(1, 600, b)
    nq = np.minimum(ctx, rng.integers(0, 300, b))
    whole = rng.random(b) < 0.4          # fresh prompts: the chunk is the whole context
    nq[whole] = ctx[whole]
    say("prefill case", seed, hkv, group, bs, ctx.tolist(), nq.tolist())
    w = wl.make_prefill("rand", seed, wl.BF16, hkv * group, hkv, 128, bs, ctx.tolist(), nq.tolist())
    err = assert_attention_close(out_f64(run_device(w)), oracle_rows(w), wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)


@pytest.mark.parametrize("seed", range(9300, 9316))
def test_random_split_prefill(seed):
    rng = np.random.default_rng(seed)
    hkv, group = int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8]))
    bs, b = int(rng.choice([16, 32])), int(rng.integers(1, 4))
    ctx = rng.integers(1, 4000, b)
    nq = np.minimum(ctx, rng.integers(0, 200, b))
    whole = rng.random(b) < 0.25
    nq[whole] = np.minimum(ctx[whole], 400)
    ctx[whole] = nq[whole]
    splits = int(rng.choice([0, 2, 3, 4, 6, 8, 11, 16, 24, 32]))
    say("split prefill case", seed, hkv, group, bs, ctx.tolist(), nq.tolist(), splits)
    w = wl.make_prefill("rsplit", seed, wl.BF16, hkv * group, hkv, 128, bs, ctx.tolist(),
                        nq.tolist())
    err = assert_attention_close(out_f64(run_split(w, splits)), oracle_rows(w), wl.BF16)
    say("max-abs %.3e row-rel %.3e" % err)
