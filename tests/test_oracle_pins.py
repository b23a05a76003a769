"""Pins of the CPU oracle to things other than itself.

Each check below is written as a function of the oracle entry points it
exercises, so the same check can be run against deliberately broken copies
of the oracle (``test_planted_mistakes_are_caught``): a plausible mistake --
a dropped scale, a flipped sign, a swapped index, a transposed operand, a
wrong grouped-query mapping, an off-by-one length -- must fail at least one
pin.

What pins what:
* brute force (pure-Python loops over tiny paged inputs): the whole decode;
* torch ``scaled_dot_product_attention`` in fp64 on *contiguous* K/V, which
  the test scatters into a permuted pool with its own code: the table walk
  and the formula (pages: attention sees a contiguous logical sequence);
* hand-worked fixtures in ``tests/golden`` (closed forms);
* closed forms: L = 1 gives v0; equal V rows; q = 0 gives the mean; a common
  key shift changes nothing; GQA equals MHA with replicated KV heads;
* invariants the pages state: any physical permutation gives the same
  result; aliased (shared) prefix blocks equal private copies; a block copy
  duplicates exactly one block and leaves the source untouched; an append
  writes exactly its slot.
* multi-token (prefill) attention: torch attention with a shifted
  lower-triangular mask on contiguous K/V; brute-force decodes of the
  sequence cut after each query position; a fresh prompt's first token gives
  v0; q = 0 gives the running mean of V; one token per sequence equals the
  decode; one chunk equals two.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- helpers
def rng_bf16(rng, shape):
    """Random bf16 bit patterns of N(0,1) values (truncation is fine here)."""
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def scatter_into_pool(seqs_k, seqs_v, block_size, num_blocks, perm, fill):
    """Place contiguous per-sequence K/V ([L, Hkv, D]) into a paged pool.

    Written independently of the oracle's gather: logical block j of
    sequence s goes to the next physical block from ``perm``.
    """
    hkv, d = seqs_k[0].shape[1:]
    k_pool = np.full((num_blocks, hkv, block_size, d), fill, dtype=seqs_k[0].dtype)
    v_pool = np.full_like(k_pool, fill)
    nblk = [-(-len(k) // block_size) for k in seqs_k]
    tables = np.full((len(seqs_k), max(max(nblk), 1)), -1, dtype=np.int32)
    it = iter(perm)
    for s, (ks, vs) in enumerate(zip(seqs_k, seqs_v)):
        for j in range(nblk[s]):
            phys = next(it)
            tables[s, j] = phys
            lo, hi = j * block_size, min(len(ks), (j + 1) * block_size)
            for t in range(lo, hi):
                for h in range(hkv):
                    k_pool[phys, h, t - lo, :] = ks[t, h]
                    v_pool[phys, h, t - lo, :] = vs[t, h]
    return k_pool, v_pool, tables


def random_contiguous(rng, lengths, hkv, d, dtype):
    if dtype == oracle.BF16:
        ks = [rng_bf16(rng, (n, hkv, d)) for n in lengths]
        vs = [rng_bf16(rng, (n, hkv, d)) for n in lengths]
    else:
        ks = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lengths]
        vs = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lengths]
    return ks, vs


def nan_fill(dtype):
    return np.uint16(0x7FC0) if dtype == oracle.BF16 else np.float32(np.nan)


# ------------------------------------------------------------------ the checks
def check_bits(bits_to_f64):
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 1 << 16, 4096, dtype=np.uint32).astype(np.uint16)
    raw = raw[(raw & 0x7F80) != 0x7F80]                       # drop inf/NaN patterns
    ref = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bits_to_f64(raw, oracle.BF16), ref)
    f = rng.standard_normal(64).astype(np.float32)
    assert np.array_equal(bits_to_f64(f, oracle.FP32), f.astype(np.float64))


def brute_force_decode(q, k_pool, v_pool, tables, lens, scale, dtype, bs):
    """Pure-Python scalar loops, written from the definition."""
    b, hq, d = q.shape
    hkv = k_pool.shape[1]
    g = hq // hkv
    toflt = (lambda x: float(oracle.bits_to_f64(np.asarray([x]), dtype)[0]))
    out = np.zeros((b, hq, d))
    for s in range(b):
        for h in range(hq):
            n = int(lens[s])
            if n == 0:
                continue
            kvh = h // g
            z = []
            for t in range(n):
                blk = int(tables[s][t // bs])
                acc = 0.0
                for i in range(d):
                    acc += toflt(q[s, h, i]) * toflt(k_pool[blk, kvh, t % bs, i])
                z.append(float(np.float32(scale)) * acc)
            m = max(z)
            w = [math.exp(x - m) for x in z]
            tot = sum(w)
            for i in range(d):
                acc = 0.0
                for t in range(n):
                    blk = int(tables[s][t // bs])
                    acc += w[t] * toflt(v_pool[blk, kvh, t % bs, i])
                out[s, h, i] = acc / tot
    return out


def check_brute_force(decode, dtype=oracle.FP32):
    rng = np.random.default_rng(7)
    lens = [0, 1, 5, 9, 4]
    hq, hkv, d, bs = 4, 2, 6, 4
    ks, vs = random_contiguous(rng, lens, hkv, d, dtype)
    nb = sum(-(-n // bs) for n in lens) + 3
    kp, vp, tab = scatter_into_pool(ks, vs, bs, nb, rng.permutation(nb), nan_fill(dtype))
    q = rng_bf16(rng, (len(lens), hq, d)) if dtype == oracle.BF16 else \
        rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    scale = np.float32(0.37)
    got = decode(q, kp, vp, tab, np.asarray(lens, np.int32), scale, dtype, bs)
    ref = brute_force_decode(q, kp, vp, tab, lens, scale, dtype, bs)
    assert np.max(np.abs(got - ref)) <= 1e-12


def check_sdpa(decode, dtype=oracle.BF16, hq=8, hkv=2):
    rng = np.random.default_rng(11)
    lens = [37, 1, 64, 50, 0, 17]
    d, bs = 16, 16
    ks, vs = random_contiguous(rng, lens, hkv, d, dtype)
    nb = sum(-(-n // bs) for n in lens) + 5
    kp, vp, tab = scatter_into_pool(ks, vs, bs, nb, rng.permutation(nb), nan_fill(dtype))
    q = rng_bf16(rng, (len(lens), hq, d)) if dtype == oracle.BF16 else \
        rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    scale = np.float32(1 / math.sqrt(d))
    got = decode(q, kp, vp, tab, np.asarray(lens, np.int32), scale, dtype, bs)
    for s, n in enumerate(lens):
        if n == 0:
            assert np.all(got[s] == 0)
            continue
        qq = torch.from_numpy(oracle.bits_to_f64(q[s], dtype))[:, None, :]          # [Hq,1,D]
        kk = torch.from_numpy(oracle.bits_to_f64(ks[s], dtype)).permute(1, 0, 2)     # [Hkv,L,D]
        vv = torch.from_numpy(oracle.bits_to_f64(vs[s], dtype)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, scale=float(scale), enable_gqa=True)[:, 0, :].numpy()
        assert np.max(np.abs(got[s] - ref)) <= 1e-12, s


def check_golden(decode, name):
    fix = json.load(open(os.path.join(GOLDEN, name)))
    bs, d = fix["block_size"], len(fix["q"])
    k = np.asarray(fix["k"], np.float32)[:, None, :]
    v = np.asarray(fix["v"], np.float32)[:, None, :]
    nb = fix["num_blocks"]
    kp = np.full((nb, 1, bs, d), np.nan, np.float32)
    vp = np.full_like(kp, np.nan)
    for t in range(len(k)):
        blk = fix["physical_blocks"][t // bs]
        kp[blk, 0, t % bs] = k[t, 0]
        vp[blk, 0, t % bs] = v[t, 0]
    tab = np.asarray([fix["physical_blocks"]], np.int32)
    q = np.asarray(fix["q"], np.float32)[None, None, :]
    got = decode(q, kp, vp, tab, np.asarray([len(k)], np.int32), np.float32(fix["scale"]),
                 oracle.FP32, bs)[0, 0]
    assert np.max(np.abs(got - np.asarray(fix["expected"]))) <= 1e-14


def paged_case(rng, lens, hq, hkv, d, bs, dtype=oracle.FP32):
    ks, vs = random_contiguous(rng, lens, hkv, d, dtype)
    nb = sum(-(-n // bs) for n in lens) + 2
    kp, vp, tab = scatter_into_pool(ks, vs, bs, nb, rng.permutation(nb), nan_fill(dtype))
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32) if dtype == oracle.FP32 \
        else rng_bf16(rng, (len(lens), hq, d))
    return q, ks, vs, kp, vp, tab


def check_closed_forms(decode):
    rng = np.random.default_rng(5)
    bs, d = 4, 8
    # L = 1 -> out = v0 exactly.
    q, ks, vs, kp, vp, tab = paged_case(rng, [1, 1], 2, 2, d, bs)
    out = decode(q, kp, vp, tab, np.asarray([1, 1], np.int32), np.float32(0.3), oracle.FP32, bs)
    for s in range(2):
        assert np.array_equal(out[s], vs[s][0].astype(np.float64))
    # All V rows equal -> out = that row.
    q, ks, vs, kp, vp, tab = paged_case(rng, [13], 2, 2, d, bs)
    vs[0][:] = vs[0][0]
    kp2, vp2, tab2 = scatter_into_pool(ks, vs, bs, kp.shape[0], tab[0][tab[0] >= 0].tolist()
                                       + [b for b in range(kp.shape[0]) if b not in tab[0]], np.nan)
    out = decode(q, kp2, vp2, tab2, np.asarray([13], np.int32), np.float32(0.3), oracle.FP32, bs)
    assert np.max(np.abs(out[0] - vs[0][0].astype(np.float64))) <= 1e-14
    # q = 0 -> uniform weights -> mean of V.
    q, ks, vs, kp, vp, tab = paged_case(rng, [11, 6], 2, 2, d, bs)
    q[:] = 0
    out = decode(q, kp, vp, tab, np.asarray([11, 6], np.int32), np.float32(0.3), oracle.FP32, bs)
    for s in range(2):
        assert np.max(np.abs(out[s] - vs[s].astype(np.float64).mean(axis=0))) <= 1e-14
    # A common key shift u changes every score by scale*q.u: softmax unchanged.
    q, ks, vs, kp, vp, tab = paged_case(rng, [10], 1, 1, d, bs)
    kp = (np.round(kp * 256) / 256).astype(np.float32)         # so that kp + u is exact
    u = np.float32(0.5) * np.ones(d, np.float32)
    base = decode(q, kp, vp, tab, np.asarray([10], np.int32), np.float32(0.3), oracle.FP32, bs)
    kp_s = kp + u                                               # NaN slack stays NaN
    shifted = decode(q, kp_s, vp, tab, np.asarray([10], np.int32), np.float32(0.3), oracle.FP32, bs)
    assert np.max(np.abs(base - shifted)) <= 1e-12


def check_gqa_equals_replicated_mha(decode):
    rng = np.random.default_rng(9)
    hq, hkv, d, bs = 8, 2, 8, 4
    lens = [7, 12, 3]
    q, ks, vs, kp, vp, tab = paged_case(rng, lens, hq, hkv, d, bs)
    g = hq // hkv
    kp_rep = np.repeat(kp, g, axis=1)       # KV head j serves query heads j*g..j*g+g-1
    vp_rep = np.repeat(vp, g, axis=1)
    a = decode(q, kp, vp, tab, np.asarray(lens, np.int32), np.float32(0.4), oracle.FP32, bs)
    b = decode(q, kp_rep, vp_rep, tab, np.asarray(lens, np.int32), np.float32(0.4), oracle.FP32, bs)
    assert np.array_equal(a, b)
    # A query head group must depend on its own KV head only.
    kp_mod = kp.copy()
    kp_mod[:, 1] = 0
    c = decode(q, kp_mod, vp, tab, np.asarray(lens, np.int32), np.float32(0.4), oracle.FP32, bs)
    assert np.array_equal(a[:, :g], c[:, :g]) and not np.array_equal(a[:, g:], c[:, g:])


def check_permutation_invariance(decode):
    rng = np.random.default_rng(13)
    lens = [33, 8, 21]
    hq = hkv = 2
    d, bs = 8, 8
    ks, vs = random_contiguous(rng, lens, hkv, d, oracle.BF16)
    nb = 20
    q = rng_bf16(rng, (3, hq, d))
    outs = []
    for seed in (1, 2, 3):
        perm = np.random.default_rng(seed).permutation(nb)
        kp, vp, tab = scatter_into_pool(ks, vs, bs, nb, perm, nan_fill(oracle.BF16))
        outs.append(decode(q, kp, vp, tab, np.asarray(lens, np.int32), np.float32(0.25),
                           oracle.BF16, bs))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def check_sharing(decode):
    """Aliased prefix blocks give the same result as private copies."""
    rng = np.random.default_rng(17)
    bs, d, h = 4, 8, 2
    prefix_blocks, nb = 3, 16
    kp = rng_bf16(rng, (nb, h, bs, d))
    vp = rng_bf16(rng, (nb, h, bs, d))
    shared = np.asarray([[0, 1, 2, 5], [0, 1, 2, 6]], np.int32)
    private = np.asarray([[0, 1, 2, 5], [7, 8, 9, 6]], np.int32)
    for src, dst in zip(range(prefix_blocks), (7, 8, 9)):
        kp[dst] = kp[src]
        vp[dst] = vp[src]
    q = rng_bf16(rng, (2, h, d))
    lens = np.asarray([15, 14], np.int32)
    a = decode(q, kp, vp, shared, lens, np.float32(0.3), oracle.BF16, bs)
    b = decode(q, kp, vp, private, lens, np.float32(0.3), oracle.BF16, bs)
    assert np.array_equal(a, b)


def check_append(append_kv, gather):
    rng = np.random.default_rng(19)
    nb, h, bs, d = 6, 3, 4, 5
    kp = rng_bf16(rng, (nb, h, bs, d))
    vp = rng_bf16(rng, (nb, h, bs, d))
    kn = rng_bf16(rng, (4, h, d))
    vn = rng_bf16(rng, (4, h, d))
    slots = np.asarray([2 * bs + 3, -1, 5 * bs + 0, 0 * bs + 1], np.int64)
    k2, v2 = append_kv(kp, vp, kn, vn, slots, bs)
    expect_k, expect_v = kp.copy(), vp.copy()
    for t, (blk, off) in {0: (2, 3), 2: (5, 0), 3: (0, 1)}.items():
        expect_k[blk, :, off] = kn[t]
        expect_v[blk, :, off] = vn[t]
    assert np.array_equal(k2, expect_k) and np.array_equal(v2, expect_v)
    assert np.array_equal(kp, expect_k) is False                    # inputs untouched
    # Reading the appended position back through a table gives the new row.
    table = np.asarray([4, 2], np.int32)                               # position 7 -> block 2, off 3
    for head in range(h):
        assert np.array_equal(gather(k2, table, 8, bs, head)[7], kn[0, head])


def check_copy(copy_blocks):
    rng = np.random.default_rng(23)
    nb, h, bs, d = 8, 2, 4, 3
    kp = rng.standard_normal((nb, h, bs, d)).astype(np.float32)
    vp = rng.standard_normal((nb, h, bs, d)).astype(np.float32)
    pairs = np.asarray([[1, 6], [3, 7]], np.int64)
    k2, v2 = copy_blocks(kp, vp, pairs)
    for src, dst in pairs:
        assert np.array_equal(k2[dst], kp[src]) and np.array_equal(v2[dst], vp[src])
    untouched = [b for b in range(nb) if b not in (6, 7)]
    assert np.array_equal(k2[untouched], kp[untouched])
    assert np.array_equal(v2[untouched], vp[untouched])
    assert not np.array_equal(k2[6], kp[6])


def check_decode_all(decode):
    check_brute_force(decode)
    check_brute_force(decode, oracle.BF16)
    check_sdpa(decode)
    check_sdpa(decode, oracle.FP32, hq=4, hkv=4)
    check_golden(decode, "attention_two_tokens.json")
    check_golden(decode, "attention_three_tokens.json")
    check_closed_forms(decode)
    check_gqa_equals_replicated_mha(decode)
    check_permutation_invariance(decode)
    check_sharing(decode)


# ------------------------------------------------------- multi-token (prefill)
def prefill_case(rng, ctx, qlens, hq, hkv, d, bs, dtype):
    """Contiguous K/V of lengths ``ctx`` scattered into a permuted pool, and a
    query chunk of ``qlens[s]`` tokens per sequence (its newest tokens)."""
    ks, vs = random_contiguous(rng, ctx, hkv, d, dtype)
    nb = sum(-(-n // bs) for n in ctx) + 3
    kp, vp, tab = scatter_into_pool(ks, vs, bs, nb, rng.permutation(nb), nan_fill(dtype))
    total = int(sum(qlens))
    q = rng_bf16(rng, (total, hq, d)) if dtype == oracle.BF16 else \
        rng.standard_normal((total, hq, d)).astype(np.float32)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return q, ks, vs, kp, vp, tab, qs


def check_prefill_sdpa(prefill, dtype=oracle.BF16, hq=8, hkv=2):
    """torch attention in fp64 on contiguous K/V with a lower-triangular mask
    shifted by the prior context (torch.tril with diagonal L - n)."""
    rng = np.random.default_rng(41)
    ctx = [37, 1, 64, 50, 0, 17, 20]
    qlens = [37, 1, 5, 50, 0, 3, 1]
    d, bs = 16, 16
    q, ks, vs, kp, vp, tab, qs = prefill_case(rng, ctx, qlens, hq, hkv, d, bs, dtype)
    scale = np.float32(1 / math.sqrt(d))
    got = prefill(q, kp, vp, tab, np.asarray(ctx, np.int32), qs, scale, dtype, bs)
    for s, (L, n) in enumerate(zip(ctx, qlens)):
        if n == 0:
            continue
        qq = torch.from_numpy(oracle.bits_to_f64(q[qs[s]:qs[s + 1]], dtype)).permute(1, 0, 2)
        kk = torch.from_numpy(oracle.bits_to_f64(ks[s], dtype)).permute(1, 0, 2)
        vv = torch.from_numpy(oracle.bits_to_f64(vs[s], dtype)).permute(1, 0, 2)
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, scale=float(scale), enable_gqa=True).permute(1, 0, 2)
        assert np.max(np.abs(got[qs[s]:qs[s + 1]] - ref.numpy())) <= 1e-12, s


def check_prefill_brute_force(prefill, dtype=oracle.FP32):
    """Each query token equals the scalar-loop brute force of a decode over
    the sequence cut after that token's position."""
    rng = np.random.default_rng(43)
    ctx, qlens = [6, 9, 3], [6, 4, 1]
    hq, hkv, d, bs = 4, 2, 5, 4
    q, ks, vs, kp, vp, tab, qs = prefill_case(rng, ctx, qlens, hq, hkv, d, bs, dtype)
    scale = np.float32(0.41)
    got = prefill(q, kp, vp, tab, np.asarray(ctx, np.int32), qs, scale, dtype, bs)
    for s, (L, n) in enumerate(zip(ctx, qlens)):
        for i in range(n):
            t = qs[s] + i
            ref = brute_force_decode(q[t][None], kp, vp, tab[s:s + 1], [L - n + i + 1], scale,
                                     dtype, bs)
            assert np.max(np.abs(got[t] - ref[0])) <= 1e-12, (s, i)


def check_prefill_closed_forms(prefill, decode):
    rng = np.random.default_rng(47)
    hq = hkv = 2
    d, bs = 8, 4
    # A fresh prompt's first token sees only itself: out = v0 exactly.
    ctx = qlens = [9, 1, 4]
    q, ks, vs, kp, vp, tab, qs = prefill_case(rng, ctx, qlens, hq, hkv, d, bs, oracle.FP32)
    out = prefill(q, kp, vp, tab, np.asarray(ctx, np.int32), qs, np.float32(0.3), oracle.FP32, bs)
    for s in range(3):
        assert np.array_equal(out[qs[s]], vs[s][0].astype(np.float64))
    # q = 0: uniform weights over the visible positions -> running mean of V.
    ctx, qlens = [11, 7], [11, 3]
    q, ks, vs, kp, vp, tab, qs = prefill_case(rng, ctx, qlens, hq, hkv, d, bs, oracle.FP32)
    q[:] = 0
    out = prefill(q, kp, vp, tab, np.asarray(ctx, np.int32), qs, np.float32(0.3), oracle.FP32, bs)
    for s, (L, n) in enumerate(zip(ctx, qlens)):
        v = vs[s].astype(np.float64)
        running = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None, None]
        for i in range(n):
            assert np.max(np.abs(out[qs[s] + i] - running[L - n + i])) <= 1e-14
    # One query token per sequence is a decode step.
    ctx = [13, 5, 1]
    q, ks, vs, kp, vp, tab, qs = prefill_case(rng, ctx, [1, 1, 1], 4, 2, d, bs, oracle.BF16)
    a = prefill(q, kp, vp, tab, np.asarray(ctx, np.int32), qs, np.float32(0.3), oracle.BF16, bs)
    b = decode(q, kp, vp, tab, np.asarray(ctx, np.int32), np.float32(0.3), oracle.BF16, bs)
    assert np.array_equal(a, b)


def check_prefill_chunking(prefill):
    """A prompt processed as one chunk equals the same prompt processed as two
    chunks (the first with only its own tokens cached)."""
    rng = np.random.default_rng(53)
    L, first = 23, 9
    hq, hkv, d, bs = 4, 1, 8, 4
    q, ks, vs, kp, vp, tab, qs = prefill_case(rng, [L], [L], hq, hkv, d, bs, oracle.BF16)
    whole = prefill(q, kp, vp, tab, np.asarray([L], np.int32), qs, np.float32(0.35),
                    oracle.BF16, bs)
    a = prefill(q[:first], kp, vp, tab, np.asarray([first], np.int32),
                np.asarray([0, first], np.int32), np.float32(0.35), oracle.BF16, bs)
    b = prefill(q[first:], kp, vp, tab, np.asarray([L], np.int32),
                np.asarray([0, L - first], np.int32), np.float32(0.35), oracle.BF16, bs)
    assert np.array_equal(whole, np.concatenate([a, b]))


def check_prefill_all(prefill, decode):
    check_prefill_sdpa(prefill)
    check_prefill_sdpa(prefill, oracle.FP32, hq=3, hkv=3)
    check_prefill_brute_force(prefill)
    check_prefill_closed_forms(prefill, decode)
    check_prefill_chunking(prefill)


# ------------------------------------------------------------------- the tests
def test_bits_widening_matches_torch():
    check_bits(oracle.bits_to_f64)


def test_decode_matches_brute_force():
    check_brute_force(oracle.decode)
    check_brute_force(oracle.decode, oracle.BF16)


@pytest.mark.parametrize("dtype,hq,hkv", [(oracle.BF16, 8, 2), (oracle.FP32, 4, 4), (oracle.BF16, 6, 1)])
def test_decode_matches_torch_sdpa_on_contiguous(dtype, hq, hkv):
    check_sdpa(oracle.decode, dtype, hq, hkv)


@pytest.mark.parametrize("name", ["attention_two_tokens.json", "attention_three_tokens.json"])
def test_decode_hand_worked_fixtures(name):
    check_golden(oracle.decode, name)


def test_decode_closed_forms():
    check_closed_forms(oracle.decode)


def test_gqa_equals_replicated_mha():
    check_gqa_equals_replicated_mha(oracle.decode)


def test_physical_permutation_invariance():
    check_permutation_invariance(oracle.decode)


def test_shared_prefix_equals_private_copies():
    check_sharing(oracle.decode)


def test_append_writes_exactly_its_slots():
    check_append(oracle.append_kv, oracle.gather_sequence)


def test_copy_duplicates_exactly_the_named_blocks():
    check_copy(oracle.copy_blocks)


def test_large_scores_stay_finite():
    rng = np.random.default_rng(29)
    q, ks, vs, kp, vp, tab = paged_case(rng, [40, 3], 2, 2, 16, 8)
    q = (q * 30).astype(np.float32)
    out = oracle.decode(q, kp, vp, tab, np.asarray([40, 3], np.int32), np.float32(0.25),
                        oracle.FP32, 8)
    assert np.all(np.isfinite(out))
    # and it still equals torch's attention on the contiguous data
    for s, n in enumerate([40, 3]):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s].astype(np.float64))[:, None, :],
            torch.from_numpy(ks[s].astype(np.float64)).permute(1, 0, 2),
            torch.from_numpy(vs[s].astype(np.float64)).permute(1, 0, 2), scale=0.25)[:, 0, :]
        assert np.max(np.abs(out[s] - ref.numpy())) <= 1e-12


def test_rows_subset_equals_full():
    rng = np.random.default_rng(31)
    q, ks, vs, kp, vp, tab = paged_case(rng, [9, 17, 4], 4, 2, 8, 4)
    lens = np.asarray([9, 17, 4], np.int32)
    full = oracle.decode(q, kp, vp, tab, lens, np.float32(0.3), oracle.FP32, 4)
    rows = [(1, 3), (0, 0), (2, 1)]
    part = oracle.decode(q, kp, vp, tab, lens, np.float32(0.3), oracle.FP32, 4, rows=rows)
    for s, h in rows:
        assert np.array_equal(part[s, h], full[s, h])


def test_prefill_matches_torch_sdpa_with_shifted_causal_mask():
    check_prefill_sdpa(oracle.prefill)
    check_prefill_sdpa(oracle.prefill, oracle.FP32, hq=3, hkv=3)


def test_prefill_matches_brute_force():
    check_prefill_brute_force(oracle.prefill)
    check_prefill_brute_force(oracle.prefill, oracle.BF16)


def test_prefill_closed_forms():
    check_prefill_closed_forms(oracle.prefill, oracle.decode)


def test_prefill_one_chunk_equals_two():
    check_prefill_chunking(oracle.prefill)


# ------------------------------------------------------- planted mistakes (CPU)
def _mutants():
    """Plausible oracle bugs, each as (name, patches to oracle.paged_attention)."""
    def no_scale(q_row, keys, values, scale):
        z = keys @ q_row
        w = np.exp(z - z.max())
        return (w @ values) / w.sum()

    def flipped_sign(q_row, keys, values, scale):
        z = -np.float64(scale) * (keys @ q_row)
        w = np.exp(z - z.max())
        return (w @ values) / w.sum()

    def k_for_v(q_row, keys, values, scale):
        z = np.float64(scale) * (keys @ q_row)
        w = np.exp(z - z.max())
        return (w @ keys) / w.sum()

    def unnormalised(q_row, keys, values, scale):
        z = np.float64(scale) * (keys @ q_row)
        return np.exp(z - z.max()) @ values

    def swapped_offset(cache, table_row, length, block_size, kv_head):
        pos = np.arange(int(length))
        blocks = np.asarray(table_row, np.int64)[np.minimum(pos % block_size, len(table_row) - 1)]
        return cache[blocks, kv_head, np.minimum(pos // block_size, block_size - 1), :]

    def identity_table(cache, table_row, length, block_size, kv_head):
        pos = np.arange(int(length))
        return cache[pos // block_size, kv_head, pos % block_size, :]

    def one_short(cache, table_row, length, block_size, kv_head):
        pos = np.arange(max(int(length) - 1, 0))
        return cache[np.asarray(table_row, np.int64)[pos // block_size], kv_head, pos % block_size, :]

    def modulo_heads(q_head, num_q_heads, num_kv_heads):
        return q_head % num_kv_heads

    return [
        ("no_scale", {"attention_rows": no_scale}),
        ("flipped_sign", {"attention_rows": flipped_sign}),
        ("k_for_v", {"attention_rows": k_for_v}),
        ("unnormalised", {"attention_rows": unnormalised}),
        ("swapped_offset", {"gather_sequence": swapped_offset}),
        ("identity_table", {"gather_sequence": identity_table}),
        ("one_short", {"gather_sequence": one_short}),
        ("modulo_heads", {"kv_head_for": modulo_heads}),
    ]


@pytest.mark.parametrize("name,patches", _mutants(), ids=[m[0] for m in _mutants()])
def test_planted_mistakes_are_caught(monkeypatch, name, patches):
    for attr, fn in patches.items():
        monkeypatch.setattr(pa, attr, fn)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        check_decode_all(pa.decode)


@pytest.mark.parametrize("name,patches", _mutants(), ids=[m[0] for m in _mutants()])
def test_planted_mistakes_are_caught_by_prefill_pins(monkeypatch, name, patches):
    for attr, fn in patches.items():
        monkeypatch.setattr(pa, attr, fn)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        check_prefill_all(pa.prefill, oracle.decode)


def _prefill_mutants():
    return [
        ("self_excluded", {"visible_keys": lambda p: int(p)}),
        ("one_ahead", {"visible_keys": lambda p: int(p) + 2}),
        ("sees_whole_context", {"visible_keys": lambda p: 1 << 30}),
        ("ignores_prior_context", {"query_position": lambda L, n, i: int(i)}),
        ("chunk_from_the_front", {"query_position": lambda L, n, i: int(L) - int(n) + int(i) - 1
                                  if int(i) > 0 else 0}),
    ]


@pytest.mark.parametrize("name,patches", _prefill_mutants(), ids=[m[0] for m in _prefill_mutants()])
def test_planted_prefill_mistakes_are_caught(monkeypatch, name, patches):
    for attr, fn in patches.items():
        monkeypatch.setattr(pa, attr, fn)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        check_prefill_all(pa.prefill, oracle.decode)


def test_planted_append_and_copy_mistakes_are_caught(monkeypatch):
    def append_wrong_offset(k_cache, v_cache, k_new, v_new, slot_mapping, block_size):
        k, v = k_cache.copy(), v_cache.copy()
        for t, slot in enumerate(slot_mapping.tolist()):
            if slot >= 0:
                blk, off = divmod(slot, block_size)
                k[blk, :, (off + 1) % block_size] = k_new[t]
                v[blk, :, (off + 1) % block_size] = v_new[t]
        return k, v

    def copy_k_only(k_cache, v_cache, block_mapping):
        k = k_cache.copy()
        for src, dst in block_mapping.tolist():
            k[dst] = k_cache[src]
        return k, v_cache.copy()

    with pytest.raises(AssertionError):
        check_append(append_wrong_offset, oracle.gather_sequence)
    with pytest.raises(AssertionError):
        check_copy(copy_k_only)
