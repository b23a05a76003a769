"""Seeded synthetic inputs for the paged decode path.

This module only makes data: lengths, block tables, slot mappings, copy
lists and N(0, 1) values.  It holds none of the attention, append or copy
arithmetic, and both the HIP path and the CPU oracle consume what it makes.

Element data is returned as raw bits: ``uint16`` for bfloat16 (rounded to
nearest-even from float32 draws), ``float32`` for fp32.

Workloads (shapes follow the serving setups the pages discuss: OPT-13B and
LLaMA-13B attention heads, 16-token blocks, mixed lengths, shared prefixes):

=====================  =====================================================
tiny_fp32              4 seqs, 8/8 heads, d 64, bs 16, fp32, lengths U[1,128]
                       before a 1-token append, 64-block permuted pool, plus
                       a copy of 2 random in-use blocks into free blocks
opt13b_mha             64 seqs, 40/40 heads, d 128, bs 16, bf16, lengths
                       U[64,2048], pool 1.25x need, no append
llama13b_long          32 seqs, 40/40 heads, d 128, bs 16, bf16, lengths
                       lognormal(median 4096, sigma ln 2) clipped to
                       [1024,16384], pool 1.25x need, 1-token append
shared_prefix_steady   16 groups x 8 samples, 40/40, d 128, bs 16, bf16: a
                       1024-token prefix shared (refcount 8) plus private
                       tails U[16,256]; 1-token append into private blocks
shared_prefix_fork     same groups forked at 1024 + U[1,15] tokens: the
                       shared tail block is partly filled, so 7 of 8 samples
                       copy it on their first write (112 copies)
gqa_pareto_bs16/32     256 seqs, 64 query heads over 8 KV heads, d 128,
                       bf16, Pareto(alpha 1.2, x_m 128) lengths capped at
                       32768, pool 1.25x need, 1-token append
gqa_single_4k/32k      one sequence, 64/8 heads, d 128, bs 16, bf16, 4096 or
                       32768 tokens after a 1-token append, pool 1.25x need
                       (the latency regime: one segment per KV head)
=====================  =====================================================

Draw order per workload (one ``numpy.random.default_rng(seed)``): lengths,
pool permutation, q, K pool, V pool, new K, new V, random copy pairs.
With ``poison=True`` every slot no sequence has written (free blocks, tail
slack, the slot the step's append will fill) holds NaN, and unused table
entries are -1, so a kernel that reads outside the sequence is caught.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .block_manager import BlockManager, blocks_needed

BF16 = "bf16"
FP32 = "fp32"
_BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 24


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) values as raw bits of ``dtype``, drawn in fixed-size chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        draw = rng.standard_normal(stop - start, dtype=np.float32)
        out[start:stop] = f32_to_bf16_bits(draw) if dtype == BF16 else draw
    return out.reshape(shape)


def nan_bits(dtype: str):
    return _BF16_NAN if dtype == BF16 else np.float32(np.nan)


def elem_bytes(dtype: str) -> int:
    return 2 if dtype == BF16 else 4


@dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: np.float32
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    k_new: Optional[np.ndarray] = None
    v_new: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None
    block_mapping: Optional[np.ndarray] = None
    # Groups of sequences sharing a prefix (pa_decode_shared): group g is the
    # sequences group_start[g] .. group_start[g+1]-1; prefix_lens[s] tokens at
    # the start of sequence s sit in blocks every member's table shares.
    group_start: Optional[np.ndarray] = None
    prefix_lens: Optional[np.ndarray] = None
    notes: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode step reads: every cached token's
        K and V row for every KV head."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads \
            * self.head_dim * elem_bytes(self.dtype)

    @property
    def has_append(self) -> bool:
        return self.slot_mapping is not None

    @property
    def kv_shared_read_bytes(self) -> Optional[int]:
        """K/V bytes a decode step reads when each group's shared tokens are
        read once: per group, its first member's shared tokens in whole
        16-token chunks, plus every sequence's remaining tokens (None without
        groups)."""
        if self.group_start is None:
            return None
        lens = self.context_lens.astype(np.int64)
        shared = (np.minimum(np.maximum(self.prefix_lens.astype(np.int64), 0), lens) // 16) * 16
        firsts = self.group_start[:-1][np.diff(self.group_start) > 0]
        tokens = int(shared[firsts].sum()) + int((lens - shared).sum())
        return tokens * 2 * self.num_kv_heads * self.head_dim * elem_bytes(self.dtype)


def _pool_size(need_blocks: int, factor: float = 1.25) -> int:
    return int(math.ceil(factor * need_blocks))


def _assemble(name, rng, dtype, hq, hkv, d, bs, num_blocks, mgr: BlockManager,
              seqs: List[int], decode_lens: np.ndarray, max_blocks: int,
              append_slots: Optional[List[int]], copies: List[Tuple[int, int]],
              poison: bool, random_copies: int = 0) -> Workload:
    """Draw values and build the arrays once the block layout is fixed."""
    b = len(seqs)
    q = normal_bits(rng, (b, hq, d), dtype)
    k_cache = normal_bits(rng, (num_blocks, hkv, bs, d), dtype)
    v_cache = normal_bits(rng, (num_blocks, hkv, bs, d), dtype)
    k_new = v_new = slot_mapping = None
    if append_slots is not None:
        k_new = normal_bits(rng, (b, hkv, d), dtype)
        v_new = normal_bits(rng, (b, hkv, d), dtype)
        slot_mapping = np.asarray(append_slots, dtype=np.int64)
    tables = mgr.block_table_array(seqs, max_blocks)
    if random_copies:
        in_use = np.unique(tables[tables >= 0])
        free = np.setdiff1d(np.arange(num_blocks), in_use)
        src = rng.choice(in_use, size=random_copies, replace=False)
        dst = rng.choice(free, size=random_copies, replace=False)
        copies = list(copies) + list(zip(src.tolist(), dst.tolist()))
    block_mapping = np.asarray(copies, dtype=np.int64).reshape(-1, 2) if copies else None

    if poison:
        nan = nan_bits(dtype)
        # Slots holding a token before this step: the tables as they were
        # before the step's copies (a copy destination is still free then).
        before_copy = {dst: src for src, dst in copies}
        written = np.zeros((num_blocks, bs), dtype=bool)
        for i, seq in enumerate(seqs):
            cached = int(decode_lens[i]) - (1 if append_slots is not None else 0)
            for j, blk in enumerate(mgr.tables[seq]):
                n_here = max(0, min(bs, cached - j * bs))
                written[before_copy.get(blk, blk), :n_here] = True
        mask = ~written
        k_cache.transpose(0, 2, 1, 3)[mask] = nan
        v_cache.transpose(0, 2, 1, 3)[mask] = nan

    return Workload(
        name=name, dtype=dtype, num_seqs=b, num_q_heads=hq, num_kv_heads=hkv,
        head_dim=d, block_size=bs, num_blocks=num_blocks,
        scale=np.float32(1.0 / math.sqrt(d)), q=q, k_cache=k_cache, v_cache=v_cache,
        block_tables=tables, context_lens=np.asarray(decode_lens, dtype=np.int32),
        k_new=k_new, v_new=v_new, slot_mapping=slot_mapping,
        block_mapping=block_mapping,
    )


def make_simple(name: str, seed: int, dtype: str, num_q_heads: int, num_kv_heads: int,
                head_dim: int, block_size: int, decode_lens, append: bool, poison: bool,
                num_blocks: Optional[int] = None, max_len: Optional[int] = None,
                random_copies: int = 0, rng: Optional[np.random.Generator] = None) -> Workload:
    """Independent sequences scattered over a permuted pool.

    ``decode_lens`` are lengths after the step's append.  With ``append``
    the last token of each sequence is the one the step writes (its slot is
    returned in ``slot_mapping`` and its values in ``k_new``/``v_new``).
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    decode_lens = np.asarray(decode_lens, dtype=np.int64)
    if append and (decode_lens < 1).any():
        raise ValueError("a sequence that appends holds at least one token")
    need = sum(blocks_needed(x, block_size) for x in decode_lens)
    if num_blocks is None:
        num_blocks = max(1, _pool_size(need))
    perm = rng.permutation(num_blocks)
    mgr = BlockManager(num_blocks, block_size, free_order=perm)
    seqs = list(range(len(decode_lens)))
    slots = [] if append else None
    for s in seqs:
        n = int(decode_lens[s])
        mgr.add_sequence(s, n - 1 if append else n)
        if append:
            slot, copy = mgr.append_slot(s)
            assert copy is None
            slots.append(slot)
    cap = int(max_len) if max_len is not None else int(max(decode_lens.max(initial=0), 1))
    max_blocks = max(1, blocks_needed(cap, block_size))
    return _assemble(name, rng, dtype, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, mgr, seqs, decode_lens, max_blocks, slots, [], poison,
                     random_copies=random_copies)


def _shared_prefix(name: str, seed: int, fork: bool, poison: bool) -> Workload:
    """16 groups x 8 samples sharing a 1024-token prefix (40/40 heads, d 128)."""
    groups, per_group, prefix, bs = 16, 8, 1024, 16
    rng = np.random.default_rng(seed)
    b = groups * per_group
    if fork:
        extra = rng.integers(1, 16, groups)               # partial shared tail block
        pre_lens = np.repeat(prefix + extra, per_group)
        need = int(sum(blocks_needed(prefix + int(e), bs) for e in extra)) + groups * (per_group - 1)
    else:
        tails = rng.integers(16, 257, b)                 # private tails, group-major
        pre_lens = prefix + tails
        need = groups * (prefix // bs) + int(sum(blocks_needed(int(t) + 1, bs) for t in tails))
    num_blocks = _pool_size(need)
    perm = rng.permutation(num_blocks)
    mgr = BlockManager(num_blocks, bs, free_order=perm)
    for g in range(groups):
        parent = g * per_group
        mgr.add_sequence(parent, int(pre_lens[parent]) if fork else prefix)
        for i in range(1, per_group):
            mgr.fork(parent, parent + i)
    if not fork:
        for s in range(b):                               # grow private tails
            for _ in range(int(pre_lens[s]) - prefix):
                _, copy = mgr.append_slot(s)
                assert copy is None
    slots, copies = [], []
    for s in range(b):
        slot, copy = mgr.append_slot(s)
        slots.append(slot)
        if copy is not None:
            copies.append(copy)
    if fork:
        assert len(copies) == groups * (per_group - 1)
    else:
        assert not copies
    decode_lens = pre_lens + 1
    max_len = prefix + 256 + 1
    max_blocks = blocks_needed(max_len, bs)
    wl = _assemble(name, rng, BF16, 40, 40, 128, bs, num_blocks, mgr, list(range(b)),
                   decode_lens, max_blocks, slots, copies, poison)
    # Each group's 8 samples share the prefix's 64 whole blocks (after the
    # fork step's copies, the partial 65th block is private to each sample).
    wl.group_start = np.arange(0, b + 1, per_group, dtype=np.int32)
    wl.prefix_lens = np.full(b, prefix, dtype=np.int32)
    wl.notes["unique_tokens"] = int(groups * prefix + (decode_lens - prefix).sum()) if not fork \
        else int(sum(int(pre_lens[g * per_group]) for g in range(groups)) + b)
    return wl


def common_prefix_lens(tables: np.ndarray, lens: np.ndarray, group_start: np.ndarray,
                       block_size: int, appended: bool) -> np.ndarray:
    """Per sequence, the tokens its group shares physically: the leading
    block-table entries equal in every member (within every member's blocks),
    as tokens, at most the shortest member's length (less the token this
    step appends, which is never shared)."""
    out = np.zeros(len(lens), dtype=np.int32)
    for g in range(len(group_start) - 1):
        lo, hi = int(group_start[g]), int(group_start[g + 1])
        if hi <= lo:
            continue
        lmin = int(lens[lo:hi].min()) - (1 if appended else 0)
        nblk = blocks_needed(max(lmin, 0), block_size)
        same = 0
        while same < nblk and np.all(tables[lo:hi, same] == tables[lo, same]):
            same += 1
        out[lo:hi] = max(0, min(same * block_size, lmin))
    return out


def make_shared_groups(name: str, seed: int, dtype: str, num_q_heads: int, num_kv_heads: int,
                       head_dim: int, block_size: int, group_sizes, prefix_tokens, tail_range,
                       append: bool, poison: bool,
                       rng: Optional[np.random.Generator] = None) -> Workload:
    """Groups of sequences forked from a common parent: group g's parent holds
    ``prefix_tokens[g]`` tokens when ``group_sizes[g]`` members are forked from
    it; each member then grows a private tail of U[tail_range] tokens (the
    first divergent write into a shared partial block copies it, as the host
    block manager does), and with ``append`` the step appends one more token
    per member (copying a still-shared tail block in the step itself:
    ``block_mapping``).  ``prefix_lens`` are the tokens each group's members
    still share physically after the step's copies.

    Draw order: tails, pool permutation, then the values as ``_assemble``."""
    rng = np.random.default_rng(seed) if rng is None else rng
    sizes = [int(x) for x in group_sizes]
    prefix = [int(x) for x in prefix_tokens]
    b = sum(sizes)
    tails = rng.integers(int(tail_range[0]), int(tail_range[1]) + 1, b)
    # Blocks: each parent's prefix once, then per member its tail, a possible
    # copy of a partial shared block and the step's append.
    need = sum(blocks_needed(p, block_size) for p in prefix)
    need += sum(blocks_needed(int(t) + 2, block_size) + 1 for t in tails)
    num_blocks = max(1, _pool_size(need))
    perm = rng.permutation(num_blocks)
    mgr = BlockManager(num_blocks, block_size, free_order=perm)
    seq = 0
    for g, m in enumerate(sizes):
        parent = seq
        mgr.add_sequence(parent, prefix[g])
        for i in range(1, m):
            mgr.fork(parent, parent + i)
        seq += m
    for s in range(b):                      # private tails (copies happen before this step)
        for _ in range(int(tails[s])):
            mgr.append_slot(s)
    slots, copies = ([], []) if append else (None, [])
    if append:
        for s in range(b):
            slot, copy = mgr.append_slot(s)
            slots.append(slot)
            if copy is not None:
                copies.append(copy)
    lens = np.array([mgr.lengths[s] for s in range(b)], dtype=np.int64)
    max_blocks = max(1, max(len(mgr.tables[s]) for s in range(b)))
    wl = _assemble(name, rng, dtype, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   mgr, list(range(b)), lens, max_blocks, slots, copies, poison)
    wl.group_start = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    wl.prefix_lens = common_prefix_lens(wl.block_tables, lens, wl.group_start, block_size, append)
    return wl


def _lognormal_lengths(rng, n):
    return np.clip(np.rint(rng.lognormal(math.log(4096), math.log(2), n)), 1024, 16384).astype(np.int64)


def _pareto_lengths(rng, n):
    u = rng.random(n)
    return np.minimum(np.floor(128.0 * (1.0 - u) ** (-1.0 / 1.2)), 32768).astype(np.int64)


WORKLOADS = ("tiny_fp32", "opt13b_mha", "llama13b_long", "shared_prefix_steady",
             "shared_prefix_fork", "gqa_pareto_bs16", "gqa_pareto_bs32", "gqa_single_4k",
             "gqa_single_32k")


def make_workload(name: str, poison: bool = True) -> Workload:
    """Build one named workload (see the module docstring)."""
    if name == "tiny_fp32":
        rng = np.random.default_rng(3101)
        pre = rng.integers(1, 129, 4)
        return make_simple(name, 3101, FP32, 8, 8, 64, 16, pre + 1, append=True, poison=poison,
                           num_blocks=64, max_len=129, random_copies=2, rng=rng)
    if name == "opt13b_mha":
        rng = np.random.default_rng(3102)
        lens = rng.integers(64, 2049, 64)
        return make_simple(name, 3102, BF16, 40, 40, 128, 16, lens, append=False, poison=poison,
                           max_len=2048, rng=rng)
    if name == "llama13b_long":
        rng = np.random.default_rng(3103)
        lens = _lognormal_lengths(rng, 32)
        return make_simple(name, 3103, BF16, 40, 40, 128, 16, lens, append=True, poison=poison,
                           max_len=16384, rng=rng)
    if name == "shared_prefix_steady":
        return _shared_prefix(name, 3104, fork=False, poison=poison)
    if name == "shared_prefix_fork":
        return _shared_prefix(name, 3104, fork=True, poison=poison)
    if name in ("gqa_pareto_bs16", "gqa_pareto_bs32"):
        rng = np.random.default_rng(3105)
        lens = _pareto_lengths(rng, 256)
        bs = 16 if name.endswith("16") else 32
        return make_simple(name, 3105, BF16, 64, 8, 128, bs, lens, append=True, poison=poison,
                           max_len=32768, rng=rng)
    if name in ("gqa_single_4k", "gqa_single_32k"):
        n = 4096 if name.endswith("4k") else 32768
        return make_simple(name, 3106, BF16, 64, 8, 128, 16, [n], append=True, poison=poison,
                           rng=np.random.default_rng(3106))
    raise KeyError(f"unknown workload {name!r}; choose from {WORKLOADS}")


def workload_lengths(name: str) -> np.ndarray:
    """Decode lengths of a named workload without drawing its values."""
    if name == "tiny_fp32":
        return np.random.default_rng(3101).integers(1, 129, 4) + 1
    if name == "opt13b_mha":
        return np.random.default_rng(3102).integers(64, 2049, 64)
    if name == "llama13b_long":
        return _lognormal_lengths(np.random.default_rng(3103), 32)
    if name == "shared_prefix_steady":
        return 1024 + np.random.default_rng(3104).integers(16, 257, 128) + 1
    if name == "shared_prefix_fork":
        return np.repeat(1024 + np.random.default_rng(3104).integers(1, 16, 16), 8) + 1
    if name in ("gqa_pareto_bs16", "gqa_pareto_bs32"):
        return _pareto_lengths(np.random.default_rng(3105), 256)
    if name in ("gqa_single_4k", "gqa_single_32k"):
        return np.array([4096 if name.endswith("4k") else 32768])
    raise KeyError(name)


# --------------------------------------------------------- multi-token queries
@dataclass
class PrefillWorkload:
    """Inputs of one multi-token (prompt / chunked prompt) attention call.

    Sequence ``s`` holds ``context_lens[s]`` tokens; its newest
    ``n_s = query_start[s+1] - query_start[s]`` tokens are the query chunk.
    ``k_new``/``v_new`` are the chunk's rows and ``slot_mapping`` their slots
    (append them first); with ``poison=True`` those slots, and every slot no
    sequence holds, are NaN in the pools until the append fills them.
    """
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: np.float32
    q: np.ndarray                 # [num_query_tokens, num_q_heads, head_dim]
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray      # int32 [num_seqs, max_blocks]
    context_lens: np.ndarray      # int32 [num_seqs]
    query_start: np.ndarray       # int32 [num_seqs + 1]
    k_new: np.ndarray             # [num_query_tokens, num_kv_heads, head_dim]
    v_new: np.ndarray
    slot_mapping: np.ndarray      # int64 [num_query_tokens]

    @property
    def num_query_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start.astype(np.int64))

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0


def make_prefill(name: str, seed: int, dtype: str, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, context_lens, query_lens, poison: bool = True,
                 rng: Optional[np.random.Generator] = None) -> PrefillWorkload:
    """Sequences of ``context_lens`` tokens whose newest ``query_lens`` tokens
    form the query chunk, blocks scattered over a pool 1.25x the need.

    Draw order: pool permutation, q, K pool, V pool, new K, new V."""
    rng = np.random.default_rng(seed) if rng is None else rng
    ctx = np.asarray(context_lens, dtype=np.int64)
    nq = np.asarray(query_lens, dtype=np.int64)
    if ctx.shape != nq.shape or np.any(nq < 0) or np.any(nq > ctx):
        raise ValueError("need 0 <= query_lens <= context_lens, one per sequence")
    b, bs = len(ctx), block_size
    per_seq = [blocks_needed(int(n), bs) for n in ctx]
    num_blocks = max(_pool_size(sum(per_seq)), 1)
    perm = rng.permutation(num_blocks)
    tables = np.full((b, max(max(per_seq, default=1), 1)), -1, dtype=np.int32)
    used = 0
    for s, k in enumerate(per_seq):
        tables[s, :k] = perm[used:used + k]
        used += k
    starts = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    total = int(starts[-1])
    q = normal_bits(rng, (total, num_q_heads, head_dim), dtype)
    k_cache = normal_bits(rng, (num_blocks, num_kv_heads, bs, head_dim), dtype)
    v_cache = normal_bits(rng, (num_blocks, num_kv_heads, bs, head_dim), dtype)
    k_new = normal_bits(rng, (total, num_kv_heads, head_dim), dtype)
    v_new = normal_bits(rng, (total, num_kv_heads, head_dim), dtype)
    slots = np.empty(total, dtype=np.int64)
    held = np.zeros((num_blocks, bs), dtype=bool)      # slots holding an earlier token
    for s in range(b):
        L, n = int(ctx[s]), int(nq[s])
        for p in range(L):
            blk, off = int(tables[s, p // bs]), p % bs
            if p < L - n:
                held[blk, off] = True
            else:
                slots[starts[s] + p - (L - n)] = blk * bs + off
    if poison:
        blk, off = np.nonzero(~held)
        k_cache[blk, :, off, :] = nan_bits(dtype)
        v_cache[blk, :, off, :] = nan_bits(dtype)
    return PrefillWorkload(name, dtype, b, num_q_heads, num_kv_heads, head_dim, bs, num_blocks,
                           np.float32(1.0 / math.sqrt(head_dim)), q, k_cache, v_cache, tables,
                           ctx.astype(np.int32), starts, k_new, v_new, slots)


PREFILL_WORKLOADS = ("llama13b_prefill", "gqa_chunked_prefill", "gqa_single_chunk_32k")


def make_prefill_workload(name: str, poison: bool = True) -> PrefillWorkload:
    """Named multi-token workloads (the pages give no prompt workload; these
    keep the decode workloads' head shapes and block size):

    * llama13b_prefill: 8 fresh prompts, lengths U[512, 2048], 40/40 heads,
      d 128, bs 16, bf16 -- the whole prompt is the chunk;
    * gqa_chunked_prefill: 16 sequences, 64 query heads over 8 KV heads, d 128,
      bs 16, bf16, a 512-token chunk on top of an earlier context of
      lognormal(median 2048, sigma ln 2) tokens clipped to [256, 8192];
    * gqa_single_chunk_32k: one sequence, 64 query heads over 8 KV heads, d 128,
      bs 16, bf16, a 64-token chunk on top of 32,704 earlier tokens (a long
      conversation's next turn: few query rows, many keys).
    """
    if name == "llama13b_prefill":
        rng = np.random.default_rng(3110)
        lens = rng.integers(512, 2049, 8)
        return make_prefill(name, 3110, BF16, 40, 40, 128, 16, lens, lens, poison, rng)
    if name == "gqa_chunked_prefill":
        rng = np.random.default_rng(3111)
        prior = np.clip(np.rint(rng.lognormal(math.log(2048), math.log(2), 16)), 256, 8192)
        prior = prior.astype(np.int64)
        return make_prefill(name, 3111, BF16, 64, 8, 128, 16, prior + 512,
                            np.full(16, 512), poison, rng)
    if name == "gqa_single_chunk_32k":
        return make_prefill(name, 3112, BF16, 64, 8, 128, 16, [32768], [64], poison)
    raise KeyError(f"unknown prefill workload {name!r}; choose from {PREFILL_WORKLOADS}")
