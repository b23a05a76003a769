"""Plain, slow, obviously-correct CPU oracle for paged decode attention,
paged multi-token (prefill) attention, the paged KV append and the
copy-on-write block copy.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.  It shares no code
with the HIP path and imports nothing from it.  Floating point is fp64;
data movement works on raw bit patterns, so it is exact.

Sources (the three web pages about "Efficient Memory Management for Large
Language Model Serving with PagedAttention"; cited by page and section):

* [P1] phantomic12.github.io catalogue note, method paragraph: the KV cache
  is cut into fixed-size blocks, and each request keeps a block table that
  the attention kernels read through.
* [P3] zeroshotmind.com essay, sections "Paging the cache", "Block tables:
  logical order, physical scatter", "Sharing a prefix without copying it".

The pages give no attention formula.  The oracle uses the textbook scaled
dot-product attention ``softmax(q . K^T * scale) . V`` over every cached
token of the sequence, including the one written this step (no other mask).
For a chunk of several query tokens (``prefill``) each query token sees the
positions up to and including its own (causal attention).

Memory layout read by the oracle (a reading: the pages fix no layout):

* ``k_cache``, ``v_cache``: ``[num_blocks, num_kv_heads, block_size, head_dim]``
  holding raw element bits: ``uint16`` for bfloat16, ``float32`` for fp32.
* ``block_tables``: int32 ``[num_seqs, max_blocks_per_seq]``, logical block
  index -> physical block number.  Entries past ``ceil(len / block_size)``
  are never read.
* ``context_lens``: int32 ``[num_seqs]``, tokens cached after this step's
  append.
* ``slot_mapping``: int64 ``[num_tokens]``; ``slot = block * block_size +
  offset``; a negative slot means "no write".
* ``block_mapping``: int64 ``[num_pairs, 2]`` of ``(src, dst)``.
* GQA: query head ``h`` reads KV head ``h // (num_q_heads // num_kv_heads)``.

Every function is pinned by tests in ``tests/test_oracle_pins.py`` against
closed forms, brute force, ``torch.nn.functional.scaled_dot_product_attention``
in fp64 on contiguous data, hand-worked fixtures and the invariants the pages
state.  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


def bits_to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored element bits to float64.

    bfloat16 is the upper half of an IEEE float32, so ``bits << 16`` viewed
    as float32 is the same number; float32 -> float64 is exact.
    """
    if dtype == BF16:
        if raw.dtype != np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == FP32:
        if raw.dtype != np.float32:
            raise TypeError("fp32 data must be passed as float32")
        return raw.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def append_kv(k_cache, v_cache, k_new, v_new, slot_mapping, block_size):
    """Paged KV append: write each new token's K/V rows into its slot.

    [P3] "Paging the cache": a sequence's cache lives in fixed-size blocks
    that are allocated on demand; a new token lands in the tail block.  The
    slot names (physical block, offset) as ``block * block_size + offset``.
    ``k_new``/``v_new`` are ``[num_tokens, num_kv_heads, head_dim]``.
    Tokens are written in order; a negative slot writes nothing.  Returns new
    pools; every byte not named by a slot is unchanged.
    """
    k_out = k_cache.copy()
    v_out = v_cache.copy()
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), int(block_size))
        k_out[block, :, offset, :] = k_new[t]
        v_out[block, :, offset, :] = v_new[t]
    return k_out, v_out


def copy_blocks(k_cache, v_cache, block_mapping):
    """Copy-on-write block copy.

    [P3] "Sharing a prefix without copying it": on a write into a shared
    block the system duplicates just that one block into a private copy.
    For every ``(src, dst)`` pair the whole block (all KV heads, all slots)
    of both pools is copied; reads come from the pools as they were before
    the call, so ``src`` itself never changes.
    """
    k_out = k_cache.copy()
    v_out = v_cache.copy()
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2).tolist():
        k_out[dst] = k_cache[src]
        v_out[dst] = v_cache[src]
    return k_out, v_out


def gather_sequence(cache, table_row, length, block_size, kv_head):
    """Gather one sequence's rows for one KV head in logical order.

    [P3] "Block tables: logical order, physical scatter": attention walks
    the logical indices in order, looks each one up in the table to find its
    physical block, and reads the keys/values from there.  Position ``j``
    lives in logical block ``j // block_size`` at offset ``j % block_size``.
    Returns ``[length, head_dim]`` raw element bits.
    """
    positions = np.arange(int(length))
    physical = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    return cache[physical, kv_head, positions % block_size, :]


def attention_rows(q_row, keys, values, scale):
    """Scaled dot-product attention of one query row over ``n`` keys, fp64.

    ``z_j = scale * (q . k_j)``; ``out = sum_j softmax(z)_j v_j``.  The
    maximum is subtracted before exponentiating (an identity that keeps the
    exponentials finite).  An empty key set gives the zero vector.
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    z = np.float64(scale) * (keys @ q_row)
    w = np.exp(z - z.max())
    return (w @ values) / w.sum()


def kv_head_for(q_head, num_q_heads, num_kv_heads):
    """Grouped-query mapping: consecutive query heads share one KV head
    (query head ``h`` reads KV head ``h // (num_q_heads // num_kv_heads)``).
    With equal head counts this is the identity (multi-head attention)."""
    return q_head // (num_q_heads // num_kv_heads)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
           block_size, rows=None):
    """Decode-step paged attention, fp64.

    ``q``: ``[num_seqs, num_q_heads, head_dim]`` raw bits of ``dtype``.
    ``scale`` is the float32 value the caller passes to the kernel; it is
    widened exactly to fp64 here.  ``rows``: optional iterable of
    ``(seq, q_head)`` pairs to evaluate (the others stay zero), so single
    outputs can be checked at full size.  Returns fp64
    ``[num_seqs, num_q_heads, head_dim]``.

    [P1] method paragraph: attention kernels read through the block table.
    [P3] "Block tables": the kernel sees a contiguous logical sequence, so
    the result is plain attention over the gathered keys and values.
    """
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    scale64 = np.float64(np.float32(scale))
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    if rows is None:
        rows = [(s, h) for s in range(num_seqs) for h in range(num_q_heads)]
    cached = {}
    for s, h in rows:
        length = int(context_lens[s])
        kv_head = kv_head_for(h, num_q_heads, num_kv_heads)
        key = (s, kv_head)
        if key not in cached:
            k = bits_to_f64(gather_sequence(k_cache, block_tables[s], length,
                                            block_size, kv_head), dtype)
            v = bits_to_f64(gather_sequence(v_cache, block_tables[s], length,
                                            block_size, kv_head), dtype)
            cached = {key: (k, v)}
        k, v = cached[key]
        out[s, h] = attention_rows(bits_to_f64(q[s, h], dtype), k, v, scale64)
    return out


def query_position(context_len, query_len, i):
    """Position of the ``i``-th token of a sequence's query chunk.

    A chunk of ``query_len`` query tokens is the sequence's newest tokens:
    their keys/values are already cached, so the sequence holds
    ``context_len`` tokens and query token ``i`` sits at position
    ``context_len - query_len + i``.  (A reading: the pages describe prompt
    processing only as attention read through the block table -- [P1] method
    paragraph -- and fix no chunk convention; this is the one a decode step
    generalises, since a chunk of one token is exactly a decode step.)
    """
    return int(context_len) - int(query_len) + int(i)


def visible_keys(position):
    """Number of leading positions a query at ``position`` attends to: every
    position up to and including its own (causal attention in a decoder)."""
    return int(position) + 1


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype,
            block_size, rows=None):
    """Multi-token (prompt / chunked prompt) paged attention, fp64.

    ``q``: ``[num_query_tokens, num_q_heads, head_dim]`` raw bits; the query
    tokens of sequence ``s`` are rows ``query_start[s] .. query_start[s+1]-1``
    (int32 ``query_start`` of length ``num_seqs + 1``).  Their keys/values
    are already in the pools (written by an append through the slot mapping).
    Query token ``i`` of sequence ``s`` at position ``p`` attends to the
    sequence's positions ``0 .. p`` read through its block table:
    ``out = sum_{j <= p} softmax_j(scale * q . k_j) v_j``.

    [P1] method paragraph: attention kernels read through the block table.
    [P3] "Block tables": the logical order is the sequence's order, so the
    result is plain causal attention over the gathered keys and values.
    ``rows``: optional iterable of ``(query_token, q_head)`` pairs to evaluate
    (the others stay zero).  Returns fp64 ``[num_query_tokens, num_q_heads,
    head_dim]``.
    """
    num_tokens, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    starts = np.asarray(query_start, dtype=np.int64)
    seq_of = np.zeros(num_tokens, dtype=np.int64)
    for s in range(len(starts) - 1):
        seq_of[starts[s]:starts[s + 1]] = s
    scale64 = np.float64(np.float32(scale))
    out = np.zeros((num_tokens, num_q_heads, head_dim), dtype=np.float64)
    if rows is None:
        rows = [(t, h) for t in range(num_tokens) for h in range(num_q_heads)]
    cached = {}
    for t, h in rows:
        s = int(seq_of[t])
        length = int(context_lens[s])
        n = int(starts[s + 1] - starts[s])
        position = query_position(length, n, t - starts[s])
        kv_head = kv_head_for(h, num_q_heads, num_kv_heads)
        key = (s, kv_head)
        if key not in cached:
            k = bits_to_f64(gather_sequence(k_cache, block_tables[s], length,
                                            block_size, kv_head), dtype)
            v = bits_to_f64(gather_sequence(v_cache, block_tables[s], length,
                                            block_size, kv_head), dtype)
            cached = {key: (k, v)}
        k, v = cached[key]
        m = visible_keys(position)
        out[t, h] = attention_rows(bits_to_f64(q[t, h], dtype), k[:m], v[:m], scale64)
    return out
