/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV-cache library (libpa.so).
 *
 * Three device operations on a pool of fixed-size KV blocks:
 *   pa_append_kv    write new tokens' keys/values into the slots a slot mapping names;
 *   pa_copy_blocks  copy whole blocks (the copy in copy-on-write);
 *   pa_decode       one decode step of attention for every sequence, reading each
 *                   sequence's keys/values through its block table
 *                   (pa_decode_shared: the same, reading tokens that groups of
 *                   sequences share once per group);
 *   pa_prefill      attention of a multi-token query chunk per sequence (a prompt,
 *                   or a piece of one) with a causal mask, through the block table;
 * and, for a model whose layers each own a pool, layer-batched forms of the
 * first two (pa_append_kv_layers, pa_copy_blocks_layers): one call serves
 * every layer.
 *
 * Sources: the pages on "Efficient Memory Management for Large Language Model
 * Serving with PagedAttention" -- zeroshotmind.com essay, sections "Paging the
 * cache" (fixed-size blocks, 16 tokens by default, allocated on demand),
 * "Block tables: logical order, physical scatter" (per-sequence table, logical
 * block index -> physical block number; attention walks the logical order),
 * "Sharing a prefix without copying it" (ref-counted shared blocks; a write
 * into a shared block duplicates that one block); phantomic12.github.io
 * catalogue note, method paragraph (attention kernels read through the block
 * table).  The attention itself is scaled dot-product attention
 * softmax(q . K^T * scale) . V over all cached tokens of the sequence.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer to caller-owned, contiguous,
 *    row-major memory, 16-byte aligned.  The library allocates nothing,
 *    frees nothing and keeps no pointer after returning.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; results are visible in stream order.
 *  - `dtype` (pa_dtype) is the element type of q, out, both pools and the
 *    new K/V; there is no conversion anywhere, so data movement is bit-exact.
 *  - Pools: k_cache, v_cache are [num_blocks, num_kv_heads, block_size, head_dim].
 *    Slot s of the pool is physical block s / block_size, offset s % block_size.
 *  - Supported: head_dim in {64, 128}; block_size in {16, 32}; dtype fp32 or
 *    bf16; num_q_heads a multiple of num_kv_heads.
 *  - Return value: PA_OK (0) or a pa_status error.  Scalar arguments are
 *    checked before any HIP call.  Index data lives on the device and is NOT
 *    checked by default (that would need a device->host copy): out-of-range
 *    blocks or slots, duplicate slots, or copy pairs that alias are undefined
 *    behaviour.  With the environment variable PA_CHECK=1 every call copies
 *    its index arrays to the host, synchronising `stream`, and returns
 *    PA_ERR_INDEX instead of launching when they break the contract.
 *  - Without PA_CHECK a call only launches kernels on `stream`, so a sequence
 *    of calls can be captured in a HIP graph and replayed, provided the
 *    caller allocates the workspace and outputs beforehand.  Under PA_CHECK=1
 *    a call copies to the host and synchronizes, and cannot be captured.
 *  - The library never prints, throws or aborts.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* bad scalar argument or NULL pointer              */
  PA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, block_size, dtype */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  PA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed       */
  PA_ERR_INDEX = 5        /* PA_CHECK=1 found index data breaking the contract */
} pa_status;

typedef enum pa_dtype { PA_DTYPE_FP32 = 0, PA_DTYPE_BF16 = 1 } pa_dtype;

/* Paged KV append.  Page: "Paging the cache" (a new token goes into the
 * sequence's tail block, a fresh block only when the tail is full; the host
 * block manager picks the slot).
 *   k_new, v_new   [num_tokens, num_kv_heads, head_dim]      read
 *   slot_mapping   int64 [num_tokens]; slot < 0 = skip token  read
 *   k_cache[slot / block_size, :, slot % block_size, :] = k_new[t]  (same for V)
 * Every other byte of the pools is left unchanged.  Contract: slots in
 * [0, num_blocks*block_size) or negative; no slot repeats.  num_tokens == 0
 * is a no-op. */
int pa_append_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                 const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                 int num_kv_heads, int block_size, int head_dim, int dtype, void* stream);

/* Copy-on-write block copy.  Page: "Sharing a prefix without copying it"
 * (duplicate just the one shared block being written).
 *   block_mapping  int64 [num_pairs][2] = (src, dst)           read
 *   k_cache[dst] = k_cache[src]; v_cache[dst] = v_cache[src]  (all heads, all slots)
 * Contract: ids in [0, num_blocks); no dst repeats; no dst equals any src of the
 * same call (so the result never depends on copy order).  num_pairs == 0 is a
 * no-op. */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                   int64_t num_blocks, int num_kv_heads, int block_size, int head_dim,
                   int dtype, void* stream);

/* Layer-batched append.  Each layer of a model caches its own keys and
 * values, all under one block table per sequence (pages: "Paging the cache",
 * "Block tables: logical order, physical scatter" -- a token's slot is chosen
 * once, so every layer writes the same slot of its own pool).  For every layer
 * l in [0, num_layers) this does exactly what
 *   pa_append_kv(k_caches[l], v_caches[l], k_new[l], v_new[l], slot_mapping, ...)
 * does, in one launch per 32 layers instead of one per layer.
 *   k_caches, v_caches  HOST arrays of num_layers device pointers to pools
 *                       [num_blocks, num_kv_heads, block_size, head_dim]
 *   k_new, v_new        HOST arrays of num_layers device pointers to
 *                       [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping        int64 [num_tokens], device, shared by all layers
 * The host arrays are read during the call only.  Every pointer in them must
 * be non-NULL and 16-byte aligned (else PA_ERR_INVALID); pools of different
 * layers must not overlap.  num_tokens == 0 or num_layers == 0 is a no-op.
 * Same slot contract and PA_CHECK behaviour as pa_append_kv. */
int pa_append_kv_layers(void* const* k_caches, void* const* v_caches,
                        const void* const* k_new, const void* const* v_new, int num_layers,
                        const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                        int num_kv_heads, int block_size, int head_dim, int dtype, void* stream);

/* Layer-batched copy-on-write copy (page: "Sharing a prefix without copying
 * it"): a shared block is shared in every layer's pool at once, so its
 * duplication copies the block in every layer.  For every layer l this does
 * exactly what pa_copy_blocks(k_caches[l], v_caches[l], block_mapping, ...)
 * does, in one launch per 32 layers (and per 65535 pairs).
 *   k_caches, v_caches  HOST arrays of num_layers device pointers to pools
 *   block_mapping       int64 [num_pairs][2] = (src, dst), device, shared by all layers
 * Pointer rules as pa_append_kv_layers; copy-pair contract and PA_CHECK
 * behaviour as pa_copy_blocks.  num_pairs == 0 or num_layers == 0 is a no-op. */
int pa_copy_blocks_layers(void* const* k_caches, void* const* v_caches, int num_layers,
                          const int64_t* block_mapping, int64_t num_pairs, int64_t num_blocks,
                          int num_kv_heads, int block_size, int head_dim, int dtype,
                          void* stream);

/* Bytes of device workspace pa_decode needs for these sizes and `num_workers`
 * (0 = the library's default for the current device).  Writes *bytes.  The
 * workspace holds, per worker, a 48-byte merge record (the record array is
 * padded to 256 bytes) and partial results of the context split:
 * num_workers * 2 * (num_q_heads / num_kv_heads) * (head_dim + 4) floats.
 * It needs no initialisation; one workspace serves successive calls of any
 * shape in stream order (never two calls at once). */
int pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int num_workers, size_t* bytes);

/* Upper bound of the number of workers (64-lane wavefronts, one per
 * workgroup) pa_decode uses by default on the current device -- the count
 * pa_decode_workspace_size assumes for num_workers = 0.  Writes *num_workers. */
int pa_decode_default_workers(int* num_workers);

/* Decode-step paged attention.  Pages: "Block tables: logical order, physical
 * scatter" (walk logical blocks in order through the table, gather K/V) and
 * the catalogue note's method paragraph (attention reads through the table).
 *   out            [num_seqs, num_q_heads, head_dim]                 written
 *   q              [num_seqs, num_q_heads, head_dim]                 read
 *   block_tables   int32 [num_seqs, max_blocks_per_seq]              read
 *   context_lens   int32 [num_seqs]: tokens cached for the sequence
 *                  AFTER this step's append (0 = empty -> out row is 0)
 *   For query head h, KV head kvh = h / (num_q_heads / num_kv_heads):
 *     out[s,h] = sum_j softmax_j(scale * q[s,h] . K_j) V_j over positions
 *     j < context_lens[s], position j stored in block
 *     block_tables[s][j / block_size] at offset j % block_size.
 *   Fused append: k_new, v_new ([num_seqs, num_kv_heads, head_dim]) and
 *     slot_mapping (int64 [num_seqs]) are all NULL, or all set.  When set,
 *     token s is sequence s's newest token: the call behaves exactly like
 *     pa_append_kv(k_new, v_new, slot_mapping, num_seqs) followed by
 *     pa_decode without them.  Contract: slot_mapping[s] is negative or the
 *     slot of position context_lens[s]-1 of sequence s.
 *   workspace      see pa_decode_workspace_size (read/written)
 *   num_workers    0 = default: workers resident at once (3 per compute
 *                  unit on the matrix-core kernel, 21 per 8 compute units on
 *                  the vector kernel, 3 per compute unit there when T below
 *                  is under 65,536), but at most about
 *                  10 sqrt(T) (and 160 per segment) on the matrix-core
 *                  kernel and 7 sqrt(T) on the vector kernel, T = segments
 *                  x 16-token chunks of the table width (a segment is a
 *                  (sequence, KV head) pair on the matrix-core kernel, a
 *                  (sequence, query head) pair otherwise; the vector
 *                  kernel's bound is at least 20 per segment), rounded up
 *                  to a multiple of 8, so that small
 *                  batches do not spend more time merging split pieces than
 *                  they gain.  Otherwise the exact number of workers.  A
 *                  tuning knob that changes only the fp32 summation order.
 * Contract: 0 <= context_lens[s] <= max_blocks_per_seq * block_size; table
 * entries for the blocks a sequence uses lie in [0, num_blocks); entries past
 * them are never read. */
int pa_decode(void* out, const void* q, void* k_cache, void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq,
              const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
              int head_dim, int block_size, int64_t num_blocks, float scale,
              const void* k_new, const void* v_new, const int64_t* slot_mapping,
              void* workspace, size_t workspace_bytes, int num_workers,
              int dtype, void* stream);

/* Bytes of device workspace pa_decode_shared needs for these sizes and
 * num_workers (0 = the library's default for the current device), whichever
 * of its paths the call takes.  Writes *bytes.  It holds what pa_decode's
 * workspace holds (partial slots of 16 rows per worker) plus, per sequence
 * and KV head, two 16-byte locators and, per sequence and query head, two
 * result rows of head_dim + 4 floats.  No initialisation needed; one
 * workspace serves successive calls in stream order (never two at once). */
int pa_decode_shared_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int num_workers, size_t* bytes);

/* Decode-step paged attention for a batch whose sequences come in groups that
 * share a prefix -- samples forked from one prompt, beams of one request.
 * Page: zeroshotmind.com essay, "Sharing a prefix without copying it" (the
 * sharers' block tables point at the same physical blocks, so one copy of the
 * prefix serves all of them); "Block tables: logical order, physical scatter".
 * Computes exactly what pa_decode computes with the same arguments (the same
 * out, the same fused append, within the fp32 summation order), but reads
 * the shared tokens once per group instead of once per member: each shared
 * 16-token tile of a KV head is read once for all the group's query rows.
 *   group_start   int32 [num_groups + 1], device: group g is the sequences
 *                 group_start[g] <= s < group_start[g + 1] (consecutive)
 *   num_groups    0 = no groups: plain pa_decode
 *   prefix_lens   int32 [num_seqs], device: tokens at the start of sequence s
 *                 that it shares with the rest of its group (0 = none)
 *   Everything else as pa_decode; workspace per pa_decode_shared_workspace_size.
 * Contract (checked under PA_CHECK=1): group_start[0] = 0, non-decreasing,
 * group_start[num_groups] = num_seqs; 0 <= prefix_lens[s] <= context_lens[s],
 * and < context_lens[s] when the fused append writes sequence s (the new
 * token is never shared); prefix_lens equal within a group; the block-table
 * entries of the first ceil(prefix_lens[s] / block_size) blocks of every
 * member equal those of the group's first sequence.  The shared part of a
 * sequence is its first floor(prefix_lens[s] / 16) * 16 tokens; the rest is
 * read through its own table.
 * Paths: bf16, head_dim 128 and 1..16 query heads per KV head run the shared
 * kernels (one attention launch, whose workers split between the groups'
 * shared tokens and the sequences' own tokens, and one merge); other shapes
 * run pa_decode's kernels.  num_workers as pa_decode (the shared kernels use
 * at least 2).  pa_set_decode_events times the attention launch. */
int pa_decode_shared(void* out, const void* q, void* k_cache, void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                     float scale, const void* k_new, const void* v_new,
                     const int64_t* slot_mapping, const int32_t* group_start, int num_groups,
                     const int32_t* prefix_lens, void* workspace, size_t workspace_bytes,
                     int num_workers, int dtype, void* stream);

/* pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture that must not call hipMalloc, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, semantics, contract and kernels as
 * pa_decode, without the workspace: the merge records and partial results live
 * in a static device array of PA_NOALLOC_SCRATCH_BYTES bytes that each GPU the
 * library runs on holds from this entry point's first call on it until the
 * process ends.  The call allocates and frees nothing.
 *   Its need is what pa_decode needs for these sizes with bf16 head_dim 128
 *   and 2..16 query heads per KV head (the matrix-core kernel):
 *   num_workers * 2 * group * (head_dim + 4) * 4 bytes plus 48 bytes per
 *   worker (rounded up to 256); otherwise num_workers * 2 * (head_dim + 4) * 4
 *   bytes plus the same records.  The default worker count of every shape
 *   fits on a 256-CU device (at most 1,024 workers: 17.4 MB for groups of
 *   16); a need above PA_NOALLOC_SCRATCH_BYTES (an explicit num_workers) is
 *   rejected with PA_ERR_WORKSPACE before any launch.
 *   The array needs no initialisation: every call writes what it reads.
 * All calls on one GPU share its one array, so two pa_decode_noalloc calls
 * that can overlap on one GPU (different streams, or different host threads
 * without ordering) race and give wrong results; calls ordered on one stream
 * are safe.  PA_ERR_UNSUPPORTED for device ordinals of 64 and above. */
#define PA_NOALLOC_SCRATCH_BYTES (24u << 20)
int pa_decode_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                      float scale, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int num_workers, int dtype, void* stream);

/* Multi-token (prompt / chunked-prompt) paged attention.  Pages: catalogue
 * note, method paragraph (attention reads through the block table) and
 * "Block tables: logical order, physical scatter" (logical order = the
 * sequence's order).  The query chunk of sequence s is its newest
 * n_s = query_start[s+1] - query_start[s] tokens, whose keys/values are
 * already in the pools (pa_append_kv / pa_append_kv_layers with their slots
 * first); query token i of the chunk sits at position
 * p = context_lens[s] - n_s + i and attends to positions 0..p (causal):
 *   out[t,h] = sum_{j <= p} softmax_j(scale * q[t,h] . K_j) V_j,
 *   t = query_start[s] + i, K_j/V_j of KV head h / (num_q_heads / num_kv_heads).
 *   out, q         [num_query_tokens, num_q_heads, head_dim]   written / read
 *   query_start    int32 [num_seqs + 1]: 0 = query_start[0] <= ... <=
 *                  query_start[num_seqs] = num_query_tokens
 *   context_lens   int32 [num_seqs]: tokens cached, chunk included
 *   max_query_len  upper bound of every n_s (sizes the grid)
 * A chunk of one token is a decode step.  Supported: bf16, head_dim 128,
 * block_size 16 or 32 (else PA_ERR_UNSUPPORTED); fp32 accumulation, P
 * rounded to bf16 for the P.V product.  Contract: n_s <= max_query_len,
 * n_s <= context_lens[s] <= max_blocks_per_seq * block_size, table entries of
 * used blocks in [0, num_blocks) -- checked under PA_CHECK=1.  No workspace.
 * num_seqs == 0, max_query_len == 0 or num_query_tokens == 0 is a no-op. */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, int max_blocks_per_seq,
               const int32_t* context_lens, const int32_t* query_start, int num_seqs,
               int max_query_len, int64_t num_query_tokens, int num_q_heads, int num_kv_heads,
               int head_dim, int block_size, int64_t num_blocks, float scale, int dtype,
               void* stream);

/* pa_prefill with each row tile's keys shared out over num_splits workgroups.
 * Splitting serves batches whose row tiles alone leave most compute units
 * idle (few sequences, short chunks, long contexts).  Each split writes an
 * unnormalised partial row: its partial sum of exp-weighted values, the max
 * it was taken relative to, and its weight sum.  A second kernel then folds
 * the partial rows by the standard log-sum-exp rescaling.  Same arguments,
 * layouts and contract as pa_prefill, plus:
 *   num_splits      0 = automatic, with tiles = the batch's row tiles (128
 *                   query rows of one KV head each) and slots = 3 workgroups
 *                   per compute unit:
 *                     - 1 while tiles >= 2 * slots;
 *                     - floor(slots / tiles), at most 32, while 16 * tiles
 *                       <= slots (one full round of workgroups);
 *                     - else the S in 2..Smax with the smallest
 *                       ceil(tiles * S / CUs) / S (an even share per compute
 *                       unit), the largest S among equals; Smax =
 *                       floor(2 * slots / tiles), at least 2, at most 16;
 *                   and never more than one split per 8 key steps of 32
 *                   keys of the longest context the tables hold.
 *                   1 = no split (then exactly pa_prefill); 2..32 = that
 *                   many; beyond 32: PA_ERR_INVALID.  Splits change only the
 *                   fp32 summation order.
 *   workspace       device memory of workspace_bytes, 16-byte aligned, at
 *                   least what pa_prefill_split_plan gives (with S splits:
 *                   S * num_query_tokens * num_q_heads * (head_dim + 4) *
 *                   4 bytes; none for S = 1), else PA_ERR_WORKSPACE.  Its
 *                   contents need no initialisation and are left undefined.
 * Two kernels on `stream`; no host synchronisation, so it can be captured in
 * a HIP graph. */
int pa_prefill_split(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                     int max_query_len, int64_t num_query_tokens, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                     float scale, int dtype, int num_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The split count pa_prefill_split uses for these sizes and num_splits
 * (0 = automatic, which reads the current device's compute-unit count) in
 * *splits, and the workspace it needs in *bytes.  PA_ERR_INVALID for sizes
 * pa_prefill would reject as invalid, or num_splits outside 0..32. */
int pa_prefill_split_plan(int num_seqs, int max_query_len, int64_t num_query_tokens,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int max_blocks_per_seq, int num_splits, int* splits, size_t* bytes);

/* Measurement hook.  `before` and `after` are hipEvent_t handles (created by
 * the caller).  While set, every pa_decode call made from this host thread
 * launches its attention kernel with `before` and `after` as the launch's
 * start and stop events (hipExtLaunchKernel): they take the kernel's own
 * start and end times, without the small kernel that merges split context
 * pieces and without marker packets between the kernels, so the attention
 * kernel alone can be timed at no cost to the step.  Pass NULL, NULL to
 * stop.  Returns PA_ERR_INVALID if exactly one is NULL. */
int pa_set_decode_events(void* before, void* after);

/* Read-bandwidth probe (measurement only; not a step of the paged path).
 * Reads num_tiles tiles of tile_bytes (4096 or 8192) bytes from `base`: tile i
 * is the one at byte offset tile_ids[i] * tile_bytes, or i * tile_bytes when
 * tile_ids is NULL.  The reads use the decode kernels' pattern: one-wave
 * workers, each taking an equal consecutive share of the list, 16-byte loads
 * (1 KiB per wave load) and 16 KiB in flight per worker; nontemporal = 1
 * marks every load non-temporal (as the decode kernels mark V).  Timed around
 * the call, it gives the device's bandwidth for that access pattern -- the
 * ceiling the attention kernels are compared against.
 *   checksum    uint32 [workers]: worker w writes the XOR of every 32-bit word
 *               it read (the XOR over all workers is the XOR of every word of
 *               every listed tile, each counted once per listing)
 *   base        device memory of base_bytes bytes, 16-byte aligned
 *   tile_ids    int32 [num_tiles] or NULL
 *   num_workers 0 = 4 per compute unit of the current device
 * Contract: every tile id in [0, base_bytes / tile_bytes) -- checked under
 * PA_CHECK=1; with tile_ids NULL, num_tiles * tile_bytes <= base_bytes is
 * checked always.  num_tiles == 0 is a no-op. */
int pa_read_probe(uint32_t* checksum, const void* base, int64_t base_bytes,
                  const int32_t* tile_ids, int64_t num_tiles, int tile_bytes, int nontemporal,
                  int num_workers, void* stream);

/* Static description of a status code (never NULL). */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
