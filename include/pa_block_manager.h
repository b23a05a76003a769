/* Host-side KV block manager of the paged KV cache (libpabm.so, C ABI).
 *
 * It decides where every cached token lives: which physical blocks each
 * sequence owns (its block table), which slot the next token of a sequence
 * goes to (the slot mapping pa_append_kv / pa_decode consume) and which
 * blocks must be duplicated before a write (the copy pairs pa_copy_blocks
 * consumes).  It runs on the CPU and never touches device memory.
 *
 * What it implements (pages on "Efficient Memory Management for Large
 * Language Model Serving with PagedAttention"):
 *  - zeroshotmind.com essay, "Paging the cache": fixed-size blocks allocated
 *    one at a time as a sequence grows, so a sequence holds exactly
 *    ceil(length / block_size) blocks and at most one partly filled block;
 *  - same essay, "Block tables: logical order, physical scatter": one table
 *    per sequence, logical block index -> physical block;
 *  - same essay, "Sharing a prefix without copying it": shared blocks are
 *    reference counted; a write into a shared block duplicates that one block,
 *    repoints the writer at the copy and decrements the original's count;
 *  - phantomic12.github.io catalogue note, method paragraph: prefix blocks are
 *    reused by identity.  The pages name a block hash but define none; this
 *    library keys a full block by the chained 64-bit FNV-1a hash of (the key
 *    of the block before it, the block's token ids), and confirms every hit by
 *    comparing the block's token ids, so a hash collision never shares a
 *    block;
 *  - zeroshotmind.com essay, "The fragmentation arithmetic": tail slack per
 *    sequence is at most block_size - 1 tokens (pa_bm_stats).
 *
 * Conventions: every function returns a pa_bm_status (0 = OK) and never
 * aborts or prints.  Sequence ids are caller-chosen non-negative int64.  A
 * failing call changes nothing (all-or-nothing).  A manager is not thread
 * safe: one thread at a time per handle.  Memory: O(num_blocks) plus, with
 * the prefix cache, num_blocks * block_size token ids. */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_BM_OK = 0,
  PA_BM_INVALID = 1,      /* bad argument (null pointer, negative size, id out of range) */
  PA_BM_EXHAUSTED = 2,    /* not enough free blocks; nothing was changed */
  PA_BM_UNKNOWN_SEQ = 3,  /* sequence id not registered */
  PA_BM_EXISTS = 4,       /* sequence id already registered */
  PA_BM_NOMEM = 5,        /* host allocation failed */
  PA_BM_CORRUPT = 6       /* pa_bm_check found a broken invariant */
} pa_bm_status;

typedef struct pa_bm pa_bm;   /* opaque; owned by the caller between create and destroy */

typedef struct {
  int64_t num_blocks;
  int64_t block_size;
  int64_t free_blocks;         /* blocks no sequence references (the free list) */
  int64_t cached_free_blocks;  /* free blocks still holding a reusable prefix block */
  int64_t used_blocks;         /* blocks referenced by at least one sequence */
  int64_t shared_blocks;       /* blocks referenced by two or more sequences */
  int64_t sequences;
  int64_t tokens;              /* sum of sequence lengths */
  int64_t table_slots;         /* sum over sequences of (blocks held) * block_size */
  int64_t tail_slack;          /* sum over sequences of unused slots in the last block */
  int64_t cached_blocks;       /* blocks registered in the prefix cache */
  int64_t prefix_hit_blocks;   /* blocks reused from the prefix cache since creation */
  int64_t copies;              /* copy-on-write pairs issued since creation */
} pa_bm_stats;

/* Creates a manager over physical blocks [0, num_blocks) of block_size slots.
 * free_order: NULL, or a permutation of [0, num_blocks) giving the order in
 * which blocks are first handed out (first in, first out; released blocks go
 * to the back).  prefix_cache: nonzero enables reuse of full blocks by their
 * token ids.  Writes the handle to *out. */
int pa_bm_create(int64_t num_blocks, int block_size, const int64_t* free_order, int prefix_cache,
                 pa_bm** out);

/* Frees the handle and everything it owns (NULL is a no-op). */
void pa_bm_destroy(pa_bm* bm);

/* Registers sequence `seq` holding `length` tokens.  tokens: NULL, or its
 * `length` token ids; with the prefix cache enabled, the longest run of
 * leading full blocks already cached with the same token ids is shared
 * instead of allocated, and the sequence's new full blocks are cached.
 * *reused_tokens (may be NULL) receives the number of tokens shared. */
int pa_bm_add_sequence(pa_bm* bm, int64_t seq, const int32_t* tokens, int64_t length,
                       int64_t* reused_tokens);

/* One decode step: reserves the slot of the next token of each of the n
 * distinct sequences seqs[0..n).  tokens: NULL or the n new token ids (needed
 * to cache the blocks they complete).  Writes slots[i] = block * block_size +
 * offset and appends (src, dst) copy pairs to copies (room for n pairs) for
 * every shared, partly filled tail block that had to be duplicated first;
 * *num_copies receives their count.  A fresh block is taken only when the tail
 * block is full. */
int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int64_t n,
                       int64_t* slots, int64_t* copies, int64_t* num_copies);

/* Registers `child` sharing every block of `parent` (reference counted). */
int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Releases the sequence's blocks; blocks whose count reaches zero go to the
 * back of the free list (a cached prefix block stays reusable until a later
 * allocation takes it). */
int pa_bm_free_sequence(pa_bm* bm, int64_t seq);

/* Batched pa_bm_fork: registers children[i] sharing every block of
 * parents[i], for i in [0, n) in order, so a child made by an earlier pair may
 * be the parent of a later one.  Checked before anything changes: every
 * parent known (or made earlier in the batch), every child new and listed
 * once; a failure changes nothing. */
int pa_bm_fork_many(pa_bm* bm, const int64_t* parents, const int64_t* children, int64_t n);

/* Batched pa_bm_free_sequence over n distinct registered sequences (a
 * sequence listed twice is PA_BM_INVALID); a failure changes nothing. */
int pa_bm_free_many(pa_bm* bm, const int64_t* seqs, int64_t n);

/* Length of a registered sequence. */
int pa_bm_length(const pa_bm* bm, int64_t seq, int64_t* length);

/* Writes the block tables (row i = seqs[i], int32 [n][max_blocks], padded
 * with `pad`) and, if context_lens is not NULL, the lengths (int32 [n]). */
int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int64_t n, int64_t max_blocks,
                       int32_t pad, int32_t* tables, int32_t* context_lens);

/* The leading tokens each sequence shares physically with the rest of its
 * group -- what pa_decode_shared (pa.h) takes as prefix_lens.  The n
 * sequences seqs[0..n) form num_groups groups of consecutive entries,
 * group g = seqs[group_start[g] .. group_start[g+1]) (group_start[0] = 0,
 * non-decreasing, group_start[num_groups] = n).  For a group of two or more,
 * every member gets (the number of leading block-table entries that are the
 * same physical block in every member) * block_size, at most the shortest
 * member's length; a group of one gets 0.  Call it after the step's
 * pa_bm_append_slots: every sequence's newest token then sits in a block of
 * its own (a shared partly filled tail block is copied before the write), so
 * it is never counted as shared.  Writes prefix_lens[0..n). */
int pa_bm_shared_prefix(const pa_bm* bm, const int64_t* seqs, int64_t n,
                        const int64_t* group_start, int64_t num_groups, int32_t* prefix_lens);

/* Reference count of one block. */
int pa_bm_refcount(const pa_bm* bm, int64_t block, int64_t* refcount);

/* Pool and fragmentation counters (see pa_bm_stats). */
int pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out);

/* Checks every invariant: reference counts equal table references, the free
 * list holds exactly the unreferenced blocks once each, every sequence holds
 * ceil(length / block_size) blocks, cache entries point at blocks carrying
 * their key.  PA_BM_OK or PA_BM_CORRUPT. */
int pa_bm_check(const pa_bm* bm);

/* The 64-bit FNV-1a hash of `bytes` bytes, continuing from `seed`
 * (14695981039346656037 starts a fresh hash) -- exported so callers can
 * reproduce block keys. */
uint64_t pa_bm_fnv1a64(uint64_t seed, const void* data, int64_t bytes);

/* Static description of a status code. */
const char* pa_bm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
