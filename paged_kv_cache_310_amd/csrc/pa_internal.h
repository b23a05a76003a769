// Internal declarations shared by the HIP translation units of libpa.so.
// Not part of the public ABI (that is include/pa.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// CDNA4 (gfx950) dispatches consecutive workgroup ids round-robin over its
// 8 accelerator dies (XCDs), each with a private L2.
constexpr int kNumXcd = 8;
// Tokens handled per decode inner-loop step ("chunk"); block sizes are
// multiples of it.
constexpr int kChunk = 16;

enum DType : int { kFp32 = 0, kBf16 = 1 };

inline int elem_bytes(int dtype) { return dtype == kBf16 ? 2 : 4; }

// What the merge kernel needs about the split segment a worker closes (the
// segment holding the worker's first chunk, begun by an earlier worker and
// ending inside this worker's range).  valid == 0: the worker closes none.
struct MergeRecord {
  int64_t W;          // chunks in the line
  int64_t NW;         // workers with chunks
  int64_t seg_start;  // first chunk of the segment
  int64_t first;      // worker holding that chunk
  int32_t seq, head;
  int32_t valid;
  int32_t first_slot; // partial slot (0 or 1) the segment's piece has in worker `first`
};

static_assert(sizeof(MergeRecord) == 48, "merge record layout");

// Work units a segment costs in the split besides its chunks (one unit per
// chunk), per attention kernel: about the measured per-segment time over the
// per-chunk time, then tuned by timing.  On the matrix cores 3 beat 2 by
// 1.5-1.8% (Pareto batches, interleaved in one process) and 0.5-1.9% (bench
// runs); 1 and 4 were slower than 3.  The vector kernel's 1 and 3 tied 2.
constexpr int kSegCostValu = 2;
constexpr int kSegCostMfma = 3;
// The shared-prefix kernel's lines (3 was within 1% of 2 there).
constexpr int kSegCostShared = 2;

// Everything the decode kernels read, in one POD passed by value.
struct DecodeArgs {
  void* out;
  const void* q;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* k_new;          // fused append, or nullptr
  const void* v_new;
  const int64_t* slot_mapping;
  MergeRecord* records;       // [workers]
  float* partials;            // [workers][2][piece_rows][head_dim + 4]: acc, max, sum, pad
  int64_t max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // num_q_heads / num_kv_heads
  int heads_per_seg;          // query heads one work segment covers (1, or group on MFMA)
  int piece_rows;             // rows (query heads) per partial piece slot: heads_per_seg
  int seg_cost;               // work units a segment costs besides its chunks
  float scale_log2;           // scale * log2(e): scores live in the exp2 domain
};

// Workspace: one MergeRecord per worker, then the partial pieces: two slots
// per worker (the segment it continues, the segment it begins) and query head
// of a segment, each a record of head_dim + 4 floats: the unnormalised
// accumulator, the running max, the sum and two floats of padding (records
// stay 16-byte aligned).  Everything is written before it is read in the same
// call, so the workspace needs no initialisation.
constexpr int kPartialExtra = 4;
__host__ __device__ inline int partial_floats(int head_dim) { return head_dim + kPartialExtra; }
inline size_t records_bytes(int workers) {
  return ((size_t)workers * sizeof(MergeRecord) + 255) & ~(size_t)255;
}
inline size_t partials_bytes(int workers, int rows, int head_dim) {
  return records_bytes(workers) +
         (size_t)workers * 2 * (size_t)rows * (size_t)partial_floats(head_dim) * sizeof(float);
}

// Decode with groups of sequences sharing a prefix (pa_decode_shared): what
// the kernels read and write besides DecodeArgs.  A sequence's attention is
// then the fold of two parts, each one result row (acc, max, sum) or a run of
// split pieces: its shared prefix, computed once for the whole group by the
// prefix line, and its own tail, computed by the tail line.  For every such
// sequence and KV head a locator entry says where each part's pieces are:
// (first worker, piece count, partial slot of the first piece, first row),
// piece count 0 meaning "whole: the row in res_pre / res_tail".
struct ShareArgs {
  const int32_t* group_start;   // [num_groups + 1]: group g = sequences [gs[g], gs[g+1])
  const int32_t* prefix_lens;   // [num_seqs]: leading tokens the sequence shares
  int32_t* loc_pre;             // [num_kv_heads][num_seqs][4] locators of the prefix part
  int32_t* loc_tail;            // [num_kv_heads][num_seqs][4] locators of the tail part
  float* res_pre;               // [num_kv_heads][num_seqs][group][head_dim + 4]
  float* res_tail;              // [num_kv_heads][num_seqs][group][head_dim + 4]
  int num_groups;
  int members_per_block;        // whole members per 16-row MFMA tile: 16 / group
};

// Rows of a partial piece slot in a shared-prefix decode: one 16-row MFMA
// tile (the prefix line's members x query heads; the tail line uses `group`).
constexpr int kSharedPieceRows = 16;

// Workspace of pa_decode_shared: records, partial pieces (16 rows per slot),
// the two locator arrays and the two result arrays, each 256-byte aligned.
struct SharedLayout {
  size_t records, partials, loc_pre, loc_tail, res_pre, res_tail, total;
};
inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
inline SharedLayout shared_layout(int workers, int num_seqs, int num_q_heads, int num_kv_heads,
                                  int head_dim) {
  SharedLayout L;
  const size_t rec = (size_t)partial_floats(head_dim) * sizeof(float);
  L.records = 0;
  L.partials = records_bytes(workers);
  L.loc_pre = L.partials + round256((size_t)workers * 2 * kSharedPieceRows * rec);
  L.loc_tail = L.loc_pre + round256((size_t)num_kv_heads * num_seqs * 16);
  L.res_pre = L.loc_tail + round256((size_t)num_kv_heads * num_seqs * 16);
  L.res_tail = L.res_pre + round256((size_t)num_seqs * num_q_heads * rec);
  L.total = L.res_tail + round256((size_t)num_seqs * num_q_heads * rec);
  return L;
}

// The shared-prefix decode kernels run for bf16, head_dim 128 and 1..16 query
// heads per KV head (the matrix-core body).
bool shared_supported(int dtype, int head_dim, int group);
// Launches the shared-prefix attention kernel (with `before`/`after`, when not
// null, as its start and stop events) and its merge.  a.records/a.partials
// and the ShareArgs arrays point into one SharedLayout workspace.
hipError_t launch_decode_shared(const DecodeArgs& a, const ShareArgs& sh, int block_size,
                                int workers, hipStream_t stream, hipEvent_t before,
                                hipEvent_t after);
// Resident shared-prefix decode workers (one-wave workgroups) per CU.
hipError_t shared_resident_per_cu(int block_size, int* resident);

// Launches the attention kernel (with `before`/`after`, when not null, as its
// start and stop events) and then the merge kernel.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int workers, hipStream_t stream, hipEvent_t before, hipEvent_t after);
// Resident decode workers (one-wave workgroups) per CU for a variant.
hipError_t decode_resident_per_cu(int dtype, int head_dim, int block_size, int group,
                                  int* resident);
// Grouped-query attention on MFMA (gqa_kernel.hip): bf16, head_dim 128,
// 2 <= group <= 16.  Launches the attention kernel only, or reports its
// occupancy when resident != nullptr.
bool gqa_supported(int dtype, int head_dim, int group);
// Rows of one partial piece of pa_decode: the query heads of a segment (the
// group on the matrix-core kernel, one head on the vector kernel).
inline int decode_piece_rows(int dtype, int head_dim, int group) {
  return gqa_supported(dtype, head_dim, group) ? group : 1;
}
hipError_t launch_gqa_attention(const DecodeArgs& a, int block_size, int workers,
                                hipStream_t stream, int* resident, hipEvent_t start = nullptr,
                                hipEvent_t stop = nullptr);
// Multi-token (prefill) attention: what the kernel reads, by value.
struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;   // [num_seqs + 1]
  int64_t max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                    // num_q_heads / num_kv_heads
  int tiles_per_seq;            // row tiles per (sequence, KV head)
  float scale_log2;             // scale * log2(e)
};
// Query rows (query token x query head of one KV head) per prefill workgroup.
constexpr int kPrefillRowsPerWg = 128;
// bf16, head_dim 128, block_size 16 or 32.
bool prefill_supported(int dtype, int head_dim, int block_size);
hipError_t launch_prefill(const PrefillArgs& a, int block_size, hipStream_t stream);

// Layers served by one multi-layer append or copy launch (their pool
// pointers travel in the kernel arguments).
constexpr int kMaxLayersPerLaunch = 32;

hipError_t launch_append_layers(void* const* k_caches, void* const* v_caches,
                                const void* const* k_new, const void* const* v_new, int num_layers,
                                const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                                int block_size, int row_bytes, hipStream_t stream);
hipError_t launch_copy_layers(void* const* k_caches, void* const* v_caches, int num_layers,
                              const int64_t* block_mapping, int64_t num_pairs, int64_t block_bytes,
                              hipStream_t stream);

hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int block_size, int row_bytes, hipStream_t stream);
hipError_t launch_copy(void* k_cache, void* v_cache, const int64_t* block_mapping,
                       int64_t num_pairs, int64_t block_bytes, hipStream_t stream);

// Workers per CU of the shared-prefix decode, and the upper bound of every
// default worker count (what pa_decode_default_workers reports for sizing a
// workspace).  The shared-prefix kernel loses 8% at 3 per CU: its prefix row
// blocks and the tails of the same sequences meet in an XCD's L2 only while
// enough workers run at once.
constexpr int kWavesPerCu = 4;
// Workers per CU of pa_decode on the matrix cores (grouped queries).
// Measured interleaved against 4: 0.4-0.9% faster on the grouped-query
// Pareto batches and 3% on mid-size batches (fewer split segments to merge,
// fewer concurrent tile streams); 704-736 or 800-896 workers (uneven per CU)
// were 1.5-7% slower than 768.  Plain decode of a batch whose sequences
// share prefix blocks was 9.5% slower at 3 than at 4 (sharers re-read the
// prefix through L2 only while enough workers run at once); such batches are
// what pa_decode_shared is for.
constexpr int kDecodeWavesPerCu = 3;
// Workers per CU of the vector decode kernel, in eighths: 21 / 8 (672 on 256
// CUs).  Swept interleaved in one process from 576 to 768 workers: 672-704
// were best on the long-context batch (1.6% faster than 768) and on the
// OPT-shaped one (1.5%), 576 8% slower.  Bench runs (one process per count,
// after the settle phase) agree: long-context 6,731-6,739 GB/s at 672,
// 6,716-6,721 at 704, 6,605-6,616 at 768; OPT-shaped 6,571-6,579 at 672-704
// against 6,484-6,493 at 768; plain decode of the steady shared-prefix batch
// 6,838-6,848 at 704, 6,745-6,757 at 672, 6,689-6,700 at 768.
constexpr int kVectorWorkersPerCuX8 = 21;

}  // namespace pa
