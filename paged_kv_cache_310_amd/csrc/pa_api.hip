// Host side of the C ABI declared in include/pa.h: argument checks, optional
// index validation (PA_CHECK=1), workspace sizing and kernel dispatch.
#include <cmath>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

bool check_enabled() {
  static const bool on = [] {
    const char* v = getenv("PA_CHECK");
    return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(int dtype, int num_kv_heads, int block_size, int head_dim, int64_t num_blocks) {
  (void)dtype;
  return num_kv_heads > 0 && block_size > 0 && head_dim > 0 && num_blocks > 0;
}

int support_status(int dtype, int block_size, int head_dim) {
  if (dtype != PA_DTYPE_FP32 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

template <typename I>
bool copy_to_host(std::vector<I>& dst, const I* src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(I), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

// PA_CHECK: every non-negative slot lies in the pool and none repeats.
int validate_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_slots,
                   hipStream_t st) {
  std::vector<int64_t> slots;
  if (!copy_to_host(slots, slot_mapping, (size_t)num_tokens, st)) return PA_ERR_HIP;
  std::vector<char> seen((size_t)num_slots, 0);
  for (int64_t s : slots) {
    if (s < 0) continue;
    if (s >= num_slots || seen[(size_t)s]) return PA_ERR_INDEX;
    seen[(size_t)s] = 1;
  }
  return PA_OK;
}

// PA_CHECK: pairs in range, no destination repeats or is also a source.
int validate_pairs(const int64_t* block_mapping, int64_t num_pairs, int64_t num_blocks,
                   hipStream_t st) {
  std::vector<int64_t> pairs;
  if (!copy_to_host(pairs, block_mapping, (size_t)(2 * num_pairs), st)) return PA_ERR_HIP;
  std::vector<char> role((size_t)num_blocks, 0);   // 1 = src, 2 = dst
  for (int64_t p = 0; p < num_pairs; ++p) {
    const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return PA_ERR_INDEX;
    if (role[(size_t)dst] != 0) return PA_ERR_INDEX;   // dst repeats or is a src
    if (role[(size_t)src] == 2) return PA_ERR_INDEX;   // src is an earlier dst
    role[(size_t)src] = 1;
    role[(size_t)dst] = 2;
  }
  return PA_OK;
}

// PA_CHECK of pa_decode_shared's groups (lengths, tables and slots already
// on the host): group_start runs from 0 to num_seqs without decreasing;
// every prefix length lies in [0, context length] -- below it when the fused
// append writes that sequence, so the new token is never shared -- and is
// the same for every member of a group; and every member's table holds its
// group's first member's blocks for the shared tokens.
template <typename G>
int validate_groups(const G& groups, const std::vector<int32_t>& lens,
                    const std::vector<int32_t>& tables, const std::vector<int64_t>& slots,
                    bool fused, int num_seqs, int max_blocks_per_seq, int block_size,
                    hipStream_t st) {
  std::vector<int32_t> gs, plen;
  if (!copy_to_host(gs, groups.group_start, (size_t)groups.num_groups + 1, st)) return PA_ERR_HIP;
  if (!copy_to_host(plen, groups.prefix_lens, (size_t)num_seqs, st)) return PA_ERR_HIP;
  if (gs[0] != 0 || gs[(size_t)groups.num_groups] != num_seqs) return PA_ERR_INDEX;
  for (int g = 0; g < groups.num_groups; ++g) {
    const int lo = gs[(size_t)g], hi = gs[(size_t)g + 1];
    if (hi < lo) return PA_ERR_INDEX;
    for (int s = lo; s < hi; ++s) {
      const int64_t P = plen[(size_t)s], L = lens[(size_t)s];
      if (P < 0 || P > L || P != plen[(size_t)lo]) return PA_ERR_INDEX;
      if (fused && slots[(size_t)s] >= 0 && P > L - 1) return PA_ERR_INDEX;
      const int64_t nblk = (P + block_size - 1) / block_size;
      for (int64_t j = 0; j < nblk; ++j)
        if (tables[(size_t)s * max_blocks_per_seq + j] !=
            tables[(size_t)lo * max_blocks_per_seq + j])
          return PA_ERR_INDEX;
    }
  }
  return PA_OK;
}

// Every entry of a host array of num_layers device pointers is non-null and
// 16-byte aligned.
template <typename P>
bool layer_pointers_ok(const P* ptrs, int num_layers) {
  if (!ptrs) return false;
  for (int l = 0; l < num_layers; ++l)
    if (!ptrs[l] || !aligned16(ptrs[l])) return false;
  return true;
}

// Compute units of the current device (cached per device).
int current_device_cus(int* out) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return PA_ERR_HIP;
    cache[dev] = cus;
  }
  *out = cache[dev];
  return PA_OK;
}

// Upper bound of the default worker count: CUs x kWavesPerCu.
int default_workers_for_current_device(int* out) {
  int cus = 0;
  const int st = current_device_cus(&cus);
  if (st != PA_OK) return st;
  *out = cus * pa::kWavesPerCu;
  return PA_OK;
}

// Default workers of one kernel variant: every worker resident at once.
// `small` (may be null) receives the count for small batches on the vector
// kernel: the resident count up to kDecodeWavesPerCu per CU.
int default_workers_for_variant(int dtype, int head_dim, int block_size, int group, int* out,
                                int* small = nullptr) {
  int cus = 0;
  const int st = current_device_cus(&cus);
  if (st != PA_OK) return st;
  int resident = 0;
  if (pa::decode_resident_per_cu(dtype, head_dim, block_size, group, &resident) != hipSuccess ||
      resident <= 0)
    return PA_ERR_HIP;
  const int per_cu = resident < pa::kDecodeWavesPerCu ? resident : pa::kDecodeWavesPerCu;
  if (pa::gqa_supported(dtype, head_dim, group) || resident < pa::kDecodeWavesPerCu)
    *out = cus * per_cu;
  else
    *out = cus * pa::kVectorWorkersPerCuX8 / 8;
  if (small != nullptr) *small = cus * per_cu;
  return PA_OK;
}

// Default workers of one call: the variant's count, or fewer for small
// batches: about c sqrt(T) workers (c = 7 on the vector kernel, 10 on the
// matrix-core kernel; the history below) for T = segments x 16-token chunks of the
// table width (a segment is a (sequence, head) pair of the attention
// kernel's line; the table width is the host's only bound on the contexts).
// A segment split over more workers gains kernel time but costs the merge
// more pieces, and the best chunks per worker grow with the batch: swept
// over one to four 64/8-head sequences of 1k-64k tokens, 8/8 heads at 8k and
// 32k and 32/4 heads at 32k (128-768 workers, interleaved), the best count
// was 192 at T = 1,024 chunks, 384 at 2,048 and 4,096, 640 at 8,192 and
// 640-768 beyond; 7 sqrt(T) lands within 0-4% of the best on every one
// (the rule it replaced, 16-64 pieces per segment from the table width, was
// up to 24% slower at 32k on 4 KV heads and 17% on 8 heads of the vector
// kernel).  Shorter batches are flat in the count.  Once the merge ran on
// the XCD whose L2 holds the pieces, the matrix-core kernel's best counts
// rose: 448 against 320 at one 64/8-head sequence of 4k (15.0 -> 14.3 us),
// 768 at 16k; so it takes 10 sqrt(T), at most 160 pieces per segment (32/4
// heads at 32k: 640 beat 768 by 3.5%).  Measured default against default:
// 2k-8k contexts and four sequences at 4k 1.6-5% faster, 1k and 16k-64k,
// 32/4 and 16/2 heads at 32k and the Pareto batch within +-0.8%.
constexpr double kWorkersPerSqrtChunk = 7.0;
constexpr double kWorkersPerSqrtChunkMfma = 10.0;
constexpr int64_t kMaxPiecesPerSegmentMfma = 160;
// The vector kernel's segments are single query heads, so its pieces are a
// head's row, and many heads per sequence give many short segments.  Below
// kVectorSmallBatch chunks of T it takes 3 workers per CU (not 21 per 8 CUs)
// and at least kVectorPiecesPerSegment pieces per segment under the cap.
// Swept on 32- and 40-head sequences of 1k-16k tokens (T = 2,560-40,960):
// 768 workers were the fastest count on each, 2-13% faster than the earlier
// default (352 at 1k, 672 beyond); at T = 82k 672 and 768 tie, and from
// 164k (the OPT-shaped batch) 672 is 1-1.6% faster.
constexpr double kVectorSmallBatch = 65536.0;
constexpr int64_t kVectorPiecesPerSegment = 20;
int default_workers_for_call(int dtype, int head_dim, int block_size, int max_blocks_per_seq,
                             int num_seqs, int num_q_heads, int num_kv_heads, int* out) {
  const int group = num_q_heads / num_kv_heads;
  int workers = 0, small = 0;
  const int st = default_workers_for_variant(dtype, head_dim, block_size, group, &workers, &small);
  if (st != PA_OK) return st;
  const bool mfma = pa::gqa_supported(dtype, head_dim, group);
  const int64_t segments = (int64_t)num_seqs * (mfma ? num_kv_heads : num_q_heads);
  const int64_t chunks = (int64_t)max_blocks_per_seq * block_size / 16;
  const double t = (double)segments * (double)(chunks > 0 ? chunks : 1);
  const double per_sqrt = mfma ? kWorkersPerSqrtChunkMfma : kWorkersPerSqrtChunk;
  int64_t cap = (int64_t)(per_sqrt * std::sqrt(t));
  const int64_t most = kMaxPiecesPerSegmentMfma * segments;
  if (mfma && cap > most) cap = most;
  if (!mfma && t < kVectorSmallBatch) {
    workers = small > workers ? small : workers;
    const int64_t least = kVectorPiecesPerSegment * segments;
    cap = least > cap ? least : cap;
  }
  cap = (cap + pa::kNumXcd - 1) / pa::kNumXcd * pa::kNumXcd;
  if (cap < pa::kNumXcd) cap = pa::kNumXcd;
  *out = cap < workers ? (int)cap : workers;
  return PA_OK;
}

// Default workers of a shared-prefix call: every worker of the shared
// kernel resident at once, but at most P per tail-line (sequence, KV head)
// segment: P = one piece per 8 16-token chunks of the table width, clamped to
// [16, 48] (the rule pa_decode used before its square-root one; the shared
// kernel's batches have many segments, where the cap rarely binds).
constexpr int64_t kChunksPerPiece = 8;
constexpr int64_t kMinPiecesPerSegment = 16;
constexpr int64_t kMaxPiecesPerSegment = 48;
int default_workers_for_shared(int block_size, int max_blocks_per_seq, int num_seqs,
                               int num_kv_heads, int* out) {
  int cus = 0;
  int st = current_device_cus(&cus);
  if (st != PA_OK) return st;
  int resident = 0;
  if (pa::shared_resident_per_cu(block_size, &resident) != hipSuccess || resident <= 0)
    return PA_ERR_HIP;
  const int workers = cus * (resident < pa::kWavesPerCu ? resident : pa::kWavesPerCu);
  const int64_t segments = (int64_t)num_seqs * num_kv_heads;
  const int64_t chunks = (int64_t)max_blocks_per_seq * block_size / 16;
  int64_t pieces = chunks / kChunksPerPiece;
  pieces = pieces < kMinPiecesPerSegment ? kMinPiecesPerSegment : pieces;
  pieces = pieces > kMaxPiecesPerSegment ? kMaxPiecesPerSegment : pieces;
  int64_t cap = pieces * segments;
  cap = (cap + pa::kNumXcd - 1) / pa::kNumXcd * pa::kNumXcd;
  *out = cap < workers ? (int)(cap > 2 ? cap : 2) : workers;
  return PA_OK;
}

// Events pa_set_decode_events installed for this host thread.
thread_local hipEvent_t tl_before = nullptr;
thread_local hipEvent_t tl_after = nullptr;

}  // namespace

extern "C" {

int pa_set_decode_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return PA_ERR_INVALID;
  tl_before = static_cast<hipEvent_t>(before);
  tl_after = static_cast<hipEvent_t>(after);
  return PA_OK;
}

}  // extern "C"

namespace pa {
// Read-bandwidth probe (probe_kernel.hip): tile_bytes 4096 or 8192.
hipError_t launch_read_probe(uint32_t* checksum, const void* base, const int32_t* tile_ids,
                             int64_t num_tiles, int tile_bytes, int nontemporal, int workers,
                             hipStream_t stream);
}  // namespace pa

extern "C" {

int pa_read_probe(uint32_t* checksum, const void* base, int64_t base_bytes,
                  const int32_t* tile_ids, int64_t num_tiles, int tile_bytes, int nontemporal,
                  int num_workers, void* stream) {
  if (num_tiles < 0 || base_bytes < 0 || num_workers < 0 ||
      (tile_bytes != 4096 && tile_bytes != 8192) || (nontemporal != 0 && nontemporal != 1))
    return PA_ERR_INVALID;
  if (num_tiles == 0) return PA_OK;
  if (!checksum || !base || !aligned16(base)) return PA_ERR_INVALID;
  const int64_t tiles_in_base = base_bytes / tile_bytes;
  if (tile_ids == nullptr && num_tiles > tiles_in_base) return PA_ERR_INVALID;
  int workers = num_workers;
  if (workers == 0) {
    const int st = default_workers_for_current_device(&workers);
    if (st != PA_OK) return st;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tile_ids != nullptr && check_enabled()) {
    std::vector<int32_t> ids;
    if (!copy_to_host(ids, tile_ids, (size_t)num_tiles, st)) return PA_ERR_HIP;
    for (int32_t id : ids)
      if (id < 0 || id >= tiles_in_base) return PA_ERR_INDEX;
  }
  return pa::launch_read_probe(checksum, base, tile_ids, num_tiles, tile_bytes, nontemporal,
                               workers, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or dtype";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_INDEX: return "index data breaks the contract (PA_CHECK)";
    default: return "unknown status";
  }
}

int pa_append_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                 const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                 int num_kv_heads, int block_size, int head_dim, int dtype, void* stream) {
  if (num_tokens < 0 || !shape_ok(dtype, num_kv_heads, block_size, head_dim, num_blocks))
    return PA_ERR_INVALID;
  const int sup = support_status(dtype, block_size, head_dim);
  if (sup != PA_OK) return sup;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    const int vs = validate_slots(slot_mapping, num_tokens, num_blocks * block_size, st);
    if (vs != PA_OK) return vs;
  }
  const int row_bytes = head_dim * pa::elem_bytes(dtype);
  return pa::launch_append(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens, num_kv_heads,
                           block_size, row_bytes, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                   int64_t num_blocks, int num_kv_heads, int block_size, int head_dim,
                   int dtype, void* stream) {
  if (num_pairs < 0 || !shape_ok(dtype, num_kv_heads, block_size, head_dim, num_blocks))
    return PA_ERR_INVALID;
  const int sup = support_status(dtype, block_size, head_dim);
  if (sup != PA_OK) return sup;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    const int vp = validate_pairs(block_mapping, num_pairs, num_blocks, st);
    if (vp != PA_OK) return vp;
  }
  const int64_t block_bytes =
      (int64_t)num_kv_heads * block_size * head_dim * pa::elem_bytes(dtype);
  return pa::launch_copy(k_cache, v_cache, block_mapping, num_pairs, block_bytes, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_append_kv_layers(void* const* k_caches, void* const* v_caches,
                        const void* const* k_new, const void* const* v_new, int num_layers,
                        const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                        int num_kv_heads, int block_size, int head_dim, int dtype, void* stream) {
  if (num_tokens < 0 || num_layers < 0 ||
      !shape_ok(dtype, num_kv_heads, block_size, head_dim, num_blocks))
    return PA_ERR_INVALID;
  const int sup = support_status(dtype, block_size, head_dim);
  if (sup != PA_OK) return sup;
  if (num_tokens == 0 || num_layers == 0) return PA_OK;
  if (!slot_mapping || !layer_pointers_ok(k_caches, num_layers) ||
      !layer_pointers_ok(v_caches, num_layers) || !layer_pointers_ok(k_new, num_layers) ||
      !layer_pointers_ok(v_new, num_layers))
    return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    const int vs = validate_slots(slot_mapping, num_tokens, num_blocks * block_size, st);
    if (vs != PA_OK) return vs;
  }
  const int row_bytes = head_dim * pa::elem_bytes(dtype);
  return pa::launch_append_layers(k_caches, v_caches, k_new, v_new, num_layers, slot_mapping,
                                  num_tokens, num_kv_heads, block_size, row_bytes,
                                  st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_copy_blocks_layers(void* const* k_caches, void* const* v_caches, int num_layers,
                          const int64_t* block_mapping, int64_t num_pairs, int64_t num_blocks,
                          int num_kv_heads, int block_size, int head_dim, int dtype,
                          void* stream) {
  if (num_pairs < 0 || num_layers < 0 ||
      !shape_ok(dtype, num_kv_heads, block_size, head_dim, num_blocks))
    return PA_ERR_INVALID;
  const int sup = support_status(dtype, block_size, head_dim);
  if (sup != PA_OK) return sup;
  if (num_pairs == 0 || num_layers == 0) return PA_OK;
  if (!block_mapping || !layer_pointers_ok(k_caches, num_layers) ||
      !layer_pointers_ok(v_caches, num_layers))
    return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    const int vp = validate_pairs(block_mapping, num_pairs, num_blocks, st);
    if (vp != PA_OK) return vp;
  }
  const int64_t block_bytes =
      (int64_t)num_kv_heads * block_size * head_dim * pa::elem_bytes(dtype);
  return pa::launch_copy_layers(k_caches, v_caches, num_layers, block_mapping, num_pairs,
                                block_bytes, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_decode_default_workers(int* num_workers) {
  if (!num_workers) return PA_ERR_INVALID;
  return default_workers_for_current_device(num_workers);
}

int pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int num_workers, size_t* bytes) {
  if (!bytes || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_workers < 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID;
  int workers = num_workers;
  if (workers == 0) {
    const int st = default_workers_for_current_device(&workers);
    if (st != PA_OK) return st;
  }
  *bytes = pa::partials_bytes(workers, num_q_heads / num_kv_heads, head_dim);
  return PA_OK;
}

}  // extern "C"

namespace {

// pa_decode's checks and launch.  `workspace` is the caller's workspace, or
// -- for pa_decode_noalloc -- null, with `scratch` the current device's static
// scratch array: the need is then checked against its size.
// Groups of sequences that share a prefix (pa_decode_shared), or none.
struct SharedGroups {
  const int32_t* group_start;
  int num_groups;
  const int32_t* prefix_lens;
};

int decode_impl(void* out, const void* q, void* k_cache, void* v_cache,
                const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                int head_dim, int block_size, int64_t num_blocks, float scale,
                const void* k_new, const void* v_new, const int64_t* slot_mapping,
                void* workspace, size_t workspace_bytes, bool use_scratch, int num_workers,
                int dtype, void* stream, const SharedGroups* groups = nullptr);

}  // namespace

extern "C" int pa_decode(void* out, const void* q, void* k_cache, void* v_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                         float scale, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, void* workspace, size_t workspace_bytes,
                         int num_workers, int dtype, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     k_new, v_new, slot_mapping, workspace, workspace_bytes, false, num_workers,
                     dtype, stream);
}

// ---------------------------------------------------------------------------
// Decode without any allocation: the workspace is a file-scope device array.
// Each device that runs the library holds its own copy of `scratch` until the
// process ends.  In host code its name is only a host-side stand-in: the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is ever handed to kernels.
static_assert(PA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return PA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int64_t num_blocks, float scale, const void* k_new,
                                 const void* v_new, const int64_t* slot_mapping, int num_workers,
                                 int dtype, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     k_new, v_new, slot_mapping, nullptr, 0, true, num_workers, dtype, stream);
}

namespace {

int decode_impl(void* out, const void* q, void* k_cache, void* v_cache,
                const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                int head_dim, int block_size, int64_t num_blocks, float scale,
                const void* k_new, const void* v_new, const int64_t* slot_mapping,
                void* workspace, size_t workspace_bytes, bool use_scratch, int num_workers,
                int dtype, void* stream, const SharedGroups* groups) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 || num_workers < 0 ||
      !shape_ok(dtype, num_kv_heads, block_size, head_dim, num_blocks) ||
      num_q_heads % num_kv_heads != 0 || !(scale == scale))
    return PA_ERR_INVALID;
  const int sup = support_status(dtype, block_size, head_dim);
  if (sup != PA_OK) return sup;
  const int fused = (k_new != nullptr) + (v_new != nullptr) + (slot_mapping != nullptr);
  if (fused != 0 && fused != 3) return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (fused && (!aligned16(k_new) || !aligned16(v_new))))
    return PA_ERR_INVALID;
  if ((int64_t)num_seqs * num_q_heads > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  if (groups && (groups->num_groups < 0 || groups->num_groups > num_seqs ||
                 (groups->num_groups > 0 && (!groups->group_start || !groups->prefix_lens))))
    return PA_ERR_INVALID;
  // The shared-prefix kernels serve bf16 head_dim 128 with 1..16 query heads
  // per KV head; other shapes (and calls without groups) run plain decode,
  // which computes the same attention.
  const bool use_shared =
      groups && groups->num_groups > 0 && pa::shared_supported(dtype, head_dim, group);

  int workers = num_workers;
  if (workers == 0) {
    const int st = use_shared
                       ? default_workers_for_shared(block_size, max_blocks_per_seq, num_seqs,
                                                    num_kv_heads, &workers)
                       : default_workers_for_call(dtype, head_dim, block_size, max_blocks_per_seq,
                                                  num_seqs, num_q_heads, num_kv_heads, &workers);
    if (st != PA_OK) return st;
  }
  if (use_shared && workers < 2) workers = 2;   // one worker per line at least
  const pa::SharedLayout lay =
      pa::shared_layout(workers, num_seqs, num_q_heads, num_kv_heads, head_dim);
  const size_t need =
      use_shared ? lay.total
                 : pa::partials_bytes(workers, pa::decode_piece_rows(dtype, head_dim, group),
                                      head_dim);
  if (use_scratch) {
    if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
    const int sc = scratch_for_current_device(&workspace);
    if (sc != PA_OK) return sc;
    workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    std::vector<int32_t> lens, tables;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, st)) return PA_ERR_HIP;
    if (!copy_to_host(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq, st))
      return PA_ERR_HIP;
    std::vector<int64_t> slots;
    if (fused && !copy_to_host(slots, slot_mapping, (size_t)num_seqs, st)) return PA_ERR_HIP;
    for (int s = 0; s < num_seqs; ++s) {
      const int64_t L = lens[(size_t)s];
      if (L < 0 || L > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_INDEX;
      const int64_t nblk = (L + block_size - 1) / block_size;
      for (int64_t j = 0; j < nblk; ++j) {
        const int64_t b = tables[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks) return PA_ERR_INDEX;
      }
      if (fused && slots[(size_t)s] >= 0) {
        if (L < 1) return PA_ERR_INDEX;
        const int64_t last = L - 1;
        const int64_t want =
            (int64_t)tables[(size_t)s * max_blocks_per_seq + last / block_size] * block_size +
            last % block_size;
        if (slots[(size_t)s] != want) return PA_ERR_INDEX;
      }
    }
    if (groups && groups->num_groups > 0) {
      const int vg = validate_groups(*groups, lens, tables, slots, fused != 0, num_seqs,
                                     max_blocks_per_seq, block_size, st);
      if (vg != PA_OK) return vg;
    }
  }

  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.records = static_cast<pa::MergeRecord*>(workspace);
  a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + pa::records_bytes(workers));
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (use_shared) {
    char* base = static_cast<char*>(workspace);
    a.partials = reinterpret_cast<float*>(base + lay.partials);
    pa::ShareArgs sh;
    sh.group_start = groups->group_start;
    sh.prefix_lens = groups->prefix_lens;
    sh.loc_pre = reinterpret_cast<int32_t*>(base + lay.loc_pre);
    sh.loc_tail = reinterpret_cast<int32_t*>(base + lay.loc_tail);
    sh.res_pre = reinterpret_cast<float*>(base + lay.res_pre);
    sh.res_tail = reinterpret_cast<float*>(base + lay.res_tail);
    sh.num_groups = groups->num_groups;
    sh.members_per_block = pa::kSharedPieceRows / group;
    return pa::launch_decode_shared(a, sh, block_size, workers, st, tl_before, tl_after) ==
                   hipSuccess
               ? PA_OK
               : PA_ERR_HIP;
  }
  return pa::launch_decode(a, dtype, head_dim, block_size, workers, st, tl_before, tl_after) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

}  // namespace

extern "C" int pa_decode_shared_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                               int head_dim, int num_workers, size_t* bytes) {
  if (!bytes || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_workers < 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID;
  int workers = num_workers;
  if (workers == 0) {
    const int st = default_workers_for_current_device(&workers);
    if (st != PA_OK) return st;
  }
  if (workers < 2) workers = 2;
  const size_t shared =
      pa::shared_layout(workers, num_seqs, num_q_heads, num_kv_heads, head_dim).total;
  const size_t plain = pa::partials_bytes(workers, num_q_heads / num_kv_heads, head_dim);
  *bytes = shared > plain ? shared : plain;
  return PA_OK;
}

extern "C" int pa_decode_shared(void* out, const void* q, void* k_cache, void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size,
                                int64_t num_blocks, float scale, const void* k_new,
                                const void* v_new, const int64_t* slot_mapping,
                                const int32_t* group_start, int num_groups,
                                const int32_t* prefix_lens, void* workspace,
                                size_t workspace_bytes, int num_workers, int dtype,
                                void* stream) {
  const SharedGroups groups{group_start, num_groups, prefix_lens};
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     k_new, v_new, slot_mapping, workspace, workspace_bytes, false, num_workers,
                     dtype, stream, &groups);
}

namespace pa {
// Prefill with the context split over num_splits workgroups per row tile
// (prefill_kernel.hip).  partials may be null when num_splits is 1.
hipError_t launch_prefill_split(const PrefillArgs& a, int block_size, int num_splits,
                                float* partials, int64_t num_query_tokens, hipStream_t stream);
}  // namespace pa

namespace {

constexpr int kPrefillMaxSplits = 32;
constexpr int kPrefillWgsPerCu = 3;        // resident prefill workgroups per CU
constexpr int kPrefillMinStepsPerSplit = 8;
constexpr int kPrefillBalancedMaxSplits = 16;   // cap of the balanced choice
constexpr int kPrefillSplitWgsPerCu = 2;        // target of the many-split choice

// Splits pa_prefill_split picks for num_splits = 0.  None while the row tiles
// alone fill the device's workgroup slots (3 per compute unit) twice.  When
// even 16 splits would not fill one round of slots, as many as make two
// workgroups per compute unit (at most 32): on one 64/8-head sequence's
// 64-token chunk over 32k, 16 splits (512 workgroups) took 89.4 us against
// 92.3 at 24 (a full round), and on 40 heads' 64-token chunk over 32k, 12
// (480) took 134.7 us against 161.8-186.2 at 20-32.  Otherwise S in
// [2, Smax], Smax = floor(2 slots / tiles) (at least 2, at most 16), with the
// smallest per-CU share ceil(tiles S / CUs) / S
// of one tile's work -- splits that leave some CUs a workgroup more than
// others lose -- and among equal shares the most splits (more resident
// workgroups).  Either way at most one split per 8 key steps of the longest
// context the tables allow.
int prefill_auto_splits(int num_seqs, int max_query_len, int group, int num_kv_heads,
                        int max_blocks_per_seq, int block_size, int* splits) {
  int cus = 0;
  const int st = current_device_cus(&cus);
  if (st != PA_OK) return st;
  const int64_t tiles =
      ((int64_t)max_query_len * group + pa::kPrefillRowsPerWg - 1) / pa::kPrefillRowsPerWg;
  const int64_t wgs = tiles * num_seqs * num_kv_heads;
  const int64_t slots = (int64_t)cus * kPrefillWgsPerCu;
  const int64_t max_steps = ((int64_t)max_blocks_per_seq * block_size + 31) / 32;
  const int64_t by_steps = max_steps / kPrefillMinStepsPerSplit;
  int64_t best = 1;
  if (wgs > 0 && wgs * kPrefillBalancedMaxSplits <= slots) {
    best = (int64_t)cus * kPrefillSplitWgsPerCu / wgs;
    best = best < kPrefillMaxSplits ? best : kPrefillMaxSplits;
  } else if (wgs > 0 && wgs < 2 * slots) {
    int64_t smax = 2 * slots / wgs;
    smax = smax > 2 ? smax : 2;
    smax = smax < kPrefillBalancedMaxSplits ? smax : kPrefillBalancedMaxSplits;
    smax = smax < by_steps ? smax : by_steps;
    int64_t best_load = 0;
    for (int64_t n = 2; n <= smax; ++n) {
      const int64_t load = (wgs * n + cus - 1) / cus;   // workgroups on the busiest CU
      // load / n <= best_load / best, exactly
      if (best == 1 || load * best <= best_load * n) {
        best = n;
        best_load = load;
      }
    }
  }
  best = best < by_steps ? best : by_steps;
  *splits = (int)(best > 1 ? best : 1);
  return PA_OK;
}

size_t prefill_partials_bytes(int splits, int64_t num_query_tokens, int num_q_heads,
                              int head_dim) {
  return splits > 1 ? (size_t)splits * num_query_tokens * num_q_heads * (head_dim + 4) * 4 : 0;
}

int prefill_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int max_blocks_per_seq,
                 const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                 int max_query_len, int64_t num_query_tokens, int num_q_heads, int num_kv_heads,
                 int head_dim, int block_size, int64_t num_blocks, float scale, int dtype,
                 int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_query_len < 0 || num_query_tokens < 0 ||
      num_splits < 0 || num_splits > kPrefillMaxSplits ||
      num_q_heads <= 0 || !shape_ok(dtype, num_kv_heads, block_size, head_dim, num_blocks) ||
      num_q_heads % num_kv_heads != 0 || !(scale == scale))
    return PA_ERR_INVALID;
  const int sup = support_status(dtype, block_size, head_dim);
  if (sup != PA_OK) return sup;
  if (!pa::prefill_supported(dtype, head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0 || num_query_tokens == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID;
  const int group = num_q_heads / num_kv_heads;
  const int64_t tiles =
      ((int64_t)max_query_len * group + pa::kPrefillRowsPerWg - 1) / pa::kPrefillRowsPerWg;
  const int64_t pair_rounds = ((int64_t)num_seqs * num_kv_heads + pa::kNumXcd - 1) / pa::kNumXcd;
  if (tiles * pa::kNumXcd * pair_rounds > INT32_MAX || num_query_tokens * num_q_heads > INT32_MAX)
    return PA_ERR_UNSUPPORTED;

  if (num_splits == 0) {
    const int sp = prefill_auto_splits(num_seqs, max_query_len, group, num_kv_heads,
                                       max_blocks_per_seq, block_size, &num_splits);
    if (sp != PA_OK) return sp;
  }
  if (tiles * pa::kNumXcd * pair_rounds * num_splits > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (num_splits > 1) {
    const size_t need = prefill_partials_bytes(num_splits, num_query_tokens, num_q_heads,
                                               head_dim);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_ERR_WORKSPACE;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    std::vector<int32_t> lens, starts, tables;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, st)) return PA_ERR_HIP;
    if (!copy_to_host(starts, query_start, (size_t)num_seqs + 1, st)) return PA_ERR_HIP;
    if (!copy_to_host(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq, st))
      return PA_ERR_HIP;
    if (starts[0] != 0 || starts[(size_t)num_seqs] != num_query_tokens) return PA_ERR_INDEX;
    for (int s = 0; s < num_seqs; ++s) {
      const int64_t L = lens[(size_t)s];
      const int64_t nq = (int64_t)starts[(size_t)s + 1] - starts[(size_t)s];
      if (nq < 0 || nq > max_query_len || nq > L) return PA_ERR_INDEX;
      if (L > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_INDEX;
      const int64_t nblk = (L + block_size - 1) / block_size;
      for (int64_t j = 0; j < nblk; ++j) {
        const int64_t b = tables[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks) return PA_ERR_INDEX;
      }
    }
  }

  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.tiles_per_seq = (int)tiles;
  a.scale_log2 = scale * 1.4426950408889634f;
  return pa::launch_prefill_split(a, block_size, num_splits, static_cast<float*>(workspace),
                                  num_query_tokens, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}


}  // namespace

extern "C" {

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, int max_blocks_per_seq,
               const int32_t* context_lens, const int32_t* query_start, int num_seqs,
               int max_query_len, int64_t num_query_tokens, int num_q_heads, int num_kv_heads,
               int head_dim, int block_size, int64_t num_blocks, float scale, int dtype,
               void* stream) {
  return prefill_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                      query_start, num_seqs, max_query_len, num_query_tokens, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, 1, nullptr, 0,
                      stream);
}

int pa_prefill_split_plan(int num_seqs, int max_query_len, int64_t num_query_tokens,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int max_blocks_per_seq, int num_splits, int* splits, size_t* bytes) {
  if (!splits || !bytes || num_seqs < 0 || max_query_len < 0 || num_query_tokens < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0 || num_splits < 0 ||
      num_splits > kPrefillMaxSplits)
    return PA_ERR_INVALID;
  int n = num_splits;
  if (n == 0) {
    const int st = prefill_auto_splits(num_seqs, max_query_len, num_q_heads / num_kv_heads,
                                       num_kv_heads, max_blocks_per_seq, block_size, &n);
    if (st != PA_OK) return st;
  }
  *splits = n;
  *bytes = prefill_partials_bytes(n, num_query_tokens, num_q_heads, head_dim);
  return PA_OK;
}

int pa_prefill_split(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                     int max_query_len, int64_t num_query_tokens, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                     float scale, int dtype, int num_splits, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return prefill_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                      query_start, num_seqs, max_query_len, num_query_tokens, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, num_splits,
                      workspace, workspace_bytes, stream);
}

}  // extern "C"
