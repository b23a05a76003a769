// Multi-token (prompt / chunked-prompt) paged attention on the gfx950 matrix
// cores: bf16, head_dim 128, block size 16 or 32.
//
// What is computed (pages on "Efficient Memory Management for Large Language
// Model Serving with PagedAttention": catalogue note, method paragraph --
// attention reads keys and values through the block table; zeroshotmind.com
// essay, "Block tables: logical order, physical scatter"): the query chunk of
// a sequence is its newest tokens, already appended to the pool; query token
// i of an n-token chunk sits at position L - n + i of the L cached tokens and
// attends to positions 0..L - n + i, gathered through the sequence's table.
//
// Work: one workgroup (kWaves waves) per kWaves * 32 query rows of one
// (sequence, KV head) pair, the pairs dealt to the XCDs so that a pair's
// workgroups share its K/V in one L2.  A row is a (query token, query head)
// pair of the KV head's group, token-major, so grouped query heads share
// every K/V tile.  Each wave owns 32 consecutive rows as two 16-row MFMA
// tiles.  The workgroup walks the keys in steps of 32 (two 16-token halves).  A step's K and V rows go from the pool
// straight into one of two LDS buffers (buffer loads with an LDS destination,
// no trip through registers), issued one step ahead, so they arrive while the
// step before is computed; one barrier per step publishes them.  The
// sequence's block-table entries are staged in LDS (kTableCap at a time), so
// no step waits on a table read before it can address its K/V rows.
//
// Per step and 16-row tile (lane l, lane group g = l/16, column n = l%16):
//  * S^T[16 keys x 16 rows] = K . Q^T for each 16-key half, four
//    v_mfma_f32_16x16x32_bf16 over the 128 dims.  K (A operand) is read from
//    LDS, Q^T (B operand) stays in registers for the whole key walk.  Lane l
//    receives the scores of keys 4g+i (i = 0..3) of the half for row n.
//  * Causal mask (key position > row position -> -inf), online softmax in
//    the exp2 domain (the scale is applied in the exponent's fma); the mask
//    is evaluated only on steps that reach past the wave's lowest row
//    position.  The row's tile max is agreed on by the four lanes holding
//    column n (two permlane swaps).  The reference max a row's
//    weights are taken against moves only when the tile max exceeds it by
//    more than kRescaleSlack (so weights stay below 2^kRescaleSlack), and
//    the accumulators are rescaled only in a step where some row's moved:
//    after the first steps that is rare, and the result (acc / sum) does not
//    depend on the reference.  P is rounded to bf16 for the product, and the
//    running sum adds the same rounded values (v_dot2_f32_bf16 with (1, 1)).
//  * O^T[128 dims x 16 rows] += V^T . P^T, eight v_mfma_f32_16x16x32_bf16
//    (one per c = 0..7) per row tile, issued after both tiles' softmax so
//    that one V^T operand read serves both tiles.  The 32 keys of the
//    k-dimension are ordered so that lane l's eight P values are exactly its
//    B operand: k = 8g+i is key 4g+i and k = 8g+4+i is key 16+4g+i.  The A operand of MFMA c (dims
//    16c..16c+15) comes from two transposing LDS reads (ds_read_b64_tr_b16)
//    of the V tile (its LDS layout is below), so lane l ends up holding dims
//    16c + 4g + i of row n.
#include "decode_common.h"

namespace pa {
namespace {

using namespace dev;

constexpr int kPD = 128;                      // head_dim
constexpr int kPRow = kPD * 2;                // bytes of one token row
constexpr int kKeys = 32;                     // keys per step
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowTiles = 2;                  // 16-row MFMA tiles per wave
constexpr int kRowsPerWave = 16 * kRowTiles;
static_assert(kWaves * kRowsPerWave == kPrefillRowsPerWg, "rows per workgroup");
// A step's K and V tiles in LDS, 32 keys x 256 bytes each, unpadded: the
// loads that fill them write 1 KiB runs (lane i of a load writes bytes
// 16 i..16 i + 15 of its run), so the layout is chosen by which pool chunk
// each lane fetches.  With r a key of the step and ch a 16-byte chunk of its
// row (dims 8 ch..8 ch + 7):
//  * K chunk (r, ch) sits at (r / 16) 4096 + 256 ch + 16 (r % 16): a 256-byte
//    line per chunk index and 16-key half, one slot per key;
//  * V chunk (r, ch) sits at (r / 16) 4096 + 256 (2 (ch / 2) + (r % 16) / 8)
//    + 16 (2 (r % 8) + ch % 2): a line per chunk pair and 8 keys.
// The A-operand reads of K (16 keys, one chunk index per 16 lanes) and the
// transposing reads of V (16 keys x two chunks per 32 lanes) then touch each
// of the 64 banks at most once per cycle, and every read address is a
// per-lane constant plus an immediate.
constexpr int kKBytes = kKeys * kPRow;
constexpr int kVBytes = kKeys * kPRow;
constexpr int kBufBytes = kKBytes + kVBytes;
constexpr int kHalfBytes = kBufBytes / 4;   // one 16-key half of the K (or V) tile
// Block-table entries held in LDS at a time (refilled every
// kTableCap * BS / kKeys steps).
constexpr int kTableCap = 1024;
// log2 of the largest weight the lazy rescale lets through.
constexpr float kRescaleSlack = 8.f;
// Dim tiles whose V^T operand is read ahead of its P.V products: the first
// ones' LDS reads are issued before the softmax, and each product's operand
// that many tiles before it is used.  One tile ahead is 4-5% faster than
// none; two (166 registers, no spills) measured from 2.5% faster to 1.5%
// slower on different boxes; four spill at three workgroups per CU.
constexpr int kVAhead = 1;

typedef uint32_t __attribute__((address_space(3))) lds_u32;

__device__ __forceinline__ u32x4 lds_load16(const char* base, int offset) {
  return *reinterpret_cast<const u32x4*>(base + offset);
}
typedef __attribute__((address_space(3))) void lds_void;
// One 16-byte pool chunk per lane into LDS: lane i's chunk (at `offset` +
// `soffset` in the range of r, or 0 outside it) lands at dst + 16 i.  dst is
// wave-uniform.
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, char* dst, int offset,
                                            int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, offset, soffset, 0, 0);
}

typedef short i16x4_t_lds __attribute__((ext_vector_type(4)));
typedef i16x4_t_lds __attribute__((address_space(3))) lds_i16x4;
// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element j % 4
// of the 8-byte fragments that lanes 4e + j / 4 (e = 0..3) address, as its
// element e.
__device__ __forceinline__ uint64_t lds_read_tr16(const char* base, int offset) {
  const i16x4_t_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(const_cast<char*>(base) + offset));
  return __builtin_bit_cast(uint64_t, v);
}

// Maximum of scores straight from the matrix cores.  The scores are finite
// or -inf (masked keys), so the NaN-propagating maximum gives fmaxf's value,
// and it maps to v_maximum3_f32 without the quieting copies fmaxf needs on
// values the compiler cannot prove canonical.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// Maximum over the four lanes that share l%16 (two permlane swaps).
__device__ __forceinline__ float group4_smax(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = smax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return smax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
// (1, 1) in bf16, for pair sums with v_dot2_f32_bf16.
__device__ constexpr bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};
// Two floats to two bf16 (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Context split: the key steps of every row tile are shared out over
// num_splits workgroups, which write unnormalized partial rows (acc[D],
// reference max, sum) to `partials` for prefill_merge_kernel.  num_splits 1:
// each workgroup walks all its keys and writes `out` directly.
struct SplitArgs {
  int num_splits;
  float* partials;              // [num_splits][num_query_tokens][num_q_heads][kPartRow]
  int64_t num_query_tokens;
};
constexpr int kPartRow = kPD + 4;   // acc[128], max, sum, 2 floats of padding

// kSplit: the workgroup takes one split of its row tile's key steps and
// writes partial rows (compiled apart, so the unsplit kernel keeps its
// registers).
template <int BS, bool kSplit>
// Three workgroups (12 waves) per CU: the register budget this sets (168)
// costs a few spilled registers and measured faster than two workgroups.
__global__ __launch_bounds__(kThreads, 3) void prefill_kernel(const PrefillArgs a,
                                                               const SplitArgs sp) {
  // Two step buffers as two LDS objects, each accessed by name in the
  // (two-fold unrolled) step loop: the compiler can then tell a buffer's
  // reads from the other buffer's in-flight loads, and does not wait for
  // those loads before reading.
  __shared__ __attribute__((aligned(16))) char lds0[kBufBytes];
  __shared__ __attribute__((aligned(16))) char lds1[kBufBytes];
  __shared__ int32_t tab[kTableCap];
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);   // wave-uniform: what derives from it stays scalar
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int n = lane & 15;
  const int HKV = a.num_kv_heads;
  const int HQ = a.num_q_heads;
  const int G = a.group;

  // Workgroup ids are dealt round-robin to the 8 XCDs (each with its own
  // L2).  XCD x (ids congruent to x mod 8) takes the (sequence, KV head)
  // pairs x, x + 8, ...: a pair's tiles run on one XCD and share its K/V
  // through that XCD's L2 instead of each fetching it from HBM, and dealing
  // pairs round-robin keeps the XCDs' shares of every sequence equal.  The
  // order within an XCD follows where the work varies.  Chunks on top of
  // long earlier contexts cost about the same per tile but differ per pair:
  // pair by pair, each pair's tiles back to back.  Fresh prompts differ per
  // tile (a tile's rows see more keys the later they sit): tile level by
  // tile level, heaviest first, across the XCD's pairs.  Every workgroup
  // takes the same decision from the batch: causal work (n^2 / 2 per
  // sequence) against work on the earlier context (n (L - n)).
  // (Each wave sums over all sequences itself, so no barrier is needed.)
  // Lane q < 64 keeps sequence q's chunk start, end and length, so that a
  // batch of up to 64 sequences needs no second round trip for its own.
  float causal_all = 0.f, earlier_all = 0.f;
  int own_q0 = 0, own_q1 = 0, own_len = 0;
  for (int q = lane; q < a.num_seqs; q += 64) {
    const int qs = a.query_start[q], qe = a.query_start[q + 1], lq = a.context_lens[q];
    if (q == lane) {
      own_q0 = qs;
      own_q1 = qe;
      own_len = lq;
    }
    const float nq_s = (float)(qe - qs);
    causal_all += 0.5f * nq_s * nq_s;
    earlier_all += nq_s * ((float)lq - nq_s);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    causal_all += __shfl_xor(causal_all, d);
    earlier_all += __shfl_xor(earlier_all, d);
  }
  const int pairs = a.num_seqs * HKV;
  const int per_xcd = (pairs + kNumXcd - 1) / kNumXcd;
  const int xcd = (int)blockIdx.x % kNumXcd;
  // The splits of one row tile are consecutive workgroups of one XCD.
  const int num_splits = kSplit ? sp.num_splits : 1;
  const int split = ((int)blockIdx.x / kNumXcd) % num_splits;
  const int slot = (int)blockIdx.x / kNumXcd / num_splits;   // in [0, tiles_per_seq * per_xcd)
  int pair, tile;
  // Equal on every lane (a butterfly gives every lane the same sum); moved
  // to a scalar so that everything derived from the pair stays scalar.
  const bool tile_major = uniform(causal_all > earlier_all ? 1 : 0) != 0;
  if (tile_major) {
    pair = (slot % per_xcd) * kNumXcd + xcd;
    tile = a.tiles_per_seq - 1 - slot / per_xcd;
  } else {
    pair = (slot / a.tiles_per_seq) * kNumXcd + xcd;
    tile = a.tiles_per_seq - 1 - slot % a.tiles_per_seq;
  }
  if (pair >= pairs) return;
  const int s = pair / HKV;
  const int hk = pair % HKV;
  const bool own = a.num_seqs <= 64;
  const int q0 = own ? __builtin_amdgcn_readlane(own_q0, s) : a.query_start[s];
  const int nq = (own ? __builtin_amdgcn_readlane(own_q1, s) : a.query_start[s + 1]) - q0;
  const int L = own ? __builtin_amdgcn_readlane(own_len, s) : a.context_lens[s];
  const int rows = nq * G;
  const int row0 = tile * kPrefillRowsPerWg;
  if (row0 >= rows) return;                       // the whole workgroup leaves
  const int last_row = min(row0 + kPrefillRowsPerWg, rows) - 1;
  const int p_max = L - nq + last_row / G;       // highest position a row here has
  const int steps = p_max / kKeys + 1;
  // This workgroup's share of the key steps (all of them without a split).
  const int split_steps = (steps + num_splits - 1) / num_splits;
  const int t_begin = kSplit ? min(steps, split * split_steps) : 0;
  const int t_end = kSplit ? min(steps, t_begin + split_steps) : steps;

  // Row tile rt of wave w covers rows row0 + 16 (w kRowTiles + rt) .. +16:
  // a wave's two tiles are adjacent, so under the causal mask its lower tile
  // computes at most one step of keys none of its rows sees (interleaving the
  // waves' tiles instead evens out the waves' key counts but makes the lower
  // tile of every wave compute two such steps: 16% more matrix work on fresh
  // prompts against 5%, and 1.5-2% slower).
  auto tile_row0 = [&](int rt) { return row0 + 16 * (wave * kRowTiles + rt); };
  const bool wave_rows = tile_row0(0) < rows;
  int wave_last = -1;                              // last real row of this wave
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
    if (tile_row0(rt) < rows) wave_last = min(tile_row0(rt) + 15, rows - 1);
  const int wave_pmax = wave_rows ? L - nq + wave_last / G : -1;
  const int wave_pmin = L - nq + tile_row0(0) / G;   // lowest position of a row in this wave

  // The weights are 2^(cexp s - m), cexp = |scale log2(e)| >= 0: a negative
  // scale flips the sign of q instead (exact in bf16).
  const float cexp = fabsf(a.scale_log2);
  const u32x4 qsign = a.scale_log2 < 0.f ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                                         : u32x4{0u, 0u, 0u, 0u};
  // This lane's row of each tile: position and Q^T operand (dims 32c+8g..+8).
  int pos[kRowTiles];
  u32x4 qop[kRowTiles][4];
  const char* qbase = static_cast<const char*>(a.q);
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = tile_row0(rt) + n;
    const bool real = r < rows;
    const int token = real ? r / G : 0;
    const int head = hk * G + (real ? r % G : 0);
    pos[rt] = real ? L - nq + token : p_max;
    const char* row = qbase + ((int64_t)(q0 + token) * HQ + head) * kPRow + g4 * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qop[rt][c] = real ? *reinterpret_cast<const u32x4*>(row + c * 64) ^ qsign
                        : u32x4{0u, 0u, 0u, 0u};
  }

  // Block-table entries [first, first + kTableCap) of the blocks the keys up
  // to p_max use, staged in LDS.
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  // Keys fetched stay below min(L, p_max + kKeys); entries past
  // ceil(L / BS) are never read.
  const int used_blocks = min(L, p_max + kKeys) / BS + 1;
  const int table_len = min(used_blocks, (L + BS - 1) / BS);
  auto stage_table = [&](int first) {
    for (int i = tid; i < kTableCap && first + i < table_len; i += kThreads)
      tab[i] = table[first + i];
  };
  constexpr int kStepsPerTable = kTableCap * BS / kKeys;

  // Step loads.  Wave w fills lines 4 (2 (w % 2) + h) .. + 3 of half w / 2
  // of both tiles (h = 0, 1): a half's 16 keys lie in one block (BS is a
  // multiple of 16 and a step starts at a multiple of 32), so the block, its
  // table entry and its buffer range are wave-uniform.  The range holds the
  // block's rows below L: rows past it (or a block past the context) load as
  // zeros.  Lane i of load h fetches, for K, chunk 4 (2 (w % 2) + h) + i / 16
  // of the half's key i % 16; for V, chunk 4 (2 (w % 2) + h) + 2 (i / 32)
  // + i % 2 of key 8 ((i / 16) % 2) + (i % 16) / 2: the layouts above.  Its
  // offset in the range is fixed but for h (64 bytes apart).
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const int fetch_half = wave >> 1;
  const int fetch_run = 2 * (wave & 1);           // first of the wave's two 1 KiB runs in the half
  const int kkey = (16 * fetch_half + (lane & 15)) % BS;
  const int vkey = (16 * fetch_half + 8 * ((lane >> 4) & 1) + ((lane & 15) >> 1)) % BS;
  const int koff = kkey * kPRow + 64 * fetch_run + 16 * (lane >> 4);
  const int voff = vkey * kPRow + 64 * fetch_run + 32 * (lane >> 5) + 16 * (lane & 1);
  const int64_t block_bytes = (int64_t)HKV * BS * kPRow;
  const int64_t head_bytes = (int64_t)hk * BS * kPRow;
  // direct: the block's table entry is read from the table itself (the
  // first step, issued while the window is being staged).
  auto fetch = [&](int k0, char* buf, bool direct) {
    const int bi = (k0 + 16 * fetch_half) / BS;   // non-negative: shifts only
    const int rows_valid = uniform(min(max(L - bi * BS, 0), BS));
    const int64_t pb =
        rows_valid > 0 ? (int64_t)uniform(direct ? table[bi] : tab[bi % kTableCap]) : 0;
    const int64_t base = pb * block_bytes + head_bytes;
    const int bytes = rows_valid * kPRow;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + base, bytes);
    char* kdst = buf + fetch_half * kHalfBytes + fetch_run * 1024;
    char* vdst = kdst + kKBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      load_to_lds(rk, kdst + 1024 * h, koff, 64 * h);
      load_to_lds(rv, vdst + 1024 * h, voff, 64 * h);
    }
  };
  // Where this lane's operand reads start in a buffer's K and V tiles (the
  // layouts above): K chunk 4c + g4 of key 16 half + n at kread + 1024 c
  // + 4096 half; V chunk 2c + (n % 4) / 2 of key 4 g4 + n / 4 at vread
  // + 512 c, byte 8 (n % 2) of it (keys 16.. 4096 bytes on).
  const int kread = 256 * g4 + 16 * n;
  const int vread = 256 * (g4 >> 1) + 16 * (8 * (g4 & 1) + 2 * (n >> 2) + ((n >> 1) & 1)) + 8 * (n & 1);

  f32x4_t acc[kRowTiles][8];
  float m_run[kRowTiles], l_run[kRowTiles];
  // The lazy-rescale bound in raw score units, (m + kRescaleSlack) / cexp:
  // a lane whose raw maximum passes it may move its row's reference.  With
  // cexp == 0 it is -inf until the first step (m = -inf) and +inf after it
  // (m = 0), as the scaled test would be.
  float raw_bound[kRowTiles];
  const float inv_cexp = 1.f / cexp;
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    m_run[rt] = -INFINITY;
    raw_bound[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[rt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Step t_begin + 2i goes to LDS buffer lds0, step t_begin + 2i + 1 to
  // lds1, each loaded during the step before it: the buffer held the step
  // two back, which every wave finished before the barrier that closed the
  // step before.  That barrier also waits for the loads (a barrier waits for
  // the wave's outstanding memory operations).
  if (!kSplit || t_begin < t_end) stage_table(t_begin / kStepsPerTable * kTableCap);
  if (t_begin < t_end) fetch(t_begin * kKeys, lds0, true);
  __syncthreads();
  auto step = [&](const char* kb, char* next, int t) __attribute__((always_inline)) {
    const int k0 = t * kKeys;
    const int ahead = t + 1;
    if (ahead < t_end) {
      if (ahead % kStepsPerTable == 0) {
        // Step `ahead` needs the next table window; every fetch of the
        // current one has been issued, so refill it between two barriers.
        __syncthreads();
        stage_table(ahead / kStepsPerTable * kTableCap);
        __syncthreads();
      }
      fetch(ahead * kKeys, next, false);
    }
    if (wave_rows && k0 <= wave_pmax) {
      // Some key of the step lies past some row's position (this includes
      // every key at or past L).
      const bool diagonal = k0 + kKeys - 1 > wave_pmin;
      const char* vb = kb + kKBytes;
      // V^T operand of dim tile c (dims 16c..16c+15): lane n of group g
      // needs V[key][16c + n] for its eight keys (k = 8g..8g+7: keys
      // 4g..4g+3, then 16+4g..16+4g+3).  In each of two transposing reads,
      // lane n of the group addresses key 4g + n/4 (+16), dims 16c + 4(n%4)
      // ..+4 (chunk 2c + (n%4)/2, its half n%2), and receives
      // V[4g + e (+16)][16c + n], e = 0..3.
      auto v_operand = [&](int c) {
        const uint64_t lo = lds_read_tr16(vb, vread + 512 * c);
        const uint64_t hi = lds_read_tr16(vb, vread + 512 * c + kHalfBytes);
        return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
      };
      // Scores of both row tiles first, the four independent accumulators
      // interleaved, so one tile's softmax overlaps the other's products.
      f32x4_t scores[kRowTiles][2];
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
        for (int half = 0; half < 2; ++half) scores[rt][half] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // K operands of dims 32c + 8g..+8 (chunk 4c + g): key 16*half + n.
        u32x4 kop[2];
#pragma unroll
        for (int half = 0; half < 2; ++half)
          kop[half] = lds_load16(kb, kread + 1024 * c + kHalfBytes * half);
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
          for (int half = 0; half < 2; ++half)
            scores[rt][half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, kop[half]),
                __builtin_bit_cast(bf16x8_t, qop[rt][c]), scores[rt][half], 0, 0, 0);
      }
      // V^T operands of the first kVAhead dim tiles are read before the
      // softmax, so their LDS latency hides behind it; later ones are read
      // kVAhead tiles before their products.
      u32x4 vop[8];
#pragma unroll
      for (int c = 0; c < kVAhead; ++c) vop[c] = v_operand(c);
      u32x4 pop[kRowTiles];
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        const f32x4_t* sc = scores[rt];
        // Raw scores.  On steps that reach past the wave's lowest row
        // position (a wave-uniform branch), keys past a row's position are
        // set to -inf: left out of the max, weight 0 below.
        float x[8];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 * half + i] = sc[half][i];
        if (diagonal) {
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (k0 + 16 * half + 4 * g4 + i > pos[rt]) x[4 * half + i] = -INFINITY;
        }
        const float mx_lane = smax(smax(smax(x[0], x[1]), smax(x[2], x[3])),
                                   smax(smax(x[4], x[5]), smax(x[6], x[7])));
        // A row's reference moves only if its tile max (the max over its four
        // lanes) passes it by the slack, i.e. only if one of its lanes' own
        // max does: the four-lane max is taken only in a step where some
        // lane's does (in the exp2 domain; cexp >= 0 keeps the order).
        const bool lane_grow = mx_lane > raw_bound[rt];
        if (__builtin_amdgcn_ballot_w64(lane_grow)) {
          float mx = group4_smax(mx_lane);
          mx = mx == -INFINITY ? -INFINITY : mx * cexp;
          const bool grow = mx > m_run[rt] + kRescaleSlack;
          const float m_new = grow ? mx : m_run[rt];
          // 1 where the reference stays (also for a row still at m = -inf,
          // where the difference would be NaN).
          const float alpha =
              !kSplit || grow ? fast_exp2(m_run[rt] - m_new) : 1.f;
          m_run[rt] = m_new;
          raw_bound[rt] = (m_new + kRescaleSlack) * inv_cexp;
          l_run[rt] *= alpha;
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) acc[rt][cc] *= alpha;
        }
        // Weights 2^(cexp x - m), rounded to bf16; the running sum adds the
        // rounded pairs with one dot product each.
        uint32_t pb[4];
        // A row that has seen no key yet (possible only in a later split)
        // keeps m = -inf: its weights are then 2^-inf = 0.
        const float neg_m = kSplit && m_run[rt] == -INFINITY ? 0.f : -m_run[rt];
        // x = -inf gives 2^-inf = 0 for cexp > 0; with cexp == 0 the product
        // would be NaN, so masked weights are zeroed explicitly then.
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = fast_exp2(fmaf(x[j], cexp, neg_m));
        if (diagonal && cexp == 0.f) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = x[j] == -INFINITY ? 0.f : w[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[j] = cvt_bf16x2(w[2 * j], w[2 * j + 1]);
          l_run[rt] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pb[j]), kOnes, l_run[rt], false);
        }
        pop[rt] = u32x4{pb[0], pb[1], pb[2], pb[3]};
      }
      // O^T += V^T . P^T, one V^T operand per dim tile for both row tiles.
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + kVAhead < 8) vop[c + kVAhead] = v_operand(c + kVAhead);
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
          acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, vop[c]), __builtin_bit_cast(bf16x8_t, pop[rt]),
              acc[rt][c], 0, 0, 0);
      }
    }
    __syncthreads();
  };
  for (int t = t_begin; t < t_end; t += 2) {
    step(lds0, lds1, t);
    if (t + 1 < t_end) step(lds1, lds0, t + 1);
  }

  if constexpr (kSplit) {
    // Unnormalized partial row for the merge: acc relative to the row's
    // reference max, the max and the sum.
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      const float total = group4_sum(l_run[rt]);
      const int r = tile_row0(rt) + n;
      if (r >= rows) continue;
      float* prow = sp.partials +
                    (((int64_t)split * sp.num_query_tokens + q0 + r / G) * HQ + hk * G + r % G) *
                        kPartRow;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<float4*>(prow + 16 * c + 4 * g4) =
            make_float4(acc[rt][c][0], acc[rt][c][1], acc[rt][c][2], acc[rt][c][3]);
      if (g4 == 0) *reinterpret_cast<float2*>(prow + kPD) = make_float2(m_run[rt], total);
    }
    return;
  }

  // Normalise and store: lane l holds dims 16c + 4g + i (i = 0..3) of its
  // row in acc[rt][c].
  char* obase = static_cast<char*>(a.out);
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const float total = group4_sum(l_run[rt]);
    const int r = tile_row0(rt) + n;
    if (r >= rows) continue;
    const float inv = 1.f / total;
    char* row = obase + ((int64_t)(q0 + r / G) * HQ + hk * G + r % G) * kPRow + g4 * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint2 v = make_uint2(cvt_bf16x2(acc[rt][c][0] * inv, acc[rt][c][1] * inv),
                                 cvt_bf16x2(acc[rt][c][2] * inv, acc[rt][c][3] * inv));
      *reinterpret_cast<uint2*>(row + c * 32) = v;
    }
  }
}

// Folds the num_splits partial rows of every (query token, query head) row
// into `out`: with M the largest reference max, out = sum_s acc_s 2^(m_s - M)
// / sum_s l_s 2^(m_s - M).  Splits that saw no key of the row carry
// m = -inf and add nothing; the first split always holds key 0, which every
// row sees.  Four waves of two rows each per workgroup, four dims per lane.
constexpr int kMergeRowsPerWg = 8;
constexpr int kMaxSplits = 32;
// kCap: split slots one lane holds in registers (16 or 32; the 32-slot
// instance needs about twice the registers, so it serves only counts past 16).
template <int kCap>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a,
                                                            const SplitArgs sp) {
  const int64_t rows = sp.num_query_tokens * a.num_q_heads;
  const int64_t row = (int64_t)blockIdx.x * kMergeRowsPerWg + threadIdx.x / 32;
  if (row >= rows) return;
  const int d0 = (threadIdx.x % 32) * 4;
  const int64_t split_stride = rows * kPartRow;
  const float* base = sp.partials + row * kPartRow;
  const int n = sp.num_splits;
  // Every split's loads are issued before the first is used (the bound is
  // the constant kCap; splits past n are skipped by a uniform branch).
  float2 ml[kCap];
  float4 o[kCap];
#pragma unroll
  for (int s = 0; s < kCap; ++s) {
    if (s < n) {
      const float* p = base + s * split_stride;
      ml[s] = *reinterpret_cast<const float2*>(p + kPD);
      o[s] = *reinterpret_cast<const float4*>(p + d0);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kCap; ++s)
    if (s < n) M = fmaxf(M, ml[s].x);
  float S = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kCap; ++s) {
    if (s < n) {
      const float f = ml[s].x == -INFINITY ? 0.f : fast_exp2(ml[s].x - M);
      S = fmaf(ml[s].y, f, S);
      O[0] = fmaf(o[s].x, f, O[0]);
      O[1] = fmaf(o[s].y, f, O[1]);
      O[2] = fmaf(o[s].z, f, O[2]);
      O[3] = fmaf(o[s].w, f, O[3]);
    }
  }
  const float inv = 1.f / S;
  *reinterpret_cast<uint2*>(static_cast<char*>(a.out) + (row * kPD + d0) * 2) =
      make_uint2(cvt_bf16x2(O[0] * inv, O[1] * inv), cvt_bf16x2(O[2] * inv, O[3] * inv));
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int block_size) {
  return dtype == kBf16 && head_dim == kPD && (block_size == 16 || block_size == 32);
}

// Declared where it is called (pa_api.hip).  partials may be null when
// num_splits is 1.
hipError_t launch_prefill_split(const PrefillArgs& a, int block_size, int num_splits,
                                float* partials, int64_t num_query_tokens, hipStream_t stream) {
  // Whole rounds of 8 pairs: workgroups past the last pair leave at once.
  const int64_t blocks = (int64_t)a.tiles_per_seq * kNumXcd *
                         ((a.num_seqs * a.num_kv_heads + kNumXcd - 1) / kNumXcd) * num_splits;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX || num_splits < 1 || num_splits > kMaxSplits) return hipErrorInvalidValue;
  const SplitArgs sp{num_splits, partials, num_query_tokens};
  const dim3 grid((unsigned)blocks), wg(kThreads);
  if (num_splits == 1) {
    if (block_size == 16)
      hipLaunchKernelGGL((prefill_kernel<16, false>), grid, wg, 0, stream, a, sp);
    else
      hipLaunchKernelGGL((prefill_kernel<32, false>), grid, wg, 0, stream, a, sp);
  } else {
    if (block_size == 16)
      hipLaunchKernelGGL((prefill_kernel<16, true>), grid, wg, 0, stream, a, sp);
    else
      hipLaunchKernelGGL((prefill_kernel<32, true>), grid, wg, 0, stream, a, sp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || num_splits == 1) return e;
  const int64_t rows = num_query_tokens * a.num_q_heads;
  const int64_t wgs = (rows + kMergeRowsPerWg - 1) / kMergeRowsPerWg;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  if (num_splits <= 16)
    hipLaunchKernelGGL(prefill_merge_kernel<16>, dim3((unsigned)wgs), dim3(256), 0, stream, a, sp);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<32>, dim3((unsigned)wgs), dim3(256), 0, stream, a, sp);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int block_size, hipStream_t stream) {
  return launch_prefill_split(a, block_size, 1, nullptr, 0, stream);
}

}  // namespace pa
