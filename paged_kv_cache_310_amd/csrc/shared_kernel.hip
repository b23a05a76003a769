// Decode-step paged attention for batches whose sequences come in groups
// that share a prefix (pa_decode_shared): bf16, head_dim 128, 1..16 query
// heads per KV head, on the gfx950 matrix cores.
//
// Pages on "Efficient Memory Management for Large Language Model Serving with
// PagedAttention": zeroshotmind.com essay, "Sharing a prefix without copying
// it" (sequences forked from one prompt keep pointing at the same physical
// blocks, which hold one copy of the prefix for all of them) and "Block
// tables: logical order, physical scatter" (attention walks each sequence's
// blocks in logical order through its table).  The result is exactly the
// attention pa_decode computes; what changes is how often a shared block is
// read.  pa_decode walks every sequence's table, so a block that 8 sequences
// share is read 8 times.  Here the tokens a group shares are read once per
// (group, KV head):
//
//  * The prefix line.  Its segments are (KV head, group, row block): a row
//    block is up to 16 / group whole members of the group, whose
//    members x query-heads q rows (at most 16) form the N columns of the same
//    MFMA products the grouped-query kernel uses (gqa_body.h).  A segment
//    walks the group's shared chunks through the group's first member's table
//    (every member's table holds the same blocks there), reading each 4 KiB
//    K and V tile once for all its rows.
//  * The tail line.  Each (KV head, sequence) segment covers the sequence's
//    chunks after its shared prefix (all of them for a sequence without one),
//    through its own table, with the fused append -- the grouped-query worker
//    loop of gqa_body.h started at that chunk.
//  * One launch serves both lines: the workers are shared out in proportion
//    to the lines' work units, each line is split over its workers exactly
//    as pa_decode splits its line (equal unit shares, a segment costing its
//    chunks plus seg_cost), and each worker runs one line's loop.
//  * A prefix or tail segment of a sequence with a shared prefix leaves its
//    unnormalised result (acc, max, sum) -- one row in res_pre / res_tail
//    when one worker holds the whole segment, else split pieces in the
//    workers' partial slots -- and a locator entry per (KV head, sequence)
//    saying which.  Segments of sequences without a shared prefix behave as
//    in pa_decode (output rows, or pieces named by a merge record).
//  * The merge launch runs the usual record merge for the latter, and for
//    every (sequence with a shared prefix, query head) folds the prefix part
//    and the tail part into the output row.
//
// The number of shared chunks of a sequence is floor(P / 16) for its prefix
// length P (clamped into [0, context length]): a partial last chunk of the
// prefix is read through each member's own table, where it is the same data.
#include "gqa_body.h"
#include "merge_body.h"

namespace pa {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// The prefix line.

// Group g: members [lo, lo + nmem) (group_start clamped into [0, B]), c0
// shared chunks (the first member's prefix length, clamped into its context,
// in whole chunks), nb row blocks of mb members (0 when nothing is shared).
struct PGroup {
  int lo, nmem, c0, nb;
};

// P is `const int32_t*` (per-lane loads) or `const const_i32*` (scalar loads
// of wave-uniform data).
template <typename P>
__device__ __forceinline__ PGroup prefix_group_at(P gs, P plen, P lens, int B, int mb, int g) {
  PGroup r;
  int lo = gs[g], hi = gs[g + 1];
  lo = lo < 0 ? 0 : (lo > B ? B : lo);
  hi = hi < lo ? lo : (hi > B ? B : hi);
  r.lo = lo;
  r.nmem = hi - lo;
  r.c0 = r.nmem > 0 ? shared_chunks(lens[lo], plen[lo]) : 0;
  r.nb = r.c0 > 0 ? (r.nmem + mb - 1) / mb : 0;
  return r;
}

__device__ __forceinline__ PGroup prefix_group_lane(const ShareArgs& sh, const int32_t* lens,
                                                    int B, int g) {
  return prefix_group_at<const int32_t*>(sh.group_start, sh.prefix_lens, lens, B,
                                         sh.members_per_block, g);
}

__device__ __forceinline__ PGroup prefix_group_uniform(const ShareArgs& sh, const int32_t* lens,
                                                       int B, int g) {
  return prefix_group_at<const const_i32*>((const const_i32*)sh.group_start,
                                           (const const_i32*)sh.prefix_lens,
                                           (const const_i32*)lens, B, sh.members_per_block, g);
}

// Chunks and units of the prefix line per KV head: group g has nb segments
// of c0 chunks, each costing c0 + seg_cost units.
__device__ __forceinline__ void prefix_line_totals(const ShareArgs& sh, const int32_t* lens, int B,
                                                   int seg_cost, int lane, int64_t& wseq,
                                                   int64_t& useq) {
  int64_t n = 0, un = 0;
  for (int g = lane; g < sh.num_groups; g += 64) {
    const PGroup pg = prefix_group_lane(sh, lens, B, g);
    n += (int64_t)pg.nb * pg.c0;
    un += (int64_t)pg.nb * (pg.c0 + seg_cost);
  }
  wseq = uniform(wave_sum(n));
  useq = uniform(wave_sum(un));
}

// Where a unit target r (relative to its KV head's units) falls on the prefix
// line: group g, the units and chunks of the head before it, r's offset in
// the group's units, and the group.
struct PHit {
  bool found;
  int g;
  int64_t bu, bc, off;
  PGroup pg;
};

__device__ void prefix_locate(const ShareArgs& sh, const int32_t* lens, int B, int seg_cost,
                              int64_t r0, int64_t r1, int lane, PHit& h0, PHit& h1) {
  h0.found = false;
  h1.found = false;
  int64_t acc_u = 0, acc_c = 0;
  for (int base = 0; base < sh.num_groups && !(h0.found && h1.found); base += 64) {
    const int g = base + lane;
    PGroup pg = {0, 0, 0, 0};
    if (g < sh.num_groups) pg = prefix_group_lane(sh, lens, B, g);
    const int64_t un = (int64_t)pg.nb * (pg.c0 + seg_cost);
    const int64_t cn = (int64_t)pg.nb * pg.c0;
    const int64_t incl_u = wave_scan(un, lane);
    const int64_t incl_c = wave_scan(cn, lane);
    const int64_t tot_u = lane_value((int64_t)incl_u, 63);
    const int64_t tot_c = lane_value((int64_t)incl_c, 63);
    auto probe = [&](int64_t r, PHit& hit) {
      if (hit.found || r >= acc_u + tot_u) return;
      const int first = __ffsll((long long)__ballot(acc_u + incl_u > r)) - 1;
      hit.found = true;
      hit.g = uniform(base + first);
      hit.bu = acc_u + lane_value((int64_t)(incl_u - un), first);
      hit.bc = acc_c + lane_value((int64_t)(incl_c - cn), first);
      hit.off = r - hit.bu;
      hit.pg.lo = lane_value(pg.lo, first);
      hit.pg.nmem = lane_value(pg.nmem, first);
      hit.pg.c0 = lane_value(pg.c0, first);
      hit.pg.nb = lane_value(pg.nb, first);
    };
    probe(r0, h0);
    probe(r1, h1);
    acc_u += tot_u;
    acc_c += tot_c;
  }
}

// A worker's range on the prefix line and the segment holding its first
// chunk.
struct PSplit {
  int64_t U, W, NW, u0, u1, b0, b1;
  int64_t seg_start, seg_unit;   // line chunk / unit of that segment's first chunk / unit
  int kvh, g, rb, j;             // its KV head, group, row block; b0's chunk in it
  PGroup pg;
};

// Line chunk of unit offset `off` into a group whose head-relative units and
// chunks begin at (bu, bc): row block off / (c0 + seg_cost), and within it
// the chunk after the block's seg_cost overhead units.
__device__ __forceinline__ int64_t prefix_chunk_at(const PHit& x, int seg_cost, int64_t head_c,
                                                   int64_t* seg_start, int* rb) {
  const int64_t per = x.pg.c0 + seg_cost;
  const int64_t b = x.off / per;
  const int64_t r2 = x.off - b * per;
  const int64_t start = head_c + x.bc + b * x.pg.c0;
  if (seg_start) *seg_start = start;
  if (rb) *rb = (int)b;
  return start + (r2 < seg_cost ? 0 : r2 - seg_cost);
}

__device__ __forceinline__ bool prefix_split(const ShareArgs& sh, const int32_t* lens, int B,
                                             int num_heads, int seg_cost, int64_t wseq,
                                             int64_t useq, int nworkers, int w, int lane,
                                             PSplit& ps) {
  ps.U = useq * num_heads;
  ps.W = wseq * num_heads;
  if (ps.U == 0) return false;
  ps.NW = ps.U < nworkers ? ps.U : nworkers;
  if (w >= ps.NW) return false;
  ps.u0 = (int64_t)w * ps.U / ps.NW;
  ps.u1 = (int64_t)(w + 1) * ps.U / ps.NW;
  const int hh0 = (int)(ps.u0 / useq);
  const int hh1 = ps.u1 < ps.U ? (int)(ps.u1 / useq) : 0;
  const int64_t r1 = ps.u1 < ps.U ? ps.u1 - (int64_t)hh1 * useq : ps.U;
  PHit x0, x1;
  prefix_locate(sh, lens, B, seg_cost, ps.u0 - (int64_t)hh0 * useq, r1, lane, x0, x1);
  ps.kvh = hh0;
  ps.g = x0.g;
  ps.pg = x0.pg;
  ps.b0 = prefix_chunk_at(x0, seg_cost, (int64_t)hh0 * wseq, &ps.seg_start, &ps.rb);
  ps.seg_unit = (int64_t)hh0 * useq + x0.bu + (int64_t)ps.rb * (x0.pg.c0 + seg_cost);
  ps.j = (int)(ps.b0 - ps.seg_start);
  ps.b1 = ps.u1 < ps.U ? prefix_chunk_at(x1, seg_cost, (int64_t)hh1 * wseq, nullptr, nullptr)
                       : ps.W;
  return ps.b0 < ps.b1;
}

// Wave-uniform cursor over the prefix line: chunk j of row block rb of group
// g's shared chunks, KV head kvh.  Callers never move it past the last chunk
// of their range.
struct PCursor {
  int64_t c, seg_start;
  int kvh, g, rb, j;
  PGroup pg;
};

__device__ __forceinline__ void pcursor_next(PCursor& k, const ShareArgs& sh, const int32_t* lens,
                                             int B) {
  ++k.c;
  if (++k.j < k.pg.c0) return;
  k.j = 0;
  k.seg_start = k.c;
  if (++k.rb < k.pg.nb) return;
  k.rb = 0;
  do {
    if (++k.g == sh.num_groups) {
      k.g = 0;
      ++k.kvh;
    }
    k.pg = prefix_group_uniform(sh, lens, B, k.g);
  } while (k.pg.nb == 0);
}

// What a prefix tile carries about its segment.
struct PMeta {
  int kvh, s_lo, nm;   // KV head; the row block's members [s_lo, s_lo + nm)
  int flags;           // kFirst, kLast, kWhole, kSecond (as for ChunkMeta)
  __device__ bool first() const { return flags & kFirst; }
  __device__ bool last() const { return flags & kLast; }
  __device__ bool whole() const { return flags & kWhole; }
  __device__ int partial_slot() const { return (flags & kSecond) ? 1 : 0; }
};

__device__ __forceinline__ PMeta pmeta(const PCursor& k, int mb, int64_t b0, int64_t b1) {
  PMeta m;
  m.kvh = k.kvh;
  m.s_lo = k.pg.lo + k.rb * mb;
  const int left = k.pg.nmem - k.rb * mb;
  m.nm = left < mb ? left : mb;
  const bool seg_last = k.j == k.pg.c0 - 1;
  m.flags = ((k.c == b0 || k.j == 0) ? kFirst : 0) | ((k.c == b1 - 1 || seg_last) ? kLast : 0) |
            ((k.seg_start >= b0 && k.seg_start + k.pg.c0 <= b1) ? kWhole : 0) |
            (k.seg_start > b0 ? kSecond : 0);
  return m;
}

// The worker loop over the prefix line's chunks [ps.b0, ps.b1).  The MFMA
// layout, ring, store queue and online softmax are those of gqa_body.h; the
// differences are the rows (the row block's members x query heads, q read
// from each member's own row), the table (the group's first member's), full
// tiles only (shared chunks are whole), and the results (res_pre rows or
// pieces, with locator entries).
template <int BS>
__device__ __forceinline__ void prefix_body(const DecodeArgs& a, const ShareArgs& sh,
                                            KernelLds& lds, const PSplit& ps, int w) {
  constexpr int CPB = BS / kChunk;
  constexpr int REC = kD + kPartialExtra;
  const int lane = threadIdx.x;
  const int g4 = lane >> 4;
  const int n = lane & 15;   // MFMA column: row n = member n / G, query head n % G of the block
  const int B = a.num_seqs;
  const int HQ = a.num_q_heads;
  const int HKV = a.num_kv_heads;
  const int G = a.group;
  const int mb = sh.members_per_block;
  const int32_t* __restrict__ lens = a.context_lens;
  const int64_t b0 = ps.b0, b1 = ps.b1;

  PCursor cur;
  cur.c = b0;
  cur.seg_start = ps.seg_start;
  cur.kvh = ps.kvh;
  cur.g = ps.g;
  cur.rb = ps.rb;
  cur.j = ps.j;
  cur.pg = ps.pg;

  const int64_t block_stride = (int64_t)HKV * BS * kRow;
  const int krow_off = token_of(n) * kRow + g4 * 16;
  // q row of column n within the block's q rows: member n / G, head n % G.
  // Columns past the block's rows address past the buffer range and read 0.
  const int qoff = ((n / G) * HQ + n % G) * kRow + g4 * 16;
  auto table_of = [&](const PCursor& k) {
    return (const const_i32*)(a.block_tables + (int64_t)k.pg.lo * a.max_blocks_per_seq);
  };
  int next_pb = table_of(cur)[cur.j / CPB];

  struct Tile {
    u32x4 k[4];   // K operand: token token_of(l%16), dims 32c + 8(l/16)
    u32x4 v[4];   // V rows: load i = token 4i + l/16, dims 8(l%16)..+8
    u32x4 q[4];   // Q^T operand: row l%16, dims 32c + 8(l/16)
    PMeta meta;
  };

  StoreQueue q = queue_on(lds.queue);
  // Prefix pieces are found through locators, never through merge records.
  MergeRecord none{};
  none.valid = 0;
  queue_record(q, a.records + w, none, lane, a.out);
  // The worker closing the split segment that holds b0 writes its members'
  // locators: pieces of workers first..w, the first in slot first_slot.
  if (ps.seg_start < b0 && ps.seg_start + ps.pg.c0 <= b1) {
    const int64_t first = worker_of(ps.seg_unit + a.seg_cost, ps.U, ps.NW);
    const int first_slot = first * ps.U / ps.NW < ps.seg_unit ? 1 : 0;
    const int s_lo = ps.pg.lo + ps.rb * mb;
    const int left = ps.pg.nmem - ps.rb * mb;
    const int nm = left < mb ? left : mb;
    const int f = queue_reserve(q, 1, lane, a.out);
    if (lane < nm)
      queue_put(q, f, lane * 16, u32x4{(uint32_t)first, (uint32_t)(w - first + 1),
                                       (uint32_t)first_slot, (uint32_t)(lane * G)});
    queue_job(q, f, sh.loc_pre + ((int64_t)ps.kvh * B + s_lo) * 4, nm * 16, lane);
  }

  int64_t q_seg = -1;   // segment whose q rows the last issued tile holds
  auto issue = [&](Tile& t, const Tile& prev, bool drain) {
    t.meta = pmeta(cur, mb, b0, b1);
    if (cur.seg_start != q_seg) {
      const int rows_bytes = ((t.meta.nm - 1) * HQ + G) * kRow;
      const __amdgpu_buffer_rsrc_t qr = tile_rsrc(
          static_cast<const char*>(a.q) + ((int64_t)t.meta.s_lo * HQ + cur.kvh * G) * kRow,
          rows_bytes);
#pragma unroll
      for (int k = 0; k < 4; ++k) t.q[k] = load16(qr, qoff + k * 64);
      q_seg = cur.seg_start;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) t.q[k] = prev.q[k];
    }
    const int64_t off = (int64_t)next_pb * block_stride + (int64_t)cur.kvh * BS * kRow +
                        (int64_t)(cur.j % CPB) * kTile;
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(static_cast<const char*>(a.k_cache) + off, kTile);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(static_cast<const char*>(a.v_cache) + off, kTile);
#pragma unroll
    for (int k = 0; k < 4; ++k) t.k[k] = load16(kr, krow_off + k * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = load16_stream(vr, i * 1024 + lane * 16);
    if (drain) {
#pragma unroll
      for (int d = 0; d < kQDrain; ++d) queue_drain_one(q, lane, a.out);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (cur.c + 1 < b1) {
      pcursor_next(cur, sh, lens, B);
      next_pb = table_of(cur)[cur.j / CPB];
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4_t o[8];

  auto consume = [&](const Tile& t) {
    const PMeta& mt = t.meta;
    if (mt.first()) {
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[k]),
                                                      __builtin_bit_cast(bf16x8_t, t.q[k]),
                                                      sacc, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * a.scale_log2;
    const float mx = group4_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);   // m_new is finite: every chunk is full
    if (__ballot(alpha != 1.f)) {
      l *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
    }
    m = m_new;
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (__bf16)fast_exp2(sc[i] - m_new);
      l += (float)pb[i];
    }
    const i16x4_t pop = __builtin_bit_cast(i16x4_t, pb);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
      const int dw = k >> 1;
      const uint32_t lo = __builtin_amdgcn_perm(t.v[1][dw], t.v[0][dw], sel);
      const uint32_t hi = __builtin_amdgcn_perm(t.v[3][dw], t.v[2][dw], sel);
      const i16x4_t va = __builtin_bit_cast(i16x4_t, (uint64_t)lo | ((uint64_t)hi << 32));
      o[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pop, o[k], 0, 0, 0);
    }
    if (!mt.last()) return;

    // ---- end of this worker's part of the segment: the rows' (acc, max, sum)
    l = group4_sum(l);
    const int rows = mt.nm * G;
    const int bytes = rows * REC * 4;
    const int f = queue_reserve(q, queue_slots(bytes), lane, a.out);
    if (n < rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = (n * REC + g4 * 32 + i * 8) * 4;
        queue_put(q, f, off, f32x4_bits(o[0][i], o[1][i], o[2][i], o[3][i]));
        queue_put(q, f, off + 16, f32x4_bits(o[4][i], o[5][i], o[6][i], o[7][i]));
      }
      if (g4 == 0) queue_put(q, f, (n * REC + kD) * 4, f32x4_bits(m, l, 0.f, 0.f));
    }
    float* dst = mt.whole()
                     ? sh.res_pre + ((int64_t)mt.kvh * B + mt.s_lo) * G * REC
                     : a.partials + ((int64_t)w * 2 + mt.partial_slot()) * a.piece_rows * REC;
    queue_job(q, f, dst, bytes, lane);
    if (mt.whole()) {
      // Locators of the members: whole, result in res_pre.
      const int fl = queue_reserve(q, 1, lane, a.out);
      if (lane < mt.nm) queue_put(q, fl, lane * 16, u32x4{(uint32_t)w, 0u, 0u, (uint32_t)(lane * G)});
      queue_job(q, fl, sh.loc_pre + ((int64_t)mt.kvh * B + mt.s_lo) * 4, mt.nm * 16, lane);
    }
  };

  const int64_t count = b1 - b0;
  Tile t[kRing];
#pragma unroll
  for (int r = 0; r + 1 < kRing; ++r) issue(t[r], t[(r + kRing - 1) % kRing], false);
  for (int64_t i = 0; i < count; i += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      if (r > 0 && i + r >= count) break;
      issue(t[(r + kRing - 1) % kRing], t[(r + kRing - 2) % kRing], r == 0);
      consume(t[r]);
    }
  }
  queue_flush(q, lane, a.out);
}

// ---------------------------------------------------------------------------
// The launch: both lines, workers shared out by work units.
// Measured: with tail segments of 8.6 chunks (the steady shared-prefix
// batch) and of 1 chunk (the fork batch), the division that ran fastest
// weighted them about 10.6 and 3.8 prefix chunk times; a line through both.
constexpr int kTailChunkTime10 = 9;
constexpr int kTailSegTime10 = 29;
template <int BS>
// One-wave workgroups, one per SIMD: the kernel holds both worker loops.
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(1)))
void decode_shared_kernel(const DecodeArgs a, const ShareArgs sh) {
  const int lane = threadIdx.x;
  const int nworkers = gridDim.x;
  const int w = (nworkers % kNumXcd) ? (int)blockIdx.x
                                     : (int)(blockIdx.x % kNumXcd) * (nworkers / kNumXcd) +
                                           (int)(blockIdx.x / kNumXcd);
  const int B = a.num_seqs;
  const int HQ = a.num_q_heads;
  const int HKV = a.num_kv_heads;
  const int32_t* __restrict__ lens = a.context_lens;
  __shared__ KernelLds lds;

  // Sequences with no cached token produce zero rows.
  for (int s = w; s < B; s += nworkers) {
    if (lens[s] == 0) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<char*>(a.out) + (size_t)s * HQ * kRow);
      for (int u = lane; u < HQ * (kRow / 16); u += 64) o[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  int64_t tw, tu, pw, pu;
  tail_line_totals(lds.split, lens, sh.prefix_lens, B, a.seg_cost, lane, tw, tu);
  prefix_line_totals(sh, lens, B, a.seg_cost, lane, pw, pu);
  const int64_t UP = pu * HKV;
  // Workers are divided by the lines' estimated times, in tenths of a prefix
  // chunk's time: a tail chunk kTailChunkTime10 (a segment's last chunk is
  // partial), a tail segment kTailSegTime10 besides its chunks (its end also
  // writes its result row and locator, and with the fused append the new
  // token's rows).
  const int64_t tail_segs = (tu - tw) / a.seg_cost;
  const int64_t UT = (kTailChunkTime10 * tw + kTailSegTime10 * tail_segs) * HKV / 10;
  // Prefix workers: the prefix line's share, at least one for each line that
  // has work.
  int wp = 0;
  if (UP > 0 && UT == 0) {
    wp = nworkers;
  } else if (UP > 0) {
    const int64_t x = (UP * nworkers + (UP + UT) / 2) / (UP + UT);
    wp = (int)(x < 1 ? 1 : (x > nworkers - 1 ? nworkers - 1 : x));
  }
  if (w < wp) {
    PSplit ps;
    if (!prefix_split(sh, lens, B, HKV, a.seg_cost, pw, pu, wp, w, lane, ps)) {
      if (lane == 0) a.records[w].valid = 0;
      return;
    }
    prefix_body<BS>(a, sh, lds, ps, w);
  } else {
    LineSplit ls;
    if (!tail_split(lds.split, lens, sh.prefix_lens, B, HKV, a.seg_cost, tw, tu, nworkers - wp,
                    w - wp, lane, ls)) {
      if (lane == 0) a.records[w].valid = 0;
      return;
    }
    gqa_body<BS, true>(a, sh, lds, ls, w, wp);
  }
}

// ---------------------------------------------------------------------------
// The merge: record waves (split segments of sequences without a shared
// prefix, as in pa_decode), then one wave per (sequence, two query heads)
// folding the prefix and tail parts of sequences with a shared prefix.

// Folds one (max, sum, acc) record into the running (M, S, O).
__device__ __forceinline__ void fold_one(float2 ms, float4 o, float& M, float& S, float* O) {
  const float Mb = fmaxf(M, ms.x);
  const float Mu = Mb == -INFINITY ? 0.f : Mb;
  const float alpha = fast_exp2(M - Mu);
  const float f = fast_exp2(ms.x - Mu);
  S = fmaf(ms.y, f, S * alpha);
  O[0] = fmaf(o.x, f, O[0] * alpha);
  O[1] = fmaf(o.y, f, O[1] * alpha);
  O[2] = fmaf(o.z, f, O[2] * alpha);
  O[3] = fmaf(o.w, f, O[3] * alpha);
  M = Mb;
}

// Folds the split pieces a locator names (row `row` of each piece) into the
// running (M, S, O), kBatch pieces' loads in flight at once.  A locator that
// names pieces outside the workspace (only an out-of-contract call can leave
// one) is ignored.
__device__ __forceinline__ void fold_pieces(const DecodeArgs& a, int workers, int4 e, int row,
                                            int d0, float& M, float& S, float* O) {
  constexpr int REC = kD + kPartialExtra;
  constexpr int kBatch = 8;
  const int first = e.x, count = e.y, slot0 = e.z;
  if (first < 0 || count > workers || first > workers - count || (slot0 & ~1) || row < 0 ||
      row >= kSharedPieceRows)
    return;
  for (int p0 = 0; p0 < count; p0 += kBatch) {
    float4 ob[kBatch];
    float2 mbv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int p = p0 + b;
      if (p < count) {
        const float* rec = a.partials + (((int64_t)(first + p) * 2 + (p == 0 ? slot0 : 0)) *
                                             a.piece_rows + row) * REC;
        mbv[b] = *reinterpret_cast<const float2*>(rec + kD);
        ob[b] = *reinterpret_cast<const float4*>(rec + d0);
      } else {
        mbv[b] = make_float2(-INFINITY, 0.f);
        ob[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float Mb = M;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) Mb = fmaxf(Mb, mbv[b].x);
    const float Mu = Mb == -INFINITY ? 0.f : Mb;
    const float alpha = fast_exp2(M - Mu);
    S *= alpha;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) O[e2] *= alpha;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const float f = fast_exp2(mbv[b].x - Mu);
      S = fmaf(mbv[b].y, f, S);
      O[0] = fmaf(ob[b].x, f, O[0]);
      O[1] = fmaf(ob[b].y, f, O[1]);
      O[2] = fmaf(ob[b].z, f, O[2]);
      O[3] = fmaf(ob[b].w, f, O[3]);
    }
    M = Mb;
  }
}

__global__ __launch_bounds__(64 * kMergeWaves) void merge_shared_kernel(const DecodeArgs a,
                                                                        const ShareArgs sh,
                                                                        int workers,
                                                                        int record_waves) {
  constexpr int REC = kD + kPartialExtra;
  const int lane = threadIdx.x % 64;
  const int id = uniform((int)(blockIdx.x * kMergeWaves + threadIdx.x / 64));
  if (id < record_waves) {
    merge_record_wave<uint16_t, kD, 8>(a, workers, id, lane);
    return;
  }
  constexpr int HPW = merge_heads_per_wave<kD>();   // 2 heads of 32 lanes x 4 dims
  const int B = a.num_seqs, HQ = a.num_q_heads, G = a.group;
  const int per_seq = (HQ + HPW - 1) / HPW;
  const int v = id - record_waves;
  const int s = v / per_seq;
  if (s >= B) return;
  const int hq = (v - s * per_seq) * HPW + lane / 32;
  if (hq >= HQ) return;   // no cross-lane work follows
  const int kvh = hq / G, hh = hq - kvh * G;
  const int d0 = (lane % 32) * 4;
  // Everything the common case needs, in one round of loads: the lengths,
  // both locators and both parts' result rows (read whether or not this
  // call wrote them; used only when the locator says so).
  const int64_t idx = (int64_t)kvh * B + s;
  const int L = a.context_lens[s];
  const int P = sh.prefix_lens[s];
  const int4 ep = *reinterpret_cast<const int4*>(sh.loc_pre + idx * 4);
  const int4 et = *reinterpret_cast<const int4*>(sh.loc_tail + idx * 4);
  const float* rp = sh.res_pre + (idx * G + hh) * REC;
  const float* rt = sh.res_tail + (idx * G + hh) * REC;
  const float2 mp = *reinterpret_cast<const float2*>(rp + kD);
  const float4 op = *reinterpret_cast<const float4*>(rp + d0);
  const float2 mt = *reinterpret_cast<const float2*>(rt + kD);
  const float4 ot = *reinterpret_cast<const float4*>(rt + d0);
  const int c0 = shared_chunks(L, P);
  if (c0 == 0) return;    // no shared prefix: written by the attention or record merge
  float M = -INFINITY, S = 0.f;
  float O[4] = {0.f, 0.f, 0.f, 0.f};
  if (ep.y <= 0)
    fold_one(mp, op, M, S, O);
  else
    fold_pieces(a, workers, ep, ep.w + hh, d0, M, S, O);
  if (chunks_of(L) - c0 > 0) {
    if (et.y <= 0)
      fold_one(mt, ot, M, S, O);
    else
      fold_pieces(a, workers, et, et.w + hh, d0, M, S, O);
  }
  char* out_row = static_cast<char*>(a.out) + ((size_t)s * HQ + hq) * kRow;
  store_out4<uint16_t>(out_row + d0 * 2, O, 1.f / S);
}

}  // namespace

bool shared_supported(int dtype, int head_dim, int group) {
  return dtype == kBf16 && head_dim == kD && group >= 1 && group <= kSharedPieceRows;
}

hipError_t shared_resident_per_cu(int block_size, int* resident) {
  if (block_size == 16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        resident, reinterpret_cast<const void*>(&decode_shared_kernel<16>), 64, 0);
  if (block_size == 32)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        resident, reinterpret_cast<const void*>(&decode_shared_kernel<32>), 64, 0);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_shared(const DecodeArgs& args, const ShareArgs& sh, int block_size,
                                int workers, hipStream_t stream, hipEvent_t before,
                                hipEvent_t after) {
  DecodeArgs a = args;
  a.heads_per_seg = a.group;
  a.piece_rows = kSharedPieceRows;
  a.seg_cost = kSegCostShared;
  if (block_size == 16)
    hipExtLaunchKernelGGL((decode_shared_kernel<16>), dim3(workers), dim3(64), 0, stream, before,
                          after, 0, a, sh);
  else if (block_size == 32)
    hipExtLaunchKernelGGL((decode_shared_kernel<32>), dim3(workers), dim3(64), 0, stream, before,
                          after, 0, a, sh);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int HPW = merge_heads_per_wave<kD>();
  const int64_t record_waves = (int64_t)workers * ((a.group + HPW - 1) / HPW);
  const int64_t combine_waves = (int64_t)a.num_seqs * ((a.num_q_heads + HPW - 1) / HPW);
  const int64_t waves = record_waves + combine_waves;
  hipLaunchKernelGGL(merge_shared_kernel, dim3((unsigned)((waves + kMergeWaves - 1) / kMergeWaves)),
                     dim3(64 * kMergeWaves), 0, stream, a, sh, workers, (int)record_waves);
  return hipGetLastError();
}

}  // namespace pa
