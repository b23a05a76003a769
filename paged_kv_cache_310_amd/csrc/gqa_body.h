// Decode-step paged attention for grouped query heads (group 2..16, bf16,
// head_dim 128) on the gfx950 matrix cores.
//
// What is computed is the same as the vector kernel (pages on "Efficient
// Memory Management for Large Language Model Serving with PagedAttention":
// zeroshotmind.com essay, "Block tables: logical order, physical scatter"):
// attention of every query head over its sequence's cached keys/values,
// gathered through the block table.  With grouped queries the `group` query
// heads of one KV head share every K/V tile, so one wave handles a
// (KV head, sequence) segment and all its query heads at once: the products
// are small dense matrices and go to MFMA.
//
// Per 16-token chunk (one 4 KiB K tile and one 4 KiB V tile):
//  * S^T[16 tokens x 16 heads] = K[16 x 128] . Q^T[128 x 16] with four
//    v_mfma_f32_16x16x32_bf16 (32 dims each).  MFMA lane l supplies row
//    l%16 and k-values 8*(l/16)..+8, and receives rows 4*(l/16)+i, column
//    l%16.  Row m of the K operand is token t(m) = 4*(m%4) + m/4, so lane l
//    ends up holding the scores of tokens 4i + l/16 (i = 0..3) for query
//    head l%16 -- exactly the layout the P.V product wants for P^T.
//  * O^T[128 dims x 16 heads] += V^T . P^T with eight
//    v_mfma_f32_16x16x16bf16_1k (16 tokens each).  The V tile is read with
//    the same coalesced 1 KiB wave loads as the vector kernel (lane l, load
//    i: token 4i + l/16, dims 8*(l%16)..+8); the A operand of MFMA c is the
//    c-th bf16 of those four loads, repacked in registers with v_perm_b32,
//    so MFMA c produces dims 8*m + c.  No LDS is used.
//  * Lane l accumulates the 32 contiguous dims 32*(l/16)..+32 of query head
//    l%16; the online softmax of head n is kept in the four lanes with
//    l%16 = n, its running max agreed on with two permlane swaps per chunk.
//    P is rounded to bf16 for the MFMA, and the softmax sum adds the same
//    rounded weights, so numerator and denominator stay consistent.
// The work split, cross-segment pipeline, fused append and partial pieces
// follow the vector kernel (decode_kernel.hip).  This header holds the worker
// loop; gqa_kernel.hip runs it over every (KV head, sequence) segment, and
// shared_kernel.hip over the tails of sequences that share a prefix.
#pragma once

#include "decode_common.h"

namespace pa {
namespace dev {

constexpr int kD = 128;
constexpr int kRow = kD * 2;                 // bytes of one token row (bf16)
constexpr int kTile = kChunk * kRow;         // 4 KiB

// Token (within the chunk) of MFMA row / k-index m.
__device__ __forceinline__ int token_of(int m) { return 4 * (m & 3) + (m >> 2); }


// The 16 bytes lane `src` holds (ds_bpermute, one dword at a time).
__device__ __forceinline__ u32x4 lane_fetch16(const u32x4& v, int src) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)v[j]);
  return r;
}

__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
  const uint32_t d = v[e >> 1];
  return (e & 1) ? bf_hi(d) : bf_lo(d);
}

// Tiles per wave: one consumed while the others are in flight.  A third
// tile measured no faster.
constexpr int kRing = 2;

// The worker loop over the chunks [ls.b0, ls.b1) of a line of (KV head,
// sequence) segments.  `w` is the worker's index in the launch (its merge
// record and partial slots), `wbase` the launch index of the line's worker 0.
// kTail: the line is the tail line of a shared-prefix decode -- segments start
// after their sequence's shared prefix, and a segment of a sequence with a
// shared prefix leaves its result (whole: a row of res_tail; split: pieces)
// with a locator entry instead of writing `out`.
template <int BS, bool kTail>
__device__ __forceinline__ void gqa_body(const DecodeArgs& a, const ShareArgs& sh, KernelLds& lds,
                                         const LineSplit& ls, int w, int wbase) {
  constexpr int CPB = BS / kChunk;
  static_assert(BS % kChunk == 0, "block size must be a multiple of the chunk");
  const int lane = threadIdx.x;
  const int g4 = lane >> 4;    // lane group 0..3
  const int n = lane & 15;     // query head within the group (MFMA column / row)
  const int B = a.num_seqs;
  const int HQ = a.num_q_heads;
  const int HKV = a.num_kv_heads;
  const int G = a.group;
  const int32_t* __restrict__ lens = a.context_lens;

  const int64_t b0 = ls.b0, b1 = ls.b1;
  Cursor cur;
  if constexpr (kTail)
    tail_cursor_start(cur, lens, sh.prefix_lens, a.slot_mapping, ls);
  else
    cursor_start(cur, lds.split, lens, a.slot_mapping, ls);

  const int64_t block_stride = (int64_t)HKV * BS * kRow;
  const bool real_head = n < G;
  const int krow_off = token_of(n) * kRow + g4 * 16;
  // Padding heads (n >= G) read past the group's rows: the buffer returns 0.
  const int qoff = n * kRow + g4 * 16;
  auto table_of = [&](const Cursor& k) {
    return (const const_i32*)(a.block_tables + (int64_t)k.s * a.max_blocks_per_seq);
  };
  int next_pb = table_of(cur)[cur.j / CPB];

  struct Tile {
    u32x4 k[4];            // K operand: token token_of(l%16), dims 32c + 8(l/16)
    u32x4 v[4];            // V rows: load i = token 4i + l/16, dims 8(l%16)..+8
    u32x4 q[4];            // Q^T operand: head l%16, dims 32c + 8(l/16)
    u32x4 kn, vn;          // newest token's K/V rows (fused append): lane l holds bytes
                           // 16 (l%16)..+16, valid when meta.slot >= 0
    ChunkMeta meta;
  };

  StoreQueue q = queue_on(lds.queue);
  // This worker closes the split segment holding b0 if the segment began in
  // an earlier worker and ends inside this range.  The record goes out
  // through the store queue: a plain store ahead of the first tile would make
  // the first tile's wait include its acknowledgement.
  MergeRecord rec = merge_record(ls, a.seg_cost, cur.n - cur.j0);
  rec.first += wbase;
  if constexpr (kTail) {
    if (rec.valid && cur.j0 > 0) {
      // The split segment is the tail of a sequence with a shared prefix:
      // the merge folds its pieces with the prefix part, found through this
      // locator, instead of through the record.
      const int f = queue_reserve(q, 1, lane, a.out);
      if (lane == 0)
        queue_put(q, f, 0, u32x4{(uint32_t)rec.first, (uint32_t)(w - rec.first + 1),
                                 (uint32_t)rec.first_slot, 0u});
      queue_job(q, f, sh.loc_tail + ((int64_t)ls.h * B + ls.s) * 4, 16, lane);
      rec.valid = 0;
    }
  }
  queue_record(q, a.records + w, rec, lane, a.out);

  // Every tile issues the same tile loads, and one of the ring's issue sites
  // the queue's store (a fixed pattern keeps the compiler's in-order wait
  // counts exact).  Rows past the chunk's
  // valid tokens lie outside the tile's buffer range and read as 0.  Loads
  // that only some tiles make go first: a wait count that assumes they were
  // not issued then waits for them, not for this tile.  These are the group's
  // q rows, loaded with the first tile of each segment (the other tiles copy
  // them from the tile issued before: one load of q per segment instead of
  // one per tile measured 6% faster), and the newest token's rows, loaded
  // with a segment's last chunk.  Past the end of the range the cursor stays
  // on the last chunk: such issues reload it and are never consumed.
  int q_s = -1, q_h = -1;   // segment whose q the last issued tile holds
  auto issue = [&](Tile& t, const Tile& prev, bool drain) {
    t.meta = chunk_meta(cur, b0, b1);
    if (cur.s != q_s || cur.h != q_h) {
      const __amdgpu_buffer_rsrc_t qr = tile_rsrc(
          static_cast<const char*>(a.q) + ((size_t)cur.s * HQ + cur.h * G) * kRow, G * kRow);
#pragma unroll
      for (int k = 0; k < 4; ++k) t.q[k] = load16(qr, qoff + k * 64);
      q_s = cur.s;
      q_h = cur.h;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) t.q[k] = prev.q[k];
    }
    if (t.meta.slot >= 0) {
      const size_t row = ((size_t)cur.s * HKV + cur.h) * kRow;
      const __amdgpu_buffer_rsrc_t knr = tile_rsrc(static_cast<const char*>(a.k_new) + row, kRow);
      const __amdgpu_buffer_rsrc_t vnr = tile_rsrc(static_cast<const char*>(a.v_new) + row, kRow);
      t.kn = load16(knr, n * 16);
      t.vn = load16(vnr, n * 16);
    }
    const int64_t off = (int64_t)next_pb * block_stride + (int64_t)cur.h * BS * kRow +
                        (int64_t)(cur.j % CPB) * kTile;
    const int bytes = uniform((t.meta.valid > 0 ? t.meta.valid : 0) * kRow);
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(static_cast<const char*>(a.k_cache) + off, bytes);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(static_cast<const char*>(a.v_cache) + off, bytes);
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
      if constexpr (kTail)
        tail_cursor_next(cur, lens, sh.prefix_lens, a.slot_mapping, B);
      else
        cursor_next(cur, lens, a.slot_mapping, B);
      next_pb = table_of(cur)[cur.j / CPB];
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4_t o[8];

  auto consume = [&](const Tile& t) {
    const ChunkMeta& mt = t.meta;
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
    if (mt.valid < kChunk) {   // the segment's last chunk: lane holds tokens g4 + 4i
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = g4 + 4 * i < mt.valid ? sc[i] : -INFINITY;
    }
    const float mx = group4_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    if (__ballot(alpha != 1.f)) {       // rescale only when some running max moved
      l *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
    }
    m = m_new;
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (__bf16)fast_exp2(sc[i] - m_use);
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

    // ---- end of this worker's part of the segment
    l = group4_sum(l);   // every lane of head n now holds the head's full sum
    if (mt.slot >= 0) {
      // Pieces of the newest rows this lane needs, from the lanes of its
      // group that hold them: K dims 32k + 8 g4 (piece 4k + g4) for the
      // score, V dims 32 g4 + 8i (piece 4 g4 + i) for the accumulator.
      const int group_base = lane & 48;
      u32x4 kq[4], vq[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) kq[k] = lane_fetch16(t.kn, group_base + 4 * k + g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) vq[i] = lane_fetch16(t.vn, group_base + 4 * g4 + i);
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) d = dot16<uint16_t>(t.q[k], kq[k]) + d;
      const float s_new = group4_sum(d) * a.scale_log2;
      const float mm = fmaxf(m, s_new);
      const float al = fast_exp2(m - mm);
      const float p = fast_exp2(s_new - mm);
      l = l * al + p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k][i] = fmaf(p, bf16_elem(vq[i], k), o[k][i] * al);
      }
      m = mm;
      // Its K/V rows go to its pool slot: lanes 0..15 hold every 16-byte
      // piece of both.
      const int64_t blk = mt.slot / BS;
      const int64_t pos = mt.slot - blk * BS;
      const int64_t row_off = ((blk * HKV + mt.h) * BS + pos) * kRow;
      const int f = queue_reserve(q, 2, lane, a.out);
      if (g4 == 0) {
        queue_put(q, f, n * 16, t.kn);
        queue_put(q, f + 1, n * 16, t.vn);
      }
      queue_job(q, f, static_cast<char*>(a.k_cache) + row_off, kRow, lane);
      queue_job(q, f + 1, static_cast<char*>(a.v_cache) + row_off, kRow, lane);
    }
    // A tail segment of a sequence with a shared prefix keeps its result
    // for the fold with the prefix part.
    const bool keep = kTail && mt.grouped() && mt.whole();
    if (mt.whole() && !keep) {
      // Output rows of the group's heads: G x 256 contiguous bytes.
      const int bytes = G * kRow;
      const int f = queue_reserve(q, queue_slots(bytes), lane, a.out);
      if (real_head) {
        const float inv = 1.f / l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float vals[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) vals[k] = o[k][i];
          queue_put(q, f, n * kRow + g4 * 64 + i * 16, pack16<uint16_t>(vals, inv));
        }
      }
      queue_job(q, f, static_cast<char*>(a.out) + ((size_t)mt.s * HQ + mt.h * G) * kRow, bytes,
                lane);
    } else {
      // Partial pieces (acc, max, sum) of the group's heads for the merge
      // kernel -- or the kept result rows -- : lane (n, g4) holds dims
      // 32 g4 + 8i + k as o[k][i].
      constexpr int REC = kD + kPartialExtra;
      const int bytes = G * REC * 4;
      const int f = queue_reserve(q, queue_slots(bytes), lane, a.out);
      if (real_head) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int off = (n * REC + g4 * 32 + i * 8) * 4;
          queue_put(q, f, off, f32x4_bits(o[0][i], o[1][i], o[2][i], o[3][i]));
          queue_put(q, f, off + 16, f32x4_bits(o[4][i], o[5][i], o[6][i], o[7][i]));
        }
        if (g4 == 0) queue_put(q, f, (n * REC + kD) * 4, f32x4_bits(m, l, 0.f, 0.f));
      }
      float* dst = keep ? sh.res_tail + ((int64_t)mt.h * B + mt.s) * G * REC
                        : a.partials + ((int64_t)w * 2 + mt.partial_slot()) * a.piece_rows * REC;
      queue_job(q, f, dst, bytes, lane);
      if (keep) {
        const int fl = queue_reserve(q, 1, lane, a.out);
        if (lane == 0) queue_put(q, fl, 0, u32x4{(uint32_t)w, 0u, 0u, 0u});
        queue_job(q, fl, sh.loc_tail + ((int64_t)mt.h * B + mt.s) * 4, 16, lane);
      }
    }
  };

  // Ring of kRing tiles: kRing - 1 in flight while one is consumed.  All
  // issues are unconditional, so every consume sees the same loads in flight.
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

}  // namespace dev
}  // namespace pa
