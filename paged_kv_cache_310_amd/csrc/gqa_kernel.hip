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
// follow the vector kernel (decode_kernel.hip).
#include "decode_common.h"

namespace pa {
namespace {

using namespace dev;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kRow = kD * 2;                 // bytes of one token row (bf16)
constexpr int kTile = kChunk * kRow;         // 4 KiB

// Token (within the chunk) of MFMA row / k-index m.
__device__ __forceinline__ int token_of(int m) { return 4 * (m & 3) + (m >> 2); }

// Sum (or max) of a value over the four lanes that share l%16.
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
  const uint32_t d = v[e >> 1];
  return (e & 1) ? bf_hi(d) : bf_lo(d);
}

template <int BS>
__global__ __launch_bounds__(64, 2) void decode_gqa_kernel(const DecodeArgs a) {
  constexpr int CPB = BS / kChunk;
  static_assert(BS % kChunk == 0, "block size must be a multiple of the chunk");
  const int lane = threadIdx.x;
  const int g4 = lane >> 4;    // lane group 0..3
  const int n = lane & 15;     // query head within the group (MFMA column / row)
  const int nworkers = gridDim.x;
  const int w = (nworkers % kNumXcd) ? (int)blockIdx.x
                                     : (int)(blockIdx.x % kNumXcd) * (nworkers / kNumXcd) +
                                           (int)(blockIdx.x / kNumXcd);
  const int B = a.num_seqs;
  const int HQ = a.num_q_heads;
  const int HKV = a.num_kv_heads;
  const int G = a.group;
  const int32_t* __restrict__ lens = a.context_lens;

  for (int s = w; s < B; s += nworkers) {
    if (lens[s] == 0) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<char*>(a.out) + (size_t)s * HQ * kRow);
      for (int u = lane; u < HQ * (kRow / 16); u += 64) o[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  LineSplit ls;
  if (!split_line(lens, B, HKV, nworkers, w, lane, ls)) {
    if (lane == 0) a.records[w].valid = 0;
    return;
  }
  const int64_t b0 = ls.b0, b1 = ls.b1;
  Cursor cur;
  cur.c = b0;
  locate_segment(lens, B, ls.wseq, b0, lane, cur.h, cur.s, cur.seg_start);
  cur.L = lens[cur.s];
  cur.n = chunks_of(cur.L);
  cur.j = (int)(b0 - cur.seg_start);
  if (lane == 0) {
    MergeRecord r;
    r.W = ls.W;
    r.NW = ls.NW;
    r.seg_start = cur.seg_start;
    r.first = worker_of(cur.seg_start, ls.W, ls.NW);
    r.first_slot = cur.seg_start > r.first * ls.W / ls.NW ? 1 : 0;
    r.seq = cur.s;
    r.head = cur.h;
    r.valid = (cur.seg_start < b0 && cur.seg_start + cur.n <= b1) ? 1 : 0;
    a.records[w] = r;
  }

  const int64_t block_stride = (int64_t)HKV * BS * kRow;
  const bool real_head = n < G;
  const int krow_off = token_of(n) * kRow + g4 * 16;
  auto table_of = [&](const Cursor& k) {
    return (const const_i32*)(a.block_tables + (int64_t)k.s * a.max_blocks_per_seq);
  };
  int next_pb = table_of(cur)[cur.j / CPB];

  struct Tile {
    u32x4 k[4];            // K operand: token token_of(l%16), dims 32c + 8(l/16)
    u32x4 v[4];            // V rows: load i = token 4i + l/16, dims 8(l%16)..+8
    u32x4 q[4];            // Q^T operand of the segment, valid when meta.first
    ChunkMeta meta;
  };

  auto issue = [&](Tile& t) {
    t.meta = chunk_meta(cur, b0, b1, a.slot_mapping);
    const int64_t off = (int64_t)next_pb * block_stride + (int64_t)cur.h * BS * kRow +
                        (int64_t)(cur.j % CPB) * kTile;
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(static_cast<const char*>(a.k_cache) + off, kTile);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(static_cast<const char*>(a.v_cache) + off, kTile);
#pragma unroll
    for (int k = 0; k < 4; ++k) t.k[k] = load16(kr, krow_off + k * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = load16(vr, i * 1024 + lane * 16);
    if (t.meta.first) {
      // head n of the group, dims 32k + 8*g4 .. +8 (padding heads read head 0, zeroed later)
      const __amdgpu_buffer_rsrc_t qr = tile_rsrc(
          static_cast<const char*>(a.q) + ((size_t)cur.s * HQ + cur.h * G) * kRow, G * kRow);
      const int qoff = (real_head ? n : 0) * kRow + g4 * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) t.q[k] = load16(qr, qoff + k * 64);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (cur.c + 1 < b1) {
      cursor_next(cur, lens, B);
      next_pb = table_of(cur)[cur.j / CPB];
    }
  };

  u32x4 qf[4];
  float m = -INFINITY, l = 0.f;
  f32x4_t o[8];

  auto consume = [&](const Tile& t) {
    const ChunkMeta& mt = t.meta;
    if (mt.first) {
#pragma unroll
      for (int k = 0; k < 4; ++k) qf[k] = real_head ? t.q[k] : u32x4{0u, 0u, 0u, 0u};
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int L_pool = mt.slot >= 0 ? mt.L - 1 : mt.L;
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[k]),
                                                      __builtin_bit_cast(bf16x8_t, qf[k]),
                                                      sacc, 0, 0, 0);
    const int base = mt.j * kChunk + g4;   // lane holds tokens base + 4i
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = base + 4 * i < L_pool ? sacc[i] * a.scale_log2 : -INFINITY;
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
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = base + 4 * i < L_pool ? t.v[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
      const int dw = k >> 1;
      const uint32_t lo = __builtin_amdgcn_perm(v[1][dw], v[0][dw], sel);
      const uint32_t hi = __builtin_amdgcn_perm(v[3][dw], v[2][dw], sel);
      const i16x4_t va = __builtin_bit_cast(i16x4_t, (uint64_t)lo | ((uint64_t)hi << 32));
      o[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pop, o[k], 0, 0, 0);
    }
    if (!mt.last) return;

    // ---- end of this worker's part of the segment
    l = group4_sum(l);   // every lane of head n now holds the head's full sum
    if (mt.slot >= 0) {
      // The newest token's rows, read here (once per appended segment).
      const size_t row = ((size_t)mt.s * HKV + mt.h) * kRow;
      const __amdgpu_buffer_rsrc_t knr = tile_rsrc(static_cast<const char*>(a.k_new) + row, kRow);
      const __amdgpu_buffer_rsrc_t vnr = tile_rsrc(static_cast<const char*>(a.v_new) + row, kRow);
      u32x4 kn[4], vn[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) kn[k] = load16(knr, k * 64 + g4 * 16);   // dims 32k + 8*g4
#pragma unroll
      for (int i = 0; i < 4; ++i) vn[i] = load16(vnr, g4 * 64 + i * 16);   // dims 32*g4 + 8i
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) d = dot16<uint16_t>(qf[k], kn[k]) + d;
      const float s_new = group4_sum(d) * a.scale_log2;
      const float mm = fmaxf(m, s_new);
      const float al = fast_exp2(m - mm);
      const float p = fast_exp2(s_new - mm);
      l = l * al + p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k][i] = fmaf(p, bf16_elem(vn[i], k), o[k][i] * al);
      }
      m = mm;
      if (n == 0) {
        // lanes 0, 16, 32, 48 hold every 16-byte piece of both rows
        const int64_t blk = mt.slot / BS;
        const int64_t pos = mt.slot - blk * BS;
        char* krow = static_cast<char*>(a.k_cache) + ((blk * HKV + mt.h) * BS + pos) * kRow;
        char* vrow = static_cast<char*>(a.v_cache) + ((blk * HKV + mt.h) * BS + pos) * kRow;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          *reinterpret_cast<u32x4*>(krow + k * 64 + g4 * 16) = kn[k];
          *reinterpret_cast<u32x4*>(vrow + g4 * 64 + k * 16) = vn[k];
        }
      }
    }
    if (real_head) {
      const bool whole = mt.seg_start >= b0 && mt.seg_start + mt.n <= b1;
      if (whole) {
        char* orow = static_cast<char*>(a.out) + ((size_t)mt.s * HQ + mt.h * G + n) * kRow + g4 * 64;
        const float inv = 1.f / l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float vals[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) vals[k] = o[k][i];
          store_out16<uint16_t>(orow + i * 16, vals, inv);
        }
      } else {
        const int64_t slot = ((int64_t)w * 2 + (mt.seg_start <= b0 ? 0 : 1)) * G + n;
        float* acc = a.partials + slot * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[g4 * 32 + i * 8 + k] = o[k][i];
        }
        if (g4 == 0) {
          float* pair = a.partials + partial_pairs_offset(nworkers, G, kD) + slot * 2;
          pair[0] = m;
          pair[1] = l;
        }
      }
    }
  };

  const int64_t count = b1 - b0;
  Tile ta, tb;
  issue(ta);
  int64_t i = 0;
  for (; i + 2 < count; i += 2) {
    issue(tb);
    consume(ta);
    issue(ta);
    consume(tb);
  }
  if (i + 1 < count) {
    issue(tb);
    consume(ta);
    consume(tb);
  } else {
    consume(ta);
  }
}

}  // namespace

bool gqa_supported(int dtype, int head_dim, int group) {
  return dtype == kBf16 && head_dim == kD && group >= 2 && group <= 16;
}

hipError_t launch_gqa_attention(const DecodeArgs& a, int block_size, int workers,
                                hipStream_t stream, int* resident) {
  if (block_size == 16) {
    if (resident != nullptr)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          resident, reinterpret_cast<const void*>(&decode_gqa_kernel<16>), 64, 0);
    hipLaunchKernelGGL((decode_gqa_kernel<16>), dim3(workers), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  if (block_size == 32) {
    if (resident != nullptr)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          resident, reinterpret_cast<const void*>(&decode_gqa_kernel<32>), 64, 0);
    hipLaunchKernelGGL((decode_gqa_kernel<32>), dim3(workers), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
