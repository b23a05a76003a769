// Decode-step paged attention for gfx950 (CDNA4), vector-ALU variant.
//
// What is computed (pages on "Efficient Memory Management for Large Language
// Model Serving with PagedAttention": zeroshotmind.com essay, section "Block
// tables: logical order, physical scatter"; phantomic12.github.io catalogue
// note, method paragraph): for every sequence s and query head h, walk the
// sequence's logical blocks in order, map each through the block table to its
// physical block, gather K/V and compute scaled dot-product attention
//   out[s,h] = sum_j softmax_j(scale * q[s,h] . k_j) v_j,   j < context_lens[s].
//
// How (an MI355X design; the pages give no kernel design):
//  * Work unit: a (query head h, sequence s) "segment" is split into 16-token
//    chunks.  All chunks of all segments, ordered head-major, form one line of
//    W = num_q_heads * sum_s ceil(L_s / 16) chunks.  The grid is persistent:
//    worker w (one 64-lane wavefront) takes chunks [w*W/N, (w+1)*W/N).  Every
//    worker gets the same number of chunks (+-1) whatever the length mix, so
//    heavy-tailed batches need no separate planning kernel: each worker scans
//    context_lens itself at start-up.
//  * A chunk's K tile (16 tokens x head_dim) is 4 KiB for bf16 d128 / fp32 d64
//    and contiguous in the [block, kv_head, slot, dim] pool layout.  It is read
//    as NL coalesced 1 KiB wave loads (16 bytes per lane).  Lane l of load i
//    holds token i*TPL + l/LPT, elements (l%LPT)*EPL .. +EPL.
//  * Scores: bf16 pairs through v_dot2_f32_bf16 (fp32 accumulate), reduced
//    over the LPT lanes of a token with DPP row operations (no LDS).
//  * Online softmax in the exp2 domain, kept per token-row of the wavefront:
//    each row carries its own running max, sum and fp32 accumulator for all
//    head_dim elements, so the P.V update needs no cross-lane traffic.  Rows
//    are merged once per piece.
//  * Loads for chunk j+1 are in flight while chunk j is computed.
//  * A segment that spans two or more workers leaves (max, sum, acc) partials
//    in the workspace and a second, small kernel merges them in worker order.
//    Segments inside one worker are written directly.  (Merging inside the
//    decode launch would need a device-scope release/acquire per partial,
//    which on this multi-XCD part writes back and invalidates the XCD's L2
//    each time; measured, that cost grew with the worker count and halved
//    throughput.)
//  * Workgroup ids are remapped so that consecutive workers run on the same
//    XCD: sequences that share prefix blocks (consecutive in the chunk line)
//    then meet in one L2.
//  * Fused append: the worker that owns a segment's last chunk takes the
//    newest token from k_new/v_new (its pool slot is masked in the loop),
//    and writes it to its slot, which no other worker reads in this launch.
#include "pa_internal.h"

// No implicit a*b+c fusion in this file: a rounded score must be the same
// value in the running maximum and in its exponent (so the maximum's weight
// is exactly 1).  Every intended FMA is written as fmaf().
#pragma clang fp contract(off)

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Read-only index data (block tables) is read through the constant address
// space so that wave-uniform reads become scalar loads: they are counted by
// lgkmcnt, so waiting for a table entry never waits for in-flight tile loads.
typedef const int32_t __attribute__((address_space(4))) const_i32;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for one tile: scalar 48-bit base, byte range [0, bytes).
// Loads through it take a 32-bit per-lane offset and return 0 outside the range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
}

template <typename T, int D>
struct Geo {
  static constexpr int kElt = sizeof(T);
  static constexpr int kRowBytes = D * kElt;    // one token's row for one head
  static constexpr int kLpt = kRowBytes / 16;   // lanes that share one token row
  static constexpr int kTpl = 64 / kLpt;        // token rows per 1 KiB wave load
  static constexpr int kNl = kChunk / kTpl;     // wave loads per 16-token tile
  static constexpr int kEpl = 16 / kElt;        // elements per lane per load
  static_assert(kLpt == 8 || kLpt == 16 || kLpt == 32, "unsupported row size");
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes that hold one token row; every lane of
// the group receives the same value.
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: partner lane ^1
  x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: partner lane ^2
  x += dpp<0x141>(x);   // row_half_mirror: the other quad of the 8-lane half
  if constexpr (LPT >= 16) x += dpp<0x140>(x);   // row_mirror: the other half-row
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);                                   // round to nearest even
  return u >> 16;
}

// Reinterprets a dword as two bf16.  The element is taken by value: clang's
// __builtin_bit_cast applied directly to an ext_vector element lvalue reads
// element 0 whatever the index (seen with the ROCm 7.2 compiler).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// q . k over the 16 bytes a lane holds, accumulated in fp32.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& q, const u32x4& k);

template <>
__device__ __forceinline__ float dot16<uint16_t>(const u32x4& q, const u32x4& k) {
  float acc = 0.f;
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x),
                                        as_bf16x2(k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y),
                                        as_bf16x2(k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z),
                                        as_bf16x2(k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w),
                                        as_bf16x2(k.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<float>(const u32x4& q, const u32x4& k) {
  float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// o[e] += p * v[e] for the EPL elements of one 16-byte piece.
template <typename T>
__device__ __forceinline__ void axpy16(float* o, float p, const u32x4& v);

template <>
__device__ __forceinline__ void axpy16<uint16_t>(float* o, float p, const u32x4& v) {
  o[0] = fmaf(p, bf_lo(v.x), o[0]);
  o[1] = fmaf(p, bf_hi(v.x), o[1]);
  o[2] = fmaf(p, bf_lo(v.y), o[2]);
  o[3] = fmaf(p, bf_hi(v.y), o[3]);
  o[4] = fmaf(p, bf_lo(v.z), o[4]);
  o[5] = fmaf(p, bf_hi(v.z), o[5]);
  o[6] = fmaf(p, bf_lo(v.w), o[6]);
  o[7] = fmaf(p, bf_hi(v.w), o[7]);
}

template <>
__device__ __forceinline__ void axpy16<float>(float* o, float p, const u32x4& v) {
  o[0] = fmaf(p, __uint_as_float(v.x), o[0]);
  o[1] = fmaf(p, __uint_as_float(v.y), o[1]);
  o[2] = fmaf(p, __uint_as_float(v.z), o[2]);
  o[3] = fmaf(p, __uint_as_float(v.w), o[3]);
}

// Writes o * inv as one 16-byte piece of an output row.
template <typename T>
__device__ __forceinline__ void store_out16(void* dst, const float* o, float inv);

template <>
__device__ __forceinline__ void store_out16<uint16_t>(void* dst, const float* o, float inv) {
  uint4 r;
  r.x = f32_to_bf16(o[0] * inv) | (f32_to_bf16(o[1] * inv) << 16);
  r.y = f32_to_bf16(o[2] * inv) | (f32_to_bf16(o[3] * inv) << 16);
  r.z = f32_to_bf16(o[4] * inv) | (f32_to_bf16(o[5] * inv) << 16);
  r.w = f32_to_bf16(o[6] * inv) | (f32_to_bf16(o[7] * inv) << 16);
  *reinterpret_cast<uint4*>(dst) = r;
}

template <>
__device__ __forceinline__ void store_out16<float>(void* dst, const float* o, float inv) {
  float4 r = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  *reinterpret_cast<float4*>(dst) = r;
}

__device__ __forceinline__ int chunks_of(int len) { return (len + kChunk - 1) / kChunk; }

// Values that are equal on every lane, moved to scalar registers so that the
// compiler keeps addresses as scalar base + 32-bit lane offset.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_sum(int64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Worker that owns chunk c of the line [0, W) split over nw workers.
__device__ __forceinline__ int64_t worker_of(int64_t c, int64_t W, int64_t nw) {
  return ((c + 1) * nw + W - 1) / W - 1;
}

// Finds the sequence holding chunk offset r (0 <= r < sum of chunks) and the
// number of chunks before it.
__device__ void locate_sequence(const int32_t* lens, int num_seqs, int64_t r, int lane,
                                int& seq, int64_t& before) {
  int64_t acc = 0;
  for (int base = 0; base < num_seqs; base += 64) {
    const int s = base + lane;
    const int64_t n = s < num_seqs ? chunks_of(lens[s]) : 0;
    const int64_t incl = wave_inclusive_scan(n, lane);
    const int64_t total = uniform((int64_t)__shfl(incl, 63));
    if (r < acc + total) {
      const unsigned long long hit = __ballot(acc + incl > r);
      const int first = __ffsll((long long)hit) - 1;
      seq = uniform(base + first);
      before = uniform((int64_t)(acc + __shfl(incl - n, first)));
      return;
    }
    acc += total;
  }
  seq = num_seqs - 1;   // unreachable for r inside the line
  before = acc;
}

// The chunk line: all (head, sequence, 16-token chunk) triples, head-major,
// split into equal contiguous ranges [b0, b1) over the workers.
struct LineSplit {
  int64_t wseq;   // chunks per head: sum over sequences of ceil(L / 16)
  int64_t W;      // chunks in the line
  int64_t NW;     // workers with a non-empty range: min(workers, W)
  int64_t b0, b1;
};

// Computes the split for worker w; false when w has no chunks.
__device__ __forceinline__ bool split_line(const int32_t* lens, int num_seqs, int num_heads,
                                           int nworkers, int w, int lane, LineSplit& ls) {
  int64_t wseq = 0;
  for (int base = 0; base < num_seqs; base += 256) {
    int64_t n = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = base + k * 64 + lane;
      if (s < num_seqs) n += chunks_of(lens[s]);
    }
    wseq += uniform(wave_sum(n));
  }
  ls.wseq = wseq;
  ls.W = wseq * num_heads;
  if (ls.W == 0) return false;
  ls.NW = ls.W < nworkers ? ls.W : nworkers;
  if (w >= ls.NW) return false;
  ls.b0 = (int64_t)w * ls.W / ls.NW;
  ls.b1 = (int64_t)(w + 1) * ls.W / ls.NW;
  return true;
}

// The segment (head h, sequence s) holding chunk c, and where it starts.
__device__ __forceinline__ void locate_segment(const int32_t* lens, int num_seqs, int64_t wseq,
                                               int64_t c, int lane, int& h, int& s,
                                               int64_t& seg_start) {
  h = (int)(c / wseq);
  int64_t before = 0;
  locate_sequence(lens, num_seqs, c - (int64_t)h * wseq, lane, s, before);
  seg_start = (int64_t)h * wseq + before;
}

template <typename T, int D>
struct Tile {
  u32x4 k[Geo<T, D>::kNl];
  u32x4 v[Geo<T, D>::kNl];
};

// Minimum waves per SIMD the register budget is sized for: two 16-token tiles
// in flight cost 2 * 2 * NL * 4 VGPRs, so the 8 KiB tiles of fp32 d128 get 2.
template <typename T, int D>
constexpr int min_waves() { return Geo<T, D>::kNl >= 8 ? 2 : 4; }

template <typename T, int D, int BS>
__global__ __launch_bounds__(64, (min_waves<T, D>())) void decode_valu_kernel(const DecodeArgs a) {
  using G = Geo<T, D>;
  constexpr int LPT = G::kLpt, TPL = G::kTpl, NL = G::kNl, EPL = G::kEpl, ROW = G::kRowBytes;
  constexpr int CPB = BS / kChunk;   // chunks per block
  static_assert(BS % kChunk == 0, "block size must be a multiple of the chunk");

  const int lane = threadIdx.x;
  const int trow = lane / LPT;   // token row of this lane within a wave load
  const int col = lane % LPT;    // 16-byte piece of that row
  const int nworkers = gridDim.x;
  const int w = (nworkers % kNumXcd) ? (int)blockIdx.x
                                     : (int)(blockIdx.x % kNumXcd) * (nworkers / kNumXcd) +
                                           (int)(blockIdx.x / kNumXcd);
  const int B = a.num_seqs;
  const int HQ = a.num_q_heads;
  const int HKV = a.num_kv_heads;
  const int32_t* __restrict__ lens = a.context_lens;

  // Sequences with no cached token produce zero rows.
  for (int s = w; s < B; s += nworkers) {
    if (lens[s] == 0) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<char*>(a.out) + (size_t)s * HQ * ROW);
      for (int u = lane; u < HQ * LPT; u += 64) o[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  LineSplit ls;
  if (!split_line(lens, B, HQ, nworkers, w, lane, ls)) return;
  const int64_t b0 = ls.b0, b1 = ls.b1;
  int h = 0, s = 0;
  int64_t seg_start = 0;
  locate_segment(lens, B, ls.wseq, b0, lane, h, s, seg_start);
  int L = lens[s];
  int n = chunks_of(L);
  int64_t c = b0;

  const int64_t block_stride = (int64_t)HKV * BS * ROW;

  for (;;) {
    const int64_t seg_end = seg_start + n;
    const int64_t piece_end = seg_end < b1 ? seg_end : b1;
    const int j0 = (int)(c - seg_start);
    const int j1 = (int)(piece_end - seg_start);

    // ---------------------------------------------------------------- piece
    const int kvh = h / a.group;
    const u32x4 qv = load16(tile_rsrc(static_cast<const char*>(a.q) + ((size_t)s * HQ + h) * ROW, ROW),
                            col * 16);
    // Fused append: the worker holding the segment's last chunk owns position
    // L-1.  It masks that position in the pooled tiles, folds the token in from
    // k_new/v_new after the chunk loop and stores it to its slot, so the loop
    // itself has no conditional loads or stores.
    int64_t slot = -1;
    if (a.slot_mapping != nullptr && j1 == n) slot = a.slot_mapping[s];
    const bool app = slot >= 0;
    const int L_pool = app ? L - 1 : L;   // positions read from the pool
    u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
    if (app) {
      const char* knew = static_cast<const char*>(a.k_new) + ((size_t)s * HKV + kvh) * ROW;
      const char* vnew = static_cast<const char*>(a.v_new) + ((size_t)s * HKV + kvh) * ROW;
      kn = load16(tile_rsrc(knew, ROW), col * 16);
      vn = load16(tile_rsrc(vnew, ROW), col * 16);
    }

    const const_i32* tab =
        (const const_i32*)(a.block_tables + (int64_t)s * a.max_blocks_per_seq);
    const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * BS * ROW;
    const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * BS * ROW;

    // Physical block of the next chunk to issue, read one chunk ahead.
    int next_pb = tab[j0 / CPB];

    float m = -INFINITY, l = 0.f;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    auto issue = [&](Tile<T, D>& t, int j) {
      const int pb = next_pb;
      next_pb = tab[(j + 1 < j1 ? j + 1 : j) / CPB];
      const int64_t off = (int64_t)pb * block_stride + (int64_t)(j % CPB) * kChunk * ROW;
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kbase + off, kChunk * ROW);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vbase + off, kChunk * ROW);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        t.k[i] = load16(kr, i * 1024 + lane * 16);
        t.v[i] = load16(vr, i * 1024 + lane * 16);
      }
      // Keep the loads ahead of the math on the other tile.
      __builtin_amdgcn_sched_barrier(0);
    };

    auto consume = [&](const Tile<T, D>& t, int j) {
      float sc[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float dot = row_sum<LPT>(dot16<T>(qv, t.k[i]));
        const int tok = j * kChunk + i * TPL + trow;
        sc[i] = tok < L_pool ? dot * a.scale_log2 : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, sc[i]);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float p = fast_exp2(sc[i] - m_use);
        l += p;
        const bool ok = j * kChunk + i * TPL + trow < L_pool;
        const u32x4 vv = ok ? t.v[i] : u32x4{0u, 0u, 0u, 0u};
        axpy16<T>(o, p, vv);
      }
      m = m_new;
    };

    // Two tiles in ping-pong: the loads of one are in flight while the other
    // is consumed (no register copies, so no wait on the in-flight loads).
    // The steady-state loop issues unconditionally, so every path into a
    // consume has the same loads in flight and the compiler waits only for
    // the tile being consumed; the last one or two chunks are peeled.
    Tile<T, D> ta, tb;
    issue(ta, j0);
    int j = j0;
    for (; j + 2 < j1; j += 2) {
      issue(tb, j + 1);
      consume(ta, j);
      issue(ta, j + 2);
      consume(tb, j + 1);
    }
    if (j + 1 < j1) {
      issue(tb, j + 1);
      consume(ta, j);
      consume(tb, j + 1);
    } else {
      consume(ta, j);
    }

    if (app) {
      // The newest token joins token row 0; its K/V row goes to its slot.
      const float dot = row_sum<LPT>(dot16<T>(qv, kn));
      if (trow == 0) {
        const float sc = dot * a.scale_log2;
        const float m_new = fmaxf(m, sc);
        const float alpha = fast_exp2(m - m_new);
        const float p = fast_exp2(sc - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
        axpy16<T>(o, p, vn);
        m = m_new;
        if (h % a.group == 0) {
          const int64_t blk = slot / BS;
          const int64_t pos = slot - blk * BS;
          const int64_t row_off = ((blk * HKV + kvh) * BS + pos) * ROW + col * 16;
          *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_cache) + row_off) = kn;
          *reinterpret_cast<u32x4*>(static_cast<char*>(a.v_cache) + row_off) = vn;
        }
      }
    }

    // Merge the token rows of the wavefront (lanes with equal col).
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off);
      const float l2 = __shfl_xor(l, off);
      const float mm = fmaxf(m, m2);
      const float mu = mm == -INFINITY ? 0.f : mm;
      const float f1 = fast_exp2(m - mu);
      const float f2 = fast_exp2(m2 - mu);
      l = l * f1 + l2 * f2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[e], off);
        o[e] = o[e] * f1 + o2 * f2;
      }
      m = mm;
    }

    char* out_row = static_cast<char*>(a.out) + ((size_t)s * HQ + h) * ROW;
    if (j0 == 0 && j1 == n) {
      if (lane < LPT) store_out16<T>(out_row + col * 16, o, 1.f / l);
    } else {
      // Partial piece: publish (max, sum, acc); the merge kernel, which runs
      // after this launch, combines the pieces of the segment.
      const int which = seg_start <= b0 ? 0 : 1;
      float* P = a.partials + ((int64_t)w * 2 + which) * a.group * (D + 2);
      if (lane < LPT) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) P[col * EPL + e] = o[e];
      }
      if (lane == 0) {
        P[D] = m;
        P[D + 1] = l;
      }
    }
    // ------------------------------------------------------------ next piece
    c = piece_end;
    if (c >= b1) break;
    do {
      if (++s == B) {
        s = 0;
        ++h;
      }
      L = lens[s];
    } while (L == 0);
    n = chunks_of(L);
    seg_start = c;
  }
}

// Merges the partial pieces of every segment that spans several workers.
// Worker w's wave acts for the segment holding chunk b0 of its range when
// that segment started in an earlier worker and ends inside this range: it
// folds the pieces of workers wa..w in worker order (deterministic) and
// writes the output row.  Runs after the decode launch in stream order, so
// the partials are visible without any in-kernel fence.
template <typename T, int D>
__global__ __launch_bounds__(64) void merge_kernel(const DecodeArgs a) {
  using G = Geo<T, D>;
  constexpr int LPT = G::kLpt, EPL = G::kEpl, ROW = G::kRowBytes;
  const int lane = threadIdx.x;
  const int col = lane % LPT;
  const int w = blockIdx.x;
  LineSplit ls;
  if (!split_line(a.context_lens, a.num_seqs, a.num_q_heads, gridDim.x, w, lane, ls)) return;
  int h = 0, s = 0;
  int64_t seg_start = 0;
  locate_segment(a.context_lens, a.num_seqs, ls.wseq, ls.b0, lane, h, s, seg_start);
  const int64_t seg_end = seg_start + chunks_of(a.context_lens[s]);
  if (!(seg_start < ls.b0 && seg_end <= ls.b1)) return;
  const int64_t wa = worker_of(seg_start, ls.W, ls.NW);
  float M = -INFINITY, S = 0.f;
  float O[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) O[e] = 0.f;
  for (int64_t ww = wa; ww <= w; ++ww) {
    const int64_t bw = ww * ls.W / ls.NW;
    const float* P = a.partials + (ww * 2 + (seg_start <= bw ? 0 : 1)) * a.group * (D + 2);
    const float mp = P[D];
    const float lp = P[D + 1];
    const float mn = fmaxf(M, mp);
    const float fa = fast_exp2(M - mn);
    const float fb = fast_exp2(mp - mn);
    S = S * fa + lp * fb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] = O[e] * fa + P[col * EPL + e] * fb;
    M = mn;
  }
  char* out_row = static_cast<char*>(a.out) + ((size_t)s * a.num_q_heads + h) * ROW;
  if (lane < LPT) store_out16<T>(out_row + col * 16, O, 1.f / S);
}

template <typename T, int D, int BS>
hipError_t launch_variant(const DecodeArgs* a, int workers, hipStream_t stream, int* resident) {
  if (resident != nullptr) {
    // Resident one-wave workgroups per CU for this variant (occupancy query).
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        resident, reinterpret_cast<const void*>(&decode_valu_kernel<T, D, BS>), 64, 0);
  }
  hipLaunchKernelGGL((decode_valu_kernel<T, D, BS>), dim3(workers), dim3(64), 0, stream, *a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || workers == 1) return e;   // one worker never splits a segment
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(workers), dim3(64), 0, stream, *a);
  return hipGetLastError();
}

// Launches the variant, or (resident != nullptr) reports its occupancy.
hipError_t dispatch(const DecodeArgs* a, int dtype, int head_dim, int block_size, int workers,
                    hipStream_t stream, int* resident) {
#define PA_DISPATCH(T, DT, HD, BSZ)                                          \
  if (dtype == DT && head_dim == HD && block_size == BSZ)                    \
    return launch_variant<T, HD, BSZ>(a, workers, stream, resident);
  PA_DISPATCH(uint16_t, kBf16, 128, 16)
  PA_DISPATCH(uint16_t, kBf16, 128, 32)
  PA_DISPATCH(uint16_t, kBf16, 64, 16)
  PA_DISPATCH(uint16_t, kBf16, 64, 32)
  PA_DISPATCH(float, kFp32, 128, 16)
  PA_DISPATCH(float, kFp32, 128, 32)
  PA_DISPATCH(float, kFp32, 64, 16)
  PA_DISPATCH(float, kFp32, 64, 32)
#undef PA_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int workers, hipStream_t stream) {
  return dispatch(&a, dtype, head_dim, block_size, workers, stream, nullptr);
}

hipError_t decode_resident_per_cu(int dtype, int head_dim, int block_size, int* resident) {
  return dispatch(nullptr, dtype, head_dim, block_size, 0, nullptr, resident);
}

}  // namespace pa
