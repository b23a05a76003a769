// Device helpers shared by the decode kernels of libpa.so (gfx950).
#pragma once

#include "pa_internal.h"

// No implicit a*b+c fusion in files that include this header: a rounded
// score must be the same value in the running maximum and in its exponent
// (so the maximum's weight is exactly 1).  Every intended FMA is fmaf().
#pragma clang fp contract(off)

namespace pa {
namespace dev {


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Read-only index data (block tables) is read through the constant address
// space so that wave-uniform reads become scalar loads: they are counted by
// lgkmcnt, so waiting for a table entry never waits for in-flight tile loads.
typedef const int32_t __attribute__((address_space(4))) const_i32;
typedef const int64_t __attribute__((address_space(4))) const_i64;
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

// Wave-uniform cursor over the chunk line: chunk c is chunk j (of n) of the
// segment (head h, sequence s of length L) that starts at line chunk
// seg_start.
struct Cursor {
  int64_t c;
  int64_t seg_start;
  int h, s, L, n, j;
};

// Moves the cursor to the next chunk of the line, skipping empty sequences.
// Callers never move it past the last chunk of their range.
__device__ __forceinline__ void cursor_next(Cursor& k, const int32_t* lens_ptr, int num_seqs) {
  const const_i32* lens = (const const_i32*)lens_ptr;   // scalar loads (lgkmcnt)
  ++k.c;
  if (++k.j < k.n) return;
  do {
    if (++k.s == num_seqs) {
      k.s = 0;
      ++k.h;
    }
    k.L = lens[k.s];
  } while (k.L == 0);
  k.n = chunks_of(k.L);
  k.j = 0;
  k.seg_start = k.c;
}

// What a tile carries about its chunk, so the consumer can switch segments
// without draining the load pipeline.
struct ChunkMeta {
  int64_t seg_start;
  int64_t slot;      // fused append into this segment's last chunk (< 0: none)
  int h, s, L, n, j;
  bool first;        // first chunk of the segment in this worker's range
  bool last;         // last chunk of the segment in this worker's range
};

__device__ __forceinline__ ChunkMeta chunk_meta(const Cursor& k, int64_t b0, int64_t b1,
                                               const int64_t* slot_mapping) {
  ChunkMeta m;
  m.seg_start = k.seg_start;
  m.h = k.h;
  m.s = k.s;
  m.L = k.L;
  m.n = k.n;
  m.j = k.j;
  m.first = k.c == b0 || k.j == 0;
  m.last = k.c == b1 - 1 || k.j == k.n - 1;
  m.slot = (slot_mapping != nullptr && k.j == k.n - 1)
               ? ((const const_i64*)slot_mapping)[k.s]   // scalar load (lgkmcnt)
               : -1;
  return m;
}

}  // namespace dev
}  // namespace pa
