// Device helpers shared by the attention kernels of libpa.so (gfx950).
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
typedef int32_t __attribute__((address_space(3))) lds_i32;

// Operand and accumulator types of the 16x16 MFMA instructions.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// A 16x16 MFMA result leaves column n of the output in the four lanes with
// l%16 == n (one per lane group l/16).
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

// Buffer resource for one tile: scalar 48-bit base, byte range [0, bytes).
// Loads through it take a 32-bit per-lane offset and return 0 outside the range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
}
// The same load with the non-temporal hint (`nt`: no reuse expected).  The
// vector kernel reads both K and V tiles this way (+10% for V, then +0.9% on
// the long-context and +1.5% on the OPT-shaped batch for K as well); a batch
// whose sequences share prefix blocks re-reads them through L2 and loses 16%
// with it -- pa_decode_shared reads such blocks once instead.  The
// matrix-core loops keep K cacheable (non-temporal K measured 2.4% slower
// there; the shared-prefix line re-reads a tile once per row block).
__device__ __forceinline__ u32x4 load16_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 2);
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
// Scales EPL accumulators by inv and packs them as 16 bytes of T.
template <typename T>
__device__ __forceinline__ u32x4 pack16(const float* o, float inv);

template <>
__device__ __forceinline__ u32x4 pack16<uint16_t>(const float* o, float inv) {
  u32x4 r;
  r[0] = f32_to_bf16(o[0] * inv) | (f32_to_bf16(o[1] * inv) << 16);
  r[1] = f32_to_bf16(o[2] * inv) | (f32_to_bf16(o[3] * inv) << 16);
  r[2] = f32_to_bf16(o[4] * inv) | (f32_to_bf16(o[5] * inv) << 16);
  r[3] = f32_to_bf16(o[6] * inv) | (f32_to_bf16(o[7] * inv) << 16);
  return r;
}

template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* o, float inv) {
  return u32x4{__float_as_uint(o[0] * inv), __float_as_uint(o[1] * inv),
               __float_as_uint(o[2] * inv), __float_as_uint(o[3] * inv)};
}

__device__ __forceinline__ u32x4 f32x4_bits(float a, float b, float c, float d) {
  return u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
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

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Inclusive prefix sum over the 64 lanes with DPP row operations: shifts
// within each 16-lane row, then the rows' totals broadcast into the rows
// above (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).
// Six VALU steps instead of the LDS-crossbar round trips of a shuffle scan.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_or_zero(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, true);
}
__device__ __forceinline__ int wave_inclusive_scan32(int x) {
  x += dpp_or_zero<0x111, 0xf>(x);   // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);   // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);   // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);   // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);   // row_bcast:15
  x += dpp_or_zero<0x143, 0xc>(x);   // row_bcast:31
  return x;
}

// Lane `src`'s x (src wave-uniform), read with v_readlane: no LDS-crossbar
// round trip, unlike a shuffle.
__device__ __forceinline__ int lane_value(int x, int src) {
  return __builtin_amdgcn_readlane(x, src);
}
__device__ __forceinline__ int64_t lane_value(int64_t x, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)x, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), src);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes: the DPP scan when every value lies
// in [0, 2^24) (the total then stays below 2^31), else the shuffle scan.
__device__ __forceinline__ int64_t wave_scan(int64_t x, int lane) {
  if (__ballot(x < 0 || x >= (1 << 24)) == 0) return wave_inclusive_scan32((int)x);
  return wave_inclusive_scan(x, lane);
}

// Sum over the 64 lanes, on every lane.  When every value lies in [0, 2^24)
// the total stays below 2^31: one DPP scan and a lane read, where the
// shuffle butterfly costs six dependent LDS-crossbar round trips per 32-bit
// half (about 1 us of a short launch's start-up).
__device__ __forceinline__ int64_t wave_sum(int64_t x) {
  if (__ballot(x < 0 || x >= (1 << 24)) == 0)
    return lane_value(wave_inclusive_scan32((int)x), 63);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------------------
// Work split.
//
// The chunk line holds all (head, sequence, 16-token chunk) triples,
// head-major.  Workers get equal shares of work units rather than of chunks:
// a segment costs its chunks plus seg_cost units for what each segment adds
// besides its chunks (the end of the segment, where its output or partial is
// produced, and the switch to the next one), so a worker whose range crosses
// many short segments gets fewer chunks.  A segment's units are its seg_cost
// overhead units followed by one unit per chunk; a worker owns the chunks
// whose units fall in its unit range.  With seg_cost = 0 the split is an
// equal split of chunks.
constexpr int kLenCache = 4096;   // sequences whose lengths are cached in LDS

struct SplitLds {
  int32_t len[kLenCache];         // context length of sequence s
};

struct LineSplit {
  int64_t wseq, useq;   // chunks / units per head
  int64_t W, U;         // chunks / units in the line
  int64_t NW;           // workers with a non-empty unit range: min(workers, U)
  int64_t u0, u1;       // this worker's units
  int64_t b0, b1;       // its chunks [b0, b1)
  int h, s;             // segment holding b0
  int64_t seg_start;    // its first chunk
  int64_t seg_unit;     // its first unit
};

// Length of sequence s: from the LDS cache the split filled, else from memory.
__device__ __forceinline__ int seq_len(const SplitLds& C, const int32_t* lens, int s) {
  return s < kLenCache ? ((const lds_i32*)C.len)[s] : lens[s];
}
__device__ __forceinline__ int seq_chunks(const SplitLds& C, const int32_t* lens, int s) {
  return chunks_of(seq_len(C, lens, s));
}

// Worker that owns unit u of the line [0, U) split over nw workers.
__device__ __forceinline__ int64_t worker_of(int64_t u, int64_t U, int64_t nw) {
  return ((u + 1) * nw + U - 1) / U - 1;
}

// Where unit target r (relative to the start of its head's units) falls:
// the first chunk at or after it and its segment.
struct UnitHit {
  bool found;
  int s;
  int64_t bu, bc;   // units / chunks of the head before sequence s
  int64_t off;      // r - bu
};

// Finds the sequences holding unit targets r0 and r1 (each relative to the
// start of its head's units; every head's units are laid out alike) in one
// pass over the sequences, 64 at a time.  A sequence of n chunks has
// n + seg_cost units (0 when empty).
__device__ void locate_units(const SplitLds& C, const int32_t* lens, int num_seqs, int seg_cost,
                             int64_t r0, int64_t r1, int lane, UnitHit& h0, UnitHit& h1) {
  h0.found = false;
  h1.found = false;
  int64_t acc_u = 0, acc_ne = 0;
  for (int base = 0; base < num_seqs && !(h0.found && h1.found); base += 64) {
    const int sq = base + lane;
    const int n = sq < num_seqs ? seq_chunks(C, lens, sq) : 0;
    const int un = n > 0 ? n + seg_cost : 0;
    const unsigned long long ne = __ballot(n > 0);
    int64_t incl;
    if (__ballot(un >= (1 << 24)) == 0) {
      incl = wave_inclusive_scan32(un);   // the 64 values sum below 2^31
    } else {
      incl = wave_inclusive_scan((int64_t)un, lane);
    }
    const int64_t tot = lane_value(incl, 63);
    auto probe = [&](int64_t r, UnitHit& hit) {
      if (hit.found || r >= acc_u + tot) return;
      const unsigned long long above = __ballot(acc_u + incl > r);
      const int first = __ffsll((long long)above) - 1;
      hit.found = true;
      hit.s = uniform(base + first);
      hit.bu = acc_u + lane_value((int64_t)(incl - un), first);
      const int64_t ne_before = acc_ne + __popcll(ne & ((1ull << first) - 1));
      hit.bc = hit.bu - (int64_t)seg_cost * ne_before;
      hit.off = r - hit.bu;
    };
    probe(r0, h0);
    probe(r1, h1);
    acc_u += tot;
    acc_ne += __popcll(ne);
  }
}

// Computes the split for worker w; false when w has no chunks.  Caches the
// sequences' lengths in C on the way.
// Lane's values v[k] = a[base + 64 k + lane], k < 4 (0 past a[n - 1]): four
// range-checked loads issued together, one memory latency for 256 entries.
__device__ __forceinline__ void load_block256(const int32_t* a, int n, int base, int lane,
                                              int v[4]) {
  const int left = n - base;
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(a + base, (left < 256 ? left : 256) * 4);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    v[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(r, (k * 64 + lane) * 4, 0, 0);
}

__device__ __forceinline__ bool split_line(SplitLds& C, const int32_t* lens, int num_seqs,
                                           int num_heads, int seg_cost, int nworkers, int w,
                                           int lane, LineSplit& ls) {
  int64_t wseq = 0, useq = 0;
  for (int base = 0; base < num_seqs; base += 256) {
    int64_t n = 0, un = 0;
    int Lb[4];
    load_block256(lens, num_seqs, base, lane, Lb);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sq = base + k * 64 + lane;
      if (sq < num_seqs) {
        const int L = Lb[k];
        if (sq < kLenCache) ((lds_i32*)C.len)[sq] = L;
        const int c = chunks_of(L);
        n += c;
        un += c > 0 ? c + seg_cost : 0;
      }
    }
    wseq += uniform(wave_sum(n));
    useq += uniform(wave_sum(un));
  }
  ls.wseq = wseq;
  ls.useq = useq;
  ls.W = wseq * num_heads;
  ls.U = useq * num_heads;
  if (ls.U == 0) return false;
  ls.NW = ls.U < nworkers ? ls.U : nworkers;
  if (w >= ls.NW) return false;
  ls.u0 = (int64_t)w * ls.U / ls.NW;
  ls.u1 = (int64_t)(w + 1) * ls.U / ls.NW;
  // Both ends of the range in one pass; u1 == U is the line's end.
  const int hh0 = (int)(ls.u0 / ls.useq);
  const int hh1 = ls.u1 < ls.U ? (int)(ls.u1 / ls.useq) : 0;
  const int64_t r1 = ls.u1 < ls.U ? ls.u1 - (int64_t)hh1 * ls.useq : ls.U;
  UnitHit x0, x1;
  locate_units(C, lens, num_seqs, seg_cost, ls.u0 - (int64_t)hh0 * ls.useq, r1, lane, x0, x1);
  ls.h = hh0;
  ls.s = x0.s;
  ls.seg_start = (int64_t)hh0 * ls.wseq + x0.bc;
  ls.seg_unit = (int64_t)hh0 * ls.useq + x0.bu;
  ls.b0 = ls.seg_start + (x0.off < seg_cost ? 0 : x0.off - seg_cost);
  ls.b1 = ls.u1 < ls.U ? (int64_t)hh1 * ls.wseq + x1.bc + (x1.off < seg_cost ? 0 : x1.off - seg_cost)
                       : ls.W;
  return ls.b0 < ls.b1;
}

// What the merge kernel needs about the segment holding b0: worker `first`
// holds its first chunk, and the partial slot of the segment's piece there.
__device__ __forceinline__ MergeRecord merge_record(const LineSplit& ls, int seg_cost, int n) {
  MergeRecord r;
  r.W = ls.U;
  r.NW = ls.NW;
  r.seg_start = ls.seg_start;
  r.first = worker_of(ls.seg_unit + seg_cost, ls.U, ls.NW);
  // Slot 1 when worker `first` has chunks (of earlier segments) before this
  // segment: its unit range starts before the segment's first unit.
  r.first_slot = r.first * ls.U / ls.NW < ls.seg_unit ? 1 : 0;
  r.seq = ls.s;
  r.head = ls.h;
  r.valid = (ls.seg_start < ls.b0 && ls.seg_start + n <= ls.b1) ? 1 : 0;
  return r;
}

// Wave-uniform cursor over the chunk line: chunk c is chunk j (of n) of the
// segment (head h, sequence s of length L) that starts at line chunk
// seg_start.  slot is the sequence's fused-append slot (< 0: none), read
// together with L so that a segment switch waits for one scalar load.
struct Cursor {
  int64_t c;
  int64_t seg_start;
  int64_t slot;
  int h, s, L, n, j;
  int j0;   // the segment's first chunk on this line: 0, or on the tail line of a
            // shared-prefix decode the first chunk after the sequence's shared prefix
};

__device__ __forceinline__ int64_t append_slot(const int64_t* slot_mapping, int s) {
  return slot_mapping != nullptr ? ((const const_i64*)slot_mapping)[s] : -1;   // scalar load
}

// Places the cursor on the first chunk of a worker's range.
__device__ __forceinline__ void cursor_start(Cursor& k, const SplitLds& C, const int32_t* lens,
                                             const int64_t* slots, const LineSplit& ls) {
  k.c = ls.b0;
  k.h = ls.h;
  k.s = ls.s;
  k.seg_start = ls.seg_start;
  k.L = uniform(seq_len(C, lens, k.s));
  k.slot = append_slot(slots, k.s);
  k.n = chunks_of(k.L);
  k.j0 = 0;
  k.j = (int)(ls.b0 - k.seg_start);
}

// Moves the cursor to the next chunk of the line, skipping empty sequences.
// Callers never move it past the last chunk of their range.
__device__ __forceinline__ void cursor_next(Cursor& k, const int32_t* lens_ptr,
                                            const int64_t* slots, int num_seqs) {
  const const_i32* lens = (const const_i32*)lens_ptr;   // scalar loads (lgkmcnt)
  ++k.c;
  if (++k.j < k.n) return;
  do {
    if (++k.s == num_seqs) {
      k.s = 0;
      ++k.h;
    }
    k.L = lens[k.s];
    k.slot = append_slot(slots, k.s);
  } while (k.L == 0);
  k.n = chunks_of(k.L);
  k.j0 = 0;
  k.j = 0;
  k.seg_start = k.c;
}

// What a tile carries about its chunk, so the consumer can switch segments
// without draining the load pipeline.  Kept small: every tile in flight
// holds one in scalar registers.
enum ChunkFlags : int {
  kFirst = 1,    // first chunk of the segment in this worker's range
  kLast = 2,     // last chunk of the segment in this worker's range
  kWhole = 4,    // the whole segment lies in this worker's range
  kSecond = 8,   // the segment begins inside the range: partial slot 1
  kGrouped = 16, // tail line: the sequence's shared prefix is attended to elsewhere
};

struct ChunkMeta {
  int64_t slot;  // fused append into the segment, set on its last chunk (< 0: none)
  int h, s;
  int valid;     // cached tokens of the chunk to attend to (0..16)
  int flags;
  __device__ bool first() const { return flags & kFirst; }
  __device__ bool last() const { return flags & kLast; }
  __device__ bool whole() const { return flags & kWhole; }
  __device__ int partial_slot() const { return (flags & kSecond) ? 1 : 0; }
  __device__ bool grouped() const { return flags & kGrouped; }
};

__device__ __forceinline__ ChunkMeta chunk_meta(const Cursor& k, int64_t b0, int64_t b1) {
  ChunkMeta m;
  m.h = k.h;
  m.s = k.s;
  const bool seg_last = k.j == k.n - 1;
  m.flags = ((k.c == b0 || k.j == k.j0) ? kFirst : 0) | ((k.c == b1 - 1 || seg_last) ? kLast : 0) |
            ((k.seg_start >= b0 && k.seg_start + (k.n - k.j0) <= b1) ? kWhole : 0) |
            (k.seg_start > b0 ? kSecond : 0) | (k.j0 > 0 ? kGrouped : 0);
  m.slot = seg_last ? k.slot : -1;
  // The appended token's pool slot is not written yet: it is attended to
  // from k_new/v_new instead.
  const int pool = k.L - (m.slot >= 0 ? 1 : 0) - k.j * kChunk;
  m.valid = pool < kChunk ? pool : kChunk;
  return m;
}

// ---------------------------------------------------------------------------
// The tail line of a shared-prefix decode.  A sequence whose first P tokens
// are shared with the other members of its group has its first
// floor(P / 16) chunks attended to by the group's prefix pass; the tail line
// holds only its remaining chunks.  Per sequence the line's chunk count is
// chunks_of(L) - shared_chunks(L, P) (0: the sequence has no tail segment).

// Chunks of a sequence of length L covered by a shared prefix of P tokens
// (P clamped into [0, L]: an out-of-contract P never reads past the context).
__device__ __forceinline__ int shared_chunks(int L, int P) {
  P = P < 0 ? 0 : (P > L ? L : P);
  return P / kChunk;
}

// Line chunks and units of the tail line (per head), caching each sequence's
// line chunk count in C.len (the split's LDS cache, here holding counts).
__device__ __forceinline__ void tail_line_totals(SplitLds& C, const int32_t* lens,
                                                 const int32_t* prefix_lens, int num_seqs,
                                                 int seg_cost, int lane, int64_t& wseq,
                                                 int64_t& useq) {
  wseq = 0;
  useq = 0;
  for (int base = 0; base < num_seqs; base += 256) {
    int64_t n = 0, un = 0;
    int Lb[4], Pb[4];
    load_block256(lens, num_seqs, base, lane, Lb);
    load_block256(prefix_lens, num_seqs, base, lane, Pb);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sq = base + k * 64 + lane;
      if (sq < num_seqs) {
        const int L = Lb[k];
        const int c = chunks_of(L) - shared_chunks(L, Pb[k]);
        if (sq < kLenCache) ((lds_i32*)C.len)[sq] = c;
        n += c;
        un += c > 0 ? c + seg_cost : 0;
      }
    }
    wseq += uniform(wave_sum(n));
    useq += uniform(wave_sum(un));
  }
}

__device__ __forceinline__ int tail_count(const SplitLds& C, const int32_t* lens,
                                          const int32_t* prefix_lens, int s) {
  if (s < kLenCache) return ((const lds_i32*)C.len)[s];
  const int L = lens[s];
  return chunks_of(L) - shared_chunks(L, prefix_lens[s]);
}

// locate_units over the tail line's per-sequence counts.
__device__ void tail_locate_units(const SplitLds& C, const int32_t* lens,
                                  const int32_t* prefix_lens, int num_seqs, int seg_cost,
                                  int64_t r0, int64_t r1, int lane, UnitHit& h0, UnitHit& h1) {
  h0.found = false;
  h1.found = false;
  int64_t acc_u = 0, acc_ne = 0;
  for (int base = 0; base < num_seqs && !(h0.found && h1.found); base += 64) {
    const int sq = base + lane;
    const int n = sq < num_seqs ? tail_count(C, lens, prefix_lens, sq) : 0;
    const int un = n > 0 ? n + seg_cost : 0;
    const unsigned long long ne = __ballot(n > 0);
    int64_t incl;
    if (__ballot(un >= (1 << 24)) == 0) {
      incl = wave_inclusive_scan32(un);
    } else {
      incl = wave_inclusive_scan((int64_t)un, lane);
    }
    const int64_t tot = lane_value(incl, 63);
    auto probe = [&](int64_t r, UnitHit& hit) {
      if (hit.found || r >= acc_u + tot) return;
      const unsigned long long above = __ballot(acc_u + incl > r);
      const int first = __ffsll((long long)above) - 1;
      hit.found = true;
      hit.s = uniform(base + first);
      hit.bu = acc_u + lane_value((int64_t)(incl - un), first);
      const int64_t ne_before = acc_ne + __popcll(ne & ((1ull << first) - 1));
      hit.bc = hit.bu - (int64_t)seg_cost * ne_before;
      hit.off = r - hit.bu;
    };
    probe(r0, h0);
    probe(r1, h1);
    acc_u += tot;
    acc_ne += __popcll(ne);
  }
}

// The split of the tail line for worker w of nworkers, given its totals per
// head; false when w has no chunks.
__device__ __forceinline__ bool tail_split(const SplitLds& C, const int32_t* lens,
                                           const int32_t* prefix_lens, int num_seqs,
                                           int num_heads, int seg_cost, int64_t wseq,
                                           int64_t useq, int nworkers, int w, int lane,
                                           LineSplit& ls) {
  ls.wseq = wseq;
  ls.useq = useq;
  ls.W = wseq * num_heads;
  ls.U = useq * num_heads;
  if (ls.U == 0) return false;
  ls.NW = ls.U < nworkers ? ls.U : nworkers;
  if (w >= ls.NW) return false;
  ls.u0 = (int64_t)w * ls.U / ls.NW;
  ls.u1 = (int64_t)(w + 1) * ls.U / ls.NW;
  const int hh0 = (int)(ls.u0 / ls.useq);
  const int hh1 = ls.u1 < ls.U ? (int)(ls.u1 / ls.useq) : 0;
  const int64_t r1 = ls.u1 < ls.U ? ls.u1 - (int64_t)hh1 * ls.useq : ls.U;
  UnitHit x0, x1;
  tail_locate_units(C, lens, prefix_lens, num_seqs, seg_cost, ls.u0 - (int64_t)hh0 * ls.useq, r1,
                    lane, x0, x1);
  ls.h = hh0;
  ls.s = x0.s;
  ls.seg_start = (int64_t)hh0 * ls.wseq + x0.bc;
  ls.seg_unit = (int64_t)hh0 * ls.useq + x0.bu;
  ls.b0 = ls.seg_start + (x0.off < seg_cost ? 0 : x0.off - seg_cost);
  ls.b1 = ls.u1 < ls.U ? (int64_t)hh1 * ls.wseq + x1.bc + (x1.off < seg_cost ? 0 : x1.off - seg_cost)
                       : ls.W;
  return ls.b0 < ls.b1;
}

// Places a tail-line cursor on the first chunk of a worker's range.
__device__ __forceinline__ void tail_cursor_start(Cursor& k, const int32_t* lens,
                                                  const int32_t* prefix_lens,
                                                  const int64_t* slots, const LineSplit& ls) {
  k.c = ls.b0;
  k.h = ls.h;
  k.s = ls.s;
  k.seg_start = ls.seg_start;
  k.L = uniform(((const const_i32*)lens)[k.s]);
  k.j0 = uniform(shared_chunks(k.L, ((const const_i32*)prefix_lens)[k.s]));
  k.slot = append_slot(slots, k.s);
  k.n = chunks_of(k.L);
  k.j = k.j0 + (int)(ls.b0 - k.seg_start);
}

// Moves a tail-line cursor to the next chunk, skipping sequences without a tail.
__device__ __forceinline__ void tail_cursor_next(Cursor& k, const int32_t* lens_ptr,
                                                 const int32_t* prefix_ptr, const int64_t* slots,
                                                 int num_seqs) {
  const const_i32* lens = (const const_i32*)lens_ptr;   // scalar loads (lgkmcnt)
  const const_i32* plen = (const const_i32*)prefix_ptr;
  ++k.c;
  if (++k.j < k.n) return;
  do {
    if (++k.s == num_seqs) {
      k.s = 0;
      ++k.h;
    }
    k.L = lens[k.s];
    k.j0 = shared_chunks(k.L, plen[k.s]);
    k.slot = append_slot(slots, k.s);
  } while (chunks_of(k.L) - k.j0 == 0);
  k.n = chunks_of(k.L);
  k.j = k.j0;
  k.seg_start = k.c;
}

// ---------------------------------------------------------------------------
// Deferred stores.
//
// A wave's vector loads and stores complete through one in-order counter
// (vmcnt).  A store issued between tile loads -- an output row at the end of
// a segment -- makes the wait for every tile already in flight also wait for
// the store's acknowledgement, about one memory latency per segment end when
// the memory system is saturated.  Segment ends therefore write their rows to
// a per-wave queue of 1 KiB slots in LDS, and every pipeline step drains
// kQDrain slots with exactly kQDrain store instructions: a step with nothing
// queued stores through a zero-length buffer range, which writes nothing.
// Every step then issues the same loads and stores, and the compiler's waits
// stay exact.  A job is `bytes` (a multiple of 16) contiguous bytes for one
// destination; slot k of it covers bytes [1024k, 1024k + 1024).
constexpr int kQSlots = 16;          // slots per wave (a power of two)
constexpr int kQDrain = 1;           // slots drained per pipeline step

struct QueueLds {
  u32x4 data[kQSlots * 64];          // slot s, lane l: 16 bytes at 1024 s + 16 l
  u32x4 meta[kQSlots];               // (dst low, dst high, bytes, 0)
};

typedef u32x4 __attribute__((address_space(3))) lds_u32x4;

struct StoreQueue {
  lds_u32x4* data;
  lds_u32x4* meta;
  int head, tail;                    // wave-uniform slot counters: [head, tail) queued
};

// LDS of a decode wave: the split's chunk-count cache is dead once the
// worker's range is known, and the store queue is used only after that.
union KernelLds {
  SplitLds split;
  QueueLds queue;
};

__device__ __forceinline__ StoreQueue queue_on(QueueLds& lds) {
  StoreQueue q;
  q.data = (lds_u32x4*)lds.data;
  q.meta = (lds_u32x4*)lds.meta;
  q.head = 0;
  q.tail = 0;
  return q;
}

// One store instruction: the slot at the head, or nothing when the queue is
// empty (`any` is a valid device pointer used as the base of the empty range).
__device__ __forceinline__ void queue_drain_one(StoreQueue& q, int lane, const void* any) {
  // The counters are wave-uniform; reading them through readfirstlane lets
  // the compiler build the store's buffer resource in scalar registers.
  const int head = uniform(q.head);
  const bool have = head < uniform(q.tail);
  const int s = head & (kQSlots - 1);
  const u32x4 mt = q.meta[s];
  const u32x4 v = q.data[s * 64 + lane];
  // readfirstlane yields a signed int: widen each half as unsigned.
  const uint64_t dst = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(mt[1]) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(mt[0]);
  const int bytes = have ? __builtin_amdgcn_readfirstlane(mt[2]) : 0;
  const __amdgpu_buffer_rsrc_t r =
      tile_rsrc(have ? reinterpret_cast<const void*>(dst) : any, bytes);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, lane * 16, 0, 0);
  q.head = head + (have ? 1 : 0);
}

// Reserves `n` (<= kQSlots) consecutive slots, storing synchronously while
// the queue is too full; returns the first.  Wave-uniform control only.
__device__ __forceinline__ int queue_reserve(StoreQueue& q, int n, int lane, const void* any) {
  while (uniform(q.tail) + n - uniform(q.head) > kQSlots) queue_drain_one(q, lane, any);
  const int first = uniform(q.tail);
  q.tail = first + n;
  return first;
}

__device__ __forceinline__ int queue_slots(int bytes) { return (bytes + 1023) >> 10; }

// 16 bytes at byte offset `off` of the job whose first slot is `first`.
__device__ __forceinline__ void queue_put(const StoreQueue& q, int first, int off, const u32x4& v) {
  const int s = (first + (off >> 10)) & (kQSlots - 1);
  q.data[s * 64 + ((off & 1023) >> 4)] = v;
}

// Destination of the job: `bytes` bytes at `dst`.  All lanes call it.
__device__ __forceinline__ void queue_job(const StoreQueue& q, int first, const void* dst,
                                          int bytes, int lane) {
  if (lane < queue_slots(bytes)) {
    const uint64_t d = reinterpret_cast<uint64_t>(dst) + (uint64_t)lane * 1024;
    const int b = bytes - lane * 1024 < 1024 ? bytes - lane * 1024 : 1024;
    q.meta[(first + lane) & (kQSlots - 1)] = u32x4{(uint32_t)d, (uint32_t)(d >> 32), (uint32_t)b, 0u};
  }
}

// Queues a worker's 48-byte merge record (lanes 0..2 carry 16 bytes each).
__device__ __forceinline__ void queue_record(StoreQueue& q, MergeRecord* dst, const MergeRecord& r,
                                             int lane, const void* any) {
  static_assert(sizeof(MergeRecord) == 48, "three 16-byte pieces");
  u32x4 p[3];
  __builtin_memcpy(p, &r, sizeof(p));
  const int f = queue_reserve(q, 1, lane, any);
  const u32x4 mine = lane == 0 ? p[0] : lane == 1 ? p[1] : p[2];
  if (lane < 3) queue_put(q, f, lane * 16, mine);
  queue_job(q, f, dst, (int)sizeof(MergeRecord), lane);
}

// Stores everything still queued (end of the worker's range).
__device__ __forceinline__ void queue_flush(StoreQueue& q, int lane, const void* any) {
  while (uniform(q.head) < uniform(q.tail)) queue_drain_one(q, lane, any);
}

}  // namespace dev
}  // namespace pa
