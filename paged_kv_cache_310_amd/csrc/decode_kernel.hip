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
//    in the workspace; the last worker to finish it (device-scope counter)
//    merges them in worker order and writes the output, then resets the
//    counter.  Segments inside one worker are written directly.
//  * Workgroup ids are remapped so that consecutive workers run on the same
//    XCD: sequences that share prefix blocks (consecutive in the chunk line)
//    then meet in one L2.
//  * Fused append: the worker that owns a segment's last chunk reads the
//    newest token from k_new/v_new instead of the pool and writes it to its
//    slot, which no other worker reads in the same launch.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

  // Length of the chunk line.
  int64_t wseq = 0;
  for (int base = 0; base < B; base += 256) {
    int64_t n = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = base + k * 64 + lane;
      if (s < B) n += chunks_of(lens[s]);
    }
    wseq += uniform(wave_sum(n));
  }
  const int64_t W = wseq * HQ;
  if (W == 0) return;
  const int64_t NW = W < nworkers ? W : nworkers;
  if (w >= NW) return;
  const int64_t b0 = (int64_t)w * W / NW;
  const int64_t b1 = (int64_t)(w + 1) * W / NW;

  int h = (int)(b0 / wseq);
  int s = 0;
  int64_t before = 0;
  locate_sequence(lens, B, b0 - (int64_t)h * wseq, lane, s, before);
  int L = lens[s];
  int n = chunks_of(L);
  int64_t seg_start = (int64_t)h * wseq + before;
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
    // Fused append: this worker owns position L-1 when it holds the last chunk.
    int64_t slot = -1;
    if (a.slot_mapping != nullptr && j1 == n) slot = a.slot_mapping[s];
    const bool app = slot >= 0;
    const int app_tok = (L - 1) & (kChunk - 1);
    const char* knew = static_cast<const char*>(a.k_new) + ((size_t)s * HKV + kvh) * ROW;
    const char* vnew = static_cast<const char*>(a.v_new) + ((size_t)s * HKV + kvh) * ROW;

    const int32_t* __restrict__ tab = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int nblk = (L + BS - 1) / BS;
    const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * BS * ROW;
    const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * BS * ROW;

    int win_base = j0 / CPB;   // block-table window: entries win_base .. win_base+63
    int win = (win_base + lane < nblk) ? tab[win_base + lane] : 0;

    float m = -INFINITY, l = 0.f;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    auto issue = [&](Tile<T, D>& t, int j) {
      const int jb = j / CPB;
      if (jb - win_base >= 64) {
        win_base = jb;
        win = (win_base + lane < nblk) ? tab[win_base + lane] : 0;
      }
      const int pb = __builtin_amdgcn_readlane(win, jb - win_base);
      const int64_t off = (int64_t)pb * block_stride + (int64_t)(j % CPB) * kChunk * ROW;
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kbase + off, kChunk * ROW);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vbase + off, kChunk * ROW);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        t.k[i] = load16(kr, i * 1024 + lane * 16);
        t.v[i] = load16(vr, i * 1024 + lane * 16);
      }
      if (app && j == n - 1) {
        // The newest token comes from k_new/v_new, not from its (stale) slot.
        const __amdgpu_buffer_rsrc_t knr = tile_rsrc(knew, ROW);
        const __amdgpu_buffer_rsrc_t vnr = tile_rsrc(vnew, ROW);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if (i * TPL + trow == app_tok) {
            t.k[i] = load16(knr, col * 16);
            t.v[i] = load16(vnr, col * 16);
          }
        }
      }
    };

    auto consume = [&](const Tile<T, D>& t, int j) {
      float sc[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float dot = row_sum<LPT>(dot16<T>(qv, t.k[i]));
        const int tok = j * kChunk + i * TPL + trow;
        sc[i] = tok < L ? dot * a.scale_log2 : -INFINITY;
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
        const bool ok = j * kChunk + i * TPL + trow < L;
        const u32x4 vv = ok ? t.v[i] : u32x4{0u, 0u, 0u, 0u};
        axpy16<T>(o, p, vv);
      }
      m = m_new;
      if (app && j == n - 1 && h % a.group == 0) {
        const int64_t blk = slot / BS;
        const int64_t pos = slot - blk * BS;
        const int64_t row_off = ((blk * HKV + kvh) * BS + pos) * ROW + col * 16;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if (i * TPL + trow == app_tok) {
            *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_cache) + row_off) = t.k[i];
            *reinterpret_cast<u32x4*>(static_cast<char*>(a.v_cache) + row_off) = t.v[i];
          }
        }
      }
    };

    // Two tiles in ping-pong: the loads of one are in flight while the other
    // is consumed (no register copies, so no wait on the in-flight loads).
    Tile<T, D> ta, tb;
    issue(ta, j0);
    for (int j = j0; j < j1; j += 2) {
      if (j + 1 < j1) issue(tb, j + 1);
      consume(ta, j);
      if (j + 1 >= j1) break;
      if (j + 2 < j1) issue(ta, j + 2);
      consume(tb, j + 1);
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
      // Partial piece: publish (max, sum, acc) and let the last arrival merge.
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
      __threadfence();
      const int seg_id = h * B + s;
      int prev = 0;
      if (lane == 0) prev = atomicAdd(a.counters + seg_id, 1);
      prev = uniform(__shfl(prev, 0));
      const int64_t wa = worker_of(seg_start, W, NW);
      const int64_t wb = worker_of(seg_end - 1, W, NW);
      if (prev == wb - wa) {
        __threadfence();
        float M = -INFINITY, S = 0.f;
        float O[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) O[e] = 0.f;
        for (int64_t ww = wa; ww <= wb; ++ww) {
          const int64_t bw = ww * W / NW;
          const float* Pp = a.partials + (ww * 2 + (seg_start <= bw ? 0 : 1)) * a.group * (D + 2);
          const float mp = Pp[D];
          const float lp = Pp[D + 1];
          const float mn = fmaxf(M, mp);
          const float fa = fast_exp2(M - mn);
          const float fb = fast_exp2(mp - mn);
          S = S * fa + lp * fb;
#pragma unroll
          for (int e = 0; e < EPL; ++e) O[e] = O[e] * fa + Pp[col * EPL + e] * fb;
          M = mn;
        }
        if (lane < LPT) store_out16<T>(out_row + col * 16, O, 1.f / S);
        if (lane == 0) a.counters[seg_id] = 0;
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

template <typename T, int D, int BS>
hipError_t launch_variant(const DecodeArgs* a, int workers, hipStream_t stream, int* resident) {
  if (resident != nullptr) {
    // Resident one-wave workgroups per CU for this variant (occupancy query).
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        resident, reinterpret_cast<const void*>(&decode_valu_kernel<T, D, BS>), 64, 0);
  }
  hipLaunchKernelGGL((decode_valu_kernel<T, D, BS>), dim3(workers), dim3(64), 0, stream, *a);
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
