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
#include "merge_body.h"

namespace pa {
namespace {

using namespace dev;

// Register budget: at least 2 waves per SIMD (256 VGPRs).  The default is
// one worker per SIMD, so the budget goes to keeping two tiles, the segment's
// q and the fused-append row in registers rather than to occupancy.
template <typename T, int D>
constexpr int min_waves() { return 2; }

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

  LineSplit ls;
  __shared__ KernelLds lds;
  const bool has_chunks = split_line(lds.split, lens, B, HQ, a.seg_cost, nworkers, w, lane, ls);
  // Sequences with no cached token produce zero rows (lengths from the
  // split's LDS cache).
  for (int s = w; s < B; s += nworkers) {
    if (seq_len(lds.split, lens, s) == 0) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<char*>(a.out) + (size_t)s * HQ * ROW);
      for (int u = lane; u < HQ * LPT; u += 64) o[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (!has_chunks) {
    if (lane == 0) a.records[w].valid = 0;
    return;
  }
  const int64_t b0 = ls.b0, b1 = ls.b1;
  Cursor cur;
  cursor_start(cur, lds.split, lens, a.slot_mapping, ls);

  const int64_t block_stride = (int64_t)HKV * BS * ROW;
  auto table_of = [&](const Cursor& k) {
    return (const const_i32*)(a.block_tables + (int64_t)k.s * a.max_blocks_per_seq);
  };
  // Physical block of the chunk under the cursor, read one chunk ahead.
  int next_pb = table_of(cur)[cur.j / CPB];

  struct Tile {
    u32x4 k[NL], v[NL];
    u32x4 q;        // valid when meta.first
    u32x4 kn, vn;   // valid when meta.slot >= 0 (the newest token of the segment)
    ChunkMeta meta;
  };

  StoreQueue q = queue_on(lds.queue);
  // This worker closes the split segment holding b0 if the segment began in
  // an earlier worker and ends inside this range.  The record goes out
  // through the store queue: a plain store ahead of the first tile would make
  // the first tile's wait include its acknowledgement.
  queue_record(q, a.records + w, merge_record(ls, a.seg_cost, cur.n), lane, a.out);

  // Loads the chunk under the cursor, drains kQDrain queued store slots (at
  // one of the ring's two issue sites: the pattern of memory operations stays
  // fixed), then moves the cursor (unless it is on the range's last chunk)
  // and prefetches the next chunk's block number.  The conditional loads go
  // first: if the compiler's in-order wait count assumes they were not
  // issued, the extra wait falls on them, not on this tile's K/V loads.
  auto issue = [&](Tile& t, bool drain) {
    t.meta = chunk_meta(cur, b0, b1);
    const int kvh = cur.h / a.group;
    if (t.meta.slot >= 0) {
      const size_t row = ((size_t)cur.s * HKV + kvh) * ROW;
      t.kn = load16(tile_rsrc(static_cast<const char*>(a.k_new) + row, ROW), col * 16);
      t.vn = load16(tile_rsrc(static_cast<const char*>(a.v_new) + row, ROW), col * 16);
    }
    if (t.meta.first())
      t.q = load16(tile_rsrc(static_cast<const char*>(a.q) + ((size_t)cur.s * HQ + cur.h) * ROW,
                             ROW), col * 16);
    const int64_t off = (int64_t)next_pb * block_stride + (int64_t)kvh * BS * ROW +
                        (int64_t)(cur.j % CPB) * kChunk * ROW;
    const __amdgpu_buffer_rsrc_t kr =
        tile_rsrc(static_cast<const char*>(a.k_cache) + off, kChunk * ROW);
    const __amdgpu_buffer_rsrc_t vr =
        tile_rsrc(static_cast<const char*>(a.v_cache) + off, kChunk * ROW);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      t.k[i] = load16_stream(kr, i * 1024 + lane * 16);
      t.v[i] = load16_stream(vr, i * 1024 + lane * 16);
    }
    if (drain) {
#pragma unroll
      for (int d = 0; d < kQDrain; ++d) queue_drain_one(q, lane, a.out);
    }
    // Keep the loads ahead of the math on the other tile.
    __builtin_amdgcn_sched_barrier(0);
    if (cur.c + 1 < b1) {
      cursor_next(cur, lens, a.slot_mapping, B);
      next_pb = table_of(cur)[cur.j / CPB];
    }
  };

  // Consumer state of the segment being accumulated.
  u32x4 qv = {0u, 0u, 0u, 0u};
  float m = -INFINITY, l = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  auto consume = [&](const Tile& t) {
    const ChunkMeta& mt = t.meta;
    if (mt.first()) {
      qv = t.q;
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    }
    // Tokens past mt.valid (beyond the sequence, or the newest token whose
    // pool slot is stale in a fused append: it is added from k_new/v_new
    // below) are masked.
    float sc[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float dot = row_sum<LPT>(dot16<T>(qv, t.k[i]));
      sc[i] = trow + i * TPL < mt.valid ? dot * a.scale_log2 : -INFINITY;
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
      const u32x4 vv = trow + i * TPL < mt.valid ? t.v[i] : u32x4{0u, 0u, 0u, 0u};
      axpy16<T>(o, p, vv);
    }
    m = m_new;
    if (!mt.last()) return;

    // ---- end of this worker's part of the segment
    const int kvh = mt.h / a.group;
    if (mt.slot >= 0) {
      // The newest token joins token row 0.
      const float dot = row_sum<LPT>(dot16<T>(qv, t.kn));
      if (trow == 0) {
        const float s_new = dot * a.scale_log2;
        const float mm = fmaxf(m, s_new);
        const float al = fast_exp2(m - mm);
        const float p = fast_exp2(s_new - mm);
        l = l * al + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= al;
        axpy16<T>(o, p, t.vn);
        m = mm;
      }
      if (mt.h % a.group == 0) {
        // Its K/V rows go to its pool slot, once per KV head (by the
        // group's first query head).
        const int64_t blk = mt.slot / BS;
        const int64_t pos = mt.slot - blk * BS;
        const int64_t row_off = ((blk * HKV + kvh) * BS + pos) * ROW;
        const int f = queue_reserve(q, 2, lane, a.out);
        if (lane < LPT) {
          queue_put(q, f, col * 16, t.kn);
          queue_put(q, f + 1, col * 16, t.vn);
        }
        queue_job(q, f, static_cast<char*>(a.k_cache) + row_off, ROW, lane);
        queue_job(q, f + 1, static_cast<char*>(a.v_cache) + row_off, ROW, lane);
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
    const int f = queue_reserve(q, 1, lane, a.out);
    if (mt.whole()) {
      if (lane < LPT) queue_put(q, f, col * 16, pack16<T>(o, 1.f / l));
      queue_job(q, f, static_cast<char*>(a.out) + ((size_t)mt.s * HQ + mt.h) * ROW, ROW, lane);
    } else {
      // Partial piece: (acc, max, sum) for the merge kernel, which combines
      // the pieces after this launch.
      constexpr int REC = D + kPartialExtra;
      if (lane < LPT) {
#pragma unroll
        for (int u = 0; u < EPL / 4; ++u)
          queue_put(q, f, (col * EPL + 4 * u) * 4,
                    f32x4_bits(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]));
      }
      if (lane == 0) queue_put(q, f, D * 4, f32x4_bits(m, l, 0.f, 0.f));
      queue_job(q, f, a.partials + ((int64_t)w * 2 + mt.partial_slot()) * a.piece_rows * REC, REC * 4,
                lane);
    }
  };

  // Two tiles in ping-pong over the whole range.  Every issue is
  // unconditional -- past the range's end the cursor stays on its last chunk,
  // and such issues are never consumed -- so every consume sees the same
  // loads in flight and segment switches never drain the pipeline.
  const int64_t count = b1 - b0;
  Tile t[2];
  issue(t[0], false);
  for (int64_t i = 0; i < count; i += 2) {
    issue(t[1], true);
    consume(t[0]);
    if (i + 1 >= count) break;
    issue(t[0], false);
    consume(t[1]);
  }
  queue_flush(q, lane, a.out);
}

// Merges the partial pieces of every segment that spans several workers.
// One wave per (decode worker, group of merge_heads_per_wave query heads of
// its segment); each lane owns 4 dims of one head.  A worker that closes a split
// segment (its MergeRecord is valid) folds the pieces of workers first..w in
// worker order, kBatch pieces per batch: the batch's accumulator rows and
// (max, sum) pairs are all loaded before any is used, with a running max
// across batches, so a segment of up to kBatch pieces costs one memory
// latency after the record.  The fold order is fixed for a given worker
// count, so results are deterministic.  Runs after
// the decode launch in stream order: the partials are visible without any
// in-kernel fence.
// Pieces loaded together: 8 keeps the merge's registers low for batches of
// many segments, which have few pieces each.  When the workers average
// kMergeWideFrom or more pieces per segment (few sequences and KV heads,
// where the worker cap leaves up to 64 per segment), merge_wide_kernel folds
// each segment with a whole workgroup instead.
constexpr int kMergeBatch = 8;
constexpr int kMergeWideFrom = 16;

// Merge workgroups are placed on the XCD that ran the decode workers whose
// records they fold: the attention launch puts workers
// [x * workers / 8, (x + 1) * workers / 8) on XCD x, so a segment's pieces,
// written by consecutive workers, and its record are still in that XCD's L2
// (when the worker count divides evenly; otherwise workgroups go in order).
// Measured interleaved: one 64/8-head sequence 16.6 -> 15.6 us per step at 4k
// and 33.5 -> 31.7 at 32k; the batched workloads unchanged, outputs identical.
template <typename T, int D, int kBatch>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const DecodeArgs a, int workers) {
  const int lane = threadIdx.x % 64;
  constexpr int HPW = merge_heads_per_wave<D>();
  const int wpr = (a.heads_per_seg + HPW - 1) / HPW;   // waves per record
  const int xw = workers / kNumXcd * wpr;              // waves per XCD
  const bool by_xcd = workers % kNumXcd == 0 && xw % kMergeWaves == 0;
  const int id = uniform(by_xcd ? (int)(blockIdx.x % kNumXcd) * xw +
                                      (int)(blockIdx.x / kNumXcd) * kMergeWaves +
                                      (int)(threadIdx.x / 64)
                                : (int)(blockIdx.x * kMergeWaves + threadIdx.x / 64));
  merge_record_wave<T, D, kBatch>(a, workers, id, lane);
}

// The merge for segments of many pieces (few sequences and heads, where the
// worker cap allows up to 64 pieces per segment): one 4-wave workgroup per
// (closing worker, head group).  Wave i folds a quarter of the segment's
// pieces, all its loads in flight together (kWideBatch at a time), and the
// four partial (max, sum, acc) results are combined through LDS.  The fold
// order is fixed for a given worker count, so results are deterministic.
constexpr int kWideBatch = 16;
template <typename T, int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_wide_kernel(const DecodeArgs a,
                                                                      int workers) {
  constexpr int LPH = D / 4;                       // lanes per head
  constexpr int HPW = merge_heads_per_wave<D>();   // heads per wave
  __shared__ float4 s_acc[kMergeWaves][64];
  __shared__ float2 s_ms[kMergeWaves][64];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int hps = a.heads_per_seg;
  const int wpr = (hps + HPW - 1) / HPW;           // head groups per record
  // One workgroup per (record, head group), placed by XCD as in merge_kernel.
  const int id = workers % kNumXcd == 0
                     ? (int)(blockIdx.x % kNumXcd) * (workers / kNumXcd * wpr) +
                           (int)(blockIdx.x / kNumXcd)
                     : (int)blockIdx.x;
  const int w = id / wpr;
  if (w >= workers) return;                        // whole workgroup
  typedef __attribute__((address_space(4))) const MergeRecord const_record;
  const const_record* r = (const const_record*)a.records + w;   // scalar loads
  if (!r->valid) return;                           // whole workgroup
  const int64_t first = r->first;
  const int first_slot = r->first_slot;
  const int g = (id - w * wpr) * HPW + lane / LPH;
  const bool active = g < hps;
  const int d0 = (lane % LPH) * 4;
  const int R = a.piece_rows;
  constexpr int REC = D + kPartialExtra;
  const int npieces = w - (int)first + 1;
  const int share = (npieces + kMergeWaves - 1) / kMergeWaves;
  const int p_lo = min(npieces, wave * share);
  const int p_hi = min(npieces, p_lo + share);
  float M = -INFINITY, S = 0.f;
  float O[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = p_lo; p0 < p_hi; p0 += kWideBatch) {
    float4 ob[kWideBatch];
    float2 mb[kWideBatch];
#pragma unroll
    for (int b = 0; b < kWideBatch; ++b) {
      const int p = p0 + b;
      if (active && p < p_hi) {
        const int64_t slot = ((first + p) * 2 + (p == 0 ? first_slot : 0)) * R + g;
        const float* rec = a.partials + slot * REC;
        mb[b] = *reinterpret_cast<const float2*>(rec + D);
        ob[b] = *reinterpret_cast<const float4*>(rec + d0);
      } else {
        mb[b] = make_float2(-INFINITY, 0.f);
        ob[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float Mb = M;
#pragma unroll
    for (int b = 0; b < kWideBatch; ++b) Mb = fmaxf(Mb, mb[b].x);
    const float Mu = Mb == -INFINITY ? 0.f : Mb;
    const float alpha = fast_exp2(M - Mu);
    S *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) O[e] *= alpha;
#pragma unroll
    for (int b = 0; b < kWideBatch; ++b) {
      const float f = fast_exp2(mb[b].x - Mu);
      S = fmaf(mb[b].y, f, S);
      O[0] = fmaf(ob[b].x, f, O[0]);
      O[1] = fmaf(ob[b].y, f, O[1]);
      O[2] = fmaf(ob[b].z, f, O[2]);
      O[3] = fmaf(ob[b].w, f, O[3]);
    }
    M = Mb;
  }
  s_acc[wave][lane] = make_float4(O[0], O[1], O[2], O[3]);
  s_ms[wave][lane] = make_float2(M, S);
  __syncthreads();
  if (wave != 0 || !active) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMergeWaves; ++i) Mx = fmaxf(Mx, s_ms[i][lane].x);
  float St = 0.f, Ot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMergeWaves; ++i) {
    const float2 ms = s_ms[i][lane];
    const float4 o = s_acc[i][lane];
    const float f = ms.x == -INFINITY ? 0.f : fast_exp2(ms.x - Mx);
    St = fmaf(ms.y, f, St);
    Ot[0] = fmaf(o.x, f, Ot[0]);
    Ot[1] = fmaf(o.y, f, Ot[1]);
    Ot[2] = fmaf(o.z, f, Ot[2]);
    Ot[3] = fmaf(o.w, f, Ot[3]);
  }
  const int head = r->head * hps + g;
  char* out_row =
      static_cast<char*>(a.out) + ((size_t)r->seq * a.num_q_heads + head) * (D * sizeof(T));
  store_out4<T>(out_row + d0 * sizeof(T), Ot, 1.f / St);
}

template <typename T, int D, int BS>
hipError_t launch_valu(const DecodeArgs* a, int workers, hipStream_t stream, int* resident,
                       hipEvent_t start, hipEvent_t stop) {
  if (resident != nullptr) {
    // Resident one-wave workgroups per CU for this variant (occupancy query).
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        resident, reinterpret_cast<const void*>(&decode_valu_kernel<T, D, BS>), 64, 0);
  }
  hipExtLaunchKernelGGL((decode_valu_kernel<T, D, BS>), dim3(workers), dim3(64), 0, stream, start,
                        stop, 0, *a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_merge(const DecodeArgs& a, int workers, hipStream_t stream) {
  const int hpw = merge_heads_per_wave<D>();
  const int64_t waves = (int64_t)workers * ((a.heads_per_seg + hpw - 1) / hpw);
  const dim3 grid((unsigned)((waves + kMergeWaves - 1) / kMergeWaves)), wg(64 * kMergeWaves);
  const int64_t segments = (int64_t)a.num_seqs * (a.num_q_heads / a.heads_per_seg);
  if ((int64_t)workers >= kMergeWideFrom * segments) {
    const int64_t groups = (int64_t)workers * ((a.heads_per_seg + hpw - 1) / hpw);
    hipLaunchKernelGGL((merge_wide_kernel<T, D>), dim3((unsigned)groups), wg, 0, stream, a,
                       workers);
  } else
    hipLaunchKernelGGL((merge_kernel<T, D, kMergeBatch>), grid, wg, 0, stream, a, workers);
  return hipGetLastError();
}

// The vector-ALU attention kernel for one variant, or its occupancy.
hipError_t dispatch_valu(const DecodeArgs* a, int dtype, int head_dim, int block_size,
                         int workers, hipStream_t stream, int* resident,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
#define PA_DISPATCH(T, DT, HD, BSZ)                                          \
  if (dtype == DT && head_dim == HD && block_size == BSZ)                    \
    return launch_valu<T, HD, BSZ>(a, workers, stream, resident, start, stop);
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

hipError_t dispatch_merge(const DecodeArgs& a, int dtype, int head_dim, int workers,
                          hipStream_t stream) {
  if (dtype == kBf16 && head_dim == 128) return launch_merge<uint16_t, 128>(a, workers, stream);
  if (dtype == kBf16 && head_dim == 64) return launch_merge<uint16_t, 64>(a, workers, stream);
  if (dtype == kFp32 && head_dim == 128) return launch_merge<float, 128>(a, workers, stream);
  if (dtype == kFp32 && head_dim == 64) return launch_merge<float, 64>(a, workers, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& args, int dtype, int head_dim, int block_size,
                         int workers, hipStream_t stream, hipEvent_t before, hipEvent_t after) {
  DecodeArgs a = args;
  const bool mfma = gqa_supported(dtype, head_dim, a.group);
  a.heads_per_seg = mfma ? a.group : 1;
  a.piece_rows = a.heads_per_seg;
  a.seg_cost = mfma ? kSegCostMfma : kSegCostValu;
  // The events, when set, take the attention kernel's own start and end
  // times from its dispatch (no marker packets between the kernels).
  const hipError_t e =
      mfma ? launch_gqa_attention(a, block_size, workers, stream, nullptr, before, after)
           : dispatch_valu(&a, dtype, head_dim, block_size, workers, stream, nullptr, before,
                           after);
  if (e != hipSuccess) return e;
  if (workers == 1) return hipSuccess;   // one worker never splits a segment
  return dispatch_merge(a, dtype, head_dim, workers, stream);
}

hipError_t decode_resident_per_cu(int dtype, int head_dim, int block_size, int group,
                                  int* resident) {
  if (gqa_supported(dtype, head_dim, group))
    return launch_gqa_attention(DecodeArgs{}, block_size, 0, nullptr, resident);
  return dispatch_valu(nullptr, dtype, head_dim, block_size, 0, nullptr, resident);
}

}  // namespace pa
