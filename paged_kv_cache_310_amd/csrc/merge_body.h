// Merge of split decode pieces: one wave folds the pieces of the segment a
// closing worker's merge record names.  Shared by the decode merge kernels
// (decode_kernel.hip) and the shared-prefix merge (shared_kernel.hip).
#pragma once

#include "decode_common.h"

namespace pa {
namespace dev {

constexpr int kMergeWaves = 4;   // waves per merge workgroup

template <int D>
constexpr int merge_heads_per_wave() { return 64 / (D / 4); }

template <typename T>
__device__ __forceinline__ void store_out4(void* dst, const float* o, float inv);

template <>
__device__ __forceinline__ void store_out4<uint16_t>(void* dst, const float* o, float inv) {
  uint2 r;
  r.x = f32_to_bf16(o[0] * inv) | (f32_to_bf16(o[1] * inv) << 16);
  r.y = f32_to_bf16(o[2] * inv) | (f32_to_bf16(o[3] * inv) << 16);
  *reinterpret_cast<uint2*>(dst) = r;
}

template <>
__device__ __forceinline__ void store_out4<float>(void* dst, const float* o, float inv) {
  *reinterpret_cast<float4*>(dst) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

// One wave of the merge: wave `id` folds, for the worker w = id / waves per
// record, the split pieces of the segment its record names
// (merge_heads_per_wave query heads of the segment per wave).
template <typename T, int D, int kBatch>
__device__ __forceinline__ void merge_record_wave(const DecodeArgs& a, int workers, int id,
                                                  int lane) {
  constexpr int LPH = D / 4;                       // lanes per head
  constexpr int HPW = merge_heads_per_wave<D>();   // heads per wave
  const int hps = a.heads_per_seg;
  const int wpr = (hps + HPW - 1) / HPW;           // waves per record
  const int w = id / wpr;
  if (w >= workers) return;
  typedef __attribute__((address_space(4))) const MergeRecord const_record;
  const const_record* r = (const const_record*)a.records + w;   // scalar loads
  if (!r->valid) return;
  const int64_t first = r->first;
  const int first_slot = r->first_slot;
  const int g = (id - w * wpr) * HPW + lane / LPH;
  if (g >= hps) return;   // no cross-lane work follows
  const int d0 = (lane % LPH) * 4;
  const int R = a.piece_rows;
  constexpr int REC = D + kPartialExtra;   // acc[D], max, sum, pad
  const int npieces = w - (int)first + 1;
  float M = -INFINITY, S = 0.f;
  float O[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < npieces; p0 += kBatch) {
    float4 ob[kBatch];
    float2 mb[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int p = p0 + b;
      if (p < npieces) {
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
    for (int b = 0; b < kBatch; ++b) Mb = fmaxf(Mb, mb[b].x);
    const float Mu = Mb == -INFINITY ? 0.f : Mb;
    const float alpha = fast_exp2(M - Mu);
    S *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) O[e] *= alpha;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const float f = fast_exp2(mb[b].x - Mu);
      S = fmaf(mb[b].y, f, S);
      O[0] = fmaf(ob[b].x, f, O[0]);
      O[1] = fmaf(ob[b].y, f, O[1]);
      O[2] = fmaf(ob[b].z, f, O[2]);
      O[3] = fmaf(ob[b].w, f, O[3]);
    }
    M = Mb;
  }
  const int head = r->head * hps + g;
  char* out_row =
      static_cast<char*>(a.out) + ((size_t)r->seq * a.num_q_heads + head) * (D * sizeof(T));
  store_out4<T>(out_row + d0 * sizeof(T), O, 1.f / S);
}


}  // namespace dev
}  // namespace pa
