// Decode-step paged attention for grouped query heads (group 2..16, bf16,
// head_dim 128) on the gfx950 matrix cores: every (KV head, sequence)
// segment of the batch, with all the group's query heads at once (the worker
// loop and its design are in gqa_body.h).  Pages on "Efficient Memory
// Management for Large Language Model Serving with PagedAttention":
// zeroshotmind.com essay, "Block tables: logical order, physical scatter".
#include "gqa_body.h"

namespace pa {
namespace {

using namespace dev;

template <int BS>
// One-wave workgroups; the register budget is set for two waves per SIMD
// (256 VGPRs, no accumulation registers), so 8 workers can be resident per CU.
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(2)))
void decode_gqa_kernel(const DecodeArgs a) {
  const int lane = threadIdx.x;
  const int nworkers = gridDim.x;
  const int w = (nworkers % kNumXcd) ? (int)blockIdx.x
                                     : (int)(blockIdx.x % kNumXcd) * (nworkers / kNumXcd) +
                                           (int)(blockIdx.x / kNumXcd);
  const int B = a.num_seqs;
  const int HQ = a.num_q_heads;
  const int32_t* __restrict__ lens = a.context_lens;

  LineSplit ls;
  __shared__ KernelLds lds;
  const bool has_chunks =
      split_line(lds.split, lens, B, a.num_kv_heads, a.seg_cost, nworkers, w, lane, ls);
  // Sequences with no cached token produce zero rows (lengths from the
  // split's LDS cache).
  for (int s = w; s < B; s += nworkers) {
    if (seq_len(lds.split, lens, s) == 0) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<char*>(a.out) + (size_t)s * HQ * kRow);
      for (int u = lane; u < HQ * (kRow / 16); u += 64) o[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (!has_chunks) {
    if (lane == 0) a.records[w].valid = 0;
    return;
  }
  gqa_body<BS, false>(a, ShareArgs{}, lds, ls, w, 0);
}

}  // namespace

bool gqa_supported(int dtype, int head_dim, int group) {
  return dtype == kBf16 && head_dim == kD && group >= 2 && group <= 16;
}

hipError_t launch_gqa_attention(const DecodeArgs& a, int block_size, int workers,
                                hipStream_t stream, int* resident, hipEvent_t start,
                                hipEvent_t stop) {
  if (block_size == 16) {
    if (resident != nullptr)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          resident, reinterpret_cast<const void*>(&decode_gqa_kernel<16>), 64, 0);
    hipExtLaunchKernelGGL((decode_gqa_kernel<16>), dim3(workers), dim3(64), 0, stream, start,
                          stop, 0, a);
    return hipGetLastError();
  }
  if (block_size == 32) {
    if (resident != nullptr)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(
          resident, reinterpret_cast<const void*>(&decode_gqa_kernel<32>), 64, 0);
    hipExtLaunchKernelGGL((decode_gqa_kernel<32>), dim3(workers), dim3(64), 0, stream, start,
                          stop, 0, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
