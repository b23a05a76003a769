// Read-bandwidth probe: a measurement companion of the decode kernels, not a
// step of the paged path.  It reads tiles of a buffer the way the decode
// kernels read K/V tiles -- one-wave workers, each walking an equal share of
// the tile list with 16-byte buffer loads (1 KiB per wave load) and 16 KiB
// in flight per wave -- but does no arithmetic beyond folding the words into
// a checksum.  Timed on the pools with the decode kernels' own tile order
// (random blocks), it gives the bandwidth ceiling of that access pattern on
// the device at hand, against which the attention kernels are compared.
#include "decode_common.h"

namespace pa {
namespace {

using namespace dev;

// XOR of a value over the 64 lanes (every lane receives it).
__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  return x;
}

// L wave loads per tile (tile = L KiB), R tiles in flight, NT: non-temporal
// loads.  Worker w (workgroup id, dealt so that consecutive workers share an
// XCD) reads tiles [w T / W, (w + 1) T / W) of the list and writes the XOR of
// every 32-bit word it read to checksum[w].
template <int L, int R, int NT>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void read_probe_kernel(uint32_t* __restrict__ checksum, const char* __restrict__ base,
                       const int32_t* __restrict__ tile_ids, int64_t num_tiles) {
  const int lane = threadIdx.x;
  const int nworkers = gridDim.x;
  const int w = (nworkers % kNumXcd) ? (int)blockIdx.x
                                     : (int)(blockIdx.x % kNumXcd) * (nworkers / kNumXcd) +
                                           (int)(blockIdx.x / kNumXcd);
  const int64_t t0 = (int64_t)w * num_tiles / nworkers;
  const int64_t t1 = (int64_t)(w + 1) * num_tiles / nworkers;
  const const_i32* ids = (const const_i32*)tile_ids;   // scalar loads
  constexpr int kTileBytes = L * 1024;
  uint32_t acc = 0;
  if (t0 < t1) {
    u32x4 ring[R][L];
    // Tile t's loads; past the range end the last tile is reloaded and never
    // folded, so every step issues the same loads.
    auto issue = [&](u32x4* dst, int64_t t) {
      const int64_t tt = t < t1 ? t : t1 - 1;
      const int64_t id = ids != nullptr ? (int64_t)ids[tt] : tt;
      const __amdgpu_buffer_rsrc_t r = tile_rsrc(base + id * kTileBytes, kTileBytes);
#pragma unroll
      for (int i = 0; i < L; ++i)
        dst[i] = NT ? load16_stream(r, i * 1024 + lane * 16) : load16(r, i * 1024 + lane * 16);
    };
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) issue(ring[r], t0 + r);
    for (int64_t t = t0; t < t1; t += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r > 0 && t + r >= t1) break;
        issue(ring[(r + R - 1) % R], t + r + R - 1);
#pragma unroll
        for (int i = 0; i < L; ++i) acc ^= ring[r][i].x ^ ring[r][i].y ^ ring[r][i].z ^ ring[r][i].w;
      }
    }
  }
  acc = wave_xor(acc);
  if (lane == 0) checksum[w] = acc;
}

template <int L, int R>
hipError_t launch_probe_lr(uint32_t* checksum, const char* base, const int32_t* ids,
                           int64_t num_tiles, int nt, int workers, hipStream_t stream) {
  if (nt)
    hipLaunchKernelGGL((read_probe_kernel<L, R, 1>), dim3(workers), dim3(64), 0, stream, checksum,
                       base, ids, num_tiles);
  else
    hipLaunchKernelGGL((read_probe_kernel<L, R, 0>), dim3(workers), dim3(64), 0, stream, checksum,
                       base, ids, num_tiles);
  return hipGetLastError();
}

}  // namespace

// Declared where it is called (pa_api.hip).
hipError_t launch_read_probe(uint32_t* checksum, const void* base, const int32_t* tile_ids,
                             int64_t num_tiles, int tile_bytes, int nontemporal, int workers,
                             hipStream_t stream) {
  const char* b = static_cast<const char*>(base);
  if (tile_bytes == 4096)
    return launch_probe_lr<4, 4>(checksum, b, tile_ids, num_tiles, nontemporal, workers, stream);
  if (tile_bytes == 8192)
    return launch_probe_lr<8, 2>(checksum, b, tile_ids, num_tiles, nontemporal, workers, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
