// Paged KV append and copy-on-write block copy: pure data movement.
//
// Append (page "Paging the cache", zeroshotmind.com essay on PagedAttention):
// each new token's K and V rows land in the slot the host block manager
// picked.  Copy (page section "Sharing a prefix without copying it"): a write
// into a shared block first duplicates that whole block.
//
// Both kernels move 16-byte units with one 128-bit load and store per unit;
// consecutive lanes touch consecutive 16-byte units so every wavefront
// access is a contiguous run (one KV row is 128..512 bytes).
#include "pa_internal.h"

namespace pa {
namespace {

// One thread per 16-byte unit of one (token, kv head) row, for K and V.
__global__ __launch_bounds__(256) void append_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache,
    const char* __restrict__ k_new, const char* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, int64_t num_units, int num_kv_heads,
    int block_size, int row_units) {
  const int64_t unit = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (unit >= num_units) return;
  const int u = (int)(unit % row_units);
  const int64_t row = unit / row_units;            // token * num_kv_heads + head
  const int head = (int)(row % num_kv_heads);
  const int64_t token = row / num_kv_heads;
  const int64_t slot = slot_mapping[token];
  if (slot < 0) return;
  const int64_t block = slot / block_size;
  const int64_t offset = slot - block * block_size;
  const int64_t dst = (((block * num_kv_heads + head) * block_size + offset) * row_units + u);
  const int64_t src = row * row_units + u;
  const uint4 kv = reinterpret_cast<const uint4*>(k_new)[src];
  const uint4 vv = reinterpret_cast<const uint4*>(v_new)[src];
  reinterpret_cast<uint4*>(k_cache)[dst] = kv;
  reinterpret_cast<uint4*>(v_cache)[dst] = vv;
}

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;   // 16-byte units per thread -> 16 KiB per workgroup

typedef unsigned v4u __attribute__((ext_vector_type(4)));
// A copied block goes out with non-temporal stores: written through without
// being kept in L2.  On the fork batch's 112 block copies that took the copy
// from 22.2 to 10.3 us, and the fork step (copies, then decode) from 104.7 to
// 93.7 us, so the decode that reads the copies right after does not miss them.
__device__ __forceinline__ void store_stream(uint4* to, const uint4& v) {
  __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(&v), reinterpret_cast<v4u*>(to));
}

// grid: x = piece of the block, y = pair, z = 0 (K) / 1 (V).
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int64_t* __restrict__ block_mapping, int64_t block_units) {
  const int64_t pair = blockIdx.y;
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  uint4* pool = reinterpret_cast<uint4*>(blockIdx.z == 0 ? k_cache : v_cache);
  const uint4* from = pool + src * block_units;
  uint4* to = pool + dst * block_units;
  const int64_t first = (int64_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  uint4 buf[kCopyUnroll];
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t u = first + i * kCopyThreads;
    if (u < block_units) buf[i] = from[u];
  }
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t u = first + i * kCopyThreads;
    if (u < block_units) store_stream(to + u, buf[i]);
  }
}

// Multi-layer variants: the pools of up to kMaxLayersPerLaunch layers travel
// by value in the kernel arguments, so one launch serves every layer without
// a device-side pointer table.
struct LayerPools {
  char* k[kMaxLayersPerLaunch];
  char* v[kMaxLayersPerLaunch];
  const char* k_new[kMaxLayersPerLaunch];
  const char* v_new[kMaxLayersPerLaunch];
};

// grid: x covers the units of one layer's rows, y = layer.
__global__ __launch_bounds__(256) void append_layers_kernel(
    const LayerPools p, const int64_t* __restrict__ slot_mapping, int64_t num_units,
    int num_kv_heads, int block_size, int row_units) {
  const int64_t unit = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (unit >= num_units) return;
  const int layer = blockIdx.y;
  const int u = (int)(unit % row_units);
  const int64_t row = unit / row_units;            // token * num_kv_heads + head
  const int head = (int)(row % num_kv_heads);
  const int64_t token = row / num_kv_heads;
  const int64_t slot = slot_mapping[token];
  if (slot < 0) return;
  const int64_t block = slot / block_size;
  const int64_t offset = slot - block * block_size;
  const int64_t dst = (((block * num_kv_heads + head) * block_size + offset) * row_units + u);
  const int64_t src = row * row_units + u;
  const uint4 kv = reinterpret_cast<const uint4*>(p.k_new[layer])[src];
  const uint4 vv = reinterpret_cast<const uint4*>(p.v_new[layer])[src];
  reinterpret_cast<uint4*>(p.k[layer])[dst] = kv;
  reinterpret_cast<uint4*>(p.v[layer])[dst] = vv;
}

// grid: x = piece of the block, y = pair, z = 2 * layer + (0 K / 1 V).
__global__ __launch_bounds__(kCopyThreads) void copy_layers_kernel(
    const LayerPools p, const int64_t* __restrict__ block_mapping, int64_t block_units) {
  const int64_t pair = blockIdx.y;
  const int layer = blockIdx.z >> 1;
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  uint4* pool = reinterpret_cast<uint4*>((blockIdx.z & 1) == 0 ? p.k[layer] : p.v[layer]);
  const uint4* from = pool + src * block_units;
  uint4* to = pool + dst * block_units;
  const int64_t first = (int64_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  uint4 buf[kCopyUnroll];
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t u = first + i * kCopyThreads;
    if (u < block_units) buf[i] = from[u];
  }
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int64_t u = first + i * kCopyThreads;
    if (u < block_units) store_stream(to + u, buf[i]);
  }
}

}  // namespace

hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int block_size, int row_bytes, hipStream_t stream) {
  const int row_units = row_bytes / 16;
  const int64_t units = num_tokens * num_kv_heads * row_units;
  const int threads = 256;
  const int64_t blocks = (units + threads - 1) / threads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                     slot_mapping, units, num_kv_heads, block_size, row_units);
  return hipGetLastError();
}

hipError_t launch_copy(void* k_cache, void* v_cache, const int64_t* block_mapping,
                       int64_t num_pairs, int64_t block_bytes, hipStream_t stream) {
  const int64_t units = block_bytes / 16;
  const int64_t per_wg = kCopyThreads * kCopyUnroll;
  const int64_t gx = (units + per_wg - 1) / per_wg;
  if (gx > INT32_MAX) return hipErrorInvalidValue;
  const int64_t kMaxY = 65535;   // grid y limit: launch in batches of pairs
  for (int64_t first = 0; first < num_pairs; first += kMaxY) {
    const int64_t n = num_pairs - first < kMaxY ? num_pairs - first : kMaxY;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)gx, (unsigned)n, 2), dim3(kCopyThreads), 0,
                       stream, static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                       block_mapping + 2 * first, units);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append_layers(void* const* k_caches, void* const* v_caches,
                                const void* const* k_new, const void* const* v_new, int num_layers,
                                const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                                int block_size, int row_bytes, hipStream_t stream) {
  const int row_units = row_bytes / 16;
  const int64_t units = num_tokens * num_kv_heads * row_units;
  const int threads = 256;
  const int64_t blocks = (units + threads - 1) / threads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  for (int first = 0; first < num_layers; first += kMaxLayersPerLaunch) {
    const int n = num_layers - first < kMaxLayersPerLaunch ? num_layers - first : kMaxLayersPerLaunch;
    LayerPools p{};
    for (int l = 0; l < n; ++l) {
      p.k[l] = static_cast<char*>(k_caches[first + l]);
      p.v[l] = static_cast<char*>(v_caches[first + l]);
      p.k_new[l] = static_cast<const char*>(k_new[first + l]);
      p.v_new[l] = static_cast<const char*>(v_new[first + l]);
    }
    hipLaunchKernelGGL(append_layers_kernel, dim3((unsigned)blocks, (unsigned)n), dim3(threads), 0,
                       stream, p, slot_mapping, units, num_kv_heads, block_size, row_units);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy_layers(void* const* k_caches, void* const* v_caches, int num_layers,
                              const int64_t* block_mapping, int64_t num_pairs, int64_t block_bytes,
                              hipStream_t stream) {
  const int64_t units = block_bytes / 16;
  const int64_t per_wg = kCopyThreads * kCopyUnroll;
  const int64_t gx = (units + per_wg - 1) / per_wg;
  if (gx > INT32_MAX) return hipErrorInvalidValue;
  const int64_t kMaxY = 65535;   // grid y limit: launch in batches of pairs
  for (int first = 0; first < num_layers; first += kMaxLayersPerLaunch) {
    const int n = num_layers - first < kMaxLayersPerLaunch ? num_layers - first : kMaxLayersPerLaunch;
    LayerPools p{};
    for (int l = 0; l < n; ++l) {
      p.k[l] = static_cast<char*>(k_caches[first + l]);
      p.v[l] = static_cast<char*>(v_caches[first + l]);
    }
    for (int64_t pf = 0; pf < num_pairs; pf += kMaxY) {
      const int64_t np = num_pairs - pf < kMaxY ? num_pairs - pf : kMaxY;
      hipLaunchKernelGGL(copy_layers_kernel, dim3((unsigned)gx, (unsigned)np, (unsigned)(2 * n)),
                         dim3(kCopyThreads), 0, stream, p, block_mapping + 2 * pf, units);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace pa
