// Read-bandwidth probe: the HBM read rate this GPU reaches on the access
// patterns of the step, measured beside the step's kernels as context for
// their roofline fractions. Not a step of the method.
//
// k_probe_stream: grid-stride reads of 16-byte vectors, 4 in flight per
//   thread before any is used (non-temporal: every byte is read once).
// k_probe_blocks: one wavefront per 4 KB block at a time, blocks visited in
//   the order a page table gives (the paged KV cache's pattern: K and V of
//   one kv head of one page are 4 KB each), 4 wave-wide 16-byte loads per
//   lane in flight.
// Each thread folds what it read with xor and writes one word, so no load is
// dead code and the writes are negligible next to the reads.
#include "common.hpp"

namespace wedlm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ void __launch_bounds__(kProbeThreads)
k_probe_stream(const u32x4* __restrict__ src, size_t nvec, uint32_t* __restrict__ sink) {
  const size_t tid = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
  u32x4 acc = {0, 0, 0, 0};
  size_t i = tid;
  for (; i + (kProbeUnroll - 1) * stride < nvec; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < nvec; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// A 4 KB block is 256 vectors: 4 wave-wide loads per lane.
__global__ void __launch_bounds__(kProbeThreads)
k_probe_blocks(const u32x4* __restrict__ src, const int32_t* __restrict__ order, int n_blocks,
               int n_src_blocks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * (kProbeThreads / kWave) + (threadIdx.x >> 6);
  const int n_waves = gridDim.x * (kProbeThreads / kWave);
  u32x4 acc = {0, 0, 0, 0};
  for (int j = wave; j < n_blocks; j += n_waves) {
    const int blk = min(max(order[j], 0), n_src_blocks - 1);
    const u32x4* base = src + static_cast<size_t>(blk) * 256 + lane;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(base + u * kWave);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  sink[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace wedlm

using namespace wedlm;

extern "C" int wedlm_read_probe(const void* src, size_t bytes, const int32_t* block_order,
                                int n_blocks, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || grid <= 0 || grid > (1 << 20) || bytes < 16) return WEDLM_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return WEDLM_ERR_INVALID;
  hipStream_t s = as_stream(stream);
  if (block_order == nullptr) {
    hipLaunchKernelGGL(k_probe_stream, dim3(grid), dim3(kProbeThreads), 0, s,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
  } else {
    const size_t n_src = bytes / 4096;
    if (n_blocks <= 0 || n_src == 0 || n_src > 0x7fffffff) return WEDLM_ERR_INVALID;
    hipLaunchKernelGGL(k_probe_blocks, dim3(grid), dim3(kProbeThreads), 0, s,
                       static_cast<const u32x4*>(src), block_order, n_blocks,
                       static_cast<int>(n_src), sink);
  }
  return launch_status();
}
