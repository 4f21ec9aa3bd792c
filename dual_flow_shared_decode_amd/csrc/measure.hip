// Bandwidth ceiling probe: a read of a buffer with coalesced, non-temporal
// 16-byte loads (the cache policy the attention kernels stream with), each
// workgroup streaming one contiguous range. Not part of the method; the
// attention kernels' achieved bandwidth is compared to it.
#include <hip/hip_runtime.h>

#include "dfa_internal.h"

namespace dfa {

namespace {
constexpr int kReadBlocks = 4096;
constexpr int kReadThreads = 256;
constexpr int kUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
}  // namespace

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                                     size_t per_block, uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * per_block;
  const size_t stop = min(base + per_block, n16);
  uint32_t acc = 0;
  for (size_t i = base + threadIdx.x; i < stop; i += kUnroll * kReadThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + (size_t)u * kReadThreads;
      v[u] = j < stop ? __builtin_nontemporal_load(buf + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

size_t stream_read_threads() { return (size_t)kReadBlocks * kReadThreads; }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t per_block = (n16 + kReadBlocks - 1) / kReadBlocks;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kReadBlocks), dim3(kReadThreads), 0, stream,
                     (const u32x4*)buf, n16, per_block, sink);
  return hipGetLastError();
}

}  // namespace dfa
