// RMSNorm of both flows' rows (pre-norm of the attention and MLP blocks in a
// layer stack; the flows share the weight vector of a block, as they share
// every weight of a layer: "Resumo Técnico: Dual-Flow Transformers", section
// "Arquitetura Central"):  y = x / sqrt(mean(x^2) + eps) * w.
// Workgroup = one row of one flow; the sum of squares is reduced in a fixed
// order (per thread, then lanes, then waves), so results do not depend on timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dfa_internal.h"
#include "ops_internal.h"

namespace dfa {

namespace {
constexpr int kNormThreads = 1024;  // one float4 per thread at 4096 columns: one load round trip per pass
}

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(NormParams p) {
  __shared__ float part[kNormThreads / 64];
  const int row = blockIdx.x, f = blockIdx.y;
  const float* x = (f ? p.x2 : p.x1) + (size_t)row * p.n;
  float* y = (f ? p.y2 : p.y1) + (size_t)row * p.n;
  float ss = 0.f;
  for (int i = threadIdx.x * 4; i < p.n; i += kNormThreads * 4) {
    const float4 v = *(const float4*)(x + i);
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot += part[w];
  const float inv = 1.f / sqrtf(tot / (float)p.n + p.eps);
  for (int i = threadIdx.x * 4; i < p.n; i += kNormThreads * 4) {
    const float4 v = *(const float4*)(x + i);
    const float4 w = *(const float4*)(p.w + i);
    *(float4*)(y + i) = make_float4(v.x * inv * w.x, v.y * inv * w.y, v.z * inv * w.z, v.w * inv * w.w);
  }
}

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(p.rows, 2), dim3(kNormThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dfa
