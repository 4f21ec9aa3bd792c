// Mixture-of-experts FFN with router replay: routing and output combination
// ("Resumo Técnico: Dual-Flow Transformers", section "Mecanismos Chave",
// router replay: the auxiliary flow reuses the experts the primary router
// selected, with its own mixing weights; section "Contribuições Principais",
// phase-specific MoE allocation: the two flows' expert fan-outs are set
// independently). This library's reading: experts ranked by the primary's
// router logits (ties to the smaller index); the primary takes the first k1,
// the auxiliary flow the first k2 >= k1 of the same ranking; each flow's
// mixing weights are a softmax of its own router logits over its set.
//
// The experts themselves run as grouped GEMVs (gemv.hip, grouped mode): each
// selected expert's matrices are read once for every row of both flows that
// selected it. This file holds the two small kernels around them:
//   moe_route_kernel    workgroup = sequence: the rank of every expert (the
//                       number of experts ahead of it: exact, no sort), the
//                       selection in ranking order and both flows' mixing
//                       weights (sums in ranking order);
//   moe_combine_kernel  thread = (sequence, 4 columns): both flows' weighted
//                       sums of their experts' outputs in ranking order, the
//                       residuals and the output coupling c.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dfa_internal.h"
#include "ops_internal.h"

namespace dfa {

namespace {
constexpr int kRouteThreads = 256;
constexpr int kCombineThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
}  // namespace

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(MoeRouteParams p) {
  __shared__ float r1s[kMoeMaxExperts], r2s[kMoeMaxExperts];
  __shared__ int sel_sh[kMoeMaxK];
  const int s = blockIdx.x, t = threadIdx.x, ne = p.experts;
  for (int e = t; e < ne; e += kRouteThreads) {
    r1s[e] = p.r1[(size_t)s * ne + e];
    r2s[e] = p.r2[(size_t)s * ne + e];
  }
  if (t < kMoeMaxK) sel_sh[t] = 0;  // stays 0 only for logits that do not order (NaN)
  __syncthreads();
  for (int e = t; e < ne; e += kRouteThreads) {
    const float v = r1s[e];
    int rank = 0;
    for (int q = 0; q < ne; ++q) {
      const float w = r1s[q];
      rank += (w > v) || (w == v && q < e);
    }
    if (rank < p.k2) sel_sh[rank] = e;
  }
  __syncthreads();
  if (t == 0) {
    // softmax of each flow's logits over its set, summed in ranking order
    const float m1 = r1s[sel_sh[0]];
    float m2 = -INFINITY;
    for (int q = 0; q < p.k2; ++q) m2 = fmaxf(m2, r2s[sel_sh[q]]);
    float s1 = 0.f, s2 = 0.f;
    for (int q = 0; q < p.k2; ++q) {
      if (q < p.k1) s1 += ex2((r1s[sel_sh[q]] - m1) * kLog2e);
      s2 += ex2((r2s[sel_sh[q]] - m2) * kLog2e);
    }
    for (int q = 0; q < p.k2; ++q) {
      const int e = sel_sh[q];
      p.sel[(size_t)s * p.k2 + q] = e;
      if (q < p.k1) p.g1[(size_t)s * p.k1 + q] = ex2((r1s[e] - m1) * kLog2e) / s1;
      p.g2[(size_t)s * p.k2 + q] = ex2((r2s[e] - m2) * kLog2e) / s2;
    }
  }
}

__global__ __launch_bounds__(kCombineThreads) void moe_combine_kernel(MoeCombineParams p) {
  const int groups = p.hidden / 4;
  const int item = blockIdx.x * kCombineThreads + threadIdx.x;
  if (item >= p.batch * groups) return;
  const int s = item / groups, n0 = (item - s * groups) * 4;
  float4 m1 = make_float4(0.f, 0.f, 0.f, 0.f), m2 = m1;
  for (int q = 0; q < p.k2; ++q) {
    const float* row = p.y + ((size_t)(s * p.k2 + q) * 2) * p.hidden + n0;
    if (q < p.k1) {
      const float g = p.g1[(size_t)s * p.k1 + q];
      const float4 v = *(const float4*)row;
      m1.x = fmaf(g, v.x, m1.x); m1.y = fmaf(g, v.y, m1.y); m1.z = fmaf(g, v.z, m1.z); m1.w = fmaf(g, v.w, m1.w);
    }
    const float g = p.g2[(size_t)s * p.k2 + q];
    const float4 v = *(const float4*)(row + p.hidden);
    m2.x = fmaf(g, v.x, m2.x); m2.y = fmaf(g, v.y, m2.y); m2.z = fmaf(g, v.z, m2.z); m2.w = fmaf(g, v.w, m2.w);
  }
  const size_t o = (size_t)s * p.hidden + n0;
  float4 o1 = m1, o2 = m2;
  if (p.c) {
    const float4 c = *(const float4*)(p.c + n0);
    o2.x = fmaf(c.x, m1.x, o2.x); o2.y = fmaf(c.y, m1.y, o2.y); o2.z = fmaf(c.z, m1.z, o2.z); o2.w = fmaf(c.w, m1.w, o2.w);
  }
  if (p.res1) {
    const float4 r = *(const float4*)(p.res1 + o);
    o1.x = r.x + o1.x; o1.y = r.y + o1.y; o1.z = r.z + o1.z; o1.w = r.w + o1.w;
  }
  if (p.res2) {
    const float4 r = *(const float4*)(p.res2 + o);
    o2.x = r.x + o2.x; o2.y = r.y + o2.y; o2.z = r.z + o2.z; o2.w = r.w + o2.w;
  }
  *(float4*)(p.out1 + o) = o1;
  *(float4*)(p.out2 + o) = o2;
}

hipError_t launch_moe_route(const MoeRouteParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(p.batch), dim3(kRouteThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const MoeCombineParams& p, hipStream_t stream) {
  const int items = p.batch * (p.hidden / 4);
  hipLaunchKernelGGL(moe_combine_kernel, dim3((items + kCombineThreads - 1) / kCombineThreads),
                     dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dfa
