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
constexpr int kCombineThreads = 128;
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
  if (t < kMoeMaxK) sel_sh[t] = 0;
  __syncthreads();
  // Ranks on a key with NaN read as -inf, ties to the smaller index: a strict
  // total order, so the ranks are a permutation and a selection never repeats
  // an expert, whatever the logits hold.
  for (int e = t; e < ne; e += kRouteThreads) {
    const float v0 = r1s[e];
    const float v = v0 == v0 ? v0 : -INFINITY;
    int rank = 0;
    for (int q = 0; q < ne; ++q) {
      const float w0 = r1s[q];
      const float w = w0 == w0 ? w0 : -INFINITY;
      rank += (w > v) || (w == v && q < e);
    }
    if (rank < p.k2) sel_sh[rank] = e;
  }
  __syncthreads();
  if (t < 64) {
    // softmax of each flow's logits over its set: lane q takes selection q
    // (k2 <= 32), lane 0 sums the exponentials in ranking order
    const int q = t;
    const bool in2 = q < p.k2, in1 = q < p.k1;
    const int e = in2 ? sel_sh[q] : 0;
    const float a1 = r1s[e], a2 = r2s[e];
    const float m1 = r1s[sel_sh[0]];  // the top-ranked logit is the primary's largest
    float m2 = in2 ? a2 : -INFINITY;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m2 = fmaxf(m2, __shfl_xor(m2, o));
    const float e1 = in1 ? ex2((a1 - m1) * kLog2e) : 0.f;
    const float e2 = in2 ? ex2((a2 - m2) * kLog2e) : 0.f;
    float s1 = 0.f, s2 = 0.f;
    for (int j = 0; j < p.k2; ++j) {  // every lane runs the same ordered sums
      const float x1 = __shfl(e1, j), x2 = __shfl(e2, j);
      if (j < p.k1) s1 += x1;
      s2 += x2;
    }
    if (in2) {
      p.sel[(size_t)s * p.k2 + q] = e;
      p.g2[(size_t)s * p.k2 + q] = e2 / s2;
    }
    if (in1) p.g1[(size_t)s * p.k1 + q] = e1 / s1;
  }
}

__global__ __launch_bounds__(kCombineThreads) void moe_combine_kernel(MoeCombineParams p) {
  const int groups = p.hidden / 4;
  const int item = blockIdx.x * kCombineThreads + threadIdx.x;
  if (item >= p.batch * groups) return;
  const int s = item / groups, n0 = (item - s * groups) * 4;
  const size_t o = (size_t)s * p.hidden + n0;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 c = p.c ? *(const float4*)(p.c + n0) : z;
  const float4 r1 = p.res1 ? *(const float4*)(p.res1 + o) : z;
  const float4 r2 = p.res2 ? *(const float4*)(p.res2 + o) : z;
  float4 m1 = z, m2 = z;
  // entries in batches: every load of a batch before its first product, the
  // products in ranking order
  constexpr int kBatch = 8;
  for (int q0 = 0; q0 < p.k2; q0 += kBatch) {
    float4 v1[kBatch], v2[kBatch];
    float g1[kBatch], g2[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int q = q0 + j;
      if (q < p.k2) {
        const float* row = p.y + ((size_t)(s * p.k2 + q) * 2) * p.hidden + n0;
        v2[j] = *(const float4*)(row + p.hidden);
        g2[j] = p.g2[(size_t)s * p.k2 + q];
        if (q < p.k1) {
          v1[j] = *(const float4*)row;
          g1[j] = p.g1[(size_t)s * p.k1 + q];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int q = q0 + j;
      if (q < p.k1) {
        m1.x = fmaf(g1[j], v1[j].x, m1.x); m1.y = fmaf(g1[j], v1[j].y, m1.y);
        m1.z = fmaf(g1[j], v1[j].z, m1.z); m1.w = fmaf(g1[j], v1[j].w, m1.w);
      }
      if (q < p.k2) {
        m2.x = fmaf(g2[j], v2[j].x, m2.x); m2.y = fmaf(g2[j], v2[j].y, m2.y);
        m2.z = fmaf(g2[j], v2[j].z, m2.z); m2.w = fmaf(g2[j], v2[j].w, m2.w);
      }
    }
  }
  float4 o1 = m1, o2 = m2;
  if (p.c) {
    o2.x = fmaf(c.x, m1.x, o2.x); o2.y = fmaf(c.y, m1.y, o2.y); o2.z = fmaf(c.z, m1.z, o2.z); o2.w = fmaf(c.w, m1.w, o2.w);
  }
  if (p.res1) {
    o1.x = r1.x + o1.x; o1.y = r1.y + o1.y; o1.z = r1.z + o1.z; o1.w = r1.w + o1.w;
  }
  if (p.res2) {
    o2.x = r2.x + o2.x; o2.y = r2.y + o2.y; o2.z = r2.z + o2.z; o2.w = r2.w + o2.w;
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
