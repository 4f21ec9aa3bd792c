// Split-K decode attention over a float32 KV cache, both flows from one read of
// every key and value ("Resumo Técnico: Dual-Flow Transformers", section
// "Mecanismos Chave"). Plain fp32 FMAs on the vector ALUs: the float32 cache
// is a small-model / reference-precision path, where the work is dominated by
// launch latency rather than by bandwidth.
//
// Workgroup = (split s, kv head g, sequence b), 4 waves. The scaled (and for
// flow 2 coupled) query rows sit in LDS. Each wave takes 64-position chunks:
// lane t scores position t0 + t against every row; the row max and sum are
// wave reductions; for the weighted value sum, lane owns dims lane + 64*j and
// reads the values of each position while the weight of position t is
// broadcast from lane t. Cache layout as in include/dfa.h (keys in 8-dim
// groups, values transposed in 16-position tiles), here with float elements.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "dfa_internal.h"
#include "launch.h"

namespace dfa {

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnParams p) {
  constexpr int DJ = D / 64;
  __shared__ int tbl[kMaxTableSlice];
  __shared__ __attribute__((aligned(16))) float qs[kMaxRows * D];
  __shared__ __attribute__((aligned(16))) float sm[kWaves * kMaxRows];
  __shared__ __attribute__((aligned(16))) float sl[kWaves * kMaxRows];
  __shared__ __attribute__((aligned(16))) float so[kWaves * kMaxRows * D];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  SplitRange r;
  if (!split_range<D>(p, b, g, s, r)) return;
  const int jb0 = stage_table(p, b, r, tbl);
  const int nr = p.flows * p.group;
  const float* q1 = (const float*)p.q1;
  const float* q2 = (const float*)p.q2;
  for (int idx = threadIdx.x; idx < nr * D; idx += kThreads) {
    const int row = idx / D, d = idx - row * D;
    const int f = row / p.group, h = g * p.group + (row - f * p.group);
    const size_t off = ((size_t)b * p.hq + h) * D + d;
    const float x = f ? fmaf(p.a[(size_t)h * D + d], q1[off], q2[off]) : q1[off];
    qs[idx] = x * p.qscale;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bs = 1 << p.bs_log2, bs_mask = bs - 1;
  const float* kc = (const float*)p.k + (size_t)g * bs * D;
  const float* vc = (const float*)p.v + (size_t)g * D * bs;
  float m[kMaxRows], l[kMaxRows], acc[kMaxRows][DJ];
#pragma unroll
  for (int i = 0; i < kMaxRows; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int j = 0; j < DJ; ++j) acc[i][j] = 0.f;
  }
  const int nch = (r.end - r.start + 63) >> 6;
  for (int c = wave; c < nch; c += kWaves) {
    const int t0 = r.start + 64 * c;
    const int t = t0 + lane;
    const int tc = min(t, r.end - 1);
    // key of position tc: tile tc/16, then dims 8j..8j+7 are 8 contiguous floats in group j
    const int kp = tc & bs_mask;
    const float* kr = kc + (size_t)tbl[(tc >> p.bs_log2) - jb0] * p.blk_stride + (size_t)(kp >> 4) * (D * 16) + (kp & 15) * 8;
    float sc[kMaxRows];
#pragma unroll
    for (int i = 0; i < kMaxRows; ++i) sc[i] = 0.f;
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 kv = *(const float4*)(kr + (d4 >> 1) * 128 + 4 * (d4 & 1));
#pragma unroll
      for (int i = 0; i < kMaxRows; ++i) {
        if (i < nr) {
          const float4 qv = *(const float4*)(qs + i * D + 4 * d4);
          sc[i] = fmaf(qv.x, kv.x, fmaf(qv.y, kv.y, fmaf(qv.z, kv.z, fmaf(qv.w, kv.w, sc[i]))));
        }
      }
    }
    float pr[kMaxRows];
#pragma unroll
    for (int i = 0; i < kMaxRows; ++i) {
      if (i < nr) {
        const float si = (t < r.end) ? sc[i] : -INFINITY;
        const float m_new = fmaxf(m[i], wave_max(si));
        const float alpha = fast_exp2(m[i] - m_new);
        pr[i] = fast_exp2(si - m_new);
        l[i] = l[i] * alpha + wave_sum(pr[i]);
        m[i] = m_new;
#pragma unroll
        for (int j = 0; j < DJ; ++j) acc[i][j] *= alpha;
      }
    }
    const int cnt = min(64, r.end - t0);
    for (int tt = 0; tt < cnt; ++tt) {
      const int key = t0 + tt;
      const int pos = key & bs_mask;  // value of (dim d, pos) is at tile pos/16, row d, column pos%16
      const float* vr = vc + (size_t)tbl[(key >> p.bs_log2) - jb0] * p.blk_stride + (size_t)(pos >> 4) * (D * 16) + (pos & 15);
      float v[DJ];
#pragma unroll
      for (int j = 0; j < DJ; ++j) v[j] = vr[(lane + 64 * j) * 16];
#pragma unroll
      for (int i = 0; i < kMaxRows; ++i) {
        if (i < nr) {
          const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[i]), tt));
#pragma unroll
          for (int j = 0; j < DJ; ++j) acc[i][j] = fmaf(w, v[j], acc[i][j]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxRows; ++i) {
    if (i < nr) {
      if (lane == 0) {
        sm[i * kWaves + wave] = m[i];
        sl[i * kWaves + wave] = l[i];
      }
#pragma unroll
      for (int j = 0; j < DJ; ++j) so[(wave * kMaxRows + i) * D + lane + 64 * j] = acc[i][j];
    }
  }
  __syncthreads();
  merge_waves<D, kMaxRows>(p, b, g, s, sm, sl, so);
}

hipError_t launch_attn_f32(const AttnParams& p, int head_dim, hipStream_t stream, const KernelEvents& ev) {
  const dim3 grid(p.n_splits, p.hkv, p.batch), block(kThreads);
  if (head_dim == 64) return launch_kernel(attn_f32_kernel<64>, grid, block, stream, ev, p);
  if (head_dim == 128) return launch_kernel(attn_f32_kernel<128>, grid, block, stream, ev, p);
  return hipErrorInvalidValue;
}

}  // namespace dfa
