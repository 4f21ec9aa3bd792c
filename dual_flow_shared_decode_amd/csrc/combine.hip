// Log-sum-exp combine of split records into normalised outputs. For record row
// (b, h, f) with splits s < ceil(len_b / split_len), each record holding the
// unnormalised output O_s, its max m_s and sum l_s in base-2 units:
//     M = max_s m_s,   O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// This is the same exact softmax as one pass over all positions, regrouped.
// One wave per record row; lane owns dims lane + 64*j.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "dfa_internal.h"

namespace dfa {

template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  constexpr int DJ = D / 64;
  constexpr int REC = D + kRecPad;
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (rowid >= p.batch * p.hq * p.flows) return;
  const int b = rowid / (p.hq * p.flows);
  const int rem = rowid - b * p.hq * p.flows;
  const int h = rem / p.flows, f = rem - h * p.flows;
  int len = p.ctx[b] + p.ctx_add;
  len = len < 0 ? 0 : (len > p.max_ctx ? p.max_ctx : len);
  const int ns = min((len + p.split_len - 1) / p.split_len, p.n_splits);
  const float* rec = p.part + (size_t)rowid * p.n_splits * REC;
  float* out = (f ? p.o2 : p.o1) + ((size_t)b * p.hq + h) * D;
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, rec[(size_t)s * REC + D]);
  mx = wave_max(mx);
  float acc[DJ], lsum = 0.f;
#pragma unroll
  for (int j = 0; j < DJ; ++j) acc[j] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* rs = rec + (size_t)s * REC;
    const float e = fast_exp2(rs[D] - mx);
    lsum = fmaf(e, rs[D + 1], lsum);
#pragma unroll
    for (int j = 0; j < DJ; ++j) acc[j] = fmaf(e, rs[lane + 64 * j], acc[j]);
  }
  const float inv = ns > 0 ? 1.f / lsum : 0.f;
#pragma unroll
  for (int j = 0; j < DJ; ++j) out[lane + 64 * j] = ns > 0 ? acc[j] * inv : 0.f;
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const int rows = p.batch * p.hq * p.flows;
  const dim3 grid((rows + kWaves - 1) / kWaves), block(kThreads);
  if (head_dim == 64)
    hipLaunchKernelGGL((combine_kernel<64>), grid, block, 0, stream, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL((combine_kernel<128>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dfa
