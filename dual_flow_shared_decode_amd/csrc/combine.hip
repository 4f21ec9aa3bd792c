// Log-sum-exp combine of split records into normalised outputs. For record row
// (b, h, f) and its splits s, each record holding the unnormalised output O_s,
// its max m_s and sum l_s in base-2 units:
//     M = max_s m_s,   O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// This is the same exact softmax as one pass over all positions, regrouped.
// Every split of every row has a record: a split past the end of its sequence
// holds the empty record (O = 0, m = -inf, l = 0), which adds nothing, and a
// row whose records are all empty (no position at all) gets zero output. So
// the combine needs no sequence lengths, and with up to kFastSplits splits
// every load of a row is issued at once.
// One wave per record row; lane owns dims lane + 64*j.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "dfa_internal.h"

namespace dfa {

constexpr int kFastSplits = 8;

// NS > 0: exactly NS splits, all records of the row loaded into registers at
// once; NS == 0: any number of splits, one record at a time.
template <int D, int NS>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  constexpr int DJ = D / 64;
  constexpr int REC = D + kRecPad;
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (rowid >= p.batch * p.hq * p.flows) return;
  const int b = rowid / (p.hq * p.flows);
  const int rem = rowid - b * p.hq * p.flows;
  const int h = rem / p.flows, f = rem - h * p.flows;
  const float* rec = p.part + (size_t)rowid * p.n_splits * REC;
  float* out = (f ? p.o2 : p.o1) + ((size_t)b * p.hq + h) * D;
  float acc[DJ], lsum = 0.f, mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < DJ; ++j) acc[j] = 0.f;

  if (NS > 0) {
    constexpr int N = NS > 0 ? NS : 1;
    float m[N], l[N], o[N][DJ];
#pragma unroll
    for (int s = 0; s < N; ++s) {
      const float* rs = rec + (size_t)s * REC;
      m[s] = rs[D];
      l[s] = rs[D + 1];
#pragma unroll
      for (int j = 0; j < DJ; ++j) o[s][j] = rs[lane + 64 * j];
    }
#pragma unroll
    for (int s = 0; s < N; ++s) mx = fmaxf(mx, m[s]);
    const float mref = mx == -INFINITY ? 0.f : mx;  // all empty: every weight below is 0
#pragma unroll
    for (int s = 0; s < N; ++s) {
      const float e = fast_exp2(m[s] - mref);
      lsum = fmaf(e, l[s], lsum);
#pragma unroll
      for (int j = 0; j < DJ; ++j) acc[j] = fmaf(e, o[s][j], acc[j]);
    }
  } else {
    for (int s = lane; s < p.n_splits; s += 64) mx = fmaxf(mx, rec[(size_t)s * REC + D]);
    mx = wave_max(mx);
    const float mref = mx == -INFINITY ? 0.f : mx;
    for (int s = 0; s < p.n_splits; ++s) {
      const float* rs = rec + (size_t)s * REC;
      const float e = fast_exp2(rs[D] - mref);
      lsum = fmaf(e, rs[D + 1], lsum);
#pragma unroll
      for (int j = 0; j < DJ; ++j) acc[j] = fmaf(e, rs[lane + 64 * j], acc[j]);
    }
  }
  const bool empty = mx == -INFINITY;
  const float inv = empty ? 0.f : 1.f / lsum;
#pragma unroll
  for (int j = 0; j < DJ; ++j) out[lane + 64 * j] = empty ? 0.f : acc[j] * inv;
}

template <int D>
hipError_t launch_combine_d(const CombineParams& p, dim3 grid, dim3 block, hipStream_t stream) {
  switch (p.n_splits) {
#define DFA_COMBINE_CASE(N)                                                             \
  case N:                                                                               \
    hipLaunchKernelGGL((combine_kernel<D, N>), grid, block, 0, stream, p);              \
    break;
    DFA_COMBINE_CASE(1) DFA_COMBINE_CASE(2) DFA_COMBINE_CASE(3) DFA_COMBINE_CASE(4)
    DFA_COMBINE_CASE(5) DFA_COMBINE_CASE(6) DFA_COMBINE_CASE(7) DFA_COMBINE_CASE(8)
#undef DFA_COMBINE_CASE
    default:
      hipLaunchKernelGGL((combine_kernel<D, 0>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const int rows = p.batch * p.hq * p.flows;
  const dim3 grid((rows + kWaves - 1) / kWaves), block(kThreads);
  if (head_dim == 64) return launch_combine_d<64>(p, grid, block, stream);
  if (head_dim == 128) return launch_combine_d<128>(p, grid, block, stream);
  return hipErrorInvalidValue;
}

}  // namespace dfa
