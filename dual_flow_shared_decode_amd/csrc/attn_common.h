// Device helpers shared by the attention kernels: split bounds, block-table
// staging, wave reductions, and the cross-wave merge that ends every
// workgroup (written as a normalised output or as a split record).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "dfa_internal.h"

namespace dfa {

// 2^x on the hardware exponential unit. Inputs below -126 give 0 or a value
// far below the precision of any sum it joins; -inf gives exactly 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Result of a split that holds no position of its sequence: zero outputs in
// direct mode (an empty sequence), else the empty record (O = 0, m = -inf,
// l = 0) of each row, so that every record the combine reads is written by the
// same call.
template <int D, int NT>
__device__ __forceinline__ void write_empty(const AttnParams& p, int b, int g, int s) {
  const int nr = p.flows * p.group;
  if (p.direct) {
    for (int idx = threadIdx.x; idx < nr * D; idx += NT) {
      const int row = idx / D, d = idx - row * D;
      const int f = row / p.group, h = g * p.group + (row - f * p.group);
      float* out = f ? p.o2 : p.o1;
      out[((size_t)b * p.hq + h) * D + d] = 0.f;
    }
  } else {
    for (int idx = threadIdx.x; idx < nr * (D + 2); idx += NT) {
      const int row = idx / (D + 2), d = idx - row * (D + 2);
      const int f = row / p.group, h = g * p.group + (row - f * p.group);
      float* rec = p.part + ((((size_t)b * p.hq + h) * p.flows + f) * p.n_splits + s) * (D + kRecPad);
      rec[d] = d == D ? -INFINITY : 0.f;
    }
  }
}

// Positions [start, end) handled by workgroup (split s, sequence b); returns
// false when the split holds no position of the sequence. Such a workgroup
// still writes its result: zero outputs in direct mode (an empty sequence),
// else the empty record (O = 0, m = -inf, l = 0) of each row, so that every
// record the combine reads is written by the same call.
struct SplitRange {
  int start, end, len;
};

template <int D>
__device__ __forceinline__ bool split_range(const AttnParams& p, int b, int g, int s, SplitRange& r) {
  int len = p.ctx[b] + p.ctx_add;
  len = len < 0 ? 0 : (len > p.max_ctx ? p.max_ctx : len);
  r.len = len;
  r.start = s * p.split_len;
  r.end = min(r.start + p.split_len, len);
  if (r.start < len) return true;
  write_empty<D, kThreads>(p, b, g, s);
  return false;
}

// Stages the physical block ids of the split's positions into LDS, clamped to
// [0, num_blocks) so that no cache access can leave the cache tensors. Ends
// with a workgroup barrier: the entries are read by every wave.
__device__ __forceinline__ int stage_table(const AttnParams& p, int b, const SplitRange& r, int* tbl) {
  const int jb0 = r.start >> p.bs_log2;
  const int jb1 = (r.end - 1) >> p.bs_log2;
  const int32_t* row = p.table + (size_t)b * p.max_blocks;
  for (int j = threadIdx.x; j <= jb1 - jb0; j += kThreads) {
    int blk = row[jb0 + j];
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    tbl[j] = blk;
  }
  __syncthreads();  // every wave reads entries other waves wrote
  return jb0;
}

// Stages the physical block ids of every block split s can touch (from its
// first position on; it does not need the sequence length) into LDS, clamped
// to [0, num_blocks) so that no cache access can leave the cache tensors.
// The caller issues a workgroup barrier before any wave reads the entries.
template <int NT = kThreads>
__device__ __forceinline__ int stage_split_table(const AttnParams& p, int b, int s, int* tbl) {
  const int jb0 = (s * p.split_len) >> p.bs_log2;
  const int nb = min(((p.split_len - 1) >> p.bs_log2) + 2, p.max_blocks - jb0);
  const int32_t* row = p.table + (size_t)b * p.max_blocks + jb0;
  for (int j = threadIdx.x; j < nb; j += NT) {
    int blk = row[j];
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    tbl[j] = blk;
  }
  return jb0;
}

// Bounds of split s given the raw length ctx[b]; as split_range, including
// the zero outputs / empty records of a split past the end of its sequence.
template <int D, int NT = kThreads>
__device__ __forceinline__ bool split_bounds(const AttnParams& p, int b, int g, int s, int len_raw, SplitRange& r) {
  int len = len_raw + p.ctx_add;
  len = len < 0 ? 0 : (len > p.max_ctx ? p.max_ctx : len);
  r.len = len;
  r.start = s * p.split_len;
  r.end = min(r.start + p.split_len, len);
  if (r.start < len) return true;
  write_empty<D, NT>(p, b, g, s);
  return false;
}

// Cross-wave merge. Each of the NW waves w that served a row left, for that
// row, the running max sm[row*NW+w], sum sl[row*NW+w] and unnormalised output
// so[(w*NRP+row)*D+d] (all in base-2 units); NT threads take part. Writes the normalised output in
// direct mode (one split per sequence), otherwise the split record (O, m, l)
// of each row. A thread takes four consecutive dimensions of a row, so every
// LDS read and global store moves 16 bytes. A wave that took no position
// left (m, l, O) = (-inf, 0, 0) and gets weight 0; some wave holds a position
// of a non-empty split, so the row max is finite.
template <int D, int NRP, int NW = kWaves, int NT = 64 * NW>
__device__ __forceinline__ void merge_waves(const AttnParams& p, int b, int g, int s,
                                            const float* sm, const float* sl, const float* so) {
  static_assert(NW == 4, "the four waves' (m, l) of a row are read as one float4");
  constexpr int D4 = D / 4;
  const int nr = p.flows * p.group;
  for (int idx = threadIdx.x; idx < nr * D4; idx += NT) {
    const int row = idx / D4, d = 4 * (idx - row * D4);
    const float4 m4 = *(const float4*)(sm + row * NW);
    const float4 l4 = *(const float4*)(sl + row * NW);
    const float mx = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
    const float e0 = fast_exp2(m4.x - mx), e1 = fast_exp2(m4.y - mx);
    const float e2 = fast_exp2(m4.z - mx), e3 = fast_exp2(m4.w - mx);
    const float4 v0 = *(const float4*)(so + (0 * NRP + row) * D + d);
    const float4 v1 = *(const float4*)(so + (1 * NRP + row) * D + d);
    const float4 v2 = *(const float4*)(so + (2 * NRP + row) * D + d);
    const float4 v3 = *(const float4*)(so + (3 * NRP + row) * D + d);
    float4 o;
    o.x = e0 * v0.x + e1 * v1.x + e2 * v2.x + e3 * v3.x;
    o.y = e0 * v0.y + e1 * v1.y + e2 * v2.y + e3 * v3.y;
    o.z = e0 * v0.z + e1 * v1.z + e2 * v2.z + e3 * v3.z;
    o.w = e0 * v0.w + e1 * v1.w + e2 * v2.w + e3 * v3.w;
    const float l = e0 * l4.x + e1 * l4.y + e2 * l4.z + e3 * l4.w;
    const int f = row >= p.group ? 1 : 0;  // at most two flows
    const int h = g * p.group + row - f * p.group;
    if (p.direct) {
      const float inv = 1.f / l;
      float* out = (f ? p.o2 : p.o1) + ((size_t)b * p.hq + h) * D + d;
      *(float4*)out = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
      float* rec = p.part + ((((size_t)b * p.hq + h) * p.flows + f) * p.n_splits + s) * (D + kRecPad);
      *(float4*)(rec + d) = o;
      if (d == 0) *(float2*)(rec + D) = make_float2(mx, l);
    }
  }
}

}  // namespace dfa
