// Mixture of the two flows' next-token distributions and its decoding
// ("Resumo Técnico: Dual-Flow Transformers", section "Mecanismos Chave",
// mixture objective: p_mix = alpha p_primary + (1 - alpha) p_aux, alpha set
// from the primary's collision probability, the primary keeping at least half
// of the weight). This library's reading of alpha: (1 + sum_v p1(v)^2) / 2.
//
// Three launches per call, on the flows' float32 logits [batch, vocab], the
// vocabulary cut into chunks of kMixChunk tokens:
//   mix_stats_kernel  workgroup = (chunk, sequence): each flow's largest logit
//                     and sum of exponentials over the chunk, and the
//                     primary's sum of squared exponentials;
//   mix_chunk_kernel  workgroup = (chunk, sequence): merges the sequence's
//                     chunk statistics in a fixed order (softmax normalisers,
//                     collision probability, alpha), then p_mix of the
//                     chunk's tokens (optionally stored), the chunk's mass and
//                     its first maximum;
//   mix_pick_kernel   workgroup = sequence: the chunk holding the caller's
//                     uniform u on the cumulative mass (inverse CDF), then the
//                     token inside that chunk, and the greedy token from the
//                     chunks' maxima.
// Masses are summed as integers: each token's p_mix (at most 1) is scaled by
// 2^35 and truncated, so every sum is exact, in any order, and the search
// meets the same sums at the chunk and at the token level. A token below
// 2^-35 of mass is never drawn. Exponentials are 2^((x - m) log2 e) on the
// hardware unit, the difference taken before scaling so that it is exact near
// the maximum however large the logits. Results do not depend on timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dfa_internal.h"
#include "ops_internal.h"

namespace dfa {

namespace {
constexpr int kMixThreads = 256;
constexpr int kRun = kMixChunk / kMixThreads;  // 16 tokens per thread
constexpr int kMixWaves = kMixThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFix = 34359738368.f;  // 2^35: fixed-point scale of a token's mass
static_assert(kMixMaxChunks <= kMixThreads, "one chunk record per thread of the pick kernel");
static_assert(kRun % 4 == 0, "float4 runs");

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

struct Norm {
  float m1, m2;  // largest logit of each flow
  float w1, w2;  // alpha / S1 and (1 - alpha) / S2
  float alpha;
};

// The sequence's softmax normalisers and alpha from its chunk records, in
// chunk order (every thread computes the same values).
__device__ __forceinline__ Norm merge_records(const float* rec, int chunks) {
  Norm n;
  n.m1 = -INFINITY;
  n.m2 = -INFINITY;
  for (int c = 0; c < chunks; ++c) {
    n.m1 = fmaxf(n.m1, rec[c * kMixRec]);
    n.m2 = fmaxf(n.m2, rec[c * kMixRec + 3]);
  }
  float s1 = 0.f, q1 = 0.f, s2 = 0.f;
  for (int c = 0; c < chunks; ++c) {
    const float* r = rec + c * kMixRec;
    const float e1 = ex2((r[0] - n.m1) * kLog2e);
    s1 = __builtin_fmaf(r[1], e1, s1);
    q1 = __builtin_fmaf(r[2], e1 * e1, q1);
    s2 = __builtin_fmaf(r[4], ex2((r[3] - n.m2) * kLog2e), s2);
  }
  const float collision = q1 / (s1 * s1);
  n.alpha = __builtin_fmaf(0.5f, collision, 0.5f);
  n.w1 = n.alpha / s1;
  n.w2 = (1.f - n.alpha) / s2;
  return n;
}

// p_mix of the four tokens v..v+3 (explicit fused operations: the same bits in
// every kernel that evaluates them).
__device__ __forceinline__ float4 mix4(const float* l1, const float* l2, int v, const Norm& n) {
  const float4 a = *(const float4*)(l1 + v);
  const float4 c = *(const float4*)(l2 + v);
  float4 q;
  q.x = __builtin_fmaf(n.w1, ex2((a.x - n.m1) * kLog2e), n.w2 * ex2((c.x - n.m2) * kLog2e));
  q.y = __builtin_fmaf(n.w1, ex2((a.y - n.m1) * kLog2e), n.w2 * ex2((c.y - n.m2) * kLog2e));
  q.z = __builtin_fmaf(n.w1, ex2((a.z - n.m1) * kLog2e), n.w2 * ex2((c.z - n.m2) * kLog2e));
  q.w = __builtin_fmaf(n.w1, ex2((a.w - n.m1) * kLog2e), n.w2 * ex2((c.w - n.m2) * kLog2e));
  return q;
}

__device__ __forceinline__ uint64_t fixed(float q) { return (uint64_t)(q * kFix); }

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t x, int d) {
  const uint32_t lo = __shfl_up((uint32_t)x, d), hi = __shfl_up((uint32_t)(x >> 32), d);
  return ((uint64_t)hi << 32) | lo;
}

// Exclusive prefix of x over the workgroup in thread order, and the total
// (integers: exact). sh: kMixWaves words of LDS.
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t x, uint64_t* sh, uint64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up_u64(incl, d);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint64_t before = incl - x;
  total = 0;
#pragma unroll
  for (int w = 0; w < kMixWaves; ++w) {
    if (w < wave) before += sh[w];
    total += sh[w];
  }
  return before;
}

// First maximum (largest value, smallest token on ties) over the workgroup.
__device__ __forceinline__ void block_first_max(float& v, int& i, float* shv, int* shi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m);
    const int oi = __shfl_xor(i, m);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
  __syncthreads();
  if (lane == 0) {
    shv[wave] = v;
    shi[wave] = i;
  }
  __syncthreads();
  v = shv[0];
  i = shi[0];
#pragma unroll
  for (int w = 1; w < kMixWaves; ++w)
    if (shv[w] > v || (shv[w] == v && shi[w] < i)) {
      v = shv[w];
      i = shi[w];
    }
}

// Max (is_max) or sum over the workgroup, lanes then waves in a fixed order.
__device__ __forceinline__ float block_reduce(float v, float* sh, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < kMixWaves; ++w) r = is_max ? fmaxf(r, sh[w]) : r + sh[w];
  return r;
}
}  // namespace

// rec[b][chunk][0..4] = {m1, s1, q1, m2, s2}: m = the chunk's largest logit,
// s = sum e^(x - m), q = sum e^(2 (x - m)) (primary only).
__global__ __launch_bounds__(kMixThreads) void mix_stats_kernel(MixParams p) {
  __shared__ float sh[kMixWaves];
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int v0 = chunk * kMixChunk;
  const float* l1 = p.logits1 + (size_t)b * p.vocab;
  const float* l2 = p.logits2 + (size_t)b * p.vocab;
  float x1[kRun], x2[kRun];
#pragma unroll
  for (int i = 0; i < kRun / 4; ++i) {
    const int v = v0 + (i * kMixThreads + threadIdx.x) * 4;  // coalesced float4 runs
    const bool in = v < p.vocab;
    const float4 a = in ? *(const float4*)(l1 + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    const float4 c = in ? *(const float4*)(l2 + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    x1[4 * i] = a.x; x1[4 * i + 1] = a.y; x1[4 * i + 2] = a.z; x1[4 * i + 3] = a.w;
    x2[4 * i] = c.x; x2[4 * i + 1] = c.y; x2[4 * i + 2] = c.z; x2[4 * i + 3] = c.w;
  }
  float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    m1 = fmaxf(m1, x1[i]);
    m2 = fmaxf(m2, x2[i]);
  }
  m1 = block_reduce(m1, sh, true);
  m2 = block_reduce(m2, sh, true);
  float s1 = 0.f, q1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const float e1 = ex2((x1[i] - m1) * kLog2e);  // 0 for padding (-inf)
    s1 += e1;
    q1 += e1 * e1;
    s2 += ex2((x2[i] - m2) * kLog2e);
  }
  s1 = block_reduce(s1, sh, false);
  q1 = block_reduce(q1, sh, false);
  s2 = block_reduce(s2, sh, false);
  if (threadIdx.x == 0) {
    float* r = p.rec + ((size_t)b * p.chunks + chunk) * kMixRec;
    r[0] = m1; r[1] = s1; r[2] = q1; r[3] = m2; r[4] = s2;
  }
}

// crec[b][chunk] = {mass (low, high word), first maximum's value bits, its token};
// alpha[b] from chunk 0.
__global__ __launch_bounds__(kMixThreads) void mix_chunk_kernel(MixParams p) {
  __shared__ uint64_t shm[kMixWaves];
  __shared__ float shv[kMixWaves];
  __shared__ int shi[kMixWaves];
  const int chunk = blockIdx.x, b = blockIdx.y;
  const Norm n = merge_records(p.rec + (size_t)b * p.chunks * kMixRec, p.chunks);
  const float* l1 = p.logits1 + (size_t)b * p.vocab;
  const float* l2 = p.logits2 + (size_t)b * p.vocab;
  float* pm = p.p_mix ? p.p_mix + (size_t)b * p.vocab : nullptr;
  const int v0 = chunk * kMixChunk + threadIdx.x * kRun;
  uint64_t mass = 0;
  float bv = -1.f;
  int bi = p.vocab;
#pragma unroll
  for (int i = 0; i < kRun / 4; ++i) {
    const int v = v0 + 4 * i;
    if (v < p.vocab) {
      const float4 q = mix4(l1, l2, v, n);
      if (pm) *(float4*)(pm + v) = q;
      const float qs[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mass += fixed(qs[j]);
        if (qs[j] > bv) {
          bv = qs[j];
          bi = v + j;
        }
      }
    }
  }
  uint64_t total;
  block_excl_scan(mass, shm, total);
  block_first_max(bv, bi, shv, shi);
  if (threadIdx.x == 0) {
    uint32_t* r = p.crec + ((size_t)b * p.chunks + chunk) * 4;
    *(uint4*)r = make_uint4((uint32_t)total, (uint32_t)(total >> 32), __float_as_uint(bv), (uint32_t)bi);
    if (chunk == 0) p.alpha[b] = n.alpha;
  }
}

__global__ __launch_bounds__(kMixThreads) void mix_pick_kernel(MixParams p) {
  __shared__ uint64_t shm[kMixWaves];
  __shared__ float shv[kMixWaves];
  __shared__ int shi[kMixWaves];
  __shared__ int sel_chunk, sel_tok;
  __shared__ uint64_t sel_base;
  const int b = blockIdx.x, t = threadIdx.x;
  // normalisers first: their loads overlap the chunk records'
  const Norm n = merge_records(p.rec + (size_t)b * p.chunks * kMixRec, p.chunks);
  // ---- chunk level: one chunk record per thread ----
  uint64_t mass = 0;
  float bv = -1.f;
  int bi = p.vocab;
  if (t < p.chunks) {
    const uint4 r = *(const uint4*)(p.crec + ((size_t)b * p.chunks + t) * 4);
    mass = ((uint64_t)r.y << 32) | r.x;
    bv = __uint_as_float(r.z);
    bi = (int)r.w;
  }
  uint64_t total;
  const uint64_t before = block_excl_scan(mass, shm, total);
  const float u = fminf(fmaxf(p.u[b], 0.f), 0x1.fffffep-1f);  // clamped to [0, 1)
  uint64_t target = (uint64_t)((double)u * (double)total);
  if (target >= total) target = total - 1;  // total > 0: the largest p_mix is at least 1 / vocab
  if (before <= target && target < before + mass) {  // exactly one chunk: the intervals tile [0, total)
    sel_chunk = t;
    sel_base = before;
  }
  block_first_max(bv, bi, shv, shi);  // its barriers also publish sel_chunk and sel_base
  // ---- token level inside the chosen chunk: the masses mix_chunk_kernel summed ----
  const float* l1 = p.logits1 + (size_t)b * p.vocab;
  const float* l2 = p.logits2 + (size_t)b * p.vocab;
  const int v0 = sel_chunk * kMixChunk + t * kRun;
  uint64_t m[kRun];
  uint64_t run = 0;
#pragma unroll
  for (int i = 0; i < kRun / 4; ++i) {
    const int v = v0 + 4 * i;
    float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
    if (v < p.vocab) q = mix4(l1, l2, v, n);
    m[4 * i] = fixed(q.x);
    m[4 * i + 1] = fixed(q.y);
    m[4 * i + 2] = fixed(q.z);
    m[4 * i + 3] = fixed(q.w);
    run += m[4 * i] + m[4 * i + 1] + m[4 * i + 2] + m[4 * i + 3];
  }
  const uint64_t local = target - sel_base;  // below the chunk's mass
  if (t == 0) sel_tok = min(sel_chunk * kMixChunk + kMixChunk, p.vocab) - 1;  // not reached: one thread claims
  uint64_t chunk_total;
  uint64_t cum = block_excl_scan(run, shm, chunk_total);
  if (cum <= local && local < cum + run) {  // exactly one thread
    int tok = v0 + kRun - 1;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      cum += m[j];
      if (cum > local) {
        tok = v0 + j;
        break;
      }
    }
    sel_tok = tok;
  }
  __syncthreads();
  if (t == 0) {
    p.token[b] = sel_tok;
    p.greedy[b] = bi;
  }
}

size_t mixture_chunks(int vocab) { return (size_t)((vocab + kMixChunk - 1) / kMixChunk); }

hipError_t launch_mixture(const MixParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(mix_stats_kernel, dim3(p.chunks, p.batch), dim3(kMixThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mix_chunk_kernel, dim3(p.chunks, p.batch), dim3(kMixThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mix_pick_kernel, dim3(p.batch), dim3(kMixThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dfa
