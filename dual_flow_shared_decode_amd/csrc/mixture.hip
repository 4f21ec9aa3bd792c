// Mixture of the two flows' next-token distributions and its decoding
// ("Resumo Técnico: Dual-Flow Transformers", section "Mecanismos Chave",
// mixture objective: p_mix = alpha p_primary + (1 - alpha) p_aux, alpha set
// from the primary's collision probability, the primary keeping at least half
// of the weight). This library's reading of alpha: (1 + sum_v p1(v)^2) / 2.
//
// Vocabularies of at most kMixFusedMaxVocab tokens take one launch,
// mix_fused_kernel, one workgroup per sequence holding the sequence's logits
// in registers. Larger ones take three launches on the flows' float32 logits
// [batch, vocab], the vocabulary cut into chunks of kMixChunk tokens:
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
// meets the same sums at every level (chunk or wave, row, token). A token below
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

// The sequence's chunk records copied to LDS (thread t: record t; one load
// round trip for all of them), for merge_records.
__device__ __forceinline__ void stage_records(const float* rec, int chunks, float (*srec)[kMixRec]) {
  const int t = threadIdx.x;
  if (t < chunks) {
    const float4 a = *(const float4*)(rec + (size_t)t * kMixRec);
    const float4 c = *(const float4*)(rec + (size_t)t * kMixRec + 4);
    srec[t][0] = a.x; srec[t][1] = a.y; srec[t][2] = a.z; srec[t][3] = a.w; srec[t][4] = c.x;
  }
  __syncthreads();
}

// The sequence's softmax normalisers and alpha from its chunk records (in
// LDS), in chunk order (every thread computes the same values).
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
__device__ __forceinline__ float4 mix4v(const float4& a, const float4& c, const Norm& n) {
  float4 q;
  q.x = __builtin_fmaf(n.w1, ex2((a.x - n.m1) * kLog2e), n.w2 * ex2((c.x - n.m2) * kLog2e));
  q.y = __builtin_fmaf(n.w1, ex2((a.y - n.m1) * kLog2e), n.w2 * ex2((c.y - n.m2) * kLog2e));
  q.z = __builtin_fmaf(n.w1, ex2((a.z - n.m1) * kLog2e), n.w2 * ex2((c.z - n.m2) * kLog2e));
  q.w = __builtin_fmaf(n.w1, ex2((a.w - n.m1) * kLog2e), n.w2 * ex2((c.w - n.m2) * kLog2e));
  return q;
}

__device__ __forceinline__ float4 mix4(const float* l1, const float* l2, int v, const Norm& n) {
  return mix4v(*(const float4*)(l1 + v), *(const float4*)(l2 + v), n);
}

// Integer mass of a probability: q * 2^35 truncated; 0 for NaN (a row with a
// non-finite logit), so no conversion of a non-finite value happens.
__device__ __forceinline__ uint64_t fixed(float q) { return q > 0.f ? (uint64_t)(fminf(q, 1.f) * kFix) : 0; }

// Wave all-reductions through vector ALU lane exchanges (no LDS). Step S
// gives each lane its own word and its partner's (in some order: the
// combining operation is symmetric): quad_perm xor 1 and xor 2, then the
// half-row and row mirrors -- which pair quads and half-rows as xor 4 and
// xor 8 would, once quads and then half-rows hold one value -- then the 16-
// and 32-lane permlane swaps. The combination tree is fixed: every lane ends
// with the same bits, run after run.
template <int S>
__device__ __forceinline__ void xpair(uint32_t x, uint32_t& a, uint32_t& b) {
  if constexpr (S < 4) {
    constexpr int kCtrl = S == 0 ? 0xB1 : (S == 1 ? 0x4E : (S == 2 ? 0x141 : 0x140));
    a = x;
    b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, false);
  } else if constexpr (S == 4) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = p[0];
    b = p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = p[0];
    b = p[1];
  }
}

template <int S>
__device__ __forceinline__ float xsum_step(float x) {
  uint32_t a, b;
  xpair<S>(__float_as_uint(x), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
template <int S>
__device__ __forceinline__ float xmax_step(float x) {
  uint32_t a, b;
  xpair<S>(__float_as_uint(x), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

__device__ __forceinline__ float wave_allsum(float x) {
  x = xsum_step<0>(x); x = xsum_step<1>(x); x = xsum_step<2>(x);
  x = xsum_step<3>(x); x = xsum_step<4>(x); return xsum_step<5>(x);
}
__device__ __forceinline__ float wave_allmax(float x) {
  x = xmax_step<0>(x); x = xmax_step<1>(x); x = xmax_step<2>(x);
  x = xmax_step<3>(x); x = xmax_step<4>(x); return xmax_step<5>(x);
}

template <int S>
__device__ __forceinline__ uint64_t xsum64_step(uint64_t x) {
  uint32_t al, bl, ah, bh;
  xpair<S>((uint32_t)x, al, bl);
  xpair<S>((uint32_t)(x >> 32), ah, bh);
  return (((uint64_t)ah << 32) | al) + (((uint64_t)bh << 32) | bl);
}
__device__ __forceinline__ uint64_t wave_allsum_u64(uint64_t x) {
  x = xsum64_step<0>(x); x = xsum64_step<1>(x); x = xsum64_step<2>(x);
  x = xsum64_step<3>(x); x = xsum64_step<4>(x); return xsum64_step<5>(x);
}

// (value, index) pair: the larger value, the smaller index on ties.
template <int S>
__device__ __forceinline__ void xfirstmax_step(float& v, int& i) {
  uint32_t va, vb, ia, ib;
  xpair<S>(__float_as_uint(v), va, vb);
  xpair<S>((uint32_t)i, ia, ib);
  const float fa = __uint_as_float(va), fb = __uint_as_float(vb);
  const bool take_b = fb > fa || (fb == fa && (int)ib < (int)ia);
  v = take_b ? fb : fa;
  i = take_b ? (int)ib : (int)ia;
}
__device__ __forceinline__ void wave_first_max(float& v, int& i) {
  xfirstmax_step<0>(v, i); xfirstmax_step<1>(v, i); xfirstmax_step<2>(v, i);
  xfirstmax_step<3>(v, i); xfirstmax_step<4>(v, i); xfirstmax_step<5>(v, i);
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t x, int d) {
  const uint32_t lo = __shfl_up((uint32_t)x, d), hi = __shfl_up((uint32_t)(x >> 32), d);
  return ((uint64_t)hi << 32) | lo;
}

// Exclusive prefix of x over the workgroup in thread order, and the total
// (integers: exact). sh: NW words of LDS.
template <int NW>
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
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += sh[w];
    total += sh[w];
  }
  return before;
}

// First maximum (largest value, smallest token on ties) over the workgroup.
template <int NW>
__device__ __forceinline__ void block_first_max(float& v, int& i, float* shv, int* shi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_first_max(v, i);
  __syncthreads();
  if (lane == 0) {
    shv[wave] = v;
    shi[wave] = i;
  }
  __syncthreads();
  v = shv[0];
  i = shi[0];
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (shv[w] > v || (shv[w] == v && shi[w] < i)) {
      v = shv[w];
      i = shi[w];
    }
}

// Max (is_max) or sum over the workgroup, lanes then waves in a fixed order.
__device__ __forceinline__ float block_reduce(float v, float* sh, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = is_max ? wave_allmax(v) : wave_allsum(v);
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
  __shared__ float srec[kMixMaxChunks][kMixRec];
  const int chunk = blockIdx.x, b = blockIdx.y;
  // the chunk's logits are loaded first: their round trip overlaps the records'
  const float* l1 = p.logits1 + (size_t)b * p.vocab;
  const float* l2 = p.logits2 + (size_t)b * p.vocab;
  const int v0 = chunk * kMixChunk + threadIdx.x * kRun;
  float4 la[kRun / 4], lc[kRun / 4];
#pragma unroll
  for (int i = 0; i < kRun / 4; ++i) {
    const int v = v0 + 4 * i;
    la[i] = v < p.vocab ? *(const float4*)(l1 + v) : make_float4(0.f, 0.f, 0.f, 0.f);
    lc[i] = v < p.vocab ? *(const float4*)(l2 + v) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  stage_records(p.rec + (size_t)b * p.chunks * kMixRec, p.chunks, srec);
  const Norm n = merge_records(&srec[0][0], p.chunks);
  float* pm = p.p_mix ? p.p_mix + (size_t)b * p.vocab : nullptr;
  uint64_t mass = 0;
  float bv = -1.f;
  int bi = p.vocab;
#pragma unroll
  for (int i = 0; i < kRun / 4; ++i) {
    const int v = v0 + 4 * i;
    if (v < p.vocab) {
      const float4 q = mix4v(la[i], lc[i], n);
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
  block_excl_scan<kMixWaves>(mass, shm, total);
  block_first_max<kMixWaves>(bv, bi, shv, shi);
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
  __shared__ float srec[kMixMaxChunks][kMixRec];
  const int b = blockIdx.x, t = threadIdx.x;
  // ---- chunk level: one chunk record per thread (loaded with the statistics) ----
  uint64_t mass = 0;
  float bv = -1.f;
  int bi = p.vocab;
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  if (t < p.chunks) r = *(const uint4*)(p.crec + ((size_t)b * p.chunks + t) * 4);
  stage_records(p.rec + (size_t)b * p.chunks * kMixRec, p.chunks, srec);
  const Norm n = merge_records(&srec[0][0], p.chunks);
  if (t < p.chunks) {
    mass = ((uint64_t)r.y << 32) | r.x;
    bv = __uint_as_float(r.z);
    bi = (int)r.w;
  }
  // Defaults for a row no chunk claims (a row whose mixture has no finite
  // mass, from a non-finite logit): chunk 0 at base 0. The scan's barriers
  // publish them before any thread may overwrite them.
  if (t == 0) {
    sel_chunk = 0;
    sel_base = 0;
  }
  uint64_t total;
  const uint64_t before = block_excl_scan<kMixWaves>(mass, shm, total);
  const float u = fminf(fmaxf(p.u[b], 0.f), 0x1.fffffep-1f);  // clamped to [0, 1)
  uint64_t target = (uint64_t)((double)u * (double)total);
  if (total > 0 && target >= total) target = total - 1;  // the largest p_mix is at least 1 / vocab
  if (total > 0 && before <= target && target < before + mass) {  // one chunk: the intervals tile [0, total)
    sel_chunk = t;
    sel_base = before;
  }
  block_first_max<kMixWaves>(bv, bi, shv, shi);  // its barriers also publish sel_chunk and sel_base
  if (total == 0) {  // workgroup-uniform: nothing to draw from; the defined token is the last one
    if (t == 0) {
      p.token[b] = p.vocab - 1;
      p.greedy[b] = bi < p.vocab ? bi : p.vocab - 1;
    }
    return;
  }
  // ---- token level inside the chosen chunk: the masses mix_chunk_kernel summed ----
  const float* l1 = p.logits1 + (size_t)b * p.vocab;
  const float* l2 = p.logits2 + (size_t)b * p.vocab;
  const int chunk_sel = min(max(sel_chunk, 0), p.chunks - 1);
  const int v0 = chunk_sel * kMixChunk + t * kRun;
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
  if (t == 0) sel_tok = min(chunk_sel * kMixChunk + kMixChunk, p.vocab) - 1;  // not reached: one thread claims
  uint64_t chunk_total;
  uint64_t cum = block_excl_scan<kMixWaves>(run, shm, chunk_total);
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
    p.greedy[b] = bi < p.vocab ? bi : p.vocab - 1;
  }
}

namespace {
constexpr int kFuseThreads = 1024;
constexpr int kFuseWaves = kFuseThreads / 64;
constexpr int kFuseRows = 8;  // float4 groups per lane and flow
static_assert(kFuseWaves * 64 * kFuseRows * 4 == kMixFusedMaxVocab, "one token per register slot");

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) { return wave_allsum_u64(x); }

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up_u64(x, d);
    if (lane >= d) x += o;
  }
  return x;
}

__device__ __forceinline__ float wave_max(float v) { return wave_allmax(v); }

__device__ __forceinline__ float wave_sum(float v) { return wave_allsum(v); }
}  // namespace

// The whole mixture of one sequence in one workgroup, for vocabularies of at
// most kMixFusedMaxVocab tokens: wave w holds tokens [2048 w, 2048 w + 2048)
// of both flows in registers (lane l, row i: the four tokens of group
// 64 i + l, so every load instruction reads 1 KB of consecutive logits). One
// read of the logits gives the softmax statistics, alpha, p_mix, the greedy
// token and the inverse-CDF token. The draw follows the token order from the
// outside in: the wave whose tokens hold the target (wave totals, in wave
// order), then the row of that wave (row totals, in row order), then the lane
// (a scan over the row), then the token among the lane's four. The masses and
// the rule are those of the chunked kernels: p_mix scaled by 2^35 and
// truncated, target = floor(u total).
__global__ __launch_bounds__(kFuseThreads) void mix_fused_kernel(MixParams p) {
  __shared__ float shs[kFuseWaves][3];
  __shared__ uint64_t shm[kFuseWaves];
  __shared__ float shv[kFuseWaves];
  __shared__ int shi[kFuseWaves];
  __shared__ int sel_tok;
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* l1 = p.logits1 + (size_t)b * p.vocab;
  const float* l2 = p.logits2 + (size_t)b * p.vocab;
  const int g0 = wave * (64 * kFuseRows) + lane;  // group of row 0; row i adds 64 i
  float4 x1[kFuseRows], x2[kFuseRows];
#pragma unroll
  for (int i = 0; i < kFuseRows; ++i) {
    const int v = (g0 + 64 * i) * 4;
    const bool in = v < p.vocab;  // the vocabulary is a multiple of 4: a group is all in or all out
    x1[i] = in ? *(const float4*)(l1 + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    x2[i] = in ? *(const float4*)(l2 + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  // ---- softmax statistics: maxima, then sums in a fixed order ----
  float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
  for (int i = 0; i < kFuseRows; ++i) {
    m1 = fmaxf(m1, fmaxf(fmaxf(x1[i].x, x1[i].y), fmaxf(x1[i].z, x1[i].w)));
    m2 = fmaxf(m2, fmaxf(fmaxf(x2[i].x, x2[i].y), fmaxf(x2[i].z, x2[i].w)));
  }
  m1 = wave_max(m1);
  m2 = wave_max(m2);
  if (lane == 0) {
    shs[wave][0] = m1;
    shs[wave][1] = m2;
  }
  __syncthreads();
  m1 = shs[0][0];
  m2 = shs[0][1];
#pragma unroll
  for (int w = 1; w < kFuseWaves; ++w) {
    m1 = fmaxf(m1, shs[w][0]);
    m2 = fmaxf(m2, shs[w][1]);
  }
  float s1 = 0.f, q1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < kFuseRows; ++i) {
    const float a[4] = {x1[i].x, x1[i].y, x1[i].z, x1[i].w};
    const float c[4] = {x2[i].x, x2[i].y, x2[i].z, x2[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e1 = ex2((a[j] - m1) * kLog2e);  // 0 for padding (-inf)
      s1 += e1;
      q1 += e1 * e1;
      s2 += ex2((c[j] - m2) * kLog2e);
    }
  }
  s1 = wave_sum(s1);
  q1 = wave_sum(q1);
  s2 = wave_sum(s2);
  __syncthreads();  // every wave has read the maxima
  if (lane == 0) {
    shs[wave][0] = s1;
    shs[wave][1] = q1;
    shs[wave][2] = s2;
  }
  __syncthreads();
  s1 = shs[0][0];
  q1 = shs[0][1];
  s2 = shs[0][2];
#pragma unroll
  for (int w = 1; w < kFuseWaves; ++w) {
    s1 += shs[w][0];
    q1 += shs[w][1];
    s2 += shs[w][2];
  }
  Norm n;
  n.m1 = m1;
  n.m2 = m2;
  n.alpha = __builtin_fmaf(0.5f, q1 / (s1 * s1), 0.5f);
  n.w1 = n.alpha / s1;
  n.w2 = (1.f - n.alpha) / s2;
  // ---- p_mix, the masses and the first maximum ----
  float* pm = p.p_mix ? p.p_mix + (size_t)b * p.vocab : nullptr;
  float4 q[kFuseRows];
  uint64_t mrow[kFuseRows];
  uint64_t mine = 0;
  float bv = -1.f;
  int bi = p.vocab;
#pragma unroll
  for (int i = 0; i < kFuseRows; ++i) {
    const int v = (g0 + 64 * i) * 4;
    q[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    mrow[i] = 0;
    if (v < p.vocab) {
      const float a[4] = {x1[i].x, x1[i].y, x1[i].z, x1[i].w};
      const float c[4] = {x2[i].x, x2[i].y, x2[i].z, x2[i].w};
      float r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[j] = __builtin_fmaf(n.w1, ex2((a[j] - n.m1) * kLog2e), n.w2 * ex2((c[j] - n.m2) * kLog2e));
        mrow[i] += fixed(r[j]);
        if (r[j] > bv) {  // tokens of a lane rise with i and j: the first maximum stays
          bv = r[j];
          bi = v + j;
        }
      }
      q[i] = make_float4(r[0], r[1], r[2], r[3]);
      if (pm) *(float4*)(pm + v) = q[i];
    }
    mine += mrow[i];
  }
  // ---- the draw: wave, row, lane, token ----
  const uint64_t wtot = wave_sum_u64(mine);
  if (lane == 0) shm[wave] = wtot;
  if (threadIdx.x == 0) sel_tok = p.vocab - 1;  // not reached: one lane claims
  block_first_max<kFuseWaves>(bv, bi, shv, shi);  // its barriers also publish shm and sel_tok
  uint64_t total = 0, wbefore = 0;
#pragma unroll
  for (int w = 0; w < kFuseWaves; ++w) {
    if (w < wave) wbefore += shm[w];
    total += shm[w];
  }
  const float u = fminf(fmaxf(p.u[b], 0.f), 0x1.fffffep-1f);  // clamped to [0, 1)
  uint64_t target = (uint64_t)((double)u * (double)total);
  if (total > 0 && target >= total) target = total - 1;  // the largest p_mix is at least 1 / vocab
  // total == 0 (no finite mass): no wave claims and the token stays vocab - 1
  if (total > 0 && wbefore <= target && target < wbefore + wtot) {  // one wave: the intervals tile [0, total)
    const uint64_t local = target - wbefore;
    uint64_t rbase = 0, mr = 0, lane_mass = 0;
    int row = -1;
    float4 qr = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kFuseRows; ++i) {
      const uint64_t t_i = wave_sum_u64(mrow[i]);
      if (row < 0) {
        if (local < rbase + t_i) {
          row = i;
          lane_mass = mrow[i];
          qr = q[i];
        } else {
          rbase += t_i;
        }
      }
    }
    mr = local - rbase;  // below the row's total
    const uint64_t incl = wave_incl_scan_u64(lane_mass);
    uint64_t cum = incl - lane_mass;
    if (cum <= mr && mr < incl) {  // exactly one lane
      const float r[4] = {qr.x, qr.y, qr.z, qr.w};
      const int v = (g0 + 64 * row) * 4;
      int tok = v + 3;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cum += fixed(r[j]);
        if (cum > mr) {
          tok = v + j;
          break;
        }
      }
      sel_tok = tok;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p.token[b] = sel_tok;
    p.greedy[b] = bi < p.vocab ? bi : p.vocab - 1;  // bi == vocab only for a row with no finite mass
    p.alpha[b] = n.alpha;
  }
}

size_t mixture_chunks(int vocab) { return (size_t)((vocab + kMixChunk - 1) / kMixChunk); }

hipError_t launch_mixture(const MixParams& p, hipStream_t stream) {
  if (p.vocab <= kMixFusedMaxVocab) {
    hipLaunchKernelGGL(mix_fused_kernel, dim3(p.batch), dim3(kFuseThreads), 0, stream, p);
    return hipGetLastError();
  }
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
