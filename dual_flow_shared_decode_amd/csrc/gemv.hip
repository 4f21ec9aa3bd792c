// Dual-flow GEMV: both flows' activations against one read of a shared weight
// matrix ("Resumo Técnico: Dual-Flow Transformers", section "Arquitetura
// Central": the flows share the attention, MLP and output matrices; section
// "Custos de Inferência vs. Treinamento": decode reads the unique weights once
// for both flows), with the layer's epilogues: residual add, SwiGLU with the
// MLP-intermediate coupling b, the MLP-output coupling c, and the primary-only
// KV append ("Mecanismos Chave": coupling vectors at the MLP-intermediate and
// MLP-output levels, primary to auxiliary; "Arquitetura Central": only the
// primary flow writes the cache).
//
// Y_f = X_f W^T for W [n, k] (bf16) and X_f [batch, k] (fp32), on
// v_mfma_f32_16x16x32_bf16 with the weights as the A operand (16 rows x 32
// columns of k) and the activations as B (32 k x 16 activation rows). The
// weights are stored in 16 x 8 tiles ([n/16][k/8][16][8], dfa_pack_weight), so a
// wave's operand load for one k-step reads 4 tiles = 1 KB contiguous, streamed
// with non-temporal loads. Activations are split x = hi + lo (hi = bf16(x),
// lo = bf16(x - hi)) and both halves accumulate into the same fp32 result; when
// every activation is exactly bf16 the low halves are skipped.
//
// Activation rows: flow f, sequence s is MFMA column block f*CBF + s/16, column
// s % 16 (each flow padded to CBF*16 rows), so the two flows of a sequence end
// up in the same lane and register -- the couplings are elementwise.
//
// Workgroup = 4 waves = 128 weight rows (2 tiles of 16 per wave) x one k-range
// (split-K). Per 128-column chunk the workgroup converts the activations to
// hi/lo bf16 in LDS, laid out as the B operand ([block][k/8][16][8]). Partial
// sums go to the workspace [k-split][matrix][row][n]; gemv_finalize sums them
// in a fixed order and applies the epilogue.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dfa_internal.h"

namespace dfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kTilesPerWave = 2;
constexpr int kRowsPerWg = 16 * kTilesPerWave * kGemvWaves;  // 128 weight rows
constexpr int kChunk = 128;                                  // k columns staged per step
constexpr int kKSteps = kChunk / 32;

// ---------------------------------------------------------------- packing
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                          int n, int k) {
  // one thread per 8-element group: tile (nt, kg), row r
  const size_t groups = (size_t)n * (k / 8);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < groups; i += (size_t)gridDim.x * blockDim.x) {
    const size_t row = i / (k / 8), kg = i - row * (k / 8);
    const size_t nt = row / 16, r = row - nt * 16;
    const uint4 v = *(const uint4*)(w + row * k + kg * 8);
    *(uint4*)(wt + ((nt * (k / 8) + kg) * 16 + r) * 8) = v;
  }
}

hipError_t launch_pack_weight(const uint16_t* w, uint16_t* wt, int n, int k, hipStream_t stream) {
  const size_t groups = (size_t)n * (k / 8);
  const size_t want = (groups + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_weight_kernel, dim3(blocks), dim3(256), 0, stream, w, wt, n, k);
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMV
__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// NCB: activation column blocks (flows * CBF); PAIR: a second matrix (w2) on the
// same activations; LO: split activations into hi + lo.
template <int NCB, bool PAIR, bool LO>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvParams p) {
  constexpr int NH = LO ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][NH][NCB][kChunk / 8][16][8];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int ks = blockIdx.y;
  const int k_begin = ks * p.k_range, k_end = min(k_begin + p.k_range, p.k);
  const int nchunks = (k_end - k_begin) / kChunk;
  const int kg_total = p.k / 8;
  const int tile0 = (blockIdx.x * kRowsPerWg) / 16 + wave * kTilesPerWave;  // first 16-row tile of this wave

  // stage activation chunk c (columns k_begin + c*kChunk ..) into xs[buf]
  auto stage = [&](int c, int buf) {
    const int kc = k_begin + c * kChunk;
    for (int item = threadIdx.x; item < NCB * 16 * (kChunk / 8); item += kGemvThreads) {
      const int kg = item % (kChunk / 8);
      const int m = item / (kChunk / 8);  // padded activation row: block m/16, column m%16
      const int cb = m / 16, f = cb / p.cbf, s = (cb - f * p.cbf) * 16 + (m & 15);
      float v[8];
      if (s < p.batch) {
        const float* src = (f ? p.x2 : p.x1) + (size_t)s * p.k + kc + kg * 8;
        const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
      }
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hi[j] = (__bf16)v[j];
        lo[j] = (__bf16)(v[j] - (float)hi[j]);
      }
      *(bf16x8*)&xs[buf][0][cb][kg][m & 15][0] = hi;
      if (LO) *(bf16x8*)&xs[buf][NH - 1][cb][kg][m & 15][0] = lo;
    }
  };

  // weight operands of one chunk: per tile and k-step, row `col` of the tile, 8 columns
  struct WChunk {
    bf16x8 a[kTilesPerWave][kKSteps];
    bf16x8 b[PAIR ? kTilesPerWave : 1][kKSteps];
  };
  auto load_w = [&](int c, WChunk& wc) {
    const int kg0 = (k_begin + c * kChunk) / 8;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const size_t base = (((size_t)(tile0 + t) * kg_total + kg0 + grp) * 16 + col) * 8;
#pragma unroll
      for (int st = 0; st < kKSteps; ++st) {
        wc.a[t][st] = __builtin_nontemporal_load((const bf16x8*)(p.w + base + (size_t)st * 4 * 16 * 8));
        if (PAIR) wc.b[t][st] = __builtin_nontemporal_load((const bf16x8*)(p.w2 + base + (size_t)st * 4 * 16 * 8));
      }
    }
  };

  f32x4 acc[kTilesPerWave][NCB], acc2[PAIR ? kTilesPerWave : 1][NCB];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      acc[t][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (PAIR) acc2[t][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  WChunk wnext;
  if (nchunks > 0) {
    load_w(0, wnext);
    stage(0, 0);
  }
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    WChunk wc = wnext;
    if (c + 1 < nchunks) {
      load_w(c + 1, wnext);
      stage(c + 1, buf ^ 1);
    }
#pragma unroll
    for (int st = 0; st < kKSteps; ++st) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const bf16x8 xb = *(const bf16x8*)&xs[buf][h][cb][4 * st + grp][col][0];
#pragma unroll
          for (int t = 0; t < kTilesPerWave; ++t) {
            acc[t][cb] = mfma(wc.a[t][st], xb, acc[t][cb]);
            if (PAIR) acc2[t][cb] = mfma(wc.b[t][st], xb, acc2[t][cb]);
          }
        }
      }
    }
    __syncthreads();
  }

  // partial sums: part[ks][mat][m][n], lane holds rows m = cb*16 + col, n = tile*16 + 4*grp + i
  const size_t mat_stride = (size_t)p.m_pad * p.n;
  float* out = p.part + (size_t)ks * (PAIR ? 2 : 1) * mat_stride;
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int n0 = (tile0 + t) * 16 + 4 * grp;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const size_t off = (size_t)(cb * 16 + col) * p.n + n0;
      *(f32x4*)(out + off) = acc[t][cb];
      if (PAIR) *(f32x4*)(out + mat_stride + off) = acc2[t][cb];
    }
  }
}

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ float silu(float u) { return u / (1.f + __expf(-u)); }

// Round to the nearest bf16, ties to even (finite inputs).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One thread per (sequence s, column n): both flows' sums over the k-splits
// (fixed order), then the epilogue.
__global__ __launch_bounds__(256) void gemv_finalize_kernel(GemvParams p) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int s = blockIdx.y;
  if (n >= p.n) return;
  const size_t mat_stride = (size_t)p.m_pad * p.n;
  const int mats = p.pair ? 2 : 1;
  float y[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // [flow][matrix]
  for (int f = 0; f < p.flows; ++f) {
    const size_t m = (size_t)(f * p.cbf * 16 + s);
    for (int ks = 0; ks < p.k_split; ++ks)
      for (int mat = 0; mat < mats; ++mat) y[f][mat] += p.part[((size_t)ks * mats + mat) * mat_stride + m * p.n + n];
  }
  const size_t o = (size_t)s * p.n + n;
  switch (p.epilogue) {
    case kEpiNone:
      p.y1[o] = y[0][0];
      if (p.flows == 2) p.y2[o] = y[1][0];
      break;
    case kEpiResidual:
      p.y1[o] = p.res1[o] + y[0][0];
      if (p.flows == 2) p.y2[o] = p.res2[o] + y[1][0];
      break;
    case kEpiSwiglu: {
      const float z1 = silu(y[0][0]) * y[0][1];
      p.y1[o] = z1;
      if (p.flows == 2) {
        const float z2 = silu(y[1][0]) * y[1][1];
        p.y2[o] = p.couple ? fmaf(p.couple[n], z1, z2) : z2;
      }
      break;
    }
    case kEpiResidualCoupled: {
      p.y1[o] = p.res1[o] + y[0][0];
      if (p.flows == 2) p.y2[o] = p.res2[o] + (p.couple ? fmaf(p.couple[n], y[0][0], y[1][0]) : y[1][0]);
      break;
    }
    case kEpiKvAppend: {
      // primary only: k = row n of W, v = row n of W2, appended at position ctx_lens[s]
      if (p.y1) p.y1[o] = y[0][0];
      if (p.y2) p.y2[o] = y[0][1];
      const int bs = 1 << p.kv_bs_log2;
      int pos = p.kv_ctx[s];
      pos = pos < 0 ? 0 : (pos >= p.kv_max_blocks * bs ? p.kv_max_blocks * bs - 1 : pos);
      int blk = p.kv_table[(size_t)s * p.kv_max_blocks + (pos >> p.kv_bs_log2)];
      blk = blk < 0 ? 0 : (blk >= p.kv_num_blocks ? p.kv_num_blocks - 1 : blk);
      const int g = n / p.kv_head_dim, d = n - g * p.kv_head_dim, slot = pos & (bs - 1);
      const size_t head = (size_t)blk * p.kv_hkv * p.kv_head_dim * bs + (size_t)g * p.kv_head_dim * bs;
      // keys [bs/16][D/8][16][8], values [bs/16][D][16] inside a block and kv head
      p.kv_k[head + (size_t)(slot >> 4) * p.kv_head_dim * 16 + (size_t)(d >> 3) * 128 + (slot & 15) * 8 + (d & 7)] =
          bf16_rne(y[0][0]);
      p.kv_v[head + (size_t)(slot >> 4) * p.kv_head_dim * 16 + (size_t)d * 16 + (slot & 15)] = bf16_rne(y[0][1]);
      break;
    }
  }
}

hipError_t launch_gemv(const GemvParams& p, hipStream_t stream) {
  const dim3 grid(p.n / kRowsPerWg, p.k_split), block(kGemvThreads);
  const int ncb = p.flows * p.cbf;
  const bool lo = !p.x_exact;
#define DFA_GEMV_CASE(NCB_, PAIR_, LO_)                                                          \
  if (ncb == NCB_ && p.pair == PAIR_ && lo == LO_) {                                             \
    hipLaunchKernelGGL((gemv_kernel<NCB_, PAIR_, LO_>), grid, block, 0, stream, p);              \
    return hipGetLastError();                                                                    \
  }
  DFA_GEMV_CASE(1, false, false) DFA_GEMV_CASE(1, false, true) DFA_GEMV_CASE(1, true, false)
  DFA_GEMV_CASE(1, true, true) DFA_GEMV_CASE(2, false, false) DFA_GEMV_CASE(2, false, true)
  DFA_GEMV_CASE(2, true, false) DFA_GEMV_CASE(2, true, true) DFA_GEMV_CASE(4, false, false)
  DFA_GEMV_CASE(4, false, true) DFA_GEMV_CASE(4, true, false) DFA_GEMV_CASE(4, true, true)
#undef DFA_GEMV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_finalize(const GemvParams& p, hipStream_t stream) {
  const dim3 grid((p.n + 255) / 256, p.batch), block(256);
  hipLaunchKernelGGL(gemv_finalize_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

size_t gemv_rows_per_workgroup() { return kRowsPerWg; }
size_t gemv_chunk() { return kChunk; }

}  // namespace dfa
