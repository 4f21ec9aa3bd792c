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
// up in the same lane and register.
//
// Workgroup = 8 math waves + 8 loader waves. The math waves cover 64 weight
// rows (four 16-row tiles, of each matrix; two wave groups split the k-steps
// of every stage, so each SIMD runs two math waves that share the stage's B
// operands) or 128 rows (eight tiles, one wave each) x one k-range
// (split-K). A tile takes its weights from one of up to three matrices by row
// range, so one launch can cover stacked matrices (the layer's [Wq; Wk; Wv]).
// The k-range is streamed in 128-column stages. The math waves keep three
// stages of weights in flight in registers (two for paired 128-row tiles)
// and only wait for their own loads; the loader waves keep two stages of raw
// activations in flight and, per stage, convert the next stage's activations
// to hi/lo bf16 in LDS (double-buffered; per column block, row r's 8-column
// groups are stored in slot group ^ r so that both the conversion's writes
// and the MFMA operand reads are free of bank conflicts), at raised wave
// priority since the conversion gates the stage. One barrier per stage hands
// the buffers over. Loads complete in issue order within a wave, so a wave
// that fetched both would wait for its weights before it could convert
// activations; split this way the GEMVs of the layer shapes run 8-12%
// faster. With one k-range the epilogue runs
// in the same kernel; otherwise partial sums go to the workspace
// [k-split][matrix][row][n] and gemv_finalize adds them in a fixed order and
// applies the epilogue (so the primary flow's results never depend on the
// auxiliary flow's inputs).
#include <hip/hip_runtime.h>
#include <math.h>

#include "dfa_internal.h"
#include "ops_internal.h"

namespace dfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
namespace {
constexpr int kGemvWaves = 8;  // waves on the weights and MFMAs
constexpr int kLoadWaves = 8;  // waves fetching and converting activations (4: no faster; 2: spills)
constexpr int kMathThreads = 64 * kGemvWaves;
constexpr int kLoadThreads = 64 * kLoadWaves;
constexpr int kGemvThreads = kMathThreads + kLoadThreads;
constexpr int kStage = 128;                    // k columns per pipeline stage
constexpr int kSteps = kStage / 32;            // MFMA k-steps per stage
static_assert(kStage / 8 == 16, "the LDS swizzle pairs 16 column groups with 16 rows");
}  // namespace

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float u) { return u / (1.f + __expf(-u)); }

// Round to the nearest bf16, ties to even (finite inputs).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void store4(float* dst, const float (&v)[4]) {
  *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
}

// Writes the primary flow's key k[0..3] and value v[0..3] for kv columns
// c0..c0+3 (kv head c0 / head_dim) at position ctx_lens[s] of sequence s,
// rounded to bf16.
__device__ __forceinline__ void kv_append(const GemvParams& p, int s, int c0, const float (&k)[4], const float (&v)[4]) {
  const int bs = 1 << p.kv_bs_log2;
  int pos = p.kv_ctx[s];
  pos = pos < 0 ? 0 : (pos >= p.kv_max_blocks * bs ? p.kv_max_blocks * bs - 1 : pos);
  int blk = p.kv_table[(size_t)s * p.kv_max_blocks + (pos >> p.kv_bs_log2)];
  blk = blk < 0 ? 0 : (blk >= p.kv_num_blocks ? p.kv_num_blocks - 1 : blk);
  const int g = c0 / p.kv_head_dim, d = c0 - g * p.kv_head_dim, slot = pos & (bs - 1);
  const size_t head = (size_t)blk * p.kv_hkv * p.kv_head_dim * bs + (size_t)g * p.kv_head_dim * bs;
  const size_t tile = head + (size_t)(slot >> 4) * p.kv_head_dim * 16;
  // keys [bs/16][D/8][16][8]: dims d..d+3 are consecutive inside one 8-dim group
  uint2 kb;
  kb.x = (uint32_t)bf16_rne(k[0]) | ((uint32_t)bf16_rne(k[1]) << 16);
  kb.y = (uint32_t)bf16_rne(k[2]) | ((uint32_t)bf16_rne(k[3]) << 16);
  *(uint2*)(p.kv_k + tile + (size_t)(d >> 3) * 128 + (slot & 15) * 8 + (d & 7)) = kb;
  // values [bs/16][D][16]: one element per dim
#pragma unroll
  for (int j = 0; j < 4; ++j) p.kv_v[tile + (size_t)(d + j) * 16 + (slot & 15)] = bf16_rne(v[j]);
}

// Epilogue of one sequence s and four consecutive columns n0..n0+3, from the
// sums y[flow][matrix][j] of both flows (flow 2 unused with one flow); o1, o2:
// element offsets of the outputs (and residuals) of the two flows.
__device__ __forceinline__ void apply_epilogue(const GemvParams& p, int s, size_t o1, size_t o2, int n0,
                                               const float (&y)[2][2][4]) {
  const bool two = p.flows == 2;
  float r1[4], r2[4];
  switch (p.epilogue) {
    case kEpiNone:
      store4(p.y1 + o1, y[0][0]);
      if (two) store4(p.y2 + o2, y[1][0]);
      break;
    case kEpiResidual: {
      const float4 a = *(const float4*)(p.res1 + o1);
      r1[0] = a.x + y[0][0][0]; r1[1] = a.y + y[0][0][1]; r1[2] = a.z + y[0][0][2]; r1[3] = a.w + y[0][0][3];
      store4(p.y1 + o1, r1);
      if (two) {
        const float4 b = *(const float4*)(p.res2 + o2);
        r2[0] = b.x + y[1][0][0]; r2[1] = b.y + y[1][0][1]; r2[2] = b.z + y[1][0][2]; r2[3] = b.w + y[1][0][3];
        store4(p.y2 + o2, r2);
      }
      break;
    }
    case kEpiSwiglu: {
#pragma unroll
      for (int j = 0; j < 4; ++j) r1[j] = silu(y[0][0][j]) * y[0][1][j];
      store4(p.y1 + o1, r1);
      if (two) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float z2 = silu(y[1][0][j]) * y[1][1][j];
          r2[j] = p.couple ? fmaf(p.couple[n0 + j], r1[j], z2) : z2;
        }
        store4(p.y2 + o2, r2);
      }
      break;
    }
    case kEpiResidualCoupled: {
      const float4 a = *(const float4*)(p.res1 + o1);
      r1[0] = a.x + y[0][0][0]; r1[1] = a.y + y[0][0][1]; r1[2] = a.z + y[0][0][2]; r1[3] = a.w + y[0][0][3];
      store4(p.y1 + o1, r1);
      if (two) {
        const float4 b = *(const float4*)(p.res2 + o2);
        const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          r2[j] = bb[j] + (p.couple ? fmaf(p.couple[n0 + j], y[0][0][j], y[1][0][j]) : y[1][0][j]);
        store4(p.y2 + o2, r2);
      }
      break;
    }
    case kEpiKvAppend:
      // primary only: k = rows n of W, v = rows n of W2, appended at position ctx_lens[s]
      if (p.y1) store4(p.y1 + o1, y[0][0]);
      if (p.y2) store4(p.y2 + o1, y[0][1]);
      kv_append(p, s, n0, y[0][0], y[0][1]);
      break;
    case kEpiSplitPair:
      store4(p.y1 + o1, y[0][0]);
      store4(p.y1 + o1 + p.n, y[0][1]);
      if (two) {
        store4(p.y2 + o2, y[1][0]);
        store4(p.y2 + o2 + p.n, y[1][1]);
      }
      break;
  }
}

// Raw activations of one stage held by one loader thread: the stage has
// NCB*16 rows x kStage/8 groups of 8 columns; loader thread t takes groups t,
// t + kLoadThreads, ...
template <int NCB>
struct XStage {
  static constexpr int kTotal = NCB * 16 * (kStage / 8);  // 8-column groups of one stage
  static constexpr int kItems = (kTotal + kLoadThreads - 1) / kLoadThreads;
  float4 v[kItems][2];
  bool live[kItems];  // false: the group is padding and converts to zeros
};

// GROUPED: activation column j of a flow is entry j of the workgroup's expert
// (ent[j] = sequence | slot << 16, cnt entries); its row of x_f is
// s * moe_row_s + slot * moe_row_slot + f * moe_row_f, and the primary's
// column is live only where the primary selected the expert (slot < k1).
template <int NCB, bool GROUPED>
__device__ __forceinline__ void fetch_x(const GemvParams& p, int k_begin, int st, XStage<NCB>& xr, const int* ent,
                                        int cnt) {
  const int kc = k_begin + st * kStage;
#pragma unroll
  for (int it = 0; it < XStage<NCB>::kItems; ++it) {
    const int item = (threadIdx.x - kMathThreads) + it * kLoadThreads;
    const int kg = item % (kStage / 8), m = item / (kStage / 8);
    const int cb = m >> 4, f = cb / p.cbf, j = (cb - f * p.cbf) * 16 + (m & 15);
    // groups past the stage (fewer than threads), past the batch or past the
    // expert's entries read row 0 of x1, which always exists, and are replaced
    // by zeros
    bool live;
    size_t row;
    if (GROUPED) {
      const int en = j < cnt ? ent[j] : 0;
      const int s = en & 0xFFFF, slot = en >> 16;
      live = item < XStage<NCB>::kTotal && j < cnt && (f == 1 || slot < p.moe_k1);
      row = (size_t)s * p.moe_row_s + (size_t)slot * p.moe_row_slot + (size_t)f * p.moe_row_f;
    } else {
      live = item < XStage<NCB>::kTotal && j < p.batch;
      row = j;
    }
    const float4* src = (const float4*)(live ? (f ? p.x2 : p.x1) + row * p.k + kc + kg * 8 : p.x1 + kc);
    // the values are not touched here: the conversion (put_x) is the first use,
    // so the loads stay in flight until then
    xr.v[it][0] = src[0];
    xr.v[it][1] = src[1];
    xr.live[it] = live;
  }
}

// Converts a stage to hi (and lo) bf16 B operands in LDS: xs[h][cb][row][k/8 ^ row][8].
template <int NCB, int NH>
__device__ __forceinline__ void put_x(const XStage<NCB>& xr, uint16_t* xs) {
#pragma unroll
  for (int it = 0; it < XStage<NCB>::kItems; ++it) {
    const int item = (threadIdx.x - kMathThreads) + it * kLoadThreads;
    const int kg = item % (kStage / 8), m = item / (kStage / 8);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 q0 = xr.live[it] ? xr.v[it][0] : z, q1 = xr.live[it] ? xr.v[it][1] : z;
    bf16x8 hi, lo;
    hi[0] = (__bf16)q0.x; hi[1] = (__bf16)q0.y; hi[2] = (__bf16)q0.z; hi[3] = (__bf16)q0.w;
    hi[4] = (__bf16)q1.x; hi[5] = (__bf16)q1.y; hi[6] = (__bf16)q1.z; hi[7] = (__bf16)q1.w;
    if (NH == 2) {
      lo[0] = (__bf16)(q0.x - (float)hi[0]); lo[1] = (__bf16)(q0.y - (float)hi[1]);
      lo[2] = (__bf16)(q0.z - (float)hi[2]); lo[3] = (__bf16)(q0.w - (float)hi[3]);
      lo[4] = (__bf16)(q1.x - (float)hi[4]); lo[5] = (__bf16)(q1.y - (float)hi[5]);
      lo[6] = (__bf16)(q1.z - (float)hi[6]); lo[7] = (__bf16)(q1.w - (float)hi[7]);
    }
    // row r of column block cb, 8-column group kg -> slot kg ^ r of row r: the
    // 16 groups a row's threads write land in 16 different banks, and so do
    // the 16 rows an MFMA operand read takes from one group
    const int r = m & 15;
    const size_t off = (((size_t)(m >> 4) * 16 + r) * (kStage / 8) + (kg ^ r)) * 8;
    if (item < XStage<NCB>::kTotal) {
      *(bf16x8*)(xs + off) = hi;
      if (NH == 2) *(bf16x8*)(xs + (size_t)NCB * kStage * 16 + off) = lo;
    }
  }
}

// NCB: activation column blocks (flows * CBF); PAIR: a second matrix (w2) on the
// same activations; LO: split activations into hi + lo.
//
// Math wave w works on tile w % 4 with the k-steps of wave group w / 4: group
// g takes k-steps 2g, 2g + 1 of every stage, so two waves per SIMD share the
// stage's B operands and each holds half of the weights in flight. Waves 8 to
// 15 are the loader waves.
//
// GROUPED (mixture of experts): grid row index = expert * moe_rgs + row group;
// the workgroup multiplies its expert's matrices (moe_wstride elements apart)
// with the rows of the sequences that selected the expert (moe_sel), found
// here in sequence order, and exits at once if there are none. One k-range.
template <int NCB, bool PAIR, bool LO, int TILES, bool GROUPED>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvParams p) {
  constexpr int kTiles = TILES;                  // 16-row weight tiles per workgroup (4 or 8)
  constexpr int kGroups = kGemvWaves / kTiles;   // wave groups sharing the tiles (2 or 1)
  constexpr int kRowsPerWg = 16 * kTiles;
  constexpr int kHalfSteps = kSteps / kGroups;   // k-steps of one wave group per stage
  constexpr int NH = LO ? 2 : 1;
  constexpr int MATS = PAIR ? 2 : 1;
  // weight stages in flight per math wave (deeper measured no faster; paired
  // 128-row tiles take two to stay within the 128 registers of a 16-wave
  // workgroup) and activation stages in flight per loader wave
  constexpr int WDEPTH = (PAIR && TILES == 8) ? 2 : 3;
  constexpr int XDEPTH = 2;
  static_assert(XDEPTH >= 2 && WDEPTH >= 1, "the loader converts stage st + 1 while stage st is multiplied");
  // LDS: the double-buffered B operands, reused after the loop to stage the
  // results for the epilogue (whichever is larger sets the size)
  constexpr size_t kXsBytes = 2 * NH * NCB * (kStage / 8) * 16 * 8 * sizeof(uint16_t);
  constexpr size_t kResBytes = MATS * NCB * 16 * kRowsPerWg * sizeof(float);
  __shared__ __attribute__((aligned(16))) unsigned char smem[kXsBytes > kResBytes ? kXsBytes : kResBytes];
  constexpr int kRed = kGroups == 2 ? 1 : 0;  // group 1's sums, handed to group 0
  __shared__ __attribute__((aligned(16))) float red[kRed ? MATS : 1][kRed ? NCB : 1][kRed ? kTiles : 1][64][4];
  auto xs = reinterpret_cast<uint16_t(*)[NH][NCB][16][kStage / 8][8]>(smem);  // [buf][h][cb][row][group ^ row][8]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int wt = wave & (kTiles - 1), wg = wave / kTiles;
  // Workgroups are dispatched to the 8 XCDs in turn (linear index mod 8) and
  // the k-range is the fastest-varying index, so with 4 or 8 k-ranges an XCD
  // holds the workgroups of one or two of them and its L2 keeps only their
  // activations (measured: within noise of the row-group-first order, the
  // 4096 x 4096 GEMV 16.7 -> 16.0 us).
  int rg = blockIdx.y, expert = 0, cnt = 0;
  const int ks = blockIdx.x;
  __shared__ int ent[GROUPED ? 64 : 1];
  __shared__ int ent_count;
  if (GROUPED) {
    expert = blockIdx.y / p.moe_rgs;
    rg = blockIdx.y - expert * p.moe_rgs;
    if (threadIdx.x < 64) {  // wave 0: lane s finds the slot of this expert in sequence s's selection
      const int s = threadIdx.x;
      int slot = -1;
      if (s < p.batch) {
        // eight selections in flight at a time (a sequence selects an expert at most once)
        const int* sel = p.moe_sel + s * p.moe_k2;
        for (int q0 = 0; q0 < p.moe_k2; q0 += 8) {
          int v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = q0 + j < p.moe_k2 ? sel[q0 + j] : -1;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (v[j] == expert) slot = q0 + j;
        }
      }
      const unsigned long long mask = __ballot(slot >= 0);
      if (slot >= 0) ent[__popcll(mask & ((1ull << s) - 1))] = s | (slot << 16);
      if (s == 0) ent_count = __popcll(mask);
    }
    __syncthreads();
    cnt = ent_count;
    if (cnt == 0) return;  // workgroup-uniform: no sequence selected this expert
  }
  const int tile = rg * kTiles + wt;  // this wave's 16-row weight tile
  const int k_begin = ks * p.k_range;
  const int nst = (min(k_begin + p.k_range, p.k) - k_begin) / kStage;
  const int kg_total = p.k / 8;

  // weight operands of one stage: per matrix and this group's k-steps, row `col` of the tile
  struct WStage {
    bf16x8 a[MATS][kHalfSteps];
  };
  // this wave's tile within its matrix (several matrices can share one launch, by row range)
  const int row0 = tile * 16;
  const int seg = row0 < p.seg1_row ? 0 : (row0 < p.seg2_row ? 1 : 2);
  const size_t wofs = GROUPED ? (size_t)expert * p.moe_wstride : 0;
  const uint16_t* const wmat = (seg == 0 ? p.w : (seg == 1 ? p.w_seg1 : p.w_seg2)) + wofs;
  const uint16_t* const wmat2 = PAIR ? p.w2 + wofs : nullptr;
  const int tile_in = (row0 - (seg == 0 ? 0 : (seg == 1 ? p.seg1_row : p.seg2_row))) / 16;
  auto fetch_w = [&](int st, WStage& w) __attribute__((always_inline)) {
    const int kg0 = (k_begin + st * kStage) / 8 + wg * kHalfSteps * 4;
    const size_t base = (((size_t)tile_in * kg_total + kg0 + grp) * 16 + col) * 8;
#pragma unroll
    for (int k2 = 0; k2 < kHalfSteps; ++k2) {
      w.a[0][k2] = __builtin_nontemporal_load((const bf16x8*)(wmat + base + (size_t)k2 * 4 * 16 * 8));
      if (PAIR) w.a[MATS - 1][k2] = __builtin_nontemporal_load((const bf16x8*)(wmat2 + base + (size_t)k2 * 4 * 16 * 8));
    }
  };

  f32x4 acc[MATS][NCB];
#pragma unroll
  for (int mat = 0; mat < MATS; ++mat)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[mat][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The loader waves fetch every stage's activations three stages ahead and
  // convert stage st + 1 into xs[(st + 1) & 1] while the math waves multiply
  // stage st; one barrier per stage hands the buffers over. The math waves
  // only ever wait for their own weights (loads complete in issue order, so a
  // wave that also fetched activations would wait for both), and the loader
  // waves only for activations, which the L2 serves.
  const bool loader = wave >= kGemvWaves;  // wave-uniform
  if (loader) {
    // the conversion gates every stage's barrier: the loader waves' instructions
    // go first on their SIMDs (the GEMVs of the layer shapes 3-9% faster)
    __builtin_amdgcn_s_setprio(2);
    XStage<NCB> x[XDEPTH];
#pragma unroll
    for (int j = 0; j < XDEPTH; ++j)
      if (j < nst) fetch_x<NCB, GROUPED>(p, k_begin, j, x[j], ent, cnt);
    if (nst > 0) put_x<NCB, NH>(x[0], &xs[0][0][0][0][0][0]);
    __syncthreads();
    // stage st: convert stage st + 1 (buffer xn) into xs[(st + 1) & 1], then
    // fetch stage st + XDEPTH into xj (stage st's buffer, converted before)
    auto lstep = [&](int st, XStage<NCB>& xj, const XStage<NCB>& xn, bool fetch) __attribute__((always_inline)) {
      if (st + 1 < nst) put_x<NCB, NH>(xn, &xs[(st + 1) & 1][0][0][0][0][0]);
      if (fetch) fetch_x<NCB, GROUPED>(p, k_begin, st + XDEPTH, xj, ent, cnt);
      __syncthreads();
    };
    int s0 = 0;
    for (; s0 + 2 * XDEPTH - 1 < nst; s0 += XDEPTH) {
#pragma unroll
      for (int j = 0; j < XDEPTH; ++j) lstep(s0 + j, x[j], x[(j + 1) % XDEPTH], true);
    }
    for (; s0 < nst; s0 += XDEPTH) {
#pragma unroll
      for (int j = 0; j < XDEPTH; ++j)
        if (s0 + j < nst) lstep(s0 + j, x[j], x[(j + 1) % XDEPTH], s0 + j + XDEPTH < nst);
    }
  } else {
    WStage w[WDEPTH];
#pragma unroll
    for (int j = 0; j < WDEPTH; ++j)
      if (j < nst) fetch_w(j, w[j]);
    __syncthreads();
    // stage st: multiply with weights wj (B operands in xs[st & 1]), then fetch stage st + WDEPTH into wj
    auto mstep = [&](int st, WStage& wj, bool fetch) __attribute__((always_inline)) {
      const int buf = st & 1;
#pragma unroll
      for (int k2 = 0; k2 < kHalfSteps; ++k2) {
        bf16x8 xb[NCB][NH];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int h = 0; h < NH; ++h)
            xb[cb][h] = *(const bf16x8*)&xs[buf][h][cb][col][(4 * (wg * kHalfSteps + k2) + grp) ^ col][0];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int mat = 0; mat < MATS; ++mat)
              acc[mat][cb] = mfma(wj.a[mat][k2], xb[cb][h], acc[mat][cb]);
      }
      if (fetch) fetch_w(st + WDEPTH, wj);
      __syncthreads();
    };
    // Steady state: every step fetches, so each iteration issues the same
    // loads and the wait before a stage's first use covers only that stage.
    int s0 = 0;
    for (; s0 + 2 * WDEPTH - 1 < nst; s0 += WDEPTH) {
#pragma unroll
      for (int j = 0; j < WDEPTH; ++j) mstep(s0 + j, w[j], true);
    }
    for (; s0 < nst; s0 += WDEPTH) {  // the last stages: fetch while stages remain
#pragma unroll
      for (int j = 0; j < WDEPTH; ++j)
        if (s0 + j < nst) mstep(s0 + j, w[j], s0 + j + WDEPTH < nst);
    }
  }

  // group 1 hands its sums to group 0 (fixed order: group 0 + group 1)
  if (kGroups == 2 && wg == 1 && !loader) {
#pragma unroll
    for (int mat = 0; mat < MATS; ++mat)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) *(f32x4*)&red[mat][cb][wt][lane][0] = acc[mat][cb];
  }
  __syncthreads();
  // lane of group 0 holds Y[m = cb*16 + col][n = tile*16 + 4*grp + i] in acc[mat][cb][i]
  const int n0 = tile * 16 + 4 * grp;
  if (kGroups == 2 && wg == 0 && !loader) {
#pragma unroll
    for (int mat = 0; mat < MATS; ++mat)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[mat][cb] += *(const f32x4*)&red[mat][cb][wt][lane][0];
  }
  if (p.k_split > 1) {
    if (wg == 0 && !loader) {
      const size_t mat_stride = (size_t)p.m_pad * p.n;
      float* out = p.part + (size_t)ks * MATS * mat_stride;
#pragma unroll
      for (int mat = 0; mat < MATS; ++mat)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          *(f32x4*)(out + mat * mat_stride + (size_t)(cb * 16 + col) * p.n + n0) = acc[mat][cb];
    }
    return;
  }
  // one k-range: the epilogue runs here. Results pass through LDS (the
  // activation buffers are free after the last barrier) so that each thread
  // finishes whole (sequence, 4-column) groups of both flows.
  float* res = reinterpret_cast<float*>(smem);  // [mat][m][kRowsPerWg columns]
  if (wg == 0 && !loader) {
#pragma unroll
    for (int mat = 0; mat < MATS; ++mat)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        *(f32x4*)(res + ((size_t)mat * NCB * 16 + cb * 16 + col) * kRowsPerWg + wt * 16 + 4 * grp) = acc[mat][cb];
  }
  __syncthreads();
  const int rows = GROUPED ? cnt : p.batch;  // activation columns per flow
  for (int idx = threadIdx.x; idx < rows * (kRowsPerWg / 4); idx += kGemvThreads) {
    const int j = idx / (kRowsPerWg / 4), c4 = (idx - j * (kRowsPerWg / 4)) * 4;
    float y[2][2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        const bool have = f < p.flows && mat < MATS;
        const int m = (f * p.cbf + (j >> 4)) * 16 + (j & 15);
        const float4 v = have ? *(const float4*)(res + ((size_t)(mat < MATS ? mat : 0) * NCB * 16 + m) * kRowsPerWg + c4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        y[f][mat][0] = v.x; y[f][mat][1] = v.y; y[f][mat][2] = v.z; y[f][mat][3] = v.w;
      }
    const int n0 = rg * kRowsPerWg + c4;
    if (GROUPED) {  // rows (sequence, slot, flow) of the output: [batch][k2][2][n], or [2n] per row for split pairs
      const int s = ent[j] & 0xFFFF, slot = ent[j] >> 16;
      const size_t row = p.epilogue == kEpiSplitPair ? 2 * (size_t)p.n : (size_t)p.n;
      const size_t o1 = ((size_t)(s * p.moe_k2 + slot) * 2) * row + n0;
      apply_epilogue(p, s, o1, o1 + row, n0, y);
    } else {
      const size_t o = (size_t)j * p.n + n0;
      apply_epilogue(p, j, o, o, n0, y);
    }
  }
}

// One thread per (sequence s, 4 columns): both flows' sums over the k-splits
// (fixed order), then the epilogue. KS > 0: exactly KS splits, every load
// issued before the first add; KS == 0: any number, four loads at a time.
constexpr int kFinalizeThreads = 128;  // 128 rather than 256: the reduction spreads over twice as many CUs

// Sum over the k-splits (fixed order) of partial row m, matrix mat, columns n0..n0+3.
template <int KS>
__device__ __forceinline__ void sum_splits(const GemvParams& p, int mats, int mat, size_t m, int n0, float (&y)[4]) {
  const size_t mat_stride = (size_t)p.m_pad * p.n;
  const float* src = p.part + mat * mat_stride + m * p.n + n0;
  if (KS > 0) {
    float4 v[KS > 0 ? KS : 1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) v[ks] = *(const float4*)(src + (size_t)ks * mats * mat_stride);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      y[0] += v[ks].x; y[1] += v[ks].y; y[2] += v[ks].z; y[3] += v[ks].w;
    }
  } else {
#pragma unroll 4
    for (int ks = 0; ks < p.k_split; ++ks) {
      const float4 v = *(const float4*)(src + (size_t)ks * mats * mat_stride);
      y[0] += v.x; y[1] += v.y; y[2] += v.z; y[3] += v.w;
    }
  }
}

template <int KS>
__global__ __launch_bounds__(kFinalizeThreads) void gemv_finalize_kernel(GemvParams p) {
  const int groups = p.n / 4;
  const int item = blockIdx.x * kFinalizeThreads + threadIdx.x;
  if (item >= p.batch * groups) return;
  const int s = item / groups, n0 = (item - s * groups) * 4;
  const int mats = p.pair ? 2 : 1;
  float y[2][2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int j = 0; j < 4; ++j) y[f][mat][j] = 0.f;
  if (p.epilogue == kEpiQkv) {
    // Both flows' queries (columns [0, q_cols)) and the primary's keys with
    // their values (the next kv_cols, then kv_cols more), rotated at position
    // ctx_lens[s] when rope is set. Rotate-half pairs dimension d < D/2 of a
    // head with d + D/2: the thread of the first half takes both.
    const int D = p.kv_head_dim, half = D >> 1;
    const bool in_q = n0 < p.q_cols, in_k = !in_q && n0 < p.q_cols + p.kv_cols;
    if (!in_q && !in_k) return;  // value columns: written with their keys
    const int col = in_q ? n0 : n0 - p.q_cols;
    const int d0 = col % D;
    if (p.rope == kRopeHalf && d0 >= half) return;
    const int pos = p.rope == kRopeNone ? 0 : min(max(p.kv_ctx[s], 0), p.rope_max_pos - 1);
    const float* cs = p.rope_cos + (size_t)pos * half;
    const float* sn = p.rope_sin + (size_t)pos * half;
    auto rot_pairs = [&](float (&v)[4]) __attribute__((always_inline)) {  // interleaved: (d, d + 1)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float c = cs[(d0 >> 1) + j], sv = sn[(d0 >> 1) + j], a = v[2 * j], b = v[2 * j + 1];
        v[2 * j] = a * c - b * sv;
        v[2 * j + 1] = a * sv + b * c;
      }
    };
    auto rot_halves = [&](float (&lo)[4], float (&hi)[4]) __attribute__((always_inline)) {  // (d, d + D/2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c = cs[d0 + j], sv = sn[d0 + j], a = lo[j], b = hi[j];
        lo[j] = a * c - b * sv;
        hi[j] = a * sv + b * c;
      }
    };
    float u[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};  // the second halves (rotate-half)
    if (in_q) {
      sum_splits<KS>(p, 1, 0, (size_t)s, n0, y[0][0]);
      sum_splits<KS>(p, 1, 0, (size_t)(p.cbf * 16 + s), n0, y[1][0]);
      const size_t o = (size_t)s * p.q_cols + n0;
      if (p.rope == kRopeHalf) {
        sum_splits<KS>(p, 1, 0, (size_t)s, n0 + half, u[0]);
        sum_splits<KS>(p, 1, 0, (size_t)(p.cbf * 16 + s), n0 + half, u[1]);
        rot_halves(y[0][0], u[0]);
        rot_halves(y[1][0], u[1]);
        store4(p.y1 + o + half, u[0]);
        store4(p.y2 + o + half, u[1]);
      } else if (p.rope == kRopeInterleaved) {
        rot_pairs(y[0][0]);
        rot_pairs(y[1][0]);
      }
      store4(p.y1 + o, y[0][0]);
      store4(p.y2 + o, y[1][0]);
    } else {
      sum_splits<KS>(p, 1, 0, (size_t)s, n0, y[0][0]);
      sum_splits<KS>(p, 1, 0, (size_t)s, n0 + p.kv_cols, y[0][1]);
      if (p.rope == kRopeHalf) {
        sum_splits<KS>(p, 1, 0, (size_t)s, n0 + half, u[0]);
        sum_splits<KS>(p, 1, 0, (size_t)s, n0 + p.kv_cols + half, u[1]);
        rot_halves(y[0][0], u[0]);
        kv_append(p, s, col + half, u[0], u[1]);
      } else if (p.rope == kRopeInterleaved) {
        rot_pairs(y[0][0]);
      }
      kv_append(p, s, col, y[0][0], y[0][1]);
    }
    return;
  }
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    if (f >= p.flows) break;
    const size_t m = (size_t)(f * p.cbf * 16 + s);
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      if (mat >= mats) break;
      sum_splits<KS>(p, mats, mat, m, n0, y[f][mat]);
    }
  }
  const size_t o = (size_t)s * p.n + n0;
  apply_epilogue(p, s, o, o, n0, y);
}

hipError_t launch_gemv(const GemvParams& p, hipStream_t stream) {
  const int ncb = p.flows * p.cbf;
  const bool lo = !p.x_exact;
  const int tiles = p.rows_per_wg / 16;
  if (p.moe_sel) {  // grouped: two flows, one k-range
    if (p.flows != 2 || (tiles != 4 && tiles != 8) || p.k_split != 1) return hipErrorInvalidValue;
    const dim3 grid(1, (p.n / p.rows_per_wg) * p.moe_experts), block(kGemvThreads);
#define DFA_GROUPED_CASE(NCB_, PAIR_, LO_)                                                                  \
  if (ncb == NCB_ && p.pair == PAIR_ && lo == LO_) {                                                        \
    if (tiles == 8) hipLaunchKernelGGL((gemv_kernel<NCB_, PAIR_, LO_, 8, true>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((gemv_kernel<NCB_, PAIR_, LO_, 4, true>), grid, block, 0, stream, p);            \
    return hipGetLastError();                                                                               \
  }
    DFA_GROUPED_CASE(2, true, false) DFA_GROUPED_CASE(2, true, true) DFA_GROUPED_CASE(2, false, true)
    DFA_GROUPED_CASE(4, true, false) DFA_GROUPED_CASE(4, true, true) DFA_GROUPED_CASE(4, false, true)
#undef DFA_GROUPED_CASE
    return hipErrorInvalidValue;
  }
  const dim3 grid(p.k_split, p.n / p.rows_per_wg), block(kGemvThreads);
#define DFA_GEMV_CASE(NCB_, PAIR_, LO_)                                                                      \
  if (ncb == NCB_ && p.pair == PAIR_ && lo == LO_) {                                                         \
    if (tiles == 8) hipLaunchKernelGGL((gemv_kernel<NCB_, PAIR_, LO_, 8, false>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((gemv_kernel<NCB_, PAIR_, LO_, 4, false>), grid, block, 0, stream, p);            \
    return hipGetLastError();                                                                                \
  }
  DFA_GEMV_CASE(1, false, false) DFA_GEMV_CASE(1, false, true) DFA_GEMV_CASE(1, true, false)
  DFA_GEMV_CASE(1, true, true) DFA_GEMV_CASE(2, false, false) DFA_GEMV_CASE(2, false, true)
  DFA_GEMV_CASE(2, true, false) DFA_GEMV_CASE(2, true, true) DFA_GEMV_CASE(4, false, false)
  DFA_GEMV_CASE(4, false, true) DFA_GEMV_CASE(4, true, false) DFA_GEMV_CASE(4, true, true)
#undef DFA_GEMV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_finalize(const GemvParams& p, hipStream_t stream) {
  const dim3 grid((p.batch * (p.n / 4) + kFinalizeThreads - 1) / kFinalizeThreads), block(kFinalizeThreads);
  switch (p.k_split) {
#define DFA_FINALIZE_CASE(N)                                                      \
  case N:                                                                         \
    hipLaunchKernelGGL((gemv_finalize_kernel<N>), grid, block, 0, stream, p);     \
    break;
    DFA_FINALIZE_CASE(2) DFA_FINALIZE_CASE(3) DFA_FINALIZE_CASE(4) DFA_FINALIZE_CASE(8) DFA_FINALIZE_CASE(16)
#undef DFA_FINALIZE_CASE
    default:
      hipLaunchKernelGGL((gemv_finalize_kernel<0>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

size_t gemv_chunk() { return kStage; }

}  // namespace dfa
