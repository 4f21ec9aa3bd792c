// Primary-only prefill of a batch of prompts: the prompt's keys and values
// written to the paged cache, then causal self-attention of the primary flow
// ("Resumo Técnico: Dual-Flow Transformers", section "Custos de Inferência vs.
// Treinamento": prefill costs what a standard Transformer's does, the
// auxiliary flow being skipped; section "Arquitetura Central": the primary
// flow alone writes the cache; "Dual-Flow Transformers: Decoupling the
// Primary Prefill Path from Additional Decode Computation": the auxiliary
// lane starts only at the last prompt position, a decode step over this
// cache).
//
// prefill_kv_kernel   thread = (prompt, kv head, 16-position tile, piece):
//                     keys in 16-byte pieces, values as one dimension of a
//                     tile (16 positions, written as one 32-byte run), into
//                     the cache layout of the decode kernels.
// prefill_attn_kernel workgroup = (query block, kv head, prompt), 4 waves;
//                     each wave owns 32 query rows = 2 MFMA column blocks;
//                     row r of the workgroup is position p0 + r / G and query
//                     head g * G + r % G (G query heads per kv head), so all
//                     heads of the group share every key/value tile. Keys and
//                     values stream from the cache in 32-position chunks
//                     staged through LDS (double-buffered, one copy per
//                     workgroup, the cache's own tile layout), up to the
//                     block's last position (causal).
// Per chunk and wave, on v_mfma_f32_16x16x32_bf16 (lane l: column n = l % 16,
// k-group grp = l / 16; result (m = 4*grp + i, n) in lane l, register i):
//   scores  S^T[pos][row] = K[pos] . Q[row], A = keys from LDS, B = the
//           query rows as given (exact bf16; the scale multiplies the fp32
//           scores), one product per 32 dimensions;
//   output  O^T[dim][row] += V^T . P^T, A = values from LDS (positions 4*grp..
//           of both tiles), B = the weights, split hi/lo (hi: the top 16 bits,
//           lo: the rest rounded to bf16; about 16 significant bits per
//           product), whose score layout is already the operand's.
// Online softmax in base 2 with each row's own lazy rescale; query blocks run
// longest first (the last block of a prompt attends the most positions).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dfa_internal.h"
#include "ops_internal.h"

namespace dfa {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfCb = 2;                            // 16-row column blocks per wave
constexpr int kPfRows = kPfWaves * kPfCb * 16;      // query rows per workgroup
constexpr float kPfLazy = 8.f;                      // a row's max lags its scores by at most 2^8
constexpr int kPfTable = kPrefillMaxBlocks;         // block-table entries staged in LDS

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Larger of two scores, NaN-propagating (IEEE maximum): no quieting of its
// inputs first, unlike fmaxf under the IEEE mode kernels run in.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four k-groups of an MFMA
// column). A register swapped with itself by v_permlane16_swap (odd 16-lane
// rows against even ones) or v_permlane32_swap (upper 32 lanes against lower)
// leaves each lane its own value and its partner's in the two results; these
// are VALU operations, no trip through LDS.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Physical block of position t of prompt b (clamped into the cache).
__device__ __forceinline__ int block_of(const PrefillParams& p, int b, int t) {
  return clampi(p.table[(size_t)b * p.max_blocks + (t >> p.bs_log2)], 0, p.num_blocks - 1);
}
}  // namespace

// One thread per (prompt, kv head, tile, piece): pieces [0, 2D) are the keys'
// 16-byte groups (dimension group kg = piece / 16 ... as the cache stores
// them: piece = kg * 16 + position in tile), pieces [2D, 2D + D) the values'
// dimensions (16 positions each).
template <int D>
__global__ __launch_bounds__(256) void prefill_kv_kernel(PrefillParams p) {
  const int pieces = 3 * D;
  const int tiles = p.lmax_tiles;
  const long item = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)p.batch * p.hkv * tiles * pieces;
  if (item >= total) return;
  const int piece = (int)(item % pieces);
  long rest = item / pieces;
  const int tile = (int)(rest % tiles);
  rest /= tiles;
  const int g = (int)(rest % p.hkv);
  const int b = (int)(rest / p.hkv);
  const int len = clampi(p.lens[b], 0, p.lmax);
  const int t0 = tile * 16;
  if (t0 >= len) return;
  const int blk = block_of(p, b, t0);
  const int bs = 1 << p.bs_log2;
  const size_t tile_base = ((size_t)blk * p.hkv + g) * bs * D + (size_t)((t0 & (bs - 1)) >> 4) * (16 * D);
  if (piece < 2 * D) {  // keys: position t0 + i, dimensions 8*kg .. 8*kg + 7
    const int kg = piece >> 4, i = piece & 15;
    if (t0 + i >= len) return;
    const uint4 v = *(const uint4*)(p.k + (((size_t)b * p.lmax + t0 + i) * p.hkv + g) * D + 8 * kg);
    *(uint4*)(p.k_cache + tile_base + (size_t)(kg * 16 + i) * 8) = v;
  } else {  // values: dimension d, positions t0 .. t0 + 15 (transposed within the tile)
    const int d = piece - 2 * D;
    const int n = min(16, len - t0);
    uint16_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      w[i] = i < n ? p.v[(((size_t)b * p.lmax + t0 + i) * p.hkv + g) * D + d] : (uint16_t)0;
    uint16_t* dst = p.v_cache + tile_base + (size_t)d * 16;
    if (n == 16) {
      uint4 lo, hi;
      lo.x = w[0] | (uint32_t)w[1] << 16; lo.y = w[2] | (uint32_t)w[3] << 16;
      lo.z = w[4] | (uint32_t)w[5] << 16; lo.w = w[6] | (uint32_t)w[7] << 16;
      hi.x = w[8] | (uint32_t)w[9] << 16; hi.y = w[10] | (uint32_t)w[11] << 16;
      hi.z = w[12] | (uint32_t)w[13] << 16; hi.w = w[14] | (uint32_t)w[15] << 16;
      *(uint4*)dst = lo;
      *(uint4*)(dst + 8) = hi;
    } else {  // a prompt's last, partial tile: only its own positions
      for (int i = 0; i < n; ++i) dst[i] = w[i];
    }
  }
}

template <int D>
__global__ __launch_bounds__(kPfThreads) void prefill_attn_kernel(PrefillParams p) {
  constexpr int KS = D / 32;                 // 32-dimension k-steps of a score product
  constexpr int DB = D / 16;                 // 16-dimension blocks of the output
  constexpr int kTile = 16 * D;              // elements of one 16-position tile
  constexpr int kPieces = kTile * 2 / 16;    // 16-byte pieces of one tile
  // LDS, double-buffered: keys as in the cache ([D/8][16][8] per tile); values
  // regrouped per tile as [4 position groups][D (+4 padding)][4 positions], so
  // the 16 lanes of an operand read phase (dimensions 16*db .. +15, one
  // position group) take 128 contiguous bytes (the cache's [D][16] order puts
  // dimensions 32 bytes apart: a 4-way bank conflict), and the padding keeps
  // the staging writes of the two halves of a cache row on different banks.
  // The two tiles of a chunk lie a multiple of 512 bytes apart, so one
  // ds_read2st64_b64 fetches a lane's 8 bytes of both into adjacent registers
  // (the MFMA operand) with no moves.
  constexpr int kVRow = D + 4;                                 // dimension rows of one position group
  constexpr int kVTile = ((4 * kVRow * 4 * 2 + 511) / 512) * 512 / 2;  // elements per regrouped tile (padded)
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][2][kTile];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][2][kVTile];
  __shared__ int tbl[kPfTable];  // the block-table entries of positions [0, q_end)

  // Workgroup -> (prompt, kv head, query block). Workgroups go to the 8 XCDs in
  // turn (linear index mod 8); with a multiple of 8 (prompt, kv head) pairs,
  // all query blocks of a pair run on one XCD, longest first, so the
  // workgroups resident there stream the same keys and values at the same
  // pace and the XCD's L2 serves them.
  const int nqb = gridDim.x, pairs = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + nqb * (blockIdx.y + gridDim.y * blockIdx.z);
  int pair, rank;
  if ((pairs & 7) == 0) {
    const int j = lin >> 3;
    pair = (lin & 7) + 8 * (j / nqb);
    rank = j % nqb;
  } else {
    pair = lin / nqb;
    rank = lin % nqb;
  }
  const int b = pair / p.hkv, g = pair - b * p.hkv;
  const int qb = nqb - 1 - rank;  // longest blocks first
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int gl2 = p.g_log2;
  const int pos_per_wg = kPfRows >> gl2;
  const int p0 = qb * pos_per_wg;
  const int len = clampi(p.lens[b], 0, p.lmax);
  if (p0 >= len) return;  // workgroup-uniform
  const int q_end = min(p0 + pos_per_wg, len);  // rows cover positions [p0, q_end)
  const int nch = (q_end + 31) >> 5;

  // ---- this lane's query rows (one per column block) and their operands ----
  int pos_r[kPfCb], head_r[kPfCb];
  bf16x8 qf[kPfCb][KS];
#pragma unroll
  for (int cb = 0; cb < kPfCb; ++cb) {
    const int r = (wave * kPfCb + cb) * 16 + n;
    pos_r[cb] = p0 + (r >> gl2);
    head_r[cb] = g * (1 << gl2) + (r & ((1 << gl2) - 1));
    const bool live = pos_r[cb] < q_end;
    const uint16_t* src = p.q + (((size_t)b * p.lmax + min(pos_r[cb], q_end - 1)) * p.hq + head_r[cb]) * D;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const bf16x8 v = *(const bf16x8*)(src + 32 * st + 8 * grp);
      qf[cb][st] = live ? v : bf16x8{};
    }
  }
  // the positions of this wave's first row and the last position any of its
  // rows attends (-1: every row of the wave lies past the prompt)
  const int wave_first = p0 + ((wave * kPfCb * 16) >> gl2);
  const int wave_last = wave_first < q_end ? min(p0 + ((((wave + 1) * kPfCb * 16) - 1) >> gl2), q_end - 1) : -1;

  // ---- chunk staging: 4 tiles of kPieces 16-byte pieces, one piece per thread and tile ----
  const int bs = 1 << p.bs_log2;
  const size_t head_off = (size_t)g * bs * D;
  const int last_tile = (q_end - 1) & ~15;  // tiles past it fall back onto it (their positions are masked)
  const int nblk = (last_tile >> p.bs_log2) + 1;  // at most kPfTable (checked on the host)
  for (int i = threadIdx.x; i < nblk; i += kPfThreads) tbl[i] = block_of(p, b, i << p.bs_log2);
  auto tile_of = [&](int tt) __attribute__((always_inline)) {
    // the block id is the same in every lane: scalar address arithmetic
    const int blk = __builtin_amdgcn_readfirstlane(tbl[tt >> p.bs_log2]);
    return (size_t)blk * p.blk_stride + head_off + (size_t)((tt & (bs - 1)) >> 4) * kTile;
  };
  // Every thread issues the same loads on every path (threads past a tile's
  // pieces read its last piece again), so the compiler's count of loads in
  // flight is exact and a store to LDS waits only for its own chunk.
  const int piece = min((int)threadIdx.x, kPieces - 1);
  // this thread's 16-byte piece of each tile of a chunk; two sets alternate so
  // that the loads of chunk c + 2 are in flight while chunk c is multiplied
  struct Stage {
    u32x4 k0, k1, v0, v1;
  };
  Stage sa, sb;
  auto fetch = [&](int c, Stage& st) __attribute__((always_inline)) {
    c = min(c, nch - 1);  // past the end: the last chunk again (never used); keeps the load count fixed
    const size_t t0 = tile_of(min(32 * c, last_tile)), t1 = tile_of(min(32 * c + 16, last_tile));
    // plain loads: every query block of the prompt reads these tiles again, so they stay in L2
    st.k0 = *((const u32x4*)(p.k_cache + t0) + piece);
    st.k1 = *((const u32x4*)(p.k_cache + t1) + piece);
    st.v0 = *((const u32x4*)(p.v_cache + t0) + piece);
    st.v1 = *((const u32x4*)(p.v_cache + t1) + piece);
  };
  auto put = [&](int buf, const Stage& st) __attribute__((always_inline)) {
    if (threadIdx.x < kPieces) {
      *((u32x4*)&k_lds[buf][0][0] + threadIdx.x) = st.k0;
      *((u32x4*)&k_lds[buf][1][0] + threadIdx.x) = st.k1;
      // value piece = cache row d = piece / 2, positions 8 * (piece % 2) .. +7:
      // position groups 2 * (piece % 2) and 2 * (piece % 2) + 1
      const int d = threadIdx.x >> 1, g0 = 2 * (threadIdx.x & 1);
      uint16_t* v0 = &v_lds[buf][0][0];
      uint16_t* v1 = &v_lds[buf][1][0];
      *(u32x2*)(v0 + (g0 * kVRow + d) * 4) = u32x2{st.v0[0], st.v0[1]};
      *(u32x2*)(v0 + ((g0 + 1) * kVRow + d) * 4) = u32x2{st.v0[2], st.v0[3]};
      *(u32x2*)(v1 + (g0 * kVRow + d) * 4) = u32x2{st.v1[0], st.v1[1]};
      *(u32x2*)(v1 + ((g0 + 1) * kVRow + d) * 4) = u32x2{st.v1[2], st.v1[3]};
    }
  };

  float m_run[kPfCb], l_run[kPfCb];
  f32x4 oacc[kPfCb][DB];
#pragma unroll
  for (int cb = 0; cb < kPfCb; ++cb) {
    m_run[cb] = -INFINITY;
    l_run[cb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto chunk = [&](int c, int buf) __attribute__((always_inline)) {
    const int t0 = 32 * c;
    if (t0 <= wave_last) {  // wave-uniform: some row of this wave sees a position of the chunk
      const uint16_t* kt = &k_lds[buf][0][0];
      const uint16_t* vt = &v_lds[buf][0][0];
      // scores of both tiles for both column blocks
      f32x4 sv[2][kPfCb];
      // the MFMA phases run at raised wave priority, so that while one wave
      // feeds the matrix unit the other wave on the SIMD fills the gaps with
      // its vector work (measured: 1005 -> 984 us at 4 x 4096 tokens)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 kf[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st)
          kf[st] = *(const bf16x8*)(kt + u * kTile + ((4 * st + grp) * 16 + n) * 8);
#pragma unroll
        for (int cb = 0; cb < kPfCb; ++cb) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < KS; ++st) acc = mfma(kf[st], qf[cb][st], acc);
          sv[u][cb] = acc;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // wave-uniform: only chunks that reach past a row's position need the
      // causal mask, and only the last chunk holds positions past the block
      const bool diag = t0 + 31 > wave_first;
      const bool tail = t0 + 32 > q_end;
      u32x4 pa[kPfCb];
      bf16x8 pb[kPfCb];
#pragma unroll
      for (int cb = 0; cb < kPfCb; ++cb) {
        float sc[8];  // raw scores q.k; the scale enters with the exponent
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[4 * u + i] = sv[u][cb][i];
        if (diag) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t0 + 16 * u + 4 * grp + i > pos_r[cb]) sc[4 * u + i] = -INFINITY;  // causal
        }
        float cmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) cmax = max2(cmax, sc[j]);
        cmax = max_over_groups(cmax) * p.qscale;  // base-2 units (qscale > 0)
        const bool moves = cmax > m_run[cb] + kPfLazy;  // this row's own decision
        if (__builtin_amdgcn_ballot_w64(moves) != 0) {
          const float m_new = moves ? cmax : m_run[cb];
          const float alpha = moves ? __builtin_amdgcn_exp2f(m_run[cb] - m_new) : 1.f;
          l_run[cb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[cb][db] *= alpha;
          m_run[cb] = m_new;
        }
        // weights x = 2^(scale*log2(e)*s - m), split x = hi + lo: hi = x truncated to
        // its top 16 bits (packed in pairs by one byte permute), lo = bf16(x - hi)
        const float neg_m = -m_run[cb];
        float psum = 0.f;
        uint32_t xb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = __builtin_amdgcn_exp2f(fmaf(sc[j], p.qscale, neg_m));
          psum += x;
          xb[j] = __float_as_uint(x);
          pb[cb][j] = (__bf16)(x - __uint_as_float(xb[j] & 0xFFFF0000u));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pa[cb][j] = __builtin_amdgcn_perm(xb[2 * j + 1], xb[2 * j], 0x07060302u);
        l_run[cb] += psum;
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 w0 = *(const u32x2*)(vt + (grp * kVRow + 16 * db + n) * 4);
        const u32x2 w1 = *(const u32x2*)(vt + kVTile + (grp * kVRow + 16 * db + n) * 4);
        u32x4 vw;
        vw[0] = w0[0];
        vw[1] = w0[1];
        vw[2] = w1[0];
        vw[3] = w1[1];
        if (tail) {  // positions past the block are zeroed (their cache slots may be unwritten)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int tv = t0 + 16 * (h >> 1) + 4 * grp + 2 * (h & 1);
            vw[h] &= (tv < q_end ? 0x0000FFFFu : 0u) | (tv + 1 < q_end ? 0xFFFF0000u : 0u);
          }
        }
        const bf16x8 va = __builtin_bit_cast(bf16x8, vw);
#pragma unroll
        for (int cb = 0; cb < kPfCb; ++cb) {
          oacc[cb][db] = mfma(va, __builtin_bit_cast(bf16x8, pa[cb]), oacc[cb][db]);
          oacc[cb][db] = mfma(va, pb[cb], oacc[cb][db]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  __syncthreads();  // the table slice
  fetch(0, sa);
  fetch(1, sb);
  put(0, sa);
  __syncthreads();
  // iteration c multiplies chunk c from LDS buffer c & 1, fetches chunk c + 2
  // into the register set chunk c came from, and moves chunk c + 1 (fetched a
  // whole iteration earlier) into the other LDS buffer
  for (int c = 0; c < nch; c += 2) {
    fetch(c + 2, sa);
    chunk(c, 0);
    put(1, sb);
    __syncthreads();
    if (c + 1 >= nch) break;
    fetch(c + 3, sb);
    chunk(c + 1, 1);
    put(0, sa);
    __syncthreads();
  }

  // ---- normalise and store: lane holds O[row n][dims 16*db + 4*grp .. +3] ----
#pragma unroll
  for (int cb = 0; cb < kPfCb; ++cb) {
    float l = l_run[cb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (pos_r[cb] >= q_end) continue;
    const float inv = 1.f / l;
    float* dst = p.o + (((size_t)b * p.lmax + pos_r[cb]) * p.hq + head_r[cb]) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 v = oacc[cb][db] * inv;
      *(float4*)(dst + 16 * db) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const long kv_items = (long)p.batch * p.hkv * p.lmax_tiles * 3 * head_dim;
  const dim3 kv_grid((unsigned)((kv_items + 255) / 256));
  const int pos_per_wg = kPfRows >> p.g_log2;
  const dim3 grid((p.lmax + pos_per_wg - 1) / pos_per_wg, p.hkv, p.batch);
  if (head_dim == 128) {
    hipLaunchKernelGGL(prefill_kv_kernel<128>, kv_grid, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(prefill_attn_kernel<128>, grid, dim3(kPfThreads), 0, stream, p);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(prefill_kv_kernel<64>, kv_grid, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(prefill_attn_kernel<64>, grid, dim3(kPfThreads), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


}  // namespace dfa
