// Split-K decode attention over a bf16 KV cache, both flows from one read of
// every key and value (asymmetric shared-KV attention: "Resumo Técnico:
// Dual-Flow Transformers", section "Mecanismos Chave"; the shared cache read
// once for both flows: section "Custos de Inferência vs. Treinamento").
//
// Workgroup = (split s, kv head g, sequence b), 4 waves per row set of at most
// 16 rows. The query rows of the workgroup are the G query heads of kv head g
// times the flows: row r is flow r / G, head g*G + r % G. Waves take
// 32-position chunks of the split in turn and each keeps its own
// online-softmax state; a merge in LDS ends the workgroup. More than 16 rows
// (16 heads per kv head with two flows) take a second set of four waves for
// rows 16-31, which walks the same chunks in step with the first: the second
// set's loads of a chunk follow the first set's closely and are served by L2.
//
// Cache layout (see include/dfa.h): keys [block][kv head][position/16][D/8][16][8],
// values [block][kv head][position/16][D][16]: a 16-position tile of either is
// one contiguous run of 16*D elements. A chunk is 32 positions = two tiles;
// every load instruction reads whole 128-byte lines (keys: 1 KB, values:
// 512 B), so the cache is streamed with non-temporal loads: each byte is read
// once and need not stay in L2.
//
// Per tile, on the matrix cores (lane l owns column n = l % 16 and k-group
// grp = l / 16 of each operand; result (m = 4*grp + i, n) is lane l, register i):
//   scores   S^T[pos][row] = K[pos][:] . Q[row][:]   v_mfma_f32_16x16x32_bf16,
//            A = keys (lane: position n, dims 32*st + 8*grp ..+7), B = queries
//   output   O^T[dim][row] += V^T[dim][pos] . P^T     v_mfma_f32_16x16x32_bf16,
//            A = values (lane: dim 16*db + n, positions 4*grp ..+3 of both
//            tiles), B = weights
// The score results of the two tiles (lane: row n, positions 4*grp + i of each)
// are exactly the weight operand the output product needs, so no data moves
// between lanes.
//
// Operands that are not exact bf16 (the scaled, coupled queries and the
// softmax weights) are split as x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi), so each product keeps about 16 significant bits. With at
// most 8 query rows (PACKED) the hi parts fill columns 0-7 and the lo parts
// columns 8-15 of one MFMA and a DPP row rotation by 8 adds the halves; with
// 16 rows the lo parts take a second MFMA into the same accumulator.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "dfa_internal.h"
#include "launch.h"

namespace dfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dpp_ror8(float x) {
  // lane i of each 16-lane row receives lane (i + 8) % 16
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
}

// Larger of two scores, NaN-propagating (IEEE maximum): no quieting of its
// inputs first, unlike fmaxf under the IEEE mode kernels run in.
__device__ __forceinline__ float score_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four k-groups of an MFMA
// column): v_permlane16_swap / v_permlane32_swap of a register with itself
// leave each lane its own value and its partner's, vector ALU operations with
// no trip through LDS.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = score_max(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return score_max(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct Chunk {
  bf16x8 k[2][D / 32];  // per tile: keys of position n, one 8-dim group per k-step
  u32x4 v[D / 16];      // dim 16*db + n: positions 4*grp.. of tile 0 (words 0-1), then of tile 1 (words 2-3)
};

// First position of tile u of the chunk at t0, moved back onto the last tile
// that holds a position of the split when it lies past the end (its scores are
// masked; reading it keeps every address inside an allocated block).
__device__ __forceinline__ int tile_start(int t0, int u, int end) { return min(t0 + 16 * u, (end - 1) & ~15); }

// Buffer resource word 3 for raw (untyped) buffer access on gfx9-family
// targets, and the cache-policy operand of a non-temporal load.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNT = 2;

// Largest lag (base-2 units) of a row's running max behind the scores it has
// weighted: the weights 2^(s - m_run) stay at most 2^kLazyRescale.
constexpr float kLazyRescale = 8.f;

// Waves per row set (8 measured no faster: the cache stream, not the
// arithmetic between loads, sets the pace).
constexpr int kAttnWaves = 4;

// Loads one chunk through buffer resources: a tile's base address is
// wave-uniform (scalar registers), each lane's byte offsets within the tile
// are fixed (koff for keys, voff for values), and the hardware returns zeros
// for any offset past the tile.
template <int D>
__device__ __forceinline__ void load_chunk(const AttnParams& p, const uint16_t* __restrict__ kc,
                                           const uint16_t* __restrict__ vc, const int* tbl, int jb0,
                                           int t0, int end, uint32_t koff, uint32_t voff, Chunk<D>& ch) {
  constexpr int kTileBytes = D * 16 * 2;
  const int bs_mask = (1 << p.bs_log2) - 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tt = tile_start(t0, u, end);
    const int blk = __builtin_amdgcn_readfirstlane(tbl[(tt >> p.bs_log2) - jb0]);
    const size_t tile = (size_t)blk * p.blk_stride + (size_t)((tt & bs_mask) >> 4) * (D * 16);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kc + tile), (short)0, kTileBytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vc + tile), (short)0, kTileBytes, kBufferWord3);
#pragma unroll
    for (int st = 0; st < D / 32; ++st)
      ch.k[u][st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + st * 1024, 0, kNT));
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff + db * 512, 0, kNT));
      ch.v[db][2 * u] = w[0];
      ch.v[db][2 * u + 1] = w[1];
    }
  }
}

// The sequence with the rank-th largest length (ties: lower index first), for
// batches of at most 64 (one length per lane; every wave computes the same
// permutation). Workgroups are dispatched in blockIdx order and one runs per
// CU at a time, so with one split per sequence taking sequences longest first
// (longest-processing-time order) keeps a long sequence from starting last.
// `mine` is ctx[lane] (INT_MIN for lanes past the batch).
__device__ __forceinline__ int longest_first(const AttnParams& p, int mine, int rank) {
  const int lane = threadIdx.x & 63;
  int above = 0;
  for (int j = 0; j < p.batch; ++j) {
    const int other = __builtin_amdgcn_readlane(mine, j);
    above += (other > mine) || (other == mine && j < lane);
  }
  const unsigned long long hit = __ballot(lane < p.batch && above == rank);
  return hit ? (int)__builtin_ctzll(hit) : rank;
}

// Raw query operand of one lane and k-step: 8 consecutive dimensions, as
// stored (bf16 or float32).
template <bool QF32>
struct QRaw {
  bf16x8 v;
  __device__ __forceinline__ void load(const void* base, size_t off) {
    v = *(const bf16x8*)((const uint16_t*)base + off);
  }
  __device__ __forceinline__ float at(int j) const { return (float)v[j]; }
};
template <>
struct QRaw<true> {
  float4 lo4, hi4;
  __device__ __forceinline__ void load(const void* base, size_t off) {
    const float4* q = (const float4*)((const float*)base + off);
    lo4 = q[0];
    hi4 = q[1];
  }
  __device__ __forceinline__ float at(int j) const {
    const float4& w = j < 4 ? lo4 : hi4;
    const int i = j & 3;
    return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
  }
};

template <int D, int NRP, bool QF32, int RS = 1>
__global__ __launch_bounds__(64 * kAttnWaves * RS) void attn_bf16_kernel(AttnParams p) {
  static_assert(RS == 1 || NRP == 16, "a second row set follows a full first one");
  constexpr int NT = 64 * kAttnWaves * RS;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr bool PACKED = (NRP == 8);
  constexpr int NR = NRP * RS;  // rows of the workgroup, padded
  // With two row sets, chunks pass from the first set to the second through
  // LDS: per wave of a set two slots of kPieces 16-byte pieces per lane (the
  // chunk as that lane holds it), in the space the final merge uses after the loop.
  constexpr int kPieces = 2 * KS + DB;
  constexpr int kSoFloats = kAttnWaves * NR * D;
  constexpr int kXchgFloats = RS == 1 ? 0 : kAttnWaves * 2 * kPieces * 64 * 4;
  __shared__ int tbl[kMaxTableSlice];
  __shared__ __attribute__((aligned(16))) float sm[kAttnWaves * NR];
  __shared__ __attribute__((aligned(16))) float sl[kAttnWaves * NR];
  __shared__ __attribute__((aligned(16))) float so[kSoFloats > kXchgFloats ? kSoFloats : kXchgFloats];

  const int s = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rs = RS == 1 ? 0 : wave_all / kAttnWaves;  // row set of the wave
  const int wave = RS == 1 ? wave_all : wave_all - rs * kAttnWaves;
  const int n = lane & 15, grp = lane >> 4;
  const int row = PACKED ? (n & 7) : n + NRP * rs;
  const int nr = p.flows * p.group;
  const bool two = p.flows == 2;

  // ---- prologue: the length, the queries and the split's block-table slice
  // are independent loads, issued together; the first cache loads wait only
  // for the table. Padding rows (row >= nr) load row nr - 1 and are zeroed. ----
  const int rr = min(row, nr - 1);
  const int f = rr / p.group, h = g * p.group + (rr - f * p.group);
  QRaw<QF32> q1r[KS], q2r[KS];
  float4 ar[KS][2];
  int jb0 = 0;
  auto load_prologue = [&](int bb) __attribute__((always_inline)) {
    const size_t qoff = ((size_t)bb * p.hq + h) * D;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int d0 = 32 * st + 8 * grp;
      q1r[st].load(p.q1, qoff + d0);
      if (two) {
        q2r[st].load(p.q2, qoff + d0);
        const float4* av = (const float4*)(p.a + (size_t)h * D + d0);
        ar[st][0] = av[0];
        ar[st][1] = av[1];
      }
    }
    jb0 = stage_split_table<NT>(p, bb, s, tbl);
  };
  // With longest-first order the loads for sequence blockIdx.z go out while
  // the lengths are ranked, and are issued again only if the ranking picks
  // another sequence (so uniform lengths cost no extra latency).
  int b = blockIdx.z;
  const int mine = p.longest_first && lane < p.batch ? p.ctx[lane] : INT_MIN;
  load_prologue(b);
  if (p.longest_first) {
    const int bl = longest_first(p, mine, b);
    if (bl != b) {
      b = bl;
      load_prologue(b);
    }
  }
  const int len_raw = p.ctx[b];
  __syncthreads();  // the table slice is read by every wave
  SplitRange r;
  if (!split_bounds<D, NT>(p, b, g, s, len_raw, r)) return;

  // ---- first chunk's loads, then the query operands while they are in flight ----
  const int bs = 1 << p.bs_log2;
  const uint16_t* __restrict__ kc = (const uint16_t*)p.k + (size_t)g * bs * D;
  const uint16_t* __restrict__ vc = (const uint16_t*)p.v + (size_t)g * D * bs;
  const int nchunks = (r.end - r.start + 31) >> 5;
  const uint32_t koff = (grp * 16 + n) * 16, voff = (n * 16 + 4 * grp) * 2;  // bytes within a tile
  Chunk<D> ca, cb;
  int c = wave;
  if (c < nchunks && rs == 0) load_chunk<D>(p, kc, vc, tbl, jb0, r.start + 32 * c, r.end, koff, voff, ca);

  // scaled (and for flow 2 coupled) query rows, split hi/lo
  bf16x8 qa[KS], qb[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v1 = q1r[st].at(j);
      float x = v1;
      if (two) {
        const float a = j < 4 ? (&ar[st][0].x)[j] : (&ar[st][1].x)[j - 4];
        x = f == 1 ? fmaf(a, v1, q2r[st].at(j)) : v1;
      }
      x = row < nr ? x * p.qscale : 0.f;
      const __bf16 hi = (__bf16)x;
      const __bf16 lo = (__bf16)(x - (float)hi);
      if (PACKED) {
        qa[st][j] = (n < 8) ? hi : lo;
      } else {
        qa[st][j] = hi;
        qb[st][j] = lo;
      }
    }
  }

  // ---- stream the split's positions in 32-position chunks ----
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk: scores, online softmax, weighted values. The running max of a
  // row moves only when the chunk's max of that row exceeds it by more than
  // kLazyRescale (base-2 units), so the weights 2^(s - m_run) stay below
  // 2^kLazyRescale and most chunks skip rescaling the accumulators (a
  // wave-wide vote skips the whole step when no row needs it). The decision
  // is the row's own -- other rows, the other flow's included, change neither
  // its values nor their rounding. The final (O, m, l) of a row describe the
  // same softmax whatever m_run ended as.
  auto process = [&](Chunk<D>& cur, int c) __attribute__((always_inline)) {
    const int t0 = r.start + 32 * c;
    f32x4 sv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) acc = mfma(cur.k[u][st], qa[st], acc);
      if (!PACKED) {
#pragma unroll
        for (int st = 0; st < KS; ++st) acc = mfma(cur.k[u][st], qb[st], acc);
      }
      sv[u] = acc;
    }
    float sc[8];  // sc[4*u + i]: row n, position t0 + 16*u + 4*grp + i
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * u + i] = sv[u][i];
    if (PACKED) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[j] += dpp_ror8(sc[j]);
    }
    if (t0 + 32 > r.end) {  // tail chunk (wave-uniform): mask positions past the split, zero unused values
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tv = tile_start(t0, u, r.end) + 4 * grp;  // positions of this lane's values
        uint32_t keep[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          keep[h] = (tv + 2 * h < r.end ? 0x0000FFFFu : 0u) | (tv + 2 * h + 1 < r.end ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          cur.v[db][2 * u] &= keep[0];
          cur.v[db][2 * u + 1] &= keep[1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[4 * u + i] = (t0 + 16 * u + 4 * grp + i < r.end) ? sc[4 * u + i] : -INFINITY;
      }
    }
    float cmax = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cmax = score_max(cmax, sc[j]);
    cmax = max_over_groups(cmax);
    const bool moves = cmax > m_run + kLazyRescale;  // the same in every lane of a row
    if (__builtin_amdgcn_ballot_w64(moves) != 0) {
      const float m_new = moves ? cmax : m_run;
      const float alpha = moves ? fast_exp2(m_run - m_new) : 1.f;  // 1: exact, the row is untouched
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    float pv[8], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = fast_exp2(sc[j] - m_run);
      psum += pv[j];
    }
    l_run += psum;
    // Both tiles in one product: k-slot 8*grp + j of the lane is position
    // 4*grp + j of tile 0 for j < 4 and 4*grp + j - 4 of tile 1 otherwise, in
    // the values (words 0-1, 2-3) and in the weights (pv[j]) alike.
    bf16x8 pa, pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = pv[j];
      const __bf16 hi = (__bf16)x;
      const __bf16 lo = (__bf16)(x - (float)hi);
      if (PACKED) {
        pa[j] = (n < 8) ? hi : lo;
      } else {
        pa[j] = hi;
        pb[j] = lo;
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = mfma(__builtin_bit_cast(bf16x8, cur.v[db]), pa, oacc[db]);
    if (!PACKED) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = mfma(__builtin_bit_cast(bf16x8, cur.v[db]), pb, oacc[db]);
    }
  };

  // Wave w takes chunks w, w + kAttnWaves, ...; two register buffers alternate so
  // that the next chunk's loads are in flight while the current one is used.
  if constexpr (RS == 1) {
    for (; c < nchunks; c += 2 * kAttnWaves) {
      if (c + kAttnWaves < nchunks)
        load_chunk<D>(p, kc, vc, tbl, jb0, r.start + 32 * (c + kAttnWaves), r.end, koff, voff, cb);
      process(ca, c);
      if (c + kAttnWaves >= nchunks) break;
      if (c + 2 * kAttnWaves < nchunks)
        load_chunk<D>(p, kc, vc, tbl, jb0, r.start + 32 * (c + 2 * kAttnWaves), r.end, koff, voff, ca);
      process(cb, c + kAttnWaves);
    }
  } else {
    // Two row sets: wave w of the first set loads chunk w + kAttnWaves * it (the
    // next one in flight, as above), copies it to its LDS slot it % 2 and
    // processes it; wave w of the second set processes it one step later, from
    // the slot. The cache is thus read once from HBM and once through L2 for
    // all 32 rows, and the second set works while the first waits for its
    // loads. One barrier opens every step, the same number of steps in every
    // wave (nchunks is uniform in the workgroup): a slot written in step it
    // (after its barrier) is read in step it + 1 (after the next barrier) and
    // rewritten in step it + 2, after the second set has passed that step's
    // barrier, i.e. finished reading it.
    uint4* xchg = reinterpret_cast<uint4*>(so) + (size_t)wave * 2 * kPieces * 64 + lane;
    const int steps = (nchunks + kAttnWaves - 1) / kAttnWaves;
    // The two sets run separate loops (rs is uniform in a wave), so that each
    // holds only its own registers; both pass steps + 1 barriers.
    if (rs == 0) {
      auto step0 = [&](Chunk<D>& cur, Chunk<D>& nxt, int it) __attribute__((always_inline)) {
        __syncthreads();
        const int cc = wave + kAttnWaves * it;
        if (cc + kAttnWaves < nchunks)
          load_chunk<D>(p, kc, vc, tbl, jb0, r.start + 32 * (cc + kAttnWaves), r.end, koff, voff, nxt);
        if (cc < nchunks) {
          uint4* slot = xchg + (it & 1) * kPieces * 64;
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int st = 0; st < KS; ++st) slot[(u * KS + st) * 64] = __builtin_bit_cast(uint4, cur.k[u][st]);
#pragma unroll
          for (int db = 0; db < DB; ++db) slot[(2 * KS + db) * 64] = __builtin_bit_cast(uint4, cur.v[db]);
          process(cur, cc);
        }
      };
      for (int it = 0; it <= steps; it += 2) {
        step0(ca, cb, it);
        if (it + 1 <= steps) step0(cb, ca, it + 1);
      }
    } else {
      for (int it = 0; it <= steps; ++it) {
        __syncthreads();
        const int cc = wave + kAttnWaves * (it - 1);
        if (it > 0 && cc < nchunks) {
          const uint4* slot = xchg + ((it - 1) & 1) * kPieces * 64;
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int st = 0; st < KS; ++st) ca.k[u][st] = __builtin_bit_cast(bf16x8, slot[(u * KS + st) * 64]);
#pragma unroll
          for (int db = 0; db < DB; ++db) ca.v[db] = __builtin_bit_cast(u32x4, slot[(2 * KS + db) * 64]);
          process(ca, cc);
        }
      }
    }
    __syncthreads();  // the last slots are read before the merge reuses their space
  }

  // ---- wave state to LDS, then merge the waves ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (PACKED) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[db][i] += dpp_ror8(oacc[db][i]);
  }
  if ((!PACKED || n < 8) && row < nr) {
    float* dst = so + (wave * NR + row) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)(dst + 16 * db) = oacc[db];
    if (grp == 0) {
      sm[row * kAttnWaves + wave] = m_run;
      sl[row * kAttnWaves + wave] = l_run;
    }
  }
  __syncthreads();
  merge_waves<D, NR, kAttnWaves, NT>(p, b, g, s, sm, sl, so);
}

// LDS a workgroup of attn_bf16_kernel<D, NRP> declares, and the dynamic LDS
// its launch adds so that one workgroup fills more than half of a compute
// unit's 160 KB: each CU then runs one workgroup at a time and takes the next
// one when it finishes, which balances ragged sequence lengths (two resident
// workgroups per CU were measured 4% slower on lengths U[1024, 8192] and no
// faster on uniform ones).
template <int D, int NR, int RS>
constexpr size_t one_per_cu_lds() {
  constexpr size_t kCuLds = 160 * 1024;
  constexpr size_t so = kAttnWaves * NR * D * 4;
  constexpr size_t xchg = RS == 1 ? 0 : kAttnWaves * 2 * (D / 16 + D / 16) * 64 * 16;  // two slots of 2*KS + DB pieces
  constexpr size_t stat = kMaxTableSlice * 4 + 2 * kAttnWaves * NR * 4 + (so > xchg ? so : xchg);
  return stat > kCuLds / 2 ? 0 : kCuLds / 2 + 256 - stat;
}

hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int rows_padded, hipStream_t stream,
                            const KernelEvents& ev) {
  const dim3 grid(p.n_splits, p.hkv, p.batch);
#define DFA_ATTN_CASE(D_, NRP_, RS_)                                                                         \
  if (head_dim == D_ && rows_padded == NRP_ * RS_)                                                           \
    return p.q_f32 ? launch_kernel(attn_bf16_kernel<D_, NRP_, true, RS_>, grid, dim3(64 * kAttnWaves * RS_), \
                                   stream, ev, p, one_per_cu_lds<D_, NRP_ * RS_, RS_>())                           \
                   : launch_kernel(attn_bf16_kernel<D_, NRP_, false, RS_>, grid, dim3(64 * kAttnWaves * RS_), \
                                   stream, ev, p, one_per_cu_lds<D_, NRP_ * RS_, RS_>());
  DFA_ATTN_CASE(128, 8, 1) DFA_ATTN_CASE(128, 16, 1) DFA_ATTN_CASE(64, 8, 1) DFA_ATTN_CASE(64, 16, 1)
  DFA_ATTN_CASE(128, 16, 2) DFA_ATTN_CASE(64, 16, 2)
#undef DFA_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace dfa
