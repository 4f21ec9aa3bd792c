// Internal interface between the host-side ABI (abi.cpp) and the launchers of
// the weight-streaming and output-head kernels (gemv.hip, mixture.hip,
// moe.hip, prefill.hip, norm.hip) and of the debug check (debug.hip). Plain
// structs passed by value to the kernels. The attention kernels do not
// include this file.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dfa {

enum : int32_t { kEpiNone = 0, kEpiResidual = 1, kEpiSwiglu = 2, kEpiResidualCoupled = 3, kEpiKvAppend = 4,
                 // layer-internal: rows [Wq; Wk; Wv]; columns [0, q_cols) are both flows' queries
                 // (y1/y2 [batch, q_cols]), the next kv_cols the primary's keys, then its values
                 // (appended to the cache). Split-K only (the finalize sees keys and values together).
                 kEpiQkv = 5,
                 // grouped (MoE) only: the two matrices are the two halves of one [2n, k] matrix;
                 // outputs are rows of 2n floats, matrix 0 in columns [0, n), matrix 1 in [n, 2n)
                 kEpiSplitPair = 6 };

struct GemvParams {
  const uint16_t* w;   // tiled [n/16][k/8][16][8]
  const uint16_t* w2;  // second matrix (SwiGLU up, KV append values) or null
  const float* x1;     // [batch, k]
  const float* x2;     // [batch, k] (two flows)
  const float* couple; // [n] or null
  const float* res1;   // [batch, n]
  const float* res2;
  float* y1;           // [batch, n]
  float* y2;
  float* part;         // [k_split][mats][m_pad][n]
  int32_t batch, n, k, flows, cbf, m_pad, k_split, k_range, pair, x_exact, epilogue;
  int32_t rows_per_wg;  // weight rows per workgroup: 64 or 128
  const uint16_t* w_seg1;  // rows [seg1_row, seg2_row) come from w_seg1, rows [seg2_row, n) from
  const uint16_t* w_seg2;  // w_seg2 (each tiled on its own); seg1_row = seg2_row = n: one matrix
  int32_t seg1_row, seg2_row;
  int32_t q_cols, kv_cols;  // kEpiQkv
  // Grouped (mixture-of-experts) launch when moe_sel is set: moe_sel [batch][moe_k2]
  // experts per sequence in ranking order (the first moe_k1 the primary's); the
  // matrices of expert e start e * moe_wstride elements after w (and w2);
  // moe_rgs row groups per expert. Activation row of (sequence s, slot, flow f):
  // s * moe_row_s + slot * moe_row_slot + f * moe_row_f of x_f. Outputs go to
  // rows ((s * moe_k2 + slot) * 2 + f) of y1 (= y2).
  const int32_t* moe_sel;
  int64_t moe_wstride;
  int32_t moe_k1, moe_k2, moe_experts, moe_rgs, moe_row_s, moe_row_slot, moe_row_f;
  // kEpiQkv: rotary embedding of both flows' queries and the primary's keys at
  // position ctx_lens[s] (kRopeNone, kRopeHalf: pairs (i, i + D/2) of a head,
  // kRopeInterleaved: pairs (2i, 2i + 1)); tables [rope_max_pos][D/2], D = kv_head_dim.
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope, rope_max_pos;
  uint16_t* kv_k;      // KV append target
  uint16_t* kv_v;
  const int32_t* kv_table;
  const int32_t* kv_ctx;
  int32_t kv_hkv, kv_head_dim, kv_bs_log2, kv_max_blocks, kv_num_blocks;
};

// Mixture decoding: the vocabulary is cut into chunks of kMixChunk tokens;
// at most kMixMaxChunks chunks (one per thread of the pick kernel).
constexpr int kMixChunk = 4096;
constexpr int kMixMaxChunks = 256;
constexpr int kMixRec = 8;  // floats per chunk-statistics record (5 used, 32-byte aligned)
// Vocabularies up to this size take one workgroup per sequence (the logits held in registers).
constexpr int kMixFusedMaxVocab = 32768;

struct MixParams {
  const float* logits1;  // [batch, vocab]
  const float* logits2;
  const float* u;        // [batch] uniforms in [0, 1)
  int32_t* token;        // [batch] inverse-CDF draw
  int32_t* greedy;       // [batch] first most likely token
  float* alpha;          // [batch]
  float* p_mix;          // [batch, vocab] or null
  float* rec;            // workspace: [batch][chunks][kMixRec] softmax statistics
  uint32_t* crec;        // workspace: [batch][chunks][4] mass (2 words), first maximum (value, token)
  int32_t batch, vocab, chunks;
};

// Mixture-of-experts routing and output combination.
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxK = 32;

struct MoeRouteParams {
  const float* r1;  // [batch, experts] router logits of the primary flow
  const float* r2;  // [batch, experts] of the auxiliary flow
  int32_t* sel;     // [batch, k2] experts in ranking order
  float* g1;        // [batch, k1]
  float* g2;        // [batch, k2]
  int32_t batch, experts, k1, k2;
};

struct MoeCombineParams {
  const float* y;     // [batch][k2][2][hidden] expert outputs of both flows
  const float* g1;
  const float* g2;
  const float* res1;  // [batch, hidden] or null
  const float* res2;
  const float* c;     // [hidden] or null
  float* out1;
  float* out2;
  int32_t batch, hidden, k1, k2;
};

// Primary-only prefill: the prompt's keys and values into the paged cache, then
// causal self-attention. q [batch][lmax][hq][D], k, v [batch][lmax][hkv][D]
// (bf16), o [batch][lmax][hq][D] (float32); cache layouts as the decode kernels'.
struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* lens;   // [batch] prompt lengths (clamped to [0, lmax])
  const int32_t* table;  // [batch][max_blocks] (entries clamped to [0, num_blocks))
  uint16_t* k_cache;
  uint16_t* v_cache;
  float* o;
  int32_t batch, hq, hkv, lmax, lmax_tiles, g_log2, bs_log2, max_blocks, num_blocks;
  int64_t blk_stride;  // elements per physical block: hkv * block_size * D
  float qscale;        // scale * log2(e)
};

enum : int32_t { kRopeNone = 0, kRopeHalf = 1, kRopeInterleaved = 2 };

// RMSNorm of rows of both flows: y_f = x_f / sqrt(mean(x_f^2) + eps) * w.
struct NormParams {
  const float* x1;
  const float* x2;
  const float* w;  // [n]
  float* y1;
  float* y2;
  int32_t rows, n;
  float eps;
};

// Debug aid: device-side check of a decode call's lengths and block-table entries.
enum : uint32_t { kTableBadLen = 1u, kTableBadBlock = 2u };
struct TableCheckParams {
  const int32_t* table;
  const int32_t* ctx;
  uint32_t* flags;  // [0]: bits, [1]: first offending sequence (0xFFFFFFFF: none)
  int32_t batch, max_blocks, num_blocks, max_ctx, block_size, ctx_add;
};

// Launchers return the launch status (hipGetLastError after the launch).
hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t s);
constexpr int kPrefillMaxBlocks = 2048;  // cache blocks one prompt may span (staged in LDS)
hipError_t launch_gemv(const GemvParams& p, hipStream_t s);
hipError_t launch_gemv_finalize(const GemvParams& p, hipStream_t s);
hipError_t launch_pack_weight(const uint16_t* w, uint16_t* wt, int n, int k, hipStream_t s);
size_t gemv_chunk();
hipError_t launch_mixture(const MixParams& p, hipStream_t s);
hipError_t launch_moe_route(const MoeRouteParams& p, hipStream_t s);
hipError_t launch_moe_combine(const MoeCombineParams& p, hipStream_t s);
size_t mixture_chunks(int vocab);
hipError_t launch_check_table(const TableCheckParams& p, hipStream_t s);

}  // namespace dfa
