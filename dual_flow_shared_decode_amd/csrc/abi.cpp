// extern "C" entry points of libdfa: argument validation, split planning and
// kernel dispatch. Validation is plain host code and runs before any HIP call;
// an invalid call returns a status and enqueues nothing.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/dfa.h"
#include "dfa_internal.h"
#include "ops_internal.h"

namespace {

thread_local std::string g_last_error;

dfa_status fail(dfa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

// Positions per split chosen by the library (measured on MI355X, 256 CUs): one
// workgroup per compute unit is what streams the cache at full rate -- 128
// workgroups reach about 6 TB/s of plain reads, 256 about 6.7 -- while more
// splits add records and combine traffic. So a single split per sequence when
// there are at least 256 (sequence, kv head) pairs (ragged lengths included:
// splitting them measured slower), else enough splits for about 256
// workgroups, of at least 512 positions each.
int64_t auto_split_len(const dfa_attn_desc* d) {
  const int64_t pairs = int64_t(d->batch) * d->num_kv_heads;
  const int64_t whole = (int64_t(d->max_ctx_len) + 31) / 32 * 32;
  if (pairs >= 256) return whole;
  const int64_t splits = (256 + pairs - 1) / pairs;
  int64_t len = (int64_t(d->max_ctx_len) + splits - 1) / splits;
  len = std::max<int64_t>((len + 255) / 256 * 256, 512);
  return std::min(len, whole);
}

dfa_status validate_attn(const dfa_attn_desc* d, int32_t* split_out) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  if (d->batch < 1 || d->batch > 65535) return fail(DFA_ERR_SHAPE, "batch must be in [1, 65535]");
  if (d->num_kv_heads < 1 || d->num_kv_heads > 65535)
    return fail(DFA_ERR_SHAPE, "num_kv_heads must be in [1, 65535]");
  if (d->num_q_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
    return fail(DFA_ERR_SHAPE, "num_q_heads must be a positive multiple of num_kv_heads");
  if (d->num_flows != 1 && d->num_flows != 2) return fail(DFA_ERR_SHAPE, "num_flows must be 1 or 2");
  if (d->head_dim < 1) return fail(DFA_ERR_SHAPE, "head_dim must be positive");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(DFA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int64_t group = d->num_q_heads / d->num_kv_heads;
  if (group * d->num_flows > dfa::kMaxRowsBf16)
    return fail(DFA_ERR_UNSUPPORTED, "(num_q_heads / num_kv_heads) * num_flows must be <= 32");
  if (!is_pow2(d->block_size) || d->block_size < 16)
    return fail(DFA_ERR_SHAPE, "block_size must be a power of two >= 16");
  if (d->max_blocks_per_seq < 1) return fail(DFA_ERR_SHAPE, "max_blocks_per_seq must be >= 1");
  if (d->num_blocks < 1) return fail(DFA_ERR_SHAPE, "num_blocks must be >= 1");
  if (d->max_ctx_len < 1) return fail(DFA_ERR_SHAPE, "max_ctx_len must be >= 1");
  if (int64_t(d->max_blocks_per_seq) * d->block_size < d->max_ctx_len)
    return fail(DFA_ERR_SHAPE, "max_ctx_len exceeds max_blocks_per_seq * block_size");
  if (d->split_len < 0 || d->split_len % 32 != 0)
    return fail(DFA_ERR_SHAPE, "split_len must be 0 or a positive multiple of 32");
  if (!std::isfinite(d->scale)) return fail(DFA_ERR_SHAPE, "scale must be finite");
  const bool kv_bf16 = d->kv_dtype == DFA_BF16, kv_f32 = d->kv_dtype == DFA_F32;
  const bool q_ok = d->q_dtype == DFA_BF16 || d->q_dtype == DFA_F32;
  if (!(kv_bf16 || kv_f32) || !q_ok) return fail(DFA_ERR_DTYPE, "unknown dtype");
  if (kv_f32 && d->q_dtype != DFA_F32) return fail(DFA_ERR_DTYPE, "a float32 cache needs float32 queries");
  if (kv_f32 && group * d->num_flows > dfa::kMaxRows)
    return fail(DFA_ERR_UNSUPPORTED, "with a float32 cache, (num_q_heads / num_kv_heads) * num_flows must be <= 16");
  int64_t split = d->split_len > 0 ? d->split_len : auto_split_len(d);
  // the block-table slice of one split must fit the staging buffer
  if ((split - 1) / d->block_size + 2 > dfa::kMaxTableSlice) {
    if (d->split_len > 0) return fail(DFA_ERR_UNSUPPORTED, "split_len spans too many cache blocks (max 1022)");
    split = int64_t(dfa::kMaxTableSlice - 2) * d->block_size / 128 * 128;
  }
  if (split > (int64_t(1) << 30)) split = int64_t(1) << 30;
  if (split_out) *split_out = int32_t(split);
  return DFA_OK;
}

int32_t num_splits(const dfa_attn_desc* d, int32_t split) {
  return int32_t((int64_t(d->max_ctx_len) + split - 1) / split);
}

// Workspace = one partial record per (sequence, query head, flow, split).
size_t workspace_bytes(const dfa_attn_desc* d, int32_t split) {
  return size_t(d->batch) * d->num_q_heads * d->num_flows * size_t(num_splits(d, split)) *
         (d->head_dim + dfa::kRecPad) * sizeof(float);
}

dfa_status check_tensors(const dfa_attn_desc* d, const void* q1, const void* q2, const float* a,
                         const void* k, const void* v, const int32_t* table, const int32_t* ctx) {
  if (!q1 || !k || !v || !table || !ctx) return fail(DFA_ERR_NULL, "q1, k_cache, v_cache, block_table and ctx_lens are required");
  if (d->num_flows == 2 && (!q2 || !a)) return fail(DFA_ERR_NULL, "q2 and a are required with two flows");
  const void* ptrs[] = {q1, k, v, table, ctx};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (d->num_flows == 2 && (!aligned16(q2) || !aligned16(a)))
    return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  return DFA_OK;
}

dfa::AttnParams make_params(const dfa_attn_desc* d, int32_t split, const void* q1, const void* q2,
                            const float* a, const void* k, const void* v, const int32_t* table,
                            const int32_t* ctx) {
  dfa::AttnParams p{};
  p.q1 = q1;
  p.q2 = d->num_flows == 2 ? q2 : nullptr;
  p.a = d->num_flows == 2 ? a : nullptr;
  p.k = k;
  p.v = v;
  p.table = table;
  p.ctx = ctx;
  p.batch = d->batch;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.flows = d->num_flows;
  p.bs_log2 = log2i(d->block_size);
  p.max_blocks = d->max_blocks_per_seq;
  p.num_blocks = d->num_blocks;
  p.max_ctx = d->max_ctx_len;
  p.split_len = split;
  p.n_splits = num_splits(d, split);
  p.blk_stride = int64_t(d->num_kv_heads) * d->block_size * d->head_dim;
  p.qscale = d->scale * 1.4426950408889634f;  // log2(e): scores in base-2 units
  p.q_f32 = d->q_dtype == DFA_F32;
  return p;
}

dfa_status launch_split_stage(const dfa_attn_desc* d, const dfa::AttnParams& p, hipStream_t st,
                              const dfa_kernel_events* events) {
  dfa::KernelEvents ev;
  if (events) {
    ev.start = static_cast<hipEvent_t>(events->start);
    ev.stop = static_cast<hipEvent_t>(events->stop);
  }
  hipError_t e;
  if (d->kv_dtype == DFA_F32) {
    e = dfa::launch_attn_f32(p, d->head_dim, st, ev);
  } else {
    const int rows = (d->num_q_heads / d->num_kv_heads) * d->num_flows;
    e = dfa::launch_attn_bf16(p, d->head_dim, rows <= 8 ? 8 : (rows <= 16 ? 16 : 32), st, ev);
  }
  if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return DFA_OK;
}

dfa_status launch_combine_stage(const dfa_attn_desc* d, int32_t split, const void* ws, float* o1, float* o2,
                                hipStream_t st) {
  dfa::CombineParams c{};
  c.part = static_cast<const float*>(ws);
  c.o1 = o1;
  c.o2 = d->num_flows == 2 ? o2 : nullptr;
  c.batch = d->batch;
  c.hq = d->num_q_heads;
  c.flows = d->num_flows;
  c.n_splits = num_splits(d, split);
  const hipError_t e = dfa::launch_combine(c, d->head_dim, st);
  if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("combine launch: ") + hipGetErrorString(e));
  return DFA_OK;
}

dfa_status check_workspace(const dfa_attn_desc* d, int32_t split, const void* ws, size_t bytes) {
  if (!ws) return fail(DFA_ERR_WORKSPACE, "workspace is required when more than one split runs");
  if (!aligned16(ws)) return fail(DFA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if (bytes < workspace_bytes(d, split)) return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_decode_attn_workspace_size()");
  return DFA_OK;
}

// Every host-side check of an attention call except the workspace's.
dfa_status check_attn_call(const dfa_attn_desc* desc, const void* q1, const void* q2, const float* a,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* ctx_lens, const float* o1, const float* o2, int32_t* split) {
  dfa_status st = validate_attn(desc, split);
  if (st != DFA_OK) return st;
  st = check_tensors(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens);
  if (st != DFA_OK) return st;
  if (!o1 || (desc->num_flows == 2 && !o2)) return fail(DFA_ERR_NULL, "o1 (and o2 with two flows) are required");
  if (!aligned16(o1) || (desc->num_flows == 2 && !aligned16(o2)))
    return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  return DFA_OK;
}

dfa_status attn_impl(const dfa_attn_desc* desc, const void* q1, const void* q2, const float* a, const void* k_cache,
                     const void* v_cache, const int32_t* block_table, const int32_t* ctx_lens, int32_t ctx_add,
                     void* workspace, size_t ws_bytes, float* o1, float* o2, hipStream_t hs,
                     const dfa_kernel_events* events) {
  int32_t split = 0;
  dfa_status st = check_attn_call(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, o1, o2, &split);
  if (st != DFA_OK) return st;
  const int32_t ns = num_splits(desc, split);
  if (ns > 1) {
    st = check_workspace(desc, split, workspace, ws_bytes);
    if (st != DFA_OK) return st;
  }
  dfa::AttnParams p = make_params(desc, split, q1, q2, a, k_cache, v_cache, block_table, ctx_lens);
  p.ctx_add = ctx_add;
  if (ns == 1) {
    p.direct = 1;
    // one workgroup per (sequence, kv head): take sequences longest first (the
    // kernel ranks up to 64 lengths in one wave)
    p.longest_first = desc->batch > 1 && desc->batch <= 64;
    p.o1 = o1;
    p.o2 = desc->num_flows == 2 ? o2 : nullptr;
    return launch_split_stage(desc, p, hs, events);
  }
  p.part = static_cast<float*>(workspace);
  st = launch_split_stage(desc, p, hs, events);
  if (st != DFA_OK) return st;
  return launch_combine_stage(desc, split, workspace, o1, o2, hs);
}

// ------------------------------------------------------------------ dual GEMV
struct GemvPlan {
  int32_t cbf, m_pad, k_split, k_range, mats, rows_per_wg;
  int32_t slice;  // sequences per launch: the kernels take at most 64 activation rows (both flows)
};

dfa_status validate_gemv(const dfa_gemv_desc* d, GemvPlan* plan) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  if (d->num_flows != 1 && d->num_flows != 2) return fail(DFA_ERR_SHAPE, "num_flows must be 1 or 2");
  if (d->batch < 1 || d->batch > 65535) return fail(DFA_ERR_SHAPE, "batch must be in [1, 65535]");
  if (d->n < 64 || d->n % 64 != 0) return fail(DFA_ERR_SHAPE, "n must be a positive multiple of 64");
  if (d->k < 128 || d->k % 128 != 0) return fail(DFA_ERR_SHAPE, "k must be a positive multiple of 128");
  if (d->epilogue < DFA_EPI_NONE || d->epilogue > DFA_EPI_KV_APPEND) return fail(DFA_ERR_SHAPE, "unknown epilogue");
  if (d->epilogue == DFA_EPI_KV_APPEND && d->num_flows != 1)
    return fail(DFA_ERR_SHAPE, "the KV append is the primary flow's alone (num_flows 1)");
  if (d->k_split < 0) return fail(DFA_ERR_SHAPE, "k_split must be >= 0");
  if (d->rows_per_wg != 0 && d->rows_per_wg != 64 && d->rows_per_wg != 128)
    return fail(DFA_ERR_SHAPE, "rows_per_wg must be 0, 64 or 128");
  if (d->rows_per_wg == 128 && d->n % 128 != 0) return fail(DFA_ERR_SHAPE, "rows_per_wg 128 needs n % 128 == 0");
  GemvPlan pl;
  // Larger batches run in slices of 32 sequences (two flows) or 64 (one flow),
  // one launch (and reduction) per slice, each reading the weights again.
  pl.slice = 64 / d->num_flows;
  const int32_t rows = std::min(d->batch, pl.slice);
  pl.cbf = (rows + 15) / 16;  // 16-row activation blocks per flow; kernels exist for 1, 2, 4 blocks in all
  if (d->num_flows * pl.cbf > 4) return fail(DFA_ERR_UNSUPPORTED, "too many activation rows");
  if (pl.cbf == 3) pl.cbf = 4;    // one flow, 33..48 rows: padded to 64
  pl.m_pad = d->num_flows * pl.cbf * 16;
  const int64_t chunks = d->k / int64_t(dfa::gemv_chunk());
  // Library choice of the workgroup's rows (measured on MI355X, batch 32, two
  // flows): 128 for a large matrix (at least 48 Mi elements) that is either too
  // narrow to fill the chip unsplit at 64 rows or wide enough to fill it
  // unsplit at 128 -- the activations a workgroup loads per stage then serve
  // twice the weight rows and twice the weight bytes are in flight
  // (4096 x 14336: 37.5 -> 33.4 us; 32000 x 4096: 68.3 -> 49.1 us); else 64
  // (a 14336-row matrix runs unsplit at 64 rows and is faster so than split
  // at 128).
  const bool big = int64_t(d->n) * d->k >= (int64_t(48) << 20);
  const bool wide128 = d->n % 128 == 0 && (d->n / 64 < 192 || d->n / 128 >= 192);
  pl.rows_per_wg = d->rows_per_wg > 0 ? d->rows_per_wg : ((big && wide128) ? 128 : 64);
  const int64_t row_groups = d->n / pl.rows_per_wg;
  // About one workgroup per compute unit (at most 256); a matrix with at
  // least 192 row groups runs unsplit, so its epilogue needs no second launch.
  // At most 16 k-ranges by choice: the reduction then issues all of a thread's loads at once (the
  // 64 x 4096 MoE router: 11.5 us at 32 k-ranges, 9.8 us at 16).
  int64_t ks = d->k_split > 0 ? d->k_split
                              : (row_groups >= 192 ? 1 : std::min<int64_t>(16, std::max<int64_t>(1, 256 / row_groups)));
  ks = std::min<int64_t>(ks, chunks);
  const int64_t chunks_per = (chunks + ks - 1) / ks;
  pl.k_range = int32_t(chunks_per * dfa::gemv_chunk());
  pl.k_split = int32_t((chunks + chunks_per - 1) / chunks_per);
  pl.mats = (d->epilogue == DFA_EPI_SWIGLU || d->epilogue == DFA_EPI_KV_APPEND) ? 2 : 1;
  if (plan) *plan = pl;
  return DFA_OK;
}

size_t gemv_workspace(const dfa_gemv_desc* d, const GemvPlan& pl) {
  if (pl.k_split == 1) return 0;  // the epilogue runs in the GEMV kernel
  return size_t(pl.k_split) * pl.mats * pl.m_pad * size_t(d->n) * sizeof(float);
}

dfa_status gemv_impl(const dfa_gemv_desc* d, const uint16_t* w, const uint16_t* w2, const float* x1,
                     const float* x2, const float* couple, const float* res1, const float* res2, float* y1,
                     float* y2, const dfa_kv_target* kv, void* workspace, size_t ws_bytes, hipStream_t hs) {
  {
    GemvPlan pl;
    dfa_status st = validate_gemv(d, &pl);
    if (st != DFA_OK) return st;
    const bool two = d->num_flows == 2;
    const bool pair = pl.mats == 2;
    const bool kvapp = d->epilogue == DFA_EPI_KV_APPEND;
    const bool resid = d->epilogue == DFA_EPI_RESIDUAL || d->epilogue == DFA_EPI_RESIDUAL_COUPLED;
    if (!w || !x1 || (two && !x2) || (pair && !w2)) return fail(DFA_ERR_NULL, "w, x1 (x2 with two flows, w2 for SwiGLU / KV append) are required");
    if (!kvapp && (!y1 || (two && !y2))) return fail(DFA_ERR_NULL, "y1 (and y2 with two flows) are required");
    if (resid && (!res1 || (two && !res2))) return fail(DFA_ERR_NULL, "residual inputs are required");
    if (kvapp && (!kv || !kv->k_cache || !kv->v_cache || !kv->block_table || !kv->ctx_lens))
      return fail(DFA_ERR_NULL, "the KV append needs a complete dfa_kv_target");
    const void* ptrs[] = {w, w2, x1, x2, couple, res1, res2, y1, y2, workspace};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t need = gemv_workspace(d, pl);
    if (need > 0 && !workspace) return fail(DFA_ERR_WORKSPACE, "workspace is required when k_split > 1");
    if (ws_bytes < need) return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_dual_gemv_workspace_size()");
    dfa::GemvParams p{};
    if (kvapp) {
      if (kv->num_kv_heads < 1 || kv->head_dim < 8 || kv->head_dim % 8 != 0 ||
          int64_t(kv->num_kv_heads) * kv->head_dim != d->n)
        return fail(DFA_ERR_SHAPE, "KV append: n must equal num_kv_heads * head_dim (head_dim multiple of 8)");
      if (!is_pow2(kv->block_size) || kv->block_size < 16 || kv->max_blocks_per_seq < 1 || kv->num_blocks < 1)
        return fail(DFA_ERR_SHAPE, "KV append: block_size power of two >= 16, positive table sizes");
      if (!aligned16(kv->k_cache) || !aligned16(kv->v_cache) || !aligned16(kv->block_table) || !aligned16(kv->ctx_lens))
        return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
      p.kv_k = static_cast<uint16_t*>(kv->k_cache);
      p.kv_v = static_cast<uint16_t*>(kv->v_cache);
      p.kv_table = kv->block_table;
      p.kv_ctx = kv->ctx_lens;
      p.kv_hkv = kv->num_kv_heads;
      p.kv_head_dim = kv->head_dim;
      p.kv_bs_log2 = log2i(kv->block_size);
      p.kv_max_blocks = kv->max_blocks_per_seq;
      p.kv_num_blocks = kv->num_blocks;
    }
    p.w = w;
    p.w2 = pair ? w2 : nullptr;
    p.x1 = x1;
    p.x2 = two ? x2 : nullptr;
    p.couple = two ? couple : nullptr;
    p.res1 = res1;
    p.res2 = two ? res2 : nullptr;
    p.y1 = y1;
    p.y2 = two || kvapp ? y2 : nullptr;
    p.part = static_cast<float*>(workspace);
    p.batch = d->batch;
    p.n = d->n;
    p.k = d->k;
    p.flows = d->num_flows;
    p.cbf = pl.cbf;
    p.m_pad = pl.m_pad;
    p.k_split = pl.k_split;
    p.k_range = pl.k_range;
    p.pair = pair;
    p.x_exact = d->x_exact_bf16 != 0;
    p.epilogue = d->epilogue;
    p.rows_per_wg = pl.rows_per_wg;
    p.w_seg1 = p.w_seg2 = w;  // one matrix
    p.seg1_row = p.seg2_row = d->n;
    // slices of at most pl.slice sequences, in order on the stream (they share the workspace)
    for (int32_t b0 = 0; b0 < d->batch; b0 += pl.slice) {
      dfa::GemvParams q = p;
      dfa_gemv_desc ds = *d;
      ds.batch = std::min(pl.slice, d->batch - b0);
      GemvPlan ps;
      validate_gemv(&ds, &ps);
      q.batch = ds.batch;
      q.cbf = ps.cbf;
      q.m_pad = ps.m_pad;
      q.k_split = ps.k_split;
      q.k_range = ps.k_range;
      auto row = [b0](const float* base, int32_t cols) { return base ? base + size_t(b0) * cols : nullptr; };
      q.x1 = row(p.x1, d->k);
      q.x2 = row(p.x2, d->k);
      q.res1 = row(p.res1, d->n);
      q.res2 = row(p.res2, d->n);
      q.y1 = const_cast<float*>(row(p.y1, d->n));
      q.y2 = const_cast<float*>(row(p.y2, d->n));
      if (kvapp) {
        q.kv_table = p.kv_table + size_t(b0) * p.kv_max_blocks;
        q.kv_ctx = p.kv_ctx + b0;
      }
      hipError_t e = dfa::launch_gemv(q, hs);
      if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("gemv launch: ") + hipGetErrorString(e));
      if (ps.k_split > 1) {
        e = dfa::launch_gemv_finalize(q, hs);
        if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("gemv epilogue launch: ") + hipGetErrorString(e));
      }
    }
    return DFA_OK;
  }
}

// ------------------------------------------------------------------ decode layer
struct LayerPlan {
  dfa_attn_desc attn;
  dfa_gemv_desc qkv, o, mlp_in, mlp_out;
  GemvPlan qkv_plan;
  size_t off_q, off_o, off_h, off_z, off_attn, off_gemv, total;
};

// The query, key and value projections as one GEMV over the rows [Wq; Wk; Wv]
// (the three matrices stay separate in memory): both flows are computed for
// every row (the weights are read once either way), the finalize stores both
// flows' queries and appends the primary's keys and values to the cache.
// Its plan always splits k, so that keys and values meet in the finalize.
GemvPlan plan_qkv(const dfa_gemv_desc& d) {
  GemvPlan pl;
  validate_gemv(&d, &pl);
  if (pl.k_split < 2) {
    dfa_gemv_desc d2 = d;
    d2.k_split = 2;
    validate_gemv(&d2, &pl);
  }
  return pl;
}

// Options of a layer step beyond the plain layer: pre-norm RMSNorm (norm
// weights and a buffer for the normalised rows of both flows) and rotary
// embeddings of the queries and keys.
struct LayerExtras {
  const float* norm_attn = nullptr;
  const float* norm_mlp = nullptr;
  float* norm_buf = nullptr;  // 2 * batch * hidden floats
  float eps = 0.f;
  int32_t rope = dfa::kRopeNone;
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  int32_t rope_max_pos = 0;
};

dfa_status qkv_impl(const dfa_layer_desc* d, const GemvPlan& pl, const dfa_layer_weights* w, const float* x1,
                    const float* x2, bool x_exact, const LayerExtras& ex, float* q1, float* q2,
                    const dfa_kv_target& kv, void* workspace, hipStream_t hs) {
  const int32_t qd = d->num_q_heads * d->head_dim, kd = d->num_kv_heads * d->head_dim;
  dfa::GemvParams p{};
  p.w = w->wq;
  p.w_seg1 = w->wk;
  p.w_seg2 = w->wv;
  p.seg1_row = qd;
  p.seg2_row = qd + kd;
  p.q_cols = qd;
  p.kv_cols = kd;
  p.x1 = x1;
  p.x2 = x2;
  p.y1 = q1;
  p.y2 = q2;
  p.part = static_cast<float*>(workspace);
  p.batch = d->batch;
  p.n = qd + 2 * kd;
  p.k = d->hidden;
  p.flows = 2;
  p.cbf = pl.cbf;
  p.m_pad = pl.m_pad;
  p.k_split = pl.k_split;
  p.k_range = pl.k_range;
  p.pair = 0;
  p.x_exact = x_exact;
  p.epilogue = dfa::kEpiQkv;
  p.rope = ex.rope;
  p.rope_cos = ex.rope_cos;
  p.rope_sin = ex.rope_sin;
  p.rope_max_pos = ex.rope_max_pos;
  p.rows_per_wg = pl.rows_per_wg;
  p.kv_k = static_cast<uint16_t*>(kv.k_cache);
  p.kv_v = static_cast<uint16_t*>(kv.v_cache);
  p.kv_table = kv.block_table;
  p.kv_ctx = kv.ctx_lens;
  p.kv_hkv = kv.num_kv_heads;
  p.kv_head_dim = kv.head_dim;
  p.kv_bs_log2 = log2i(kv.block_size);
  p.kv_max_blocks = kv.max_blocks_per_seq;
  p.kv_num_blocks = kv.num_blocks;
  // slices of at most pl.slice sequences, in order on the stream (they share the workspace)
  for (int32_t b0 = 0; b0 < d->batch; b0 += pl.slice) {
    dfa::GemvParams q = p;
    dfa_gemv_desc ds{std::min(pl.slice, d->batch - b0), p.n, p.k, 2, DFA_EPI_NONE, x_exact ? 1 : 0, 0, 0};
    const GemvPlan ps = plan_qkv(ds);
    q.batch = ds.batch;
    q.cbf = ps.cbf;
    q.m_pad = ps.m_pad;
    q.k_split = ps.k_split;
    q.k_range = ps.k_range;
    q.x1 = x1 + size_t(b0) * d->hidden;
    q.x2 = x2 + size_t(b0) * d->hidden;
    q.y1 = q1 + size_t(b0) * qd;
    q.y2 = q2 + size_t(b0) * qd;
    q.kv_table = kv.block_table + size_t(b0) * kv.max_blocks_per_seq;
    q.kv_ctx = kv.ctx_lens + b0;
    hipError_t e = dfa::launch_gemv(q, hs);
    if (e == hipSuccess) e = dfa::launch_gemv_finalize(q, hs);
    if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("qkv gemv launch: ") + hipGetErrorString(e));
  }
  return DFA_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

dfa_status plan_layer(const dfa_layer_desc* d, LayerPlan* lp) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  if (d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
    return fail(DFA_ERR_SHAPE, "num_q_heads must be a positive multiple of num_kv_heads");
  LayerPlan p{};
  p.attn = dfa_attn_desc{d->batch, d->num_q_heads, d->num_kv_heads, d->head_dim, d->block_size,
                         d->max_blocks_per_seq, d->num_blocks, d->max_ctx_len, 2, 0, d->scale, DFA_F32, DFA_BF16};
  const int32_t qd = d->num_q_heads * d->head_dim, kd = d->num_kv_heads * d->head_dim;
  p.qkv = dfa_gemv_desc{d->batch, qd + 2 * kd, d->hidden, 2, DFA_EPI_NONE, d->x_exact_bf16, 0, 0};
  p.o = dfa_gemv_desc{d->batch, d->hidden, qd, 2, DFA_EPI_RESIDUAL, 0, 0, 0};
  p.mlp_in = dfa_gemv_desc{d->batch, d->mlp, d->hidden, 2, DFA_EPI_SWIGLU, 0, 0, 0};
  p.mlp_out = dfa_gemv_desc{d->batch, d->hidden, d->mlp, 2, DFA_EPI_RESIDUAL_COUPLED, 0, 0, 0};
  int32_t split = 0;
  dfa_status st = validate_attn(&p.attn, &split);
  if (st != DFA_OK) return st;
  size_t gemv_ws = 0;
  for (const dfa_gemv_desc* g : {&p.qkv, &p.o, &p.mlp_in, &p.mlp_out}) {
    GemvPlan gp;
    st = validate_gemv(g, &gp);
    if (st != DFA_OK) return st;
    gemv_ws = std::max(gemv_ws, gemv_workspace(g, gp));
  }
  p.qkv_plan = plan_qkv(p.qkv);
  gemv_ws = std::max(gemv_ws, gemv_workspace(&p.qkv, p.qkv_plan));
  const size_t B = size_t(d->batch);
  p.off_q = 0;
  p.off_o = p.off_q + align256(2 * B * qd * sizeof(float));
  p.off_h = p.off_o + align256(2 * B * qd * sizeof(float));
  p.off_z = p.off_h + align256(2 * B * d->hidden * sizeof(float));
  p.off_attn = p.off_z + align256(2 * B * d->mlp * sizeof(float));
  p.off_gemv = p.off_attn + align256(workspace_bytes(&p.attn, split));
  p.total = p.off_gemv + align256(gemv_ws);
  if (lp) *lp = p;
  return DFA_OK;
}

}  // namespace

namespace dfa {
dfa_status report_error(dfa_status st, const std::string& msg) { return fail(st, msg); }

dfa_status attn_host_checks(const dfa_attn_desc* desc, const void* q1, const void* q2, const float* a,
                            const void* k_cache, const void* v_cache, const int32_t* block_table,
                            const int32_t* ctx_lens, const float* o1, const float* o2, int32_t* n_splits) {
  int32_t split = 0;
  const dfa_status st = check_attn_call(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, o1, o2, &split);
  if (st == DFA_OK && n_splits) *n_splits = num_splits(desc, split);
  return st;
}
}  // namespace dfa

extern "C" {

size_t dfa_dual_gemv_workspace_size(const dfa_gemv_desc* desc) {
  GemvPlan pl;
  if (validate_gemv(desc, &pl) != DFA_OK) return 0;
  return gemv_workspace(desc, pl);
}

dfa_status dfa_dual_gemv(const dfa_gemv_desc* d, const uint16_t* w, const uint16_t* w2, const float* x1,
                         const float* x2, const float* couple, const float* res1, const float* res2, float* y1,
                         float* y2, const dfa_kv_target* kv, void* workspace, size_t ws_bytes, void* stream) {
  try {
    return gemv_impl(d, w, w2, x1, x2, couple, res1, res2, y1, y2, kv, workspace, ws_bytes,
                     static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

size_t dfa_decode_layer_workspace_size(const dfa_layer_desc* desc) {
  LayerPlan lp;
  return plan_layer(desc, &lp) == DFA_OK ? lp.total : 0;
}

namespace {
// One layer step (the plan and arguments already validated), with the options of `ex`.
// x_exact: x1 and x2 hold exact bf16 values (the caller's inputs of a first layer only).
dfa_status layer_step(const dfa_layer_desc* d, const LayerPlan& lp, const dfa_layer_weights* w, const LayerExtras& ex,
                      bool x_exact, const float* x1, const float* x2, void* k_cache, void* v_cache,
                      const int32_t* block_table, const int32_t* ctx_lens, float* out1, float* out2, char* ws,
                      hipStream_t hs) {
  {
    dfa_status st;
    const size_t B = size_t(d->batch);
    const size_t qd = size_t(d->num_q_heads) * d->head_dim;
    float* q1 = reinterpret_cast<float*>(ws + lp.off_q);
    float* q2 = q1 + B * qd;
    float* o1 = reinterpret_cast<float*>(ws + lp.off_o);
    float* o2 = o1 + B * qd;
    float* h1 = reinterpret_cast<float*>(ws + lp.off_h);
    float* h2 = h1 + B * d->hidden;
    float* z1 = reinterpret_cast<float*>(ws + lp.off_z);
    float* z2 = z1 + B * d->mlp;
    void* aws = ws + lp.off_attn;
    void* gws = ws + lp.off_gemv;
    const size_t aws_bytes = lp.off_gemv - lp.off_attn, gws_bytes = lp.total - lp.off_gemv;
    // pre-norm of both flows (shared weights) into ex.norm_buf
    auto rmsnorm = [&](const float* a, const float* b, const float* wn, const float** n1, const float** n2) {
      dfa::NormParams np{a, b, wn, ex.norm_buf, ex.norm_buf + B * d->hidden, d->batch, d->hidden, ex.eps};
      const hipError_t e = dfa::launch_rmsnorm(np, hs);
      if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("rmsnorm launch: ") + hipGetErrorString(e));
      *n1 = np.y1;
      *n2 = np.y2;
      return DFA_OK;
    };
    const float* a1 = x1;
    const float* a2 = x2;
    if (ex.norm_attn && (st = rmsnorm(x1, x2, ex.norm_attn, &a1, &a2)) != DFA_OK) return st;
    // 1-2. both flows' queries (aux query from its own embedding input x2) and the primary's
    // keys and values (rotated when ex.rope is set), appended at position ctx_lens[b]; the
    // auxiliary flow writes no KV
    const dfa_kv_target kv{k_cache, v_cache, block_table, ctx_lens, d->num_kv_heads, d->head_dim, d->block_size,
                           d->max_blocks_per_seq, d->num_blocks};
    st = qkv_impl(d, lp.qkv_plan, w, a1, a2, x_exact && !ex.norm_attn, ex, q1, q2, kv, gws, hs);
    if (st != DFA_OK) return st;
    // 3. both flows attend the primary cache, now ctx_lens[b] + 1 positions; q2 coupled by a
    st = attn_impl(&lp.attn, q1, q2, w->a, k_cache, v_cache, block_table, ctx_lens, 1, aws, aws_bytes, o1, o2, hs,
                   nullptr);
    if (st != DFA_OK) return st;
    // 4. output projection + residual
    st = gemv_impl(&lp.o, w->wo, nullptr, o1, o2, nullptr, x1, x2, h1, h2, nullptr, gws, gws_bytes, hs);
    if (st != DFA_OK) return st;
    // 5. SwiGLU (on the pre-normed rows when ex.norm_mlp is set), MLP-intermediate coupling b
    const float* m1 = h1;
    const float* m2 = h2;
    if (ex.norm_mlp && (st = rmsnorm(h1, h2, ex.norm_mlp, &m1, &m2)) != DFA_OK) return st;
    st = gemv_impl(&lp.mlp_in, w->w_gate, w->w_up, m1, m2, w->b, nullptr, nullptr, z1, z2, nullptr, gws, gws_bytes,
                   hs);
    if (st != DFA_OK) return st;
    // 6. down projection, MLP-output coupling c, residual
    return gemv_impl(&lp.mlp_out, w->w_down, nullptr, z1, z2, w->c, h1, h2, out1, out2, nullptr, gws, gws_bytes, hs);
  }
}

dfa_status check_layer_weights(const dfa_layer_weights* w) {
  if (!w || !w->wq || !w->wk || !w->wv || !w->wo || !w->w_gate || !w->w_up || !w->w_down || !w->a)
    return fail(DFA_ERR_NULL, "every weight matrix and the coupling vector a are required");
  const void* ptrs[] = {w->wq, w->wk, w->wv, w->wo, w->w_gate, w->w_up, w->w_down, w->a, w->b, w->c};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(DFA_ERR_ALIGNMENT, "weights and couplings must be 16-byte aligned");
  return DFA_OK;
}
}  // namespace

dfa_status dfa_decode_layer(const dfa_layer_desc* d, const dfa_layer_weights* w, const float* x1, const float* x2,
                            void* k_cache, void* v_cache, const int32_t* block_table, const int32_t* ctx_lens,
                            float* out1, float* out2, void* workspace, size_t ws_bytes, void* stream) {
  try {
    LayerPlan lp;
    dfa_status st = plan_layer(d, &lp);
    if (st != DFA_OK) return st;
    if ((st = check_layer_weights(w)) != DFA_OK) return st;
    if (!x1 || !x2 || !out1 || !out2 || !k_cache || !v_cache || !block_table || !ctx_lens)
      return fail(DFA_ERR_NULL, "x1, x2, out1, out2, the caches, block_table and ctx_lens are required");
    if (!workspace) return fail(DFA_ERR_WORKSPACE, "workspace is required");
    if (!aligned16(workspace)) return fail(DFA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    if (ws_bytes < lp.total) return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_decode_layer_workspace_size()");
    return layer_step(d, lp, w, LayerExtras{}, d->x_exact_bf16 != 0, x1, x2, k_cache, v_cache, block_table,
                      ctx_lens, out1, out2, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

namespace {
struct StackPlan {
  LayerPlan lp;
  size_t off_norm, off_act, act_bytes, total;
};

dfa_status plan_stack(const dfa_stack_desc* d, StackPlan* sp) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  dfa_status st = plan_layer(&d->layer, &sp->lp);
  if (st != DFA_OK) return st;
  if (d->num_layers < 1 || d->num_layers > 4096) return fail(DFA_ERR_SHAPE, "num_layers must be in [1, 4096]");
  if (d->rope != DFA_ROPE_NONE && d->rope != DFA_ROPE_HALF && d->rope != DFA_ROPE_INTERLEAVED)
    return fail(DFA_ERR_SHAPE, "rope must be DFA_ROPE_NONE, DFA_ROPE_HALF or DFA_ROPE_INTERLEAVED");
  if (d->rope != DFA_ROPE_NONE && d->rope_max_pos < d->layer.max_ctx_len)
    return fail(DFA_ERR_SHAPE, "rope_max_pos must cover every position (>= max_ctx_len)");
  if (d->rms_norm != 0 && d->rms_norm != 1) return fail(DFA_ERR_SHAPE, "rms_norm must be 0 or 1");
  if (d->rms_norm && (!(d->rms_eps >= 0.f) || !std::isfinite(d->rms_eps)))
    return fail(DFA_ERR_SHAPE, "rms_eps must be finite and >= 0");
  const size_t act = align256(2 * size_t(d->layer.batch) * d->layer.hidden * sizeof(float));
  sp->off_norm = sp->lp.total;
  sp->off_act = sp->off_norm + act;
  sp->act_bytes = act;
  sp->total = sp->off_act + 2 * act;
  return DFA_OK;
}
}  // namespace

size_t dfa_decode_stack_workspace_size(const dfa_stack_desc* desc) {
  StackPlan sp;
  return plan_stack(desc, &sp) == DFA_OK ? sp.total : 0;
}

dfa_status dfa_decode_stack(const dfa_stack_desc* d, const dfa_stack_layer* layers, const float* rope_cos,
                            const float* rope_sin, const float* x1, const float* x2, const int32_t* block_table,
                            const int32_t* ctx_lens, float* out1, float* out2, void* workspace, size_t ws_bytes,
                            void* stream) {
  try {
    StackPlan sp;
    dfa_status st = plan_stack(d, &sp);
    if (st != DFA_OK) return st;
    if (!layers) return fail(DFA_ERR_NULL, "layers is NULL");
    if (!x1 || !x2 || !out1 || !out2 || !block_table || !ctx_lens)
      return fail(DFA_ERR_NULL, "x1, x2, out1, out2, block_table and ctx_lens are required");
    if (d->rope != DFA_ROPE_NONE && (!rope_cos || !rope_sin)) return fail(DFA_ERR_NULL, "rotary tables are required");
    for (int32_t l = 0; l < d->num_layers; ++l) {
      if ((st = check_layer_weights(&layers[l].w)) != DFA_OK) return st;
      if (!layers[l].k_cache || !layers[l].v_cache) return fail(DFA_ERR_NULL, "every layer needs its caches");
      if (d->rms_norm && (!layers[l].norm_attn || !layers[l].norm_mlp))
        return fail(DFA_ERR_NULL, "every layer needs its norm weights");
      if (d->rms_norm && (!aligned16(layers[l].norm_attn) || !aligned16(layers[l].norm_mlp)))
        return fail(DFA_ERR_ALIGNMENT, "norm weights must be 16-byte aligned");
    }
    if (!workspace || ws_bytes < sp.total) return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_decode_stack_workspace_size()");
    if (!aligned16(workspace)) return fail(DFA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    char* ws = static_cast<char*>(workspace);
    const size_t bh = size_t(d->layer.batch) * d->layer.hidden;
    float* act[2] = {reinterpret_cast<float*>(ws + sp.off_act), reinterpret_cast<float*>(ws + sp.off_act + sp.act_bytes)};
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    for (int32_t l = 0; l < d->num_layers; ++l) {
      LayerExtras ex;
      if (d->rms_norm) {
        ex.norm_attn = layers[l].norm_attn;
        ex.norm_mlp = layers[l].norm_mlp;
        ex.norm_buf = reinterpret_cast<float*>(ws + sp.off_norm);
        ex.eps = d->rms_eps;
      }
      ex.rope = d->rope;
      ex.rope_cos = rope_cos;
      ex.rope_sin = rope_sin;
      ex.rope_max_pos = d->rope_max_pos;
      const float* in1 = l == 0 ? x1 : act[(l - 1) & 1];
      const float* in2 = l == 0 ? x2 : act[(l - 1) & 1] + bh;
      float* o1 = l == d->num_layers - 1 ? out1 : act[l & 1];
      float* o2 = l == d->num_layers - 1 ? out2 : act[l & 1] + bh;
      // only the caller's inputs can be exact bf16; later layers read float32 outputs
      st = layer_step(&d->layer, sp.lp, &layers[l].w, ex, l == 0 && d->layer.x_exact_bf16 != 0, in1, in2,
                      layers[l].k_cache, layers[l].v_cache, block_table, ctx_lens, o1, o2, ws, hs);
      if (st != DFA_OK) return st;
    }
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

static dfa_status validate_mixture(const dfa_mixture_desc* d) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  if (d->batch < 1 || d->batch > 65535) return fail(DFA_ERR_SHAPE, "batch must be in [1, 65535]");
  if (d->vocab < 4 || d->vocab % 4 != 0 || d->vocab > dfa::kMixChunk * dfa::kMixMaxChunks)
    return fail(DFA_ERR_SHAPE, "vocab must be a positive multiple of 4, at most 2^20");
  return DFA_OK;
}

size_t dfa_mixture_workspace_size(const dfa_mixture_desc* d) {
  if (validate_mixture(d) != DFA_OK) return 0;
  // per (sequence, chunk): softmax statistics (kMixRec floats), then mass and maximum (4 words)
  return size_t(d->batch) * dfa::mixture_chunks(d->vocab) * (dfa::kMixRec * sizeof(float) + 4 * sizeof(uint32_t));
}

dfa_status dfa_mixture_sample(const dfa_mixture_desc* d, const float* logits1, const float* logits2,
                              const float* u, int32_t* token, int32_t* greedy, float* alpha, float* p_mix,
                              void* workspace, size_t ws_bytes, void* stream) {
  try {
    dfa_status st = validate_mixture(d);
    if (st != DFA_OK) return st;
    if (!logits1 || !logits2 || !u || !token || !greedy || !alpha)
      return fail(DFA_ERR_NULL, "logits1, logits2, u, token, greedy and alpha are required");
    if (!aligned16(logits1) || !aligned16(logits2) || (p_mix && !aligned16(p_mix)))
      return fail(DFA_ERR_ALIGNMENT, "logits and p_mix must be 16-byte aligned");
    const size_t need = dfa_mixture_workspace_size(d);
    if (!workspace || ws_bytes < need) return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_mixture_workspace_size()");
    if (!aligned16(workspace)) return fail(DFA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    dfa::MixParams p{};
    p.logits1 = logits1;
    p.logits2 = logits2;
    p.u = u;
    p.token = token;
    p.greedy = greedy;
    p.alpha = alpha;
    p.p_mix = p_mix;
    p.batch = d->batch;
    p.vocab = d->vocab;
    p.chunks = int32_t(dfa::mixture_chunks(d->vocab));
    p.rec = static_cast<float*>(workspace);
    p.crec = reinterpret_cast<uint32_t*>(p.rec + size_t(p.batch) * p.chunks * dfa::kMixRec);
    const hipError_t e = dfa::launch_mixture(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("mixture launch: ") + hipGetErrorString(e));
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

// ------------------------------------------------------------------ output head
// One call: both flows' logits (the dual GEMV over the vocabulary matrix), then the mixture
// kernels of dfa_mixture_sample on them, sharing one workspace.
struct HeadPlan {
  dfa_gemv_desc gemv;
  GemvPlan gp;
  int32_t chunks;
  size_t gemv_off, rec_off, crec_off, total;
};

static dfa_status plan_head(const dfa_head_desc* d, HeadPlan* hp) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  if (d->batch < 1 || d->batch > 65535) return fail(DFA_ERR_SHAPE, "batch must be in [1, 65535]");
  if (d->vocab < 64 || d->vocab % 64 != 0 || d->vocab > (1 << 20))
    return fail(DFA_ERR_SHAPE, "vocab must be a multiple of 64 in [64, 2^20]");
  if (d->hidden < 128 || d->hidden % 128 != 0) return fail(DFA_ERR_SHAPE, "hidden must be a positive multiple of 128");
  HeadPlan h{};
  h.gemv = dfa_gemv_desc{d->batch, d->vocab, d->hidden, 2, DFA_EPI_NONE, d->x_exact_bf16 ? 1 : 0, 0, 0};
  const dfa_status st = validate_gemv(&h.gemv, &h.gp);
  if (st != DFA_OK) return st;
  h.chunks = int32_t(dfa::mixture_chunks(d->vocab));
  const size_t B = size_t(d->batch);
  h.gemv_off = 0;
  h.rec_off = align256(gemv_workspace(&h.gemv, h.gp));
  h.crec_off = h.rec_off + align256(B * h.chunks * dfa::kMixRec * sizeof(float));
  h.total = h.crec_off + align256(B * h.chunks * 4 * sizeof(uint32_t));
  if (hp) *hp = h;
  return DFA_OK;
}

size_t dfa_output_head_workspace_size(const dfa_head_desc* d) {
  HeadPlan h;
  return plan_head(d, &h) == DFA_OK ? h.total : 0;
}

dfa_status dfa_output_head(const dfa_head_desc* d, const uint16_t* w_vocab, const float* h1, const float* h2,
                           const float* u, float* logits1, float* logits2, int32_t* token, int32_t* greedy,
                           float* alpha, float* p_mix, void* workspace, size_t ws_bytes, void* stream) {
  try {
    HeadPlan h;
    dfa_status st = plan_head(d, &h);
    if (st != DFA_OK) return st;
    if (!w_vocab || !h1 || !h2 || !u || !logits1 || !logits2 || !token || !greedy || !alpha)
      return fail(DFA_ERR_NULL, "w_vocab, h1, h2, u, logits1, logits2, token, greedy and alpha are required");
    const void* ptrs[] = {w_vocab, h1, h2, logits1, logits2, p_mix, workspace};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    if (!workspace || ws_bytes < h.total)
      return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_output_head_workspace_size()");
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    st = gemv_impl(&h.gemv, w_vocab, nullptr, h1, h2, nullptr, nullptr, nullptr, logits1, logits2, nullptr,
                   ws + h.gemv_off, h.rec_off - h.gemv_off, hs);
    if (st != DFA_OK) return st;
    dfa::MixParams p{};
    p.logits1 = logits1;
    p.logits2 = logits2;
    p.u = u;
    p.token = token;
    p.greedy = greedy;
    p.alpha = alpha;
    p.p_mix = p_mix;
    p.batch = d->batch;
    p.vocab = d->vocab;
    p.chunks = h.chunks;
    p.rec = reinterpret_cast<float*>(ws + h.rec_off);
    p.crec = reinterpret_cast<uint32_t*>(ws + h.crec_off);
    const hipError_t e = dfa::launch_mixture(p, hs);
    if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("output head mixture launch: ") + hipGetErrorString(e));
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

static dfa_status validate_moe(const dfa_moe_desc* d) {
  if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
  if (d->batch < 1 || d->batch > 65535) return fail(DFA_ERR_SHAPE, "batch must be in [1, 65535]");
  if (d->hidden < 128 || d->hidden % 128 != 0 || d->mlp < 128 || d->mlp % 128 != 0)
    return fail(DFA_ERR_SHAPE, "hidden and mlp must be positive multiples of 128");
  if (d->num_experts < 1 || d->num_experts > dfa::kMoeMaxExperts)
    return fail(DFA_ERR_SHAPE, "num_experts must be in [1, 1024]");
  if (d->k1 < 1 || d->k1 > d->k2 || d->k2 > d->num_experts || d->k2 > dfa::kMoeMaxK)
    return fail(DFA_ERR_SHAPE, "fan-outs must satisfy 1 <= k1 <= k2 <= min(num_experts, 32)");
  return DFA_OK;
}

// Sequences per pass of the expert GEMVs (their activation blocks hold 64 rows of both flows); a
// larger batch runs in slices, each reading its selected experts again.
constexpr int kMoeSlice = 32;

// Weight rows per workgroup of the grouped expert GEMVs.
constexpr int kMoeRowsUp = 128;
constexpr int kMoeRowsDown = 128;

// Routing buffer: int32 sel [batch][k2], then float g1 [batch][k1], then float g2 [batch][k2],
// each section starting on a 16-byte boundary.
struct MoeRouting {
  size_t g1_off, g2_off, bytes;
};
static MoeRouting moe_routing_layout(const dfa_moe_desc* d) {
  auto up16 = [](size_t x) { return (x + 15) & ~size_t(15); };
  MoeRouting r;
  r.g1_off = up16(size_t(d->batch) * d->k2 * sizeof(int32_t));
  r.g2_off = r.g1_off + up16(size_t(d->batch) * d->k1 * sizeof(float));
  r.bytes = r.g2_off + up16(size_t(d->batch) * d->k2 * sizeof(float));
  return r;
}

size_t dfa_moe_routing_size(const dfa_moe_desc* d) {
  if (validate_moe(d) != DFA_OK) return 0;
  return moe_routing_layout(d).bytes;
}

size_t dfa_moe_workspace_size(const dfa_moe_desc* d) {
  if (validate_moe(d) != DFA_OK) return 0;
  // both flows' expert intermediates [slice][k2][2][mlp], then expert outputs [slice][k2][2][hidden],
  // slice = min(batch, kMoeSlice) sequences (the slices of a larger batch reuse them in turn)
  return size_t(std::min(d->batch, kMoeSlice)) * d->k2 * 2 * (size_t(d->mlp) + d->hidden) * sizeof(float);
}

dfa_status dfa_moe_route(const dfa_moe_desc* d, const float* r1, const float* r2, void* routing,
                         size_t routing_bytes, void* stream) {
  try {
    dfa_status st = validate_moe(d);
    if (st != DFA_OK) return st;
    if (!r1 || !r2 || !routing) return fail(DFA_ERR_NULL, "r1, r2 and routing are required");
    if (!aligned16(r1) || !aligned16(r2) || !aligned16(routing))
      return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const MoeRouting lay = moe_routing_layout(d);
    if (routing_bytes < lay.bytes) return fail(DFA_ERR_WORKSPACE, "routing smaller than dfa_moe_routing_size()");
    char* base = static_cast<char*>(routing);
    dfa::MoeRouteParams p{};
    p.r1 = r1;
    p.r2 = r2;
    p.sel = reinterpret_cast<int32_t*>(base);
    p.g1 = reinterpret_cast<float*>(base + lay.g1_off);
    p.g2 = reinterpret_cast<float*>(base + lay.g2_off);
    p.batch = d->batch;
    p.experts = d->num_experts;
    p.k1 = d->k1;
    p.k2 = d->k2;
    const hipError_t e = dfa::launch_moe_route(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("moe route launch: ") + hipGetErrorString(e));
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

dfa_status dfa_moe_ffn(const dfa_moe_desc* d, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                       const float* b, const float* c, const float* h1, const float* h2, const float* res1,
                       const float* res2, const void* routing, float* out1, float* out2, void* workspace,
                       size_t workspace_bytes, void* stream) {
  try {
    dfa_status st = validate_moe(d);
    if (st != DFA_OK) return st;
    if (!w_gate || !w_up || !w_down || !h1 || !h2 || !routing || !out1 || !out2)
      return fail(DFA_ERR_NULL, "weights, h1, h2, routing, out1 and out2 are required");
    const void* ptrs[] = {w_gate, w_up, w_down, b, c, h1, h2, res1, res2, routing, out1, out2, workspace};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t need = dfa_moe_workspace_size(d);
    if (!workspace || workspace_bytes < need) return fail(DFA_ERR_WORKSPACE, "workspace smaller than dfa_moe_workspace_size()");
    const MoeRouting lay = moe_routing_layout(d);
    const char* rb = static_cast<const char*>(routing);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // slices of at most kMoeSlice sequences, in order on the stream (they share the workspace)
    for (int32_t b0 = 0; b0 < d->batch; b0 += kMoeSlice) {
      const int32_t nb = std::min(kMoeSlice, d->batch - b0);
      const int32_t* sel = reinterpret_cast<const int32_t*>(rb) + size_t(b0) * d->k2;
      float* z = static_cast<float*>(workspace);
      float* y = z + size_t(nb) * d->k2 * 2 * d->mlp;
      const size_t xo = size_t(b0) * d->hidden;  // row offset of the slice in [batch, hidden] tensors

      // gate and up projections of every selected expert, SwiGLU and b in the epilogue
      dfa::GemvParams g{};
      g.batch = nb;
      g.flows = 2;
      g.cbf = (nb + 15) / 16;
      g.m_pad = 2 * g.cbf * 16;
      g.k_split = 1;
      g.moe_sel = sel;
      g.moe_k1 = d->k1;
      g.moe_k2 = d->k2;
      g.moe_experts = d->num_experts;
      dfa::GemvParams up = g;
      up.w = w_gate;
      up.w2 = w_up;
      up.x1 = h1 + xo;
      up.x2 = h2 + xo;
      up.couple = b;
      up.y1 = up.y2 = z;
      up.n = d->mlp;
      up.k = d->hidden;
      up.k_range = d->hidden;
      up.pair = 1;
      up.x_exact = d->x_exact_bf16 != 0;
      up.epilogue = dfa::kEpiSwiglu;
      up.w_seg1 = up.w_seg2 = w_gate;
      up.seg1_row = up.seg2_row = d->mlp;
      up.moe_wstride = int64_t(d->mlp) * d->hidden;
      up.rows_per_wg = d->mlp % kMoeRowsUp == 0 ? kMoeRowsUp : 64;
      up.moe_rgs = d->mlp / up.rows_per_wg;
      up.moe_row_s = 1;
      hipError_t e = dfa::launch_gemv(up, hs);
      if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("moe gate/up launch: ") + hipGetErrorString(e));
      // down projection of every selected expert, from the intermediates [batch][k2][2][mlp]
      // (the two halves of each expert's matrix as the two matrices of one
      // workgroup where they tile evenly: twice the weight bytes per stage)
      dfa::GemvParams dn = g;
      const bool halves = (d->hidden / 2) % kMoeRowsDown == 0;
      dn.w = w_down;
      dn.x1 = dn.x2 = z;
      dn.y1 = dn.y2 = y;
      dn.n = halves ? d->hidden / 2 : d->hidden;
      dn.k = d->mlp;
      dn.k_range = d->mlp;
      dn.pair = halves ? 1 : 0;
      dn.w2 = halves ? w_down + size_t(dn.n) * d->mlp : nullptr;  // packed by 16-row tiles: rows [n, 2n)
      dn.x_exact = 0;
      dn.epilogue = halves ? dfa::kEpiSplitPair : dfa::kEpiNone;
      dn.w_seg1 = dn.w_seg2 = w_down;
      dn.seg1_row = dn.seg2_row = dn.n;
      dn.moe_wstride = int64_t(d->hidden) * d->mlp;
      dn.rows_per_wg = dn.n % kMoeRowsDown == 0 ? kMoeRowsDown : 64;
      dn.moe_rgs = dn.n / dn.rows_per_wg;
      dn.moe_row_s = 2 * d->k2;
      dn.moe_row_slot = 2;
      dn.moe_row_f = 1;
      e = dfa::launch_gemv(dn, hs);
      if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("moe down launch: ") + hipGetErrorString(e));
      dfa::MoeCombineParams cp{};
      cp.y = y;
      cp.g1 = reinterpret_cast<const float*>(rb + lay.g1_off) + size_t(b0) * d->k1;
      cp.g2 = reinterpret_cast<const float*>(rb + lay.g2_off) + size_t(b0) * d->k2;
      cp.res1 = res1 ? res1 + xo : nullptr;
      cp.res2 = res2 ? res2 + xo : nullptr;
      cp.c = c;
      cp.out1 = out1 + xo;
      cp.out2 = out2 + xo;
      cp.batch = nb;
      cp.hidden = d->hidden;
      cp.k1 = d->k1;
      cp.k2 = d->k2;
      e = dfa::launch_moe_combine(cp, hs);
      if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("moe combine launch: ") + hipGetErrorString(e));
    }
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

dfa_status dfa_prefill(const dfa_prefill_desc* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* prompt_lens, void* k_cache, void* v_cache, const int32_t* block_table,
                       float* o, void* stream) {
  try {
    if (!d) return fail(DFA_ERR_NULL, "desc is NULL");
    if (d->batch < 1 || d->batch > 65535) return fail(DFA_ERR_SHAPE, "batch must be in [1, 65535]");
    if (d->num_kv_heads < 1 || d->num_q_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
      return fail(DFA_ERR_SHAPE, "num_q_heads must be a positive multiple of num_kv_heads");
    const int group = d->num_q_heads / d->num_kv_heads;
    if (!is_pow2(group) || group > 16)
      return fail(DFA_ERR_UNSUPPORTED, "query heads per kv head must be 1, 2, 4, 8 or 16");
    if (d->num_kv_heads > 65535) return fail(DFA_ERR_SHAPE, "num_kv_heads must be at most 65535");
    if (d->head_dim != 64 && d->head_dim != 128) return fail(DFA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (!is_pow2(d->block_size) || d->block_size < 16 || d->max_blocks_per_seq < 1 || d->num_blocks < 1)
      return fail(DFA_ERR_SHAPE, "block_size a power of two >= 16; positive table sizes");
    if (d->max_prompt_len < 1 || int64_t(d->max_prompt_len) > int64_t(d->max_blocks_per_seq) * d->block_size)
      return fail(DFA_ERR_SHAPE, "max_prompt_len must be in [1, max_blocks_per_seq * block_size]");
    if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(DFA_ERR_SHAPE, "scale must be positive and finite");
    if ((d->max_prompt_len + d->block_size - 1) / d->block_size > dfa::kPrefillMaxBlocks)
      return fail(DFA_ERR_UNSUPPORTED, "a prompt may span at most 2048 cache blocks");
    if (!q || !k || !v || !prompt_lens || !k_cache || !v_cache || !block_table || !o)
      return fail(DFA_ERR_NULL, "every pointer is required");
    const void* ptrs[] = {q, k, v, prompt_lens, k_cache, v_cache, block_table, o};
    for (const void* x : ptrs)
      if (!aligned16(x)) return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    dfa::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.lens = prompt_lens;
    p.table = block_table;
    p.k_cache = static_cast<uint16_t*>(k_cache);
    p.v_cache = static_cast<uint16_t*>(v_cache);
    p.o = o;
    p.batch = d->batch;
    p.hq = d->num_q_heads;
    p.hkv = d->num_kv_heads;
    p.lmax = d->max_prompt_len;
    p.lmax_tiles = (d->max_prompt_len + 15) / 16;
    p.g_log2 = log2i(group);
    p.bs_log2 = log2i(d->block_size);
    p.max_blocks = d->max_blocks_per_seq;
    p.num_blocks = d->num_blocks;
    p.blk_stride = int64_t(d->num_kv_heads) * d->block_size * d->head_dim;
    p.qscale = d->scale * 1.4426950408889634f;
    const hipError_t e = dfa::launch_prefill(p, d->head_dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("prefill launch: ") + hipGetErrorString(e));
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

dfa_status dfa_pack_weight(const uint16_t* w, uint16_t* w_tiled, int32_t n, int32_t k, void* stream) {
  if (!w || !w_tiled) return fail(DFA_ERR_NULL, "w and w_tiled are required");
  if (n < 16 || n % 16 != 0 || k < 8 || k % 8 != 0) return fail(DFA_ERR_SHAPE, "n must be a multiple of 16, k of 8");
  if (!aligned16(w) || !aligned16(w_tiled)) return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(w), b0 = reinterpret_cast<uintptr_t>(w_tiled);
  const uintptr_t bytes = uintptr_t(n) * uintptr_t(k) * 2;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(DFA_ERR_SHAPE, "w and w_tiled overlap");
  const hipError_t e = dfa::launch_pack_weight(w, w_tiled, n, k, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("pack launch: ") + hipGetErrorString(e));
  return DFA_OK;
}


int32_t dfa_decode_attn_split_len(const dfa_attn_desc* desc) {
  int32_t split = 0;
  const dfa_status st = validate_attn(desc, &split);
  return st == DFA_OK ? split : -int32_t(st);
}

int32_t dfa_decode_attn_num_splits(const dfa_attn_desc* desc) {
  int32_t split = 0;
  const dfa_status st = validate_attn(desc, &split);
  return st == DFA_OK ? num_splits(desc, split) : -int32_t(st);
}

size_t dfa_decode_attn_workspace_size(const dfa_attn_desc* desc) {
  int32_t split = 0;
  if (validate_attn(desc, &split) != DFA_OK) return 0;
  return workspace_bytes(desc, split);
}

dfa_status dfa_decode_attn_timed(const dfa_attn_desc* desc, const void* q1, const void* q2, const float* a,
                                 const void* k_cache, const void* v_cache, const int32_t* block_table,
                                 const int32_t* ctx_lens, void* workspace, size_t ws_bytes, float* o1,
                                 float* o2, void* stream, const dfa_kernel_events* events) {
  try {
    return attn_impl(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, 0, workspace, ws_bytes, o1, o2,
                     static_cast<hipStream_t>(stream), events);
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

dfa_status dfa_decode_attn(const dfa_attn_desc* desc, const void* q1, const void* q2, const float* a,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* ctx_lens, void* workspace, size_t ws_bytes, float* o1,
                           float* o2, void* stream) {
  return dfa_decode_attn_timed(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, workspace, ws_bytes,
                               o1, o2, stream, nullptr);
}

dfa_status dfa_decode_attn_partials(const dfa_attn_desc* desc, const void* q1, const void* q2,
                                    const float* a, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens, void* workspace,
                                    size_t ws_bytes, void* stream) {
  try {
    int32_t split = 0;
    dfa_status st = validate_attn(desc, &split);
    if (st != DFA_OK) return st;
    st = check_tensors(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens);
    if (st != DFA_OK) return st;
    st = check_workspace(desc, split, workspace, ws_bytes);
    if (st != DFA_OK) return st;
    dfa::AttnParams p = make_params(desc, split, q1, q2, a, k_cache, v_cache, block_table, ctx_lens);
    p.part = static_cast<float*>(workspace);
    return launch_split_stage(desc, p, static_cast<hipStream_t>(stream), nullptr);
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

dfa_status dfa_combine(const dfa_attn_desc* desc, const void* workspace, size_t ws_bytes, float* o1, float* o2,
                       void* stream) {
  try {
    int32_t split = 0;
    dfa_status st = validate_attn(desc, &split);
    if (st != DFA_OK) return st;
    if (!o1 || (desc->num_flows == 2 && !o2))
      return fail(DFA_ERR_NULL, "o1 (and o2 with two flows) are required");
    if (!aligned16(o1) || (desc->num_flows == 2 && !aligned16(o2)))
      return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    st = check_workspace(desc, split, workspace, ws_bytes);
    if (st != DFA_OK) return st;
    return launch_combine_stage(desc, split, workspace, o1, o2, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

const char* dfa_status_string(dfa_status s) {
  switch (s) {
    case DFA_OK: return "ok";
    case DFA_ERR_NULL: return "required pointer is NULL";
    case DFA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case DFA_ERR_DTYPE: return "unsupported element type";
    case DFA_ERR_WORKSPACE: return "workspace missing or too small";
    case DFA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DFA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case DFA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

dfa_status dfa_check_kv_table(const dfa_attn_desc* desc, const int32_t* block_table, const int32_t* ctx_lens,
                              int32_t ctx_add, uint32_t* flags, void* stream) {
  try {
    int32_t split = 0;
    const dfa_status st = validate_attn(desc, &split);
    if (st != DFA_OK) return st;
    if (!block_table || !ctx_lens || !flags) return fail(DFA_ERR_NULL, "block_table, ctx_lens and flags are required");
    if (!aligned16(block_table) || !aligned16(ctx_lens) || !aligned16(flags))
      return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    if (ctx_add < 0 || ctx_add > 1) return fail(DFA_ERR_SHAPE, "ctx_add must be 0 or 1");
    dfa::TableCheckParams p{block_table, ctx_lens, flags, desc->batch, desc->max_blocks_per_seq, desc->num_blocks,
                            desc->max_ctx_len, desc->block_size, ctx_add};
    const hipError_t e = dfa::launch_check_table(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("table check launch: ") + hipGetErrorString(e));
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_HIP, "unexpected host exception");
  }
}

const char* dfa_last_error(void) { return g_last_error.c_str(); }

int32_t dfa_version(void) { return 100; }

size_t dfa_stream_read_sink_bytes(void) { return dfa::stream_read_threads() * sizeof(uint32_t); }

dfa_status dfa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(DFA_ERR_NULL, "buf and sink are required");
  if (bytes % 16 != 0 || bytes == 0) return fail(DFA_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned16(buf) || !aligned16(sink)) return fail(DFA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  const hipError_t e = dfa::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("stream read launch: ") + hipGetErrorString(e));
  return DFA_OK;
}

}  // extern "C"
