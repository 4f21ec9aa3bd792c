// extern "C" entry points of libdfa: argument validation, split planning and
// kernel dispatch. Validation is plain host code and runs before any HIP call;
// an invalid call returns a status and enqueues nothing.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/dfa.h"
#include "dfa_internal.h"

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

// Positions per split chosen by the library (measured on MI355X, 256 CUs): a
// single split per sequence when there are at least 128 (sequence, kv head)
// pairs -- one workgroup per pair then streams at full rate, and the combine
// launch would cost more than the extra parallelism gains; otherwise splits of
// at least 2048 positions, enough of them for about 512 workgroups.
int64_t auto_split_len(const dfa_attn_desc* d) {
  const int64_t pairs = int64_t(d->batch) * d->num_kv_heads;
  if (pairs >= 128) return (int64_t(d->max_ctx_len) + 31) / 32 * 32;
  const int64_t want = (512 + pairs - 1) / pairs;
  int64_t len = (int64_t(d->max_ctx_len) + want - 1) / want;
  len = (len + 127) / 128 * 128;
  return std::max<int64_t>(len, 2048);
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
  if (group * d->num_flows > dfa::kMaxRows)
    return fail(DFA_ERR_UNSUPPORTED, "(num_q_heads / num_kv_heads) * num_flows must be <= 16");
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
    e = dfa::launch_attn_bf16(p, d->head_dim, rows <= 8 ? 8 : 16, st, ev);
  }
  if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return DFA_OK;
}

dfa_status launch_combine_stage(const dfa_attn_desc* d, int32_t split, const int32_t* ctx,
                                const void* ws, float* o1, float* o2, hipStream_t st) {
  dfa::CombineParams c{};
  c.part = static_cast<const float*>(ws);
  c.ctx = ctx;
  c.o1 = o1;
  c.o2 = d->num_flows == 2 ? o2 : nullptr;
  c.batch = d->batch;
  c.hq = d->num_q_heads;
  c.flows = d->num_flows;
  c.split_len = split;
  c.n_splits = num_splits(d, split);
  c.max_ctx = d->max_ctx_len;
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

}  // namespace

extern "C" {

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
    int32_t split = 0;
    dfa_status st = validate_attn(desc, &split);
    if (st != DFA_OK) return st;
    st = check_tensors(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens);
    if (st != DFA_OK) return st;
    if (!o1 || (desc->num_flows == 2 && !o2)) return fail(DFA_ERR_NULL, "o1 (and o2 with two flows) are required");
    if (!aligned16(o1) || (desc->num_flows == 2 && !aligned16(o2)))
      return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const int32_t ns = num_splits(desc, split);
    if (ns > 1) {
      st = check_workspace(desc, split, workspace, ws_bytes);
      if (st != DFA_OK) return st;
    }
    dfa::AttnParams p = make_params(desc, split, q1, q2, a, k_cache, v_cache, block_table, ctx_lens);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (ns == 1) {
      p.direct = 1;
      p.o1 = o1;
      p.o2 = desc->num_flows == 2 ? o2 : nullptr;
      return launch_split_stage(desc, p, hs, events);
    }
    p.part = static_cast<float*>(workspace);
    st = launch_split_stage(desc, p, hs, events);
    if (st != DFA_OK) return st;
    return launch_combine_stage(desc, split, ctx_lens, workspace, o1, o2, hs);
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

dfa_status dfa_combine(const dfa_attn_desc* desc, const int32_t* ctx_lens, const void* workspace,
                       size_t ws_bytes, float* o1, float* o2, void* stream) {
  try {
    int32_t split = 0;
    dfa_status st = validate_attn(desc, &split);
    if (st != DFA_OK) return st;
    if (!ctx_lens || !o1 || (desc->num_flows == 2 && !o2))
      return fail(DFA_ERR_NULL, "ctx_lens, o1 (and o2 with two flows) are required");
    if (!aligned16(ctx_lens) || !aligned16(o1) || (desc->num_flows == 2 && !aligned16(o2)))
      return fail(DFA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    st = check_workspace(desc, split, workspace, ws_bytes);
    if (st != DFA_OK) return st;
    return launch_combine_stage(desc, split, ctx_lens, workspace, o1, o2, static_cast<hipStream_t>(stream));
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
