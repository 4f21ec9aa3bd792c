// Internal interface between the host-side ABI (abi.cpp) and the attention
// and measurement launchers. Plain structs passed by value to the kernels.
// The weight-streaming and output-head kernels have theirs in ops_internal.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>

#include "../../include/dfa.h"

namespace dfa {

constexpr int kWaves = 4;          // waves per attention workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 16;       // query rows (heads x flows) per float32-cache workgroup and per row set
constexpr int kMaxRowsBf16 = 32;   // query rows per bf16-cache workgroup (two row sets)
constexpr int kRecPad = 4;         // partial record = head_dim + kRecPad floats
constexpr int kMaxTableSlice = 1024;  // block-table entries staged per split

struct AttnParams {
  const void* q1;
  const void* q2;
  const float* a;
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* ctx;
  float* part;  // split records (split mode)
  float* o1;    // outputs (direct mode)
  float* o2;
  int32_t batch, hq, hkv, group, flows;
  int32_t bs_log2, max_blocks, num_blocks, max_ctx;
  int32_t split_len, n_splits;
  int64_t blk_stride;  // elements per physical block: hkv * block_size * head_dim
  float qscale;        // scale * log2(e): scores come out in base-2 units
  int32_t ctx_add;     // added to every ctx_lens entry (1 when attending a just-appended position)
  int32_t direct;      // 1: one split per sequence; normalise and write o1/o2
  int32_t q_f32;       // Q element type is float32 (else bf16)
  int32_t longest_first;  // 1: workgroup z takes sequences in descending length order
};

struct CombineParams {
  const float* part;
  float* o1;
  float* o2;
  int32_t batch, hq, flows, n_splits;
};

// Optional events recorded by the runtime at the start and end of a kernel's
// own dispatch (no extra commands on the stream).
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Sets the calling thread's error message (dfa_last_error) and returns st.
dfa_status report_error(dfa_status st, const std::string& msg);

// The host-side checks of dfa_decode_attn short of the workspace (descriptor,
// pointers, alignment); on success *n_splits is the split count of its plan.
dfa_status attn_host_checks(const dfa_attn_desc* desc, const void* q1, const void* q2, const float* a,
                            const void* k_cache, const void* v_cache, const int32_t* block_table,
                            const int32_t* ctx_lens, const float* o1, const float* o2, int32_t* n_splits);

// Launchers return the launch status (hipGetLastError after the launch).
hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int rows_padded, hipStream_t s, const KernelEvents& ev);
hipError_t launch_attn_f32(const AttnParams& p, int head_dim, hipStream_t s, const KernelEvents& ev);
hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
size_t stream_read_threads();

}  // namespace dfa
