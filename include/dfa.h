/*
 * dfa.h -- C ABI of libdfa: the decode step of a Dual-Flow Transformer on
 * AMD Instinct MI355X (gfx950).
 *
 * A Dual-Flow layer runs two residual flows over shared weights and one
 * persistent key/value cache. The primary flow writes the cache; the
 * auxiliary flow couples its query to the primary query through a learned
 * vector a, attends the primary keys and values, and never writes the cache.
 * Sources: "Resumo Técnico: Dual-Flow Transformers" (gist.science, pt),
 * sections "Arquitetura Central" (flows, shared matrices, the cache is written
 * by the primary flow only), "Mecanismos Chave" (asymmetric shared-KV
 * attention; coupling vectors a, b, c at the query, MLP-intermediate and
 * MLP-output levels, primary to auxiliary only) and "Custos de Inferência vs.
 * Treinamento" (decode does about twice the arithmetic while reading the same
 * cache and the same unique weights).
 *
 * The pages give the coupling vectors but not their formulas; this library
 * computes q2' = q2 + a * q1, z2' = z2 + b * z1 and m2' = m2 + c * m1
 * (elementwise; z = SwiGLU product, m = MLP output).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) and
 *    must be 16-byte aligned. The caller owns every buffer; the library
 *    allocates nothing, keeps no pointer after returning, and holds no global
 *    state besides a per-thread error message (and the fixed device scratch
 *    of dfa_decode_attn_noalloc), so calls are thread-safe.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; results are valid once the stream has
 *    been synchronised. Calls on one stream execute in order.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns a non-zero dfa_status and has no side effects.
 *    Device-resident sizes (ctx_lens, block_table) cannot be validated on the
 *    host: they are the caller's contract. The kernels clamp them so that no
 *    access leaves the buffers the descriptor describes: a length is clamped
 *    to [0, max_ctx_len], a block id to [0, num_blocks).
 *  - No C++ exception crosses this interface.
 *
 * Layouts (row-major, innermost last):
 *  - Q1, Q2, O1, O2:   [batch, num_q_heads, head_dim]
 *  - a:                [num_q_heads * head_dim] float32
 *  - K cache:          [num_blocks, num_kv_heads, block_size / 16,
 *                       head_dim / 8, 16, 8]
 *                      (keys in tiles of 16 positions; inside a tile, groups
 *                      of 8 dimensions, each holding the 16 positions' 8
 *                      elements: a tile is 16 * head_dim contiguous elements)
 *  - V cache:          [num_blocks, num_kv_heads, block_size / 16, head_dim, 16]
 *                      (values transposed inside tiles of 16 positions: for a
 *                      tile and a dimension, the 16 positions are contiguous)
 *  - block_table:      int32 [batch, max_blocks_per_seq]; position t of
 *                      sequence b is slot t % block_size of physical block
 *                      block_table[b][t / block_size]. A contiguous cache is
 *                      one block per sequence (block_size = capacity).
 *  - ctx_lens:         int32 [batch], cached positions attended (>= 1)
 *  - query head h reads kv head h / (num_q_heads / num_kv_heads).
 */
#ifndef DFA_H
#define DFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DFA_API __attribute__((visibility("default")))
#else
#define DFA_API
#endif

typedef enum dfa_status {
  DFA_OK = 0,
  DFA_ERR_NULL = 1,        /* a required pointer is NULL */
  DFA_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent */
  DFA_ERR_DTYPE = 3,       /* unsupported element-type combination */
  DFA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  DFA_ERR_UNSUPPORTED = 5, /* well-formed request with no kernel in this build */
  DFA_ERR_ALIGNMENT = 6,   /* a device pointer is not 16-byte aligned */
  DFA_ERR_HIP = 7          /* the HIP runtime reported an error */
} dfa_status;

typedef enum dfa_dtype { DFA_F32 = 0, DFA_BF16 = 1 } dfa_dtype;

/* Shape and policy of one decode-attention call (one layer). */
typedef struct dfa_attn_desc {
  int32_t batch;              /* sequences, >= 1 */
  int32_t num_q_heads;        /* Hq, multiple of num_kv_heads; (Hq / Hkv) * num_flows <= 32
                                 with a bf16 cache, <= 16 with a float32 cache */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t block_size;         /* positions per cache block: power of two >= 16 */
  int32_t max_blocks_per_seq; /* columns of block_table */
  int32_t num_blocks;         /* physical blocks in each cache tensor */
  int32_t max_ctx_len;        /* upper bound of ctx_lens; <= max_blocks_per_seq * block_size */
  int32_t num_flows;          /* 1 = primary only, 2 = primary and auxiliary */
  int32_t split_len;          /* positions per split (multiple of 32), 0 = library choice */
  float scale;                /* softmax scale applied to q.k (1/sqrt(D) in a standard layer) */
  dfa_dtype q_dtype;          /* element type of Q1 and Q2 */
  dfa_dtype kv_dtype;         /* element type of the K and V caches */
} dfa_attn_desc;

/*
 * Split plan. A sequence's positions are cut into splits of split_len
 * positions, processed independently and merged by a log-sum-exp combine.
 * Returns the split length the library will use for `desc` (> 0), or
 * -(dfa_status) if `desc` is invalid.
 */
DFA_API int32_t dfa_decode_attn_split_len(const dfa_attn_desc* desc);

/* Number of split slots per sequence: ceil(max_ctx_len / split_len); <= 0 on error. */
DFA_API int32_t dfa_decode_attn_num_splits(const dfa_attn_desc* desc);

/*
 * Workspace bytes needed by dfa_decode_attn (when it runs more than one
 * split) and by dfa_decode_attn_partials / dfa_combine: one partial record per
 * (sequence, query head, flow, split). 0 if `desc` is invalid. Calls that
 * share a workspace must not overlap in time.
 */
DFA_API size_t dfa_decode_attn_workspace_size(const dfa_attn_desc* desc);

/*
 * Dual-flow decode attention (asymmetric shared-KV attention, "Mecanismos
 * Chave"). For every sequence b, query head h and flow f:
 *     q^1 = Q1[b,h],  q^2 = Q2[b,h] + a[h] * Q1[b,h]
 *     O_f[b,h] = sum_t softmax_t(scale * <q^f, K_t>) V_t,  t in [0, ctx_lens[b])
 * Both flows are served from one read of every cached key and value. The
 * caches are read only (the auxiliary flow never writes KV). With one split
 * per sequence this is one kernel; with more, the split kernel is followed by
 * the log-sum-exp combine of dfa_combine on the same stream.
 *  q1, q2:   Q1, Q2 of type desc->q_dtype. q2 and a are ignored (may be NULL)
 *            when num_flows == 1.
 *  k_cache, v_cache: type desc->kv_dtype, layouts above. Never written.
 *  workspace: device scratch of workspace_bytes; required (>= the size from
 *            dfa_decode_attn_workspace_size) when more than one split runs,
 *            else may be NULL. Contents on return are unspecified.
 *  o1, o2:   float32 outputs; o2 ignored (may be NULL) when num_flows == 1.
 */
DFA_API dfa_status dfa_decode_attn(const dfa_attn_desc* desc, const void* q1, const void* q2,
                           const float* a, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens,
                           void* workspace, size_t workspace_bytes, float* o1, float* o2,
                           void* stream);

/*
 * Debug aid: checks on the device what a dfa_decode_attn call with `desc`
 * would read of ctx_lens and block_table. The attention kernels clamp a
 * length to [0, max_ctx_len] and a block id to [0, num_blocks), so that no
 * access leaves the buffers; a corrupt table is then read silently as the
 * nearest valid block. This call reports such entries instead: one small
 * kernel on `stream` writes
 *     flags[0] = DFA_TABLE_BAD_LEN   if some ctx_lens[b] + ctx_add lies outside
 *                                    [0, max_ctx_len],
 *              | DFA_TABLE_BAD_BLOCK if some entry among the first
 *                                    ceil(len_b / block_size) of row b (len_b
 *                                    the clamped length) lies outside
 *                                    [0, num_blocks);
 *     flags[1] = the smallest offending sequence index, or 0xFFFFFFFF.
 * flags: device uint32 [2] (16-byte aligned), written by the call (no
 * clearing needed). ctx_add: 0 as for dfa_decode_attn, 1 for the layer step
 * (which attends the just-appended position). Scans every row in one
 * workgroup: meant for debugging, not for the hot path.
 */
#define DFA_TABLE_BAD_LEN 1u
#define DFA_TABLE_BAD_BLOCK 2u
DFA_API dfa_status dfa_check_kv_table(const dfa_attn_desc* desc, const int32_t* block_table,
                                      const int32_t* ctx_lens, int32_t ctx_add, uint32_t* flags, void* stream);

/*
 * dfa_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, split plan, kernels and results as dfa_decode_attn, without
 * the workspace: the split records live in a device array of the library,
 * DFA_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held until the process ends. Its
 * device address is looked up on the first call on each GPU (with that GPU
 * current); no call allocates or frees memory.
 * Limit: dfa_decode_attn_workspace_size(desc) <= DFA_NOALLOC_SCRATCH_BYTES
 * whenever more than one split runs (checked on the host: DFA_ERR_WORKSPACE,
 * nothing enqueued). `stream` must belong to the current device
 * (DFA_ERR_UNSUPPORTED otherwise). Calls on one GPU share the array: calls
 * that overlap in time (on different streams) race and must not be issued.
 */
#define DFA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
DFA_API dfa_status dfa_decode_attn_noalloc(const dfa_attn_desc* desc, const void* q1, const void* q2,
                                           const float* a, const void* k_cache, const void* v_cache,
                                           const int32_t* block_table, const int32_t* ctx_lens, float* o1,
                                           float* o2, void* stream);

/*
 * Optional events for measuring the attention kernel itself: hipEvent_t
 * handles (passed as void*) that the runtime records when the attention
 * kernel's dispatch starts and ends, adding no command to the stream. NULL
 * members are not recorded. The combine kernel, if any, is not covered.
 */
typedef struct dfa_kernel_events {
  void* start;
  void* stop;
} dfa_kernel_events;

/* dfa_decode_attn with dfa_kernel_events around its attention kernel (events may be NULL). */
DFA_API dfa_status dfa_decode_attn_timed(const dfa_attn_desc* desc, const void* q1, const void* q2,
                                         const float* a, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* ctx_lens,
                                         void* workspace, size_t workspace_bytes, float* o1, float* o2,
                                         void* stream, const dfa_kernel_events* events);

/*
 * The split stage alone: writes one partial record per (b, h, f, split) to
 * `workspace` and no output. Record (b, h, f, s) starts at float index
 *     (((b * num_q_heads + h) * num_flows + f) * num_splits + s) * (head_dim + 4)
 * and holds head_dim floats of unnormalised output sum_t 2^(u_t - m) V_t, then
 * m = max_t u_t and l = sum_t 2^(u_t - m), with u_t = scale * log2(e) * <q, K_t>
 * over the split's positions, then two unused floats. A split past the end of
 * its sequence gets the empty record (O = 0, m = -inf, l = 0), so every
 * record is written. With dfa_combine this is the same computation
 * as dfa_decode_attn; the records also let a caller merge splits computed
 * elsewhere (for example other devices holding other positions).
 */
DFA_API dfa_status dfa_decode_attn_partials(const dfa_attn_desc* desc, const void* q1, const void* q2,
                                    const float* a, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Log-sum-exp combine of the partial records in `workspace` (layout above)
 * into the normalised outputs: with M = max_s m_s over the num_splits
 * records of a row,
 *     O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
 * Empty records add nothing; a row whose records are all empty (a sequence
 * with no position) gets zero outputs. Every record must have been written
 * (dfa_decode_attn_partials writes all of them).
 */
DFA_API dfa_status dfa_combine(const dfa_attn_desc* desc, const void* workspace, size_t workspace_bytes,
                               float* o1, float* o2, void* stream);

/*
 * ------------------------------------------------------------------ dual GEMV
 * Y_f = X_f W^T for both flows f from one read of a shared weight matrix W
 * ("Arquitetura Central": the flows share the attention, MLP and output
 * matrices; "Custos de Inferência vs. Treinamento": decode reads the unique
 * weights once), followed by one of the layer's epilogues. Activations and
 * outputs are float32 [batch, k] / [batch, n], row-major; weights bf16 in the
 * tiled layout written by dfa_pack_weight. Accumulation is float32; every
 * activation is split into two bf16 terms (hi = bf16(x), lo = bf16(x - hi))
 * unless x_exact_bf16 says they are exact bf16 values.
 */
typedef enum dfa_epilogue {
  DFA_EPI_NONE = 0,              /* y_f = x_f W^T */
  DFA_EPI_RESIDUAL = 1,          /* y_f = res_f + x_f W^T */
  DFA_EPI_SWIGLU = 2,            /* z_f = silu(x_f W^T) * (x_f W2^T), silu(u) = u / (1 + e^-u);
                                    y_1 = z_1; y_2 = z_2 + couple * z_1 (couple = b, may be NULL) */
  DFA_EPI_RESIDUAL_COUPLED = 3,  /* m_f = x_f W^T; y_1 = res_1 + m_1;
                                    y_2 = res_2 + m_2 + couple * m_1 (couple = c, may be NULL) */
  DFA_EPI_KV_APPEND = 4          /* one flow (primary): k = x_1 W^T, v = x_1 W2^T with n = Hkv * D,
                                    rounded to bf16 (nearest, ties to even) and written to position
                                    ctx_lens[b] of sequence b in the KV cache; y1, y2 (optional)
                                    receive k and v as float32 */
} dfa_epilogue;

typedef struct dfa_gemv_desc {
  int32_t batch;         /* sequences = rows per flow, 1..65535; one launch (and reduction) per
                            slice of 32 sequences with two flows, 64 with one: a larger batch
                            reads the weights once per slice */
  int32_t n;             /* output columns = rows of W, multiple of 64 */
  int32_t k;             /* input columns = columns of W, multiple of 128 */
  int32_t num_flows;     /* 1 (primary only) or 2 */
  int32_t epilogue;      /* dfa_epilogue */
  int32_t x_exact_bf16;  /* 1: every activation value is exactly a bf16 value */
  int32_t k_split;       /* k-ranges reduced through the workspace (1: none, the epilogue
                            runs in the GEMV kernel); 0 = library choice */
  int32_t rows_per_wg;   /* weight rows per workgroup: 64, or 128 (needs n % 128 == 0);
                            0 = library choice. Results do not depend on it. */
} dfa_gemv_desc;

/* KV cache written by DFA_EPI_KV_APPEND (same layout as dfa_decode_attn reads). */
typedef struct dfa_kv_target {
  void* k_cache;                /* bf16 [num_blocks, Hkv, block_size/16, D/8, 16, 8] */
  void* v_cache;                /* bf16 [num_blocks, Hkv, block_size/16, D, 16] */
  const int32_t* block_table;   /* int32 [batch, max_blocks_per_seq] */
  const int32_t* ctx_lens;      /* int32 [batch]: cached positions; the new one goes at ctx_lens[b] */
  int32_t num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks;
} dfa_kv_target;

/* Workspace bytes of dfa_dual_gemv for `desc` (0 if invalid or if the plan has one k-range). */
DFA_API size_t dfa_dual_gemv_workspace_size(const dfa_gemv_desc* desc);

/*
 * Runs the GEMV and its epilogue on `stream` (one launch with one k-range, else
 * two: the split GEMV and the fixed-order reduction with the epilogue). Required
 * pointers: w, x1, y1 (y1/y2 optional for KV_APPEND), x2 and y2 with two
 * flows, w2 for SWIGLU and KV_APPEND, res1 (res2 with two flows) for the
 * residual epilogues, kv for KV_APPEND. couple may be NULL. The auxiliary
 * flow's inputs (x2, res2, couple) never affect y1 or the KV cache.
 */
DFA_API dfa_status dfa_dual_gemv(const dfa_gemv_desc* desc, const uint16_t* w, const uint16_t* w2,
                                 const float* x1, const float* x2, const float* couple, const float* res1,
                                 const float* res2, float* y1, float* y2, const dfa_kv_target* kv,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Repacks a row-major bf16 weight [n, k] (nn.Linear layout) into the tiled
 * layout of dfa_dual_gemv: element (r, c) goes to
 *     ((r / 16) * (k / 8) + c / 8) * 128 + (r % 16) * 8 + c % 8.
 * n multiple of 16, k multiple of 8; w and w_tiled must not overlap.
 */
DFA_API dfa_status dfa_pack_weight(const uint16_t* w, uint16_t* w_tiled, int32_t n, int32_t k, void* stream);

/*
 * ------------------------------------------------------------ decode layer
 * One decode step of a whole dual-flow layer ("Arquitetura Central",
 * "Mecanismos Chave"), for every sequence b at its new position L = ctx_lens[b]:
 *     q_f = x_f Wq^T (both flows; x2 comes from the auxiliary flow's embedding)
 *     k, v = x_1 Wk^T, x_1 Wv^T -> bf16 -> KV cache position L   (primary only)
 *     o_f = dual-flow attention over positions [0, L] (dfa_decode_attn, with a)
 *     h_f = x_f + o_f Wo^T
 *     z_1 = silu(h_1 Wg^T) * (h_1 Wu^T),  z_2 = silu(h_2 Wg^T) * (h_2 Wu^T) + b * z_1
 *     out_1 = h_1 + z_1 Wd^T,             out_2 = h_2 + z_2 Wd^T + c * (z_1 Wd^T)
 * The query, key and value projections run as one GEMV over the rows
 * [Wq; Wk; Wv] (the matrices stay separate in memory) whose split-K reduction
 * stores the queries and appends the keys and values; each other GEMV is one
 * launch plus, when its plan splits k, a reduction launch (at the benchmark
 * shape: 8 launches). Every weight is read once for both flows (once per
 * slice of 32 sequences beyond 32). The caller advances ctx_lens afterwards.
 * Requirements: those of dfa_decode_attn (max_ctx_len >= every ctx_lens[b] +
 * 1) and of dfa_dual_gemv (hidden, mlp, num_q_heads * head_dim and
 * num_kv_heads * head_dim multiples of 128). x1, x2, out1, out2: float32 [batch, hidden].
 * The auxiliary flow's inputs (x2, a, b, c) never affect out1 or the cache.
 */
typedef struct dfa_layer_desc {
  int32_t batch, hidden, num_q_heads, num_kv_heads, head_dim, mlp;
  int32_t block_size, max_blocks_per_seq, num_blocks, max_ctx_len;
  float scale;
  int32_t x_exact_bf16;  /* 1: x1 and x2 hold exact bf16 values */
} dfa_layer_desc;

typedef struct dfa_layer_weights {
  const uint16_t* wq;      /* [num_q_heads * head_dim, hidden], tiled (dfa_pack_weight) */
  const uint16_t* wk;      /* [num_kv_heads * head_dim, hidden], tiled */
  const uint16_t* wv;      /* [num_kv_heads * head_dim, hidden], tiled */
  const uint16_t* wo;      /* [hidden, num_q_heads * head_dim], tiled */
  const uint16_t* w_gate;  /* [mlp, hidden], tiled */
  const uint16_t* w_up;    /* [mlp, hidden], tiled */
  const uint16_t* w_down;  /* [hidden, mlp], tiled */
  const float* a;          /* [num_q_heads * head_dim] query coupling */
  const float* b;          /* [mlp] MLP-intermediate coupling (NULL = 0) */
  const float* c;          /* [hidden] MLP-output coupling (NULL = 0) */
} dfa_layer_weights;

DFA_API size_t dfa_decode_layer_workspace_size(const dfa_layer_desc* desc);

DFA_API dfa_status dfa_decode_layer(const dfa_layer_desc* desc, const dfa_layer_weights* weights,
                                    const float* x1, const float* x2, void* k_cache, void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens, float* out1,
                                    float* out2, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ------------------------------------------------------------- layer stack
 * One decode step through num_layers dual-flow layers of the shape `layer`
 * (the layer of dfa_decode_layer, "Arquitetura Central", "Mecanismos Chave"),
 * each flow's output feeding the next layer, with the LLaMA-like options the
 * pages do not name (this library's choices):
 *  - rms_norm = 1: pre-norm RMSNorm before the attention block and before the
 *    MLP block, y = x / sqrt(mean(x^2) + rms_eps) * w, one weight vector per
 *    block and layer (16-byte aligned), shared by both flows; the residuals
 *    add the un-normed x and h;
 *  - rope: rotary embeddings of both flows' queries and of the primary's key
 *    at position ctx_lens[b] (before the query coupling and the cache
 *    append): dimension pairs of each head, (i, i + head_dim/2) for
 *    DFA_ROPE_HALF or (2i, 2i + 1) for DFA_ROPE_INTERLEAVED, rotated
 *    (x, y) -> (x cos - y sin, x sin + y cos) by the caller's tables
 *    rope_cos, rope_sin: float32 [rope_max_pos, head_dim / 2] (row p: the
 *    angles of position p; positions are clamped to rope_max_pos - 1).
 * Every layer appends the primary's key and value at ctx_lens[b] of its own
 * cache (all layers share block_table and ctx_lens); the caller advances
 * ctx_lens afterwards. layer.x_exact_bf16 describes x1 and x2 (the first
 * layer's input) only. With rope = DFA_ROPE_NONE and rms_norm = 0 each layer
 * is exactly dfa_decode_layer. The step allocates nothing and issues only
 * kernel launches, so it can be captured in a HIP graph.
 */
typedef enum dfa_rope { DFA_ROPE_NONE = 0, DFA_ROPE_HALF = 1, DFA_ROPE_INTERLEAVED = 2 } dfa_rope;

typedef struct dfa_stack_desc {
  dfa_layer_desc layer;  /* shape of every layer (as dfa_decode_layer) */
  int32_t num_layers;    /* 1..4096 */
  int32_t rope;          /* dfa_rope */
  int32_t rope_max_pos;  /* rows of the rotary tables (>= layer.max_ctx_len when rope is set) */
  int32_t rms_norm;      /* 0 or 1 */
  float rms_eps;         /* >= 0 */
} dfa_stack_desc;

typedef struct dfa_stack_layer {
  dfa_layer_weights w;     /* as dfa_decode_layer */
  const float* norm_attn;  /* [hidden] (rms_norm) */
  const float* norm_mlp;   /* [hidden] (rms_norm) */
  void* k_cache;           /* this layer's cache (layout of dfa_decode_attn) */
  void* v_cache;
} dfa_stack_layer;

DFA_API size_t dfa_decode_stack_workspace_size(const dfa_stack_desc* desc);

/* layers: host array [num_layers]; x1, x2, out1, out2: float32 [batch, hidden]. */
DFA_API dfa_status dfa_decode_stack(const dfa_stack_desc* desc, const dfa_stack_layer* layers, const float* rope_cos,
                                    const float* rope_sin, const float* x1, const float* x2,
                                    const int32_t* block_table, const int32_t* ctx_lens, float* out1, float* out2,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * ------------------------------------------------------ mixture decoding
 * Next token from the mixture of the two flows' distributions ("Mecanismos
 * Chave", mixture objective): with p_f = softmax(logits_f) over the vocabulary,
 *     c = sum_v p_1(v)^2           (the primary's collision probability)
 *     alpha = (1 + c) / 2          (this library's reading: the primary keeps at
 *                                   least half of the weight, more when confident)
 *     p_mix = alpha p_1 + (1 - alpha) p_2.
 * For each sequence b, with the caller's uniform u[b] (clamped to [0, 1)):
 *     token[b]  = the smallest v whose cumulative p_mix mass exceeds u[b] times
 *                 the total mass (inverse CDF);
 *     greedy[b] = the smallest v with the largest p_mix(v);
 *     alpha[b]  = alpha.
 * logits1 (primary), logits2 (auxiliary): float32 [batch, vocab], row-major,
 * 16-byte aligned, finite (a row with a non-finite logit returns token and
 * greedy vocab - 1, or the first maximum where p_mix has one; never a token
 * outside [0, vocab)). p_mix (optional, NULL to skip): float32
 * [batch, vocab], receives the mixture. u: float32 [batch]. token, greedy:
 * int32 [batch]; alpha: float32 [batch]. All device memory owned by the
 * caller; results independent of timing.
 * Masses are summed as integers (p_mix scaled by 2^35, truncated), so the
 * search is exact and independent of summation order; a token with less than
 * 2^-35 of mass is never drawn. One launch on `stream` for vocab <= 32768,
 * three above.
 * Limits: batch 1..65535; vocab a multiple of 4 in [4, 2^20]. The workspace
 * (dfa_mixture_workspace_size bytes, 16-byte aligned) holds per-chunk records
 * for vocab > 32768 (required at every size); its contents on entry do not
 * matter.
 */
typedef struct dfa_mixture_desc {
  int32_t batch;
  int32_t vocab;
} dfa_mixture_desc;

/* Workspace bytes of dfa_mixture_sample for `desc` (0 if invalid). */
DFA_API size_t dfa_mixture_workspace_size(const dfa_mixture_desc* desc);

DFA_API dfa_status dfa_mixture_sample(const dfa_mixture_desc* desc, const float* logits1, const float* logits2,
                                      const float* u, int32_t* token, int32_t* greedy, float* alpha, float* p_mix,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ------------------------------------------------------------ output head
 * The output head in one call: both flows' logits from one read of the
 * shared vocabulary matrix ("Arquitetura Central": one output matrix shared by
 * the flows), then the mixture decoding above ("Mecanismos Chave", mixture
 * objective):
 *     logits_f = h_f W^T  (W: bf16 [vocab, hidden], tiled by dfa_pack_weight)
 * and token, greedy, alpha and (optionally) p_mix exactly as
 * dfa_mixture_sample defines them for these logits: the kernels of
 * dfa_dual_gemv, then those of dfa_mixture_sample, sharing one workspace.
 *  h1, h2:          float32 [batch, hidden] final hidden states of the flows
 *  u:               float32 [batch] uniforms
 *  logits1, logits2: float32 [batch, vocab] outputs (required: the mixture
 *                   reads them back)
 *  token, greedy, alpha, p_mix: as dfa_mixture_sample (p_mix may be NULL)
 *  workspace:       dfa_output_head_workspace_size bytes, 16-byte aligned
 * Limits: batch 1..65535 (the GEMV in slices of 32 sequences); vocab a
 * multiple of 64 in [64, 2^20]; hidden a multiple of 128.
 */
typedef struct dfa_head_desc {
  int32_t batch;
  int32_t vocab;
  int32_t hidden;
  int32_t x_exact_bf16;  /* 1: h1 and h2 hold exact bf16 values */
} dfa_head_desc;

DFA_API size_t dfa_output_head_workspace_size(const dfa_head_desc* desc);

DFA_API dfa_status dfa_output_head(const dfa_head_desc* desc, const uint16_t* w_vocab, const float* h1,
                                   const float* h2, const float* u, float* logits1, float* logits2, int32_t* token,
                                   int32_t* greedy, float* alpha, float* p_mix, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * ------------------------------------------- mixture-of-experts FFN (router replay)
 * A SwiGLU mixture-of-experts FFN for both flows at one decode step ("Mecanismos
 * Chave", router replay: the auxiliary flow reuses the experts the primary
 * router selected, with its own mixing weights; "Contribuições Principais",
 * phase-specific MoE allocation: the two flows' expert fan-outs k1 and k2 are
 * independent). This library's reading, for every sequence s:
 *     experts ranked by the primary's router logits r1[s] (descending; equal
 *     logits in index order); S1 = the first k1, S2 = the first k2 (k1 <= k2)
 *     g1 = softmax of r1[s] over S1,  g2 = softmax of r2[s] over S2
 *     z_f,e = silu(h_f Wg_e^T) * (h_f Wu_e^T);  z2,e += b * z1,e for e in S1
 *     m1 = sum_{e in S1} g1(e) z1,e Wd_e^T,  m2 = sum_{e in S2} g2(e) z2,e Wd_e^T
 *     out1 = res1 + m1,  out2 = res2 + m2 + c * m1
 * Each selected expert's matrices are read once for every row of both flows
 * that selected it. The primary flow's outputs never depend on the auxiliary
 * flow's inputs (h2, r2, res2, b, c).
 */
typedef struct dfa_moe_desc {
  int32_t batch;         /* sequences: 1..65535 (the expert GEMVs run slices of 32 sequences,
                            each reading its selected experts again) */
  int32_t hidden;        /* model width: multiple of 128 */
  int32_t mlp;           /* expert width: multiple of 128 */
  int32_t num_experts;   /* 1..1024 */
  int32_t k1, k2;        /* fan-outs: 1 <= k1 <= k2 <= min(num_experts, 32) */
  int32_t x_exact_bf16;  /* 1: h1 and h2 hold exact bf16 values */
} dfa_moe_desc;

/*
 * Bytes of a routing buffer: int32 sel [batch][k2] (experts in ranking order;
 * the first k1 of a row are the primary's), then float32 g1 [batch][k1], then
 * float32 g2 [batch][k2], each section starting on a 16-byte boundary. 0 if
 * `desc` is invalid. A caller may also fill one itself (distinct experts in
 * [0, num_experts) per row).
 */
DFA_API size_t dfa_moe_routing_size(const dfa_moe_desc* desc);

/*
 * Router replay: from both flows' router logits r1, r2 (float32
 * [batch, num_experts], finite), writes the selection and both flows' mixing
 * weights into `routing` (one launch on `stream`). Equal logits rank in index
 * order; the mixing weights are summed in ranking order.
 */
DFA_API dfa_status dfa_moe_route(const dfa_moe_desc* desc, const float* r1, const float* r2, void* routing,
                                 size_t routing_bytes, void* stream);

/* Workspace bytes of dfa_moe_ffn: 4 * min(batch, 32) * k2 * 2 * (mlp + hidden); 0 if invalid. */
DFA_API size_t dfa_moe_workspace_size(const dfa_moe_desc* desc);

/*
 * The experts and their combination (three launches on `stream`): grouped
 * gate/up GEMV with SwiGLU and b, grouped down GEMV, and the weighted sums in
 * ranking order with the residuals and c.
 *  w_gate, w_up: bf16 [num_experts][mlp, hidden], w_down: bf16
 *                [num_experts][hidden, mlp]; each expert's matrix tiled by
 *                dfa_pack_weight, the experts back to back.
 *  b: float32 [mlp] or NULL (0); c: float32 [hidden] or NULL (0).
 *  h1, h2: float32 [batch, hidden] FFN inputs; res1, res2: float32
 *          [batch, hidden] residuals or NULL (0); out1, out2: float32
 *          [batch, hidden]; routing: as written by dfa_moe_route.
 * Routing entries outside [0, num_experts) select nothing (their slots then
 * read unwritten workspace). The workspace's contents on entry do not matter.
 */
DFA_API dfa_status dfa_moe_ffn(const dfa_moe_desc* desc, const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, const float* b, const float* c, const float* h1,
                               const float* h2, const float* res1, const float* res2, const void* routing,
                               float* out1, float* out2, void* workspace, size_t workspace_bytes, void* stream);

/*
 * --------------------------------------------------------- primary prefill
 * Prefill of a batch of prompts by the primary flow alone ("Custos de
 * Inferência vs. Treinamento": prefill costs what a standard Transformer's
 * does, the auxiliary flow being skipped; "Arquitetura Central": only the
 * primary flow writes the cache). Two launches on `stream`:
 *  1. the prompts' keys and values go to positions [0, L_b) of each sequence
 *     b in the paged cache (layouts above; other slots are left as they are);
 *  2. causal self-attention, for every prompt b, position t < L_b, head h:
 *       O[b,t,h] = sum_{u <= t} softmax_u(scale * <Q[b,t,h], K[b,u,g]>) V[b,u,g]
 *     with g = h / (num_q_heads / num_kv_heads), keys and values read back
 *     from the cache.
 * The auxiliary flow joins at the last prompt position ("Dual-Flow
 * Transformers: Decoupling the Primary Prefill Path from Additional Decode
 * Computation"): that first auxiliary step is dfa_decode_attn with
 * ctx_lens[b] = L_b, Q1 = the primary's queries at position L_b - 1 and Q2 the
 * auxiliary flow's.
 *  q:  bf16 [batch, max_prompt_len, num_q_heads, head_dim]
 *  k, v: bf16 [batch, max_prompt_len, num_kv_heads, head_dim]
 *  prompt_lens: int32 [batch], L_b in [0, max_prompt_len] (clamped there);
 *      rows at positions >= L_b are never read
 *  block_table: int32 [batch, max_blocks_per_seq] covering positions [0, L_b)
 *      (entries clamped to [0, num_blocks))
 *  o:  float32 [batch, max_prompt_len, num_q_heads, head_dim]; rows at
 *      positions >= L_b are not written
 * Supported: head_dim 64 or 128; 1, 2, 4, 8 or 16 query heads per kv head;
 * ceil(max_prompt_len / block_size) <= 2048 (the table slice is staged on chip).
 */
typedef struct dfa_prefill_desc {
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t max_prompt_len;  /* row stride of q, k, v and o */
  int32_t block_size, max_blocks_per_seq, num_blocks;
  float scale;
} dfa_prefill_desc;

DFA_API dfa_status dfa_prefill(const dfa_prefill_desc* desc, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* prompt_lens, void* k_cache, void* v_cache,
                               const int32_t* block_table, float* o, void* stream);

/* Short fixed description of a status code. Never NULL. */
DFA_API const char* dfa_status_string(dfa_status status);

/* Detail of the last failure reported on the calling thread ("" if none). */
DFA_API const char* dfa_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
DFA_API int32_t dfa_version(void);

/*
 * Measurement helper (not part of the method): reads `bytes` bytes at `buf`
 * with coalesced, non-temporal 16-byte loads on `stream`, the bandwidth
 * ceiling that the streaming kernels are compared to. `sink` must hold 4 bytes per launched
 * thread (dfa_stream_read_sink_bytes()); it is written only with a value that
 * keeps the loads live. bytes must be a multiple of 16.
 */
DFA_API dfa_status dfa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
DFA_API size_t dfa_stream_read_sink_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* DFA_H */
