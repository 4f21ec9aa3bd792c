"""ctypes binding of libdfa (include/dfa.h): argument marshalling only.

Each function takes torch tensors resident on the GPU (or None where the C
entry point accepts NULL), passes their device addresses and the current HIP
stream to the C function of the same name, and raises ``DfaError`` on a
non-zero status. Every step of the computation runs in the library's kernels;
there is no fallback: if libdfa.so is missing, loading fails loudly.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdfa.so")

DFA_F32, DFA_BF16 = 0, 1
STATUS = {0: "DFA_OK", 1: "DFA_ERR_NULL", 2: "DFA_ERR_SHAPE", 3: "DFA_ERR_DTYPE",
          4: "DFA_ERR_WORKSPACE", 5: "DFA_ERR_UNSUPPORTED", 6: "DFA_ERR_ALIGNMENT", 7: "DFA_ERR_HIP"}

# Every symbol include/dfa.h declares.
EXPORTS = ["dfa_decode_attn_split_len", "dfa_decode_attn_num_splits", "dfa_decode_attn_workspace_size",
           "dfa_decode_attn", "dfa_decode_attn_noalloc", "dfa_decode_attn_timed", "dfa_decode_attn_partials",
           "dfa_combine", "dfa_check_kv_table",
           "dfa_dual_gemv_workspace_size", "dfa_dual_gemv", "dfa_pack_weight",
           "dfa_decode_layer_workspace_size", "dfa_decode_layer", "dfa_decode_stack_workspace_size",
           "dfa_decode_stack",
           "dfa_mixture_workspace_size", "dfa_mixture_sample", "dfa_output_head_workspace_size", "dfa_output_head",
           "dfa_moe_routing_size", "dfa_moe_route", "dfa_moe_workspace_size", "dfa_moe_ffn", "dfa_prefill",
           "dfa_status_string", "dfa_last_error", "dfa_version", "dfa_stream_read", "dfa_stream_read_sink_bytes"]

DFA_EPI_NONE, DFA_EPI_RESIDUAL, DFA_EPI_SWIGLU, DFA_EPI_RESIDUAL_COUPLED, DFA_EPI_KV_APPEND = range(5)
DFA_ROPE_NONE, DFA_ROPE_HALF, DFA_ROPE_INTERLEAVED = range(3)


class DfaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class AttnDesc(ctypes.Structure):
    """Mirror of dfa_attn_desc."""

    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
                ("num_flows", ctypes.c_int32), ("split_len", ctypes.c_int32),
                ("scale", ctypes.c_float), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class GemvDesc(ctypes.Structure):
    """Mirror of dfa_gemv_desc."""

    _fields_ = [("batch", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("num_flows", ctypes.c_int32), ("epilogue", ctypes.c_int32), ("x_exact_bf16", ctypes.c_int32),
                ("k_split", ctypes.c_int32), ("rows_per_wg", ctypes.c_int32)]


class KvTarget(ctypes.Structure):
    """Mirror of dfa_kv_target."""

    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("ctx_lens", ctypes.c_void_p), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    """Mirror of dfa_layer_desc."""

    _fields_ = [(f, ctypes.c_int32) for f in ("batch", "hidden", "num_q_heads", "num_kv_heads", "head_dim", "mlp",
                                              "block_size", "max_blocks_per_seq", "num_blocks", "max_ctx_len")] + \
               [("scale", ctypes.c_float), ("x_exact_bf16", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    """Mirror of dfa_layer_weights."""

    _fields_ = [(f, ctypes.c_void_p) for f in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "a", "b", "c")]


class StackDesc(ctypes.Structure):
    """Mirror of dfa_stack_desc."""

    _fields_ = [("layer", LayerDesc), ("num_layers", ctypes.c_int32), ("rope", ctypes.c_int32),
                ("rope_max_pos", ctypes.c_int32), ("rms_norm", ctypes.c_int32), ("rms_eps", ctypes.c_float)]


class StackLayer(ctypes.Structure):
    """Mirror of dfa_stack_layer."""

    _fields_ = [("w", LayerWeights), ("norm_attn", ctypes.c_void_p), ("norm_mlp", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


class MixtureDesc(ctypes.Structure):
    """Mirror of dfa_mixture_desc."""

    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32)]


class HeadDesc(ctypes.Structure):
    """Mirror of dfa_head_desc."""

    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("x_exact_bf16", ctypes.c_int32)]


class MoeDesc(ctypes.Structure):
    """Mirror of dfa_moe_desc."""

    _fields_ = [(f, ctypes.c_int32) for f in ("batch", "hidden", "mlp", "num_experts", "k1", "k2", "x_exact_bf16")]


class PrefillDesc(ctypes.Structure):
    """Mirror of dfa_prefill_desc."""

    _fields_ = [(f, ctypes.c_int32) for f in ("batch", "num_q_heads", "num_kv_heads", "head_dim", "max_prompt_len",
                                              "block_size", "max_blocks_per_seq", "num_blocks")] + \
               [("scale", ctypes.c_float)]


class KernelEvents(ctypes.Structure):
    """Mirror of dfa_kernel_events (hipEvent_t handles)."""

    _fields_ = [("start", ctypes.c_void_p), ("stop", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dual_flow_shared_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(AttnDesc)
        sig = {
            "dfa_decode_attn_split_len": (ctypes.c_int32, [D]),
            "dfa_decode_attn_num_splits": (ctypes.c_int32, [D]),
            "dfa_decode_attn_workspace_size": (ctypes.c_size_t, [D]),
            "dfa_decode_attn": (ctypes.c_int, [D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
            "dfa_decode_attn_noalloc": (ctypes.c_int, [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
            "dfa_check_kv_table": (ctypes.c_int, [D, _P, _P, ctypes.c_int32, _P, _P]),
            "dfa_decode_attn_timed": (ctypes.c_int, [D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P,
                                                     ctypes.POINTER(KernelEvents)]),
            "dfa_decode_attn_partials": (ctypes.c_int, [D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "dfa_combine": (ctypes.c_int, [D, _P, ctypes.c_size_t, _P, _P, _P]),
            "dfa_dual_gemv_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(GemvDesc)]),
            "dfa_dual_gemv": (ctypes.c_int, [ctypes.POINTER(GemvDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             ctypes.POINTER(KvTarget), _P, ctypes.c_size_t, _P]),
            "dfa_pack_weight": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P]),
            "dfa_decode_layer_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc)]),
            "dfa_decode_layer": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _P, _P, _P,
                                                _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "dfa_mixture_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MixtureDesc)]),
            "dfa_mixture_sample": (ctypes.c_int, [ctypes.POINTER(MixtureDesc), _P, _P, _P, _P, _P, _P, _P, _P,
                                                  ctypes.c_size_t, _P]),
            "dfa_output_head_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(HeadDesc)]),
            "dfa_output_head": (ctypes.c_int, [ctypes.POINTER(HeadDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_size_t, _P]),
            "dfa_moe_routing_size": (ctypes.c_size_t, [ctypes.POINTER(MoeDesc)]),
            "dfa_moe_route": (ctypes.c_int, [ctypes.POINTER(MoeDesc), _P, _P, _P, ctypes.c_size_t, _P]),
            "dfa_moe_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MoeDesc)]),
            "dfa_moe_ffn": (ctypes.c_int, [ctypes.POINTER(MoeDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, ctypes.c_size_t, _P]),
            "dfa_prefill": (ctypes.c_int, [ctypes.POINTER(PrefillDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
            "dfa_decode_stack_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(StackDesc)]),
            "dfa_decode_stack": (ctypes.c_int, [ctypes.POINTER(StackDesc), ctypes.POINTER(StackLayer), _P, _P, _P, _P,
                                                _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "dfa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "dfa_last_error": (ctypes.c_char_p, []),
            "dfa_version": (ctypes.c_int32, []),
            "dfa_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
            "dfa_stream_read_sink_bytes": (ctypes.c_size_t, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    """Device address of a GPU tensor, or None (NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libdfa takes GPU tensors")
    if not t.is_contiguous():
        raise ValueError("libdfa takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status: int):
    if status != 0:
        raise DfaError(status, lib().dfa_last_error().decode())


def dfa_decode_attn_split_len(desc: AttnDesc) -> int:
    v = lib().dfa_decode_attn_split_len(ctypes.byref(desc))
    if v <= 0:
        raise DfaError(-v, lib().dfa_last_error().decode())
    return v


def dfa_decode_attn_num_splits(desc: AttnDesc) -> int:
    v = lib().dfa_decode_attn_num_splits(ctypes.byref(desc))
    if v <= 0:
        raise DfaError(-v, lib().dfa_last_error().decode())
    return v


def dfa_decode_attn_workspace_size(desc: AttnDesc) -> int:
    return int(lib().dfa_decode_attn_workspace_size(ctypes.byref(desc)))


def dfa_decode_attn(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, workspace, o1, o2,
                    stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_decode_attn(ctypes.byref(desc), _ptr(q1), _ptr(q2), _ptr(a), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(workspace),
                                 ws_bytes, _ptr(o1), _ptr(o2), _stream(stream)))


def dfa_decode_attn_noalloc(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, o1, o2, stream=None):
    """dfa_decode_attn without a workspace (the library's fixed device scratch holds the split records)."""
    _check(lib().dfa_decode_attn_noalloc(ctypes.byref(desc), _ptr(q1), _ptr(q2), _ptr(a), _ptr(k_cache),
                                         _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(o1), _ptr(o2),
                                         _stream(stream)))


DFA_TABLE_BAD_LEN, DFA_TABLE_BAD_BLOCK = 1, 2


def dfa_check_kv_table(desc, block_table, ctx_lens, flags, ctx_add=0, stream=None):
    """Device-side check of the lengths and block-table entries a decode call reads; writes flags
    (int32 tensor [2], viewed as uint32): the DFA_TABLE_BAD_* bits and the first offending sequence."""
    _check(lib().dfa_check_kv_table(ctypes.byref(desc), _ptr(block_table), _ptr(ctx_lens), ctx_add, _ptr(flags),
                                    _stream(stream)))


def _event_handle(ev):
    """Raw hipEvent_t of a torch.cuda.Event (created on its first record)."""
    if ev is None:
        return None
    if not ev.cuda_event:
        raise ValueError("record the event once before passing it, so that it exists")
    return ev.cuda_event


def dfa_decode_attn_timed(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, workspace, o1, o2,
                          stream=None, start=None, stop=None):
    """dfa_decode_attn with torch.cuda.Event `start`/`stop` recorded around its attention kernel."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ev = KernelEvents(_event_handle(start), _event_handle(stop))
    _check(lib().dfa_decode_attn_timed(ctypes.byref(desc), _ptr(q1), _ptr(q2), _ptr(a), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(workspace),
                                       ws_bytes, _ptr(o1), _ptr(o2), _stream(stream), ctypes.byref(ev)))


def dfa_decode_attn_partials(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, workspace,
                             stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_decode_attn_partials(ctypes.byref(desc), _ptr(q1), _ptr(q2), _ptr(a), _ptr(k_cache),
                                          _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens),
                                          _ptr(workspace), ws_bytes, _stream(stream)))


def dfa_combine(desc, workspace, o1, o2, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_combine(ctypes.byref(desc), _ptr(workspace), ws_bytes, _ptr(o1),
                             _ptr(o2), _stream(stream)))


def dfa_dual_gemv_workspace_size(desc: GemvDesc) -> int:
    return int(lib().dfa_dual_gemv_workspace_size(ctypes.byref(desc)))


def kv_target(k_cache, v_cache, block_table, ctx_lens, num_kv_heads, head_dim, block_size,
              max_blocks_per_seq, num_blocks) -> KvTarget:
    """Device addresses of the cache to append to; the structure keeps the tensors alive."""
    kv = KvTarget(_ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), num_kv_heads, head_dim,
                  block_size, max_blocks_per_seq, num_blocks)
    kv._tensors = (k_cache, v_cache, block_table, ctx_lens)
    return kv


def dfa_dual_gemv(desc, w, w2, x1, x2, couple, res1, res2, y1, y2, kv, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_dual_gemv(ctypes.byref(desc), _ptr(w), _ptr(w2), _ptr(x1), _ptr(x2), _ptr(couple),
                               _ptr(res1), _ptr(res2), _ptr(y1), _ptr(y2),
                               ctypes.byref(kv) if kv is not None else None, _ptr(workspace), ws_bytes,
                               _stream(stream)))


def dfa_pack_weight(w, w_tiled, n, k, stream=None):
    _check(lib().dfa_pack_weight(_ptr(w), _ptr(w_tiled), n, k, _stream(stream)))


def dfa_decode_layer_workspace_size(desc: LayerDesc) -> int:
    return int(lib().dfa_decode_layer_workspace_size(ctypes.byref(desc)))


def layer_weights(wq, wk, wv, wo, w_gate, w_up, w_down, a, b, c) -> LayerWeights:
    """Device addresses of packed weights and coupling vectors (tensors or None); the structure
    keeps the tensors alive."""
    tensors = (wq, wk, wv, wo, w_gate, w_up, w_down, a, b, c)
    lw = LayerWeights(*[_ptr(t) for t in tensors])
    lw._tensors = tensors
    return lw


def dfa_decode_layer(desc, weights, x1, x2, k_cache, v_cache, block_table, ctx_lens, out1, out2, workspace,
                     stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_decode_layer(ctypes.byref(desc), ctypes.byref(weights), _ptr(x1), _ptr(x2), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(out1), _ptr(out2),
                                  _ptr(workspace), ws_bytes, _stream(stream)))


def dfa_mixture_workspace_size(desc: MixtureDesc) -> int:
    return int(lib().dfa_mixture_workspace_size(ctypes.byref(desc)))


def dfa_mixture_sample(desc, logits1, logits2, u, token, greedy, alpha, p_mix, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_mixture_sample(ctypes.byref(desc), _ptr(logits1), _ptr(logits2), _ptr(u), _ptr(token),
                                    _ptr(greedy), _ptr(alpha), _ptr(p_mix), _ptr(workspace), ws_bytes,
                                    _stream(stream)))


def dfa_output_head_workspace_size(desc: HeadDesc) -> int:
    return lib().dfa_output_head_workspace_size(ctypes.byref(desc))


def dfa_output_head(desc, w_vocab, h1, h2, u, logits1, logits2, token, greedy, alpha, p_mix, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_output_head(ctypes.byref(desc), _ptr(w_vocab), _ptr(h1), _ptr(h2), _ptr(u), _ptr(logits1),
                                 _ptr(logits2), _ptr(token), _ptr(greedy), _ptr(alpha), _ptr(p_mix), _ptr(workspace),
                                 ws_bytes, _stream(stream)))


def dfa_moe_routing_size(desc: MoeDesc) -> int:
    return int(lib().dfa_moe_routing_size(ctypes.byref(desc)))


def dfa_moe_workspace_size(desc: MoeDesc) -> int:
    return int(lib().dfa_moe_workspace_size(ctypes.byref(desc)))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dfa_moe_route(desc, r1, r2, routing, stream=None):
    _check(lib().dfa_moe_route(ctypes.byref(desc), _ptr(r1), _ptr(r2), _ptr(routing), _nbytes(routing),
                               _stream(stream)))


def dfa_moe_ffn(desc, w_gate, w_up, w_down, b, c, h1, h2, res1, res2, routing, out1, out2, workspace, stream=None):
    _check(lib().dfa_moe_ffn(ctypes.byref(desc), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(b), _ptr(c), _ptr(h1),
                             _ptr(h2), _ptr(res1), _ptr(res2), _ptr(routing), _ptr(out1), _ptr(out2), _ptr(workspace),
                             _nbytes(workspace), _stream(stream)))


def dfa_prefill(desc, q, k, v, prompt_lens, k_cache, v_cache, block_table, o, stream=None):
    _check(lib().dfa_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(prompt_lens), _ptr(k_cache),
                             _ptr(v_cache), _ptr(block_table), _ptr(o), _stream(stream)))


def dfa_decode_stack_workspace_size(desc: StackDesc) -> int:
    return int(lib().dfa_decode_stack_workspace_size(ctypes.byref(desc)))


def stack_layers(entries):
    """A dfa_stack_layer array from (layer_weights(...), norm_attn, norm_mlp, k_cache, v_cache) tuples (tensors
    or None); the array keeps the tensors alive."""
    arr = (StackLayer * len(entries))()
    keep = []
    for i, (w, na, nm, kc, vc) in enumerate(entries):
        arr[i] = StackLayer(w, _ptr(na), _ptr(nm), _ptr(kc), _ptr(vc))
        keep.append((w, na, nm, kc, vc))
    arr._tensors = keep
    return arr


def dfa_decode_stack(desc, layers, rope_cos, rope_sin, x1, x2, block_table, ctx_lens, out1, out2, workspace,
                     stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dfa_decode_stack(ctypes.byref(desc), layers, _ptr(rope_cos), _ptr(rope_sin), _ptr(x1), _ptr(x2),
                                  _ptr(block_table), _ptr(ctx_lens), _ptr(out1), _ptr(out2), _ptr(workspace),
                                  ws_bytes, _stream(stream)))


def dfa_stream_read(buf, sink, stream=None):
    _check(lib().dfa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def dfa_stream_read_sink_bytes() -> int:
    return int(lib().dfa_stream_read_sink_bytes())


def dfa_status_string(status: int) -> str:
    return lib().dfa_status_string(status).decode()


def dfa_version() -> int:
    return int(lib().dfa_version())
