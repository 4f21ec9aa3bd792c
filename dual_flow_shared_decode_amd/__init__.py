"""Dual-flow shared-KV decode on AMD Instinct MI355X (gfx950).

The computation lives in libdfa.so (C ABI in include/dfa.h, HIP kernels under
csrc/, built by ``build``). This package is its ctypes binding (``_lib``: the
same names as the C entry points, argument marshalling only). PyTorch serves
only for device memory, streams and events.
"""
from ._lib import (DFA_BF16, DFA_EPI_KV_APPEND, DFA_ROPE_HALF, DFA_ROPE_INTERLEAVED, DFA_ROPE_NONE, DFA_EPI_NONE, DFA_EPI_RESIDUAL,  # noqa: F401
                   DFA_EPI_RESIDUAL_COUPLED, DFA_EPI_SWIGLU, DFA_F32, AttnDesc, DfaError, GemvDesc,
                   KernelEvents, KvTarget, LayerDesc, LayerWeights, MixtureDesc, MoeDesc, PrefillDesc, StackDesc, StackLayer, dfa_combine, dfa_decode_attn,
                   dfa_decode_attn_num_splits, dfa_decode_layer, dfa_decode_layer_workspace_size,
                   dfa_decode_attn_partials, dfa_decode_attn_split_len, dfa_decode_attn_timed,
                   dfa_decode_attn_workspace_size, dfa_dual_gemv, dfa_dual_gemv_workspace_size,
                   dfa_mixture_sample, dfa_mixture_workspace_size, dfa_moe_ffn, dfa_moe_route,
                   dfa_moe_routing_size, dfa_moe_workspace_size, dfa_pack_weight, dfa_prefill, dfa_status_string, dfa_stream_read, dfa_stream_read_sink_bytes,
                   dfa_version, kv_target, layer_weights, lib, dfa_decode_stack, dfa_decode_stack_workspace_size,
                   stack_layers)
