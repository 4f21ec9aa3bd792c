"""Shared helpers of the GPU tests: run libdfa on a workload, compare with the oracle."""
import sys

import numpy as np
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from oracle import attention as A
from workloads.device import upload_attn_case

# Tolerance on the row-normalised max relative error: for every output row
# (b, h, f), max_d |gpu - oracle| / max_d |oracle|. The kernels accumulate in
# float32 and split every non-bf16 MFMA operand into two bf16 terms, which
# keeps about 16 significant bits per product; observed errors are ~1e-5.
TOL = 2e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def desc_for(case, num_flows=2, split_len=0, max_ctx_len=None, q_dtype=None):
    cfg = case.cfg
    dt = {"bf16": dfa.DFA_BF16, "f32": dfa.DFA_F32}
    return dfa.AttnDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                        head_dim=cfg.head_dim, block_size=case.block_size,
                        max_blocks_per_seq=case.max_blocks_per_seq, num_blocks=case.k_cache.shape[0],
                        max_ctx_len=max_ctx_len or case.max_ctx_len, num_flows=num_flows,
                        split_len=split_len, scale=cfg.scale, q_dtype=dt[q_dtype or cfg.qtype],
                        kv_dtype=dt[cfg.dtype])


def run_attn(case, num_flows=2, split_len=0, tensors=None, desc=None):
    """GPU outputs (o1, o2 as float32 numpy; o2 None for one flow)."""
    t = tensors or upload_attn_case(case)
    d = desc or desc_for(case, num_flows, split_len)
    ws_bytes = dfa.dfa_decode_attn_workspace_size(d)
    ws = torch.zeros(max(ws_bytes // 4, 4), dtype=torch.float32, device="cuda")
    B, H, D = case.cfg.batch, case.cfg.num_q_heads, case.cfg.head_dim
    o1 = torch.full((B, H, D), float("nan"), device="cuda")
    o2 = torch.full((B, H, D), float("nan"), device="cuda") if num_flows == 2 else None
    dfa.dfa_decode_attn(d, t["q1"], t["q2"] if num_flows == 2 else None, t["a"] if num_flows == 2 else None,
                        t["k_cache"], t["v_cache"], t["block_table"], t["ctx_lens"], ws, o1, o2)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), (o2.cpu().numpy() if o2 is not None else None)


def oracle_attn(case, num_flows=2, pairs=None):
    cfg = case.cfg
    return A.decode_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache, case.block_table,
                              case.ctx_lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale,
                              block_size=case.block_size, num_flows=num_flows, q_dtype=cfg.qtype,
                              kv_dtype=cfg.dtype, pairs=pairs)


def row_rel_err(got, ref):
    """max over rows of max_d |got - ref| / max_d |ref| (rows = all but the last axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float(np.max(num / den))


def assert_close(got, ref, tol=TOL, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = row_rel_err(got, ref)
    say(f"  {what}: row-normalised max rel err {err:.3e}")
    assert err <= tol, f"{what}: {err:.3e} > {tol}"
    return err
