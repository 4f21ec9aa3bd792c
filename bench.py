#!/usr/bin/env python3
"""Dual-flow decode-attention benchmark on one MI355X.

One step = one dfa_decode_attn call over the whole batch: the attention
kernel (auxiliary query coupled in its prologue; both flows' scores, online
softmax and weighted values from one read of every cached key and value),
followed by the log-sum-exp combine when the library splits sequences. The
default workload is the largest attention workload that fits one GPU: batch
4, 32 query / 8 kv heads of 128, 131072 cached positions per sequence (2 GiB
of bf16 cache), 1% of the keys scaled by 8. The K timed steps run back to back
between two HIP events on the launch stream; `value` and `ms_per_step` come
from them. A second pass of K steps measures the attention kernel alone: each
launch carries start/stop events recorded from its own dispatch
(dfa_decode_attn_timed), and their mean is the kernel's average launch
duration used for `roofline.achieved`. Inputs are resident in HBM before
timing; when a cache is smaller than 1 GiB, copies of it are rotated between
steps so that no step finds it in the 256 MB last-level cache.

Prints one JSON line. `value` is tokens per second counting both flows (two
per sequence per step). Also reported: achieved HBM bandwidth of the step and
of the split kernel against the 8 TB/s peak, the HBM traffic per launch from
the committed counter summary of the workload (both flows and one flow), the
measured stream-read ceiling, the auxiliary flow's increment over a one-flow
run of the same kernel, the same figures for the two other attention
workloads (`other_workloads`: batch 16 x 4096 positions; batch 64 with ragged
lengths in a shuffled paged cache) and of a model with 16 query heads per kv
head (128/8 heads, batch 8 x 16384 positions: 32 query rows per kv head with
both flows), and the CPU oracle's rate on a bounded sample (context only).

    python bench.py [--steps K] [--warmup W] [--flows 1|2]
                    [--config c2|c3|c4|c5|gemv|head|moe|prefill|stack]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dual-flow decode attn: tokens/s (both flows) + achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["dual_flow_shared_decode_amd/csrc/" + f
                  for f in ("attn_bf16.hip", "attn_common.h", "dfa_internal.h", "launch.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_file(config_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"attn_bf16_{config_name}_counters.txt")


def measured_traffic(config_name: str, flows: int = 2):
    """HBM bytes per attention-kernel launch with `flows` flows from the committed counter summary
    of the workload, or None when there is none or the kernel sources changed since it was made."""
    path = counters_file(config_name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals[f"hbm_bytes_per_launch_{flows}flow"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(case, num_flows):
    """Bytes the method must move for one call: every cached key and value once, the
    queries (and a), the float32 outputs."""
    cfg = case.cfg
    esz = 2 if cfg.dtype == "bf16" else 4
    qsz = 2 if cfg.qtype == "bf16" else 4
    kv = int(case.ctx_lens.astype("int64").sum()) * cfg.num_kv_heads * cfg.head_dim * esz * 2
    rows = cfg.batch * cfg.num_q_heads * cfg.head_dim
    q = rows * qsz * num_flows + (cfg.num_q_heads * cfg.head_dim * 4 if num_flows == 2 else 0)
    out = rows * 4 * num_flows
    return kv + q + out


def cpu_baseline(case, budget_s: float):
    """The float64 oracle, as it stands, on (sequence, kv head) pairs of the same workload, taken in
    order (cycling) until the time budget is spent; the rate is scaled to tokens/s of both flows (a
    sequence is all of its kv heads)."""
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    cfg = case.cfg
    pairs = [(b, g) for b in range(cfg.batch) for g in range(cfg.num_kv_heads)]
    t0 = time.perf_counter()
    done = 0
    positions = 0
    while time.perf_counter() - t0 < budget_s:
        b, g = pairs[done % len(pairs)]
        A.decode_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache, case.block_table,
                           case.ctx_lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale,
                           block_size=case.block_size, num_flows=2, q_dtype=cfg.qtype, kv_dtype=cfg.dtype,
                           pairs=[(b, g)])
        done += 1
        positions += int(case.ctx_lens[b])
    dt = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    # a sequence-step is num_kv_heads pair evaluations of the sequence's length
    mean_len = float(case.ctx_lens.mean())
    seqs = positions / (mean_len * cfg.num_kv_heads)
    return {"value": 2.0 * seqs / dt, "unit": "tokens/s (both flows)", "cores": int(max(blas) if blas else 1),
            "kind": "oracle",
            "sample": f"{done} (sequence, kv head) evaluations ({positions} cached positions, both flows, all "
                      f"{cfg.num_q_heads // cfg.num_kv_heads} query heads of each kv head) of {cfg.name}, pairs "
                      f"taken in order from the first; float64 numpy oracle, {dt:.1f} s; rate = positions / "
                      f"(mean length x kv heads) sequence-steps per second, x2 flows",
            "host_cpus": len(os.sched_getaffinity(0))}


def layer_bytes(cfg):
    """Bytes one layer step must move: every weight once, the cache (ctx + 1 positions) once, the
    appended key/value, and the float32 activations in and out of each stage."""
    import workloads as W
    w = 2 * sum(a * b for a, b in W.weight_shapes(cfg).values())
    kv_read = cfg.batch * (cfg.ctx + 1) * cfg.num_kv_heads * cfg.head_dim * 2 * 2
    kv_write = cfg.batch * cfg.num_kv_heads * cfg.head_dim * 2 * 2
    qd = cfg.num_q_heads * cfg.head_dim
    act = 4 * cfg.batch * 2 * (cfg.hidden + qd + qd + qd + cfg.hidden + cfg.hidden + cfg.mlp + cfg.mlp + cfg.hidden)
    return w + kv_read + kv_write + act


def copy_calibration(args, rec):
    """For counter runs (--copy-calibration MIB): one plain device copy of that size after the timed
    work, so that the counters' readings of a known byte count give their scale."""
    if not args.copy_calibration:
        return
    import torch

    n = args.copy_calibration << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    rec["copy_calibration_bytes"] = n
    del src, dst


def bench_layer(args):
    """One dfa_decode_layer step of the full-layer workload (batch 32, hidden 4096, 32/8 heads of 128,
    SwiGLU MLP 14336, 4096 cached positions)."""
    import torch

    import dual_flow_shared_decode_amd as dfa
    import workloads as W
    from workloads.device import to_device

    cfg = W.C5
    log("generating c5 inputs")
    case = W.make_layer_case(cfg, W.SEEDS["c5"], pad_nan=False)
    packed = {}
    for name, w in case.w.items():
        dev = to_device(w)
        packed[name] = torch.empty_like(dev)
        dfa.dfa_pack_weight(dev, packed[name], w.shape[0], w.shape[1])
        del dev
    dev = {k: to_device(getattr(case, k)) for k in ("x1", "x2", "a", "b", "c", "k_cache", "v_cache", "block_table",
                                                    "ctx_lens")}
    desc = dfa.LayerDesc(batch=cfg.batch, hidden=cfg.hidden, num_q_heads=cfg.num_q_heads,
                         num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, mlp=cfg.mlp,
                         block_size=case.block_size, max_blocks_per_seq=case.max_blocks_per_seq,
                         num_blocks=case.k_cache.shape[0], max_ctx_len=cfg.ctx + 1, scale=cfg.scale,
                         x_exact_bf16=1)
    wts = dfa.layer_weights(packed["wq"], packed["wk"], packed["wv"], packed["wo"], packed["wg"], packed["wu"],
                            packed["wd"], dev["a"], dev["b"], dev["c"])
    ws = torch.empty(dfa.dfa_decode_layer_workspace_size(desc) // 4 + 64, dtype=torch.float32, device="cuda")
    out1 = torch.empty((cfg.batch, cfg.hidden), device="cuda")
    out2 = torch.empty_like(out1)
    stream = torch.cuda.current_stream()

    def step():  # the cache slot at ctx_lens is rewritten with the same values every step
        dfa.dfa_decode_layer(desc, wts, dev["x1"], dev["x2"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                             dev["ctx_lens"], out1, out2, ws, stream)
    # A step touches ~1 GB of weights and cache that nothing touched since upload; its first
    # passes run ~10% slower (measured: 241 us per step after 5 warm-up steps, 219 after 500),
    # so the layer warms up for at least 200 steps, as a serving loop would be.
    warmup = max(args.warmup, 200)
    for _ in range(warmup):
        step()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    nbytes = layer_bytes(cfg)
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"layer step {ms * 1e3:.1f} us, {nbytes / 1e6:.0f} MB -> {gbps:.0f} GB/s")
    rec = {"metric": "dual-flow decode layer step: tokens/s (both flows) + achieved HBM GB/s vs peak",
           "value": 2 * cfg.batch / (ms * 1e-3), "unit": "tokens/s (both flows)", "n_gpus": 1,
           "steps": args.steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "c5: one dual-flow decode layer step, batch 32, hidden 4096, 32/8 heads "
                                  "of 128, SwiGLU MLP 14336, 4096 cached positions",
                      "batch": cfg.batch},
           "achieved_gbps": gbps, "hbm_peak_gbps": HBM_PEAK_GBPS, "frac_of_peak": gbps / HBM_PEAK_GBPS,
           "algorithmic_bytes_per_step": nbytes}
    copy_calibration(args, rec)
    print(json.dumps(rec), flush=True)


GEMV_SHAPES = (  # the dense layer's weight streams at hidden 4096, 32/8 heads of 128, SwiGLU 14336
    ("qkv", 6144, 4096, "none", 1),            # [Wq; Wk; Wv], exact bf16 inputs (the layer's first GEMV)
    ("wo", 4096, 4096, "residual", 0),
    ("gate_up", 14336, 4096, "swiglu", 0),     # the SwiGLU pair: two 14336 x 4096 matrices
    ("down", 4096, 14336, "residual_coupled", 0),
)


def bench_gemv(args):
    """dfa_dual_gemv alone on the four weight streams of the layer workload (batch 32), one or two
    flows: each shape's launches (GEMV and, when split, its reduction) timed back to back, with
    enough copies of the weights rotated that the last-level cache never serves them. For HBM
    counter runs: the weights must be read once whatever the number of flows."""
    import torch

    import dual_flow_shared_decode_amd as dfa

    batch, flows = 32, args.flows
    epi = {"none": dfa.DFA_EPI_NONE, "residual": dfa.DFA_EPI_RESIDUAL, "swiglu": dfa.DFA_EPI_SWIGLU,
           "residual_coupled": dfa.DFA_EPI_RESIDUAL_COUPLED if flows == 2 else dfa.DFA_EPI_RESIDUAL}
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(2024)
    shapes, total_w, total_ms = {}, 0, 0.0
    for name, n, k, kind, exact in GEMV_SHAPES:
        mats = 2 if kind == "swiglu" else 1
        wbytes = mats * n * k * 2
        copies = max(1, -(-(768 << 20) // wbytes))
        log(f"gemv {name}: {n} x {k}{' x 2' if mats == 2 else ''}, {flows} flow(s), {copies} weight copies")
        ws_ = []
        for _ in range(copies):  # random bf16 weights (a layout change only: values do not matter here)
            pair = []
            for _ in range(mats):
                w = (torch.randn((n, k), device="cuda", generator=gen) * 0.02).to(torch.bfloat16).view(torch.int16)
                wt = torch.empty_like(w)
                dfa.dfa_pack_weight(w, wt, n, k, stream)
                pair.append(wt)
                del w
            ws_.append(pair)
        x = [torch.randn((batch, k), device="cuda", generator=gen) for _ in range(flows)]
        if exact:
            x = [t.to(torch.bfloat16).float() for t in x]
        res = [torch.randn((batch, n), device="cuda", generator=gen) for _ in range(flows)]
        couple = torch.randn(n, device="cuda", generator=gen) * 0.1 if flows == 2 and kind != "none" else None
        y = [torch.empty((batch, n), device="cuda") for _ in range(flows)]
        d = dfa.GemvDesc(batch=batch, n=n, k=k, num_flows=flows, epilogue=epi[kind], x_exact_bf16=exact, k_split=0,
                         rows_per_wg=0)
        wsb = dfa.dfa_dual_gemv_workspace_size(d)
        work = torch.empty(max(wsb // 4, 4), dtype=torch.float32, device="cuda") if wsb else None
        two = flows == 2
        use_res = kind in ("residual", "residual_coupled")

        def step(i):
            w = ws_[i % copies]
            dfa.dfa_dual_gemv(d, w[0], w[1] if mats == 2 else None, x[0], x[1] if two else None, couple,
                              res[0] if use_res else None, res[1] if (use_res and two) else None, y[0],
                              y[1] if two else None, None, work, stream)
        for i in range(max(args.warmup, 2 * copies)):
            step(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        act = 4 * batch * flows * (k + n * (1 + (1 if use_res else 0)))
        gbps = (wbytes + act) / (ms * 1e-3) / 1e9
        shapes[name] = {"n": n, "k": k, "matrices": mats, "epilogue": kind, "us": ms * 1e3, "weight_bytes": wbytes,
                        "algorithmic_bytes": wbytes + act, "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
                        "k_split": int(wsb > 0)}
        log(f"gemv {name}: {ms * 1e3:.1f} us per launch, {gbps:.0f} GB/s")
        total_w += wbytes + act
        total_ms += ms
        del ws_, x, res, y, work
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    gbps = total_w / (total_ms * 1e-3) / 1e9
    rec = {"metric": "dual GEMV on the layer's weight streams: achieved HBM GB/s vs peak", "value": gbps,
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": total_ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"dual GEMV, batch 32, {flows} flow(s): [Wq; Wk; Wv] 6144 x 4096, Wo 4096 x 4096, "
                                  "SwiGLU pair 2 x 14336 x 4096, down 4096 x 14336", "batch": batch,
                      "num_flows": flows},
           "frac_of_peak": gbps / HBM_PEAK_GBPS, "shapes": shapes}
    copy_calibration(args, rec)
    print(json.dumps(rec), flush=True)


def bench_head(args):
    """One output-head step of the head workload (batch 32, hidden 4096, vocabulary 32000): both flows'
    logits from one read of the shared vocabulary matrix, then the mixture of their distributions and a
    sampled and a greedy token per sequence, as one dfa_output_head call. The same kernels called
    separately (dfa_dual_gemv, then dfa_mixture_sample) are timed too."""
    import numpy as np
    import torch

    import dual_flow_shared_decode_amd as dfa
    import workloads as W
    from workloads.device import to_device

    cfg = W.HEAD
    log("generating head inputs")
    h1, h2, w_bits, u = W.make_head_case(cfg, W.SEEDS["head"])
    dev = to_device(w_bits)
    # two copies of the 262 MB matrix, alternated between steps: no step finds it in the last-level cache
    wts = [torch.empty_like(dev) for _ in range(2)]
    for wt in wts:
        dfa.dfa_pack_weight(dev, wt, cfg.vocab, cfg.hidden)
    del dev
    x1, x2, tu = to_device(h1), to_device(h2), to_device(u)
    gd = dfa.GemvDesc(batch=cfg.batch, n=cfg.vocab, k=cfg.hidden, num_flows=2, epilogue=dfa.DFA_EPI_NONE,
                      x_exact_bf16=1, k_split=0, rows_per_wg=0)
    gws = torch.empty(max(dfa.dfa_dual_gemv_workspace_size(gd) // 4, 4), device="cuda")
    md = dfa.MixtureDesc(batch=cfg.batch, vocab=cfg.vocab)
    mws = torch.empty(dfa.dfa_mixture_workspace_size(md) // 4, device="cuda")
    y1 = torch.empty((cfg.batch, cfg.vocab), device="cuda")
    y2 = torch.empty_like(y1)
    tok = torch.empty(cfg.batch, dtype=torch.int32, device="cuda")
    gr = torch.empty_like(tok)
    al = torch.empty(cfg.batch, device="cuda")
    hd = dfa.HeadDesc(batch=cfg.batch, vocab=cfg.vocab, hidden=cfg.hidden, x_exact_bf16=1)
    hws = torch.empty(dfa.dfa_output_head_workspace_size(hd) // 4, device="cuda")
    stream = torch.cuda.current_stream()

    def mix():
        dfa.dfa_mixture_sample(md, y1, y2, tu, tok, gr, al, None, mws, stream)

    def step_two(i):
        dfa.dfa_dual_gemv(gd, wts[i % 2], None, x1, x2, None, None, None, y1, y2, None, gws, stream)
        mix()

    def step(i):
        dfa.dfa_output_head(hd, wts[i % 2], x1, x2, tu, y1, y2, tok, gr, al, None, hws, stream)

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    warmup = max(args.warmup, 100)
    two_ms = timed(step_two, args.steps, warmup)
    ms = timed(step, args.steps, warmup)
    mix_ms = timed(lambda i: mix(), args.steps, 10)
    w_bytes = 2 * cfg.vocab * cfg.hidden
    logits = 4 * cfg.batch * cfg.vocab
    # the weight once, both flows' hidden states in, both flows' logits out and back in, the tokens out
    nbytes = w_bytes + 2 * 4 * cfg.batch * cfg.hidden + 2 * logits + 2 * logits + 12 * cfg.batch
    gbps = nbytes / (ms * 1e-3) / 1e9
    mix_bytes = 2 * logits + 2 * 4 * cfg.batch  # the mixture's own minimum: both logit rows once
    log(f"head step {ms * 1e3:.1f} us ({nbytes / 1e6:.0f} MB -> {gbps:.0f} GB/s); two calls {two_ms * 1e3:.1f} us; "
        f"mixture alone {mix_ms * 1e3:.1f} us")
    print(json.dumps({"metric": "dual-flow output head + mixture sampling: tokens/s + achieved HBM GB/s vs peak",
                      "value": cfg.batch / (ms * 1e-3), "unit": "sampled tokens/s", "n_gpus": 1,
                      "steps": args.steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "head: both flows' logits over a 32000-token vocabulary from hidden "
                                             "4096 (shared bf16 matrix), mixture, sampled and greedy tokens, "
                                             "batch 32", "batch": cfg.batch, "vocab": cfg.vocab},
                      "achieved_gbps": gbps, "hbm_peak_gbps": HBM_PEAK_GBPS, "frac_of_peak": gbps / HBM_PEAK_GBPS,
                      "algorithmic_bytes_per_step": nbytes, "two_call_us": two_ms * 1e3, "mixture_us": mix_ms * 1e3,
                      "mixture_gbps": mix_bytes / (mix_ms * 1e-3) / 1e9}), flush=True)


def bench_moe(args):
    """One mixture-of-experts FFN step with router replay (batch 32, hidden 4096, 64 experts of width
    1024, primary fan-out 4, auxiliary fan-out 8): both flows' router logits from one read of the
    shared router (dfa_dual_gemv), the selection and mixing weights (dfa_moe_route), and the experts
    (dfa_moe_ffn: grouped gate/up and down GEMVs, each selected expert read once for both flows, and
    the weighted combination)."""
    import numpy as np
    import torch

    import dual_flow_shared_decode_amd as dfa
    import workloads as W
    from workloads.device import to_device

    cfg = W.MOE
    log("generating moe inputs")
    case = W.make_moe_case(cfg, W.SEEDS["moe"])

    def pack(bits):
        ne, n, k = bits.shape
        src = to_device(bits)
        dst = torch.empty_like(src)
        for e in range(ne):
            dfa.dfa_pack_weight(src[e], dst[e], n, k)
        return dst
    wg, wu, wd = pack(case.wg), pack(case.wu), pack(case.wd)
    wr = pack(case.wr[None])[0]
    h1, h2, res1, res2 = (to_device(x) for x in (case.h1, case.h2, case.res1, case.res2))
    bvec, cvec = to_device(case.b), to_device(case.c)
    rd = dfa.GemvDesc(batch=cfg.batch, n=cfg.experts, k=cfg.hidden, num_flows=2, epilogue=dfa.DFA_EPI_NONE,
                      x_exact_bf16=1, k_split=0, rows_per_wg=0)
    rws = torch.empty(max(dfa.dfa_dual_gemv_workspace_size(rd) // 4, 4), device="cuda")
    r1 = torch.empty((cfg.batch, cfg.experts), device="cuda")
    r2 = torch.empty_like(r1)
    out1 = torch.empty((cfg.batch, cfg.hidden), device="cuda")
    out2 = torch.empty_like(out1)
    stream = torch.cuda.current_stream()

    def make(k2):
        d = dfa.MoeDesc(batch=cfg.batch, hidden=cfg.hidden, mlp=cfg.mlp, num_experts=cfg.experts, k1=cfg.k1, k2=k2,
                        x_exact_bf16=1)
        routing = torch.empty(dfa.dfa_moe_routing_size(d) // 4, dtype=torch.int32, device="cuda")
        ws = torch.empty(dfa.dfa_moe_workspace_size(d) // 4, device="cuda")

        def step():
            dfa.dfa_dual_gemv(rd, wr, None, h1, h2, None, None, None, r1, r2, None, rws, stream)
            dfa.dfa_moe_route(d, r1, r2, routing, stream)
            dfa.dfa_moe_ffn(d, wg, wu, wd, bvec, cvec, h1, h2, res1, res2, routing, out1, out2, ws, stream)
        return d, routing, step

    def timed(step, steps, warmup):
        for _ in range(warmup):
            step()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    def distinct(d, routing, k):  # experts the step reads: the union of the first k of every row
        sel = routing.cpu().numpy()[:cfg.batch * d.k2].reshape(cfg.batch, d.k2)
        return len(np.unique(sel[:, :k]))

    warmup = max(args.warmup, 20)
    d, routing, step = make(cfg.k2)
    ms = timed(step, args.steps, warmup)
    used = distinct(d, routing, cfg.k2)
    used_primary = distinct(d, routing, cfg.k1)
    d_eq, routing_eq, step_eq = make(cfg.k1)
    ms_eq = timed(step_eq, args.steps, warmup)
    expert_bytes = 3 * cfg.hidden * cfg.mlp * 2
    act = 4 * cfg.batch * cfg.hidden * 2 * 3  # h in (router and experts' first read), res in, out
    inter = 4 * cfg.batch * cfg.k2 * 2 * (cfg.mlp + cfg.hidden) * 2  # intermediates and expert outputs, out and in
    nbytes = used * expert_bytes + 2 * cfg.experts * cfg.hidden + act + inter
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"moe step {ms * 1e3:.1f} us: {used} of {cfg.experts} experts read ({used_primary} for the primary's "
        f"fan-out alone), {nbytes / 1e6:.0f} MB -> {gbps:.0f} GB/s; with k2 = k1 = {cfg.k1}: {ms_eq * 1e3:.1f} us")
    print(json.dumps({"metric": "dual-flow MoE FFN step (router replay): tokens/s (both flows) + achieved HBM GB/s",
                      "value": 2 * cfg.batch / (ms * 1e-3), "unit": "tokens/s (both flows)", "n_gpus": 1,
                      "steps": args.steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "moe: SwiGLU mixture-of-experts FFN with router replay, batch 32, "
                                             "hidden 4096, 64 experts of width 1024, primary fan-out 4, auxiliary "
                                             "fan-out 8", "batch": cfg.batch, "experts": cfg.experts,
                                 "k1": cfg.k1, "k2": cfg.k2},
                      "achieved_gbps": gbps, "hbm_peak_gbps": HBM_PEAK_GBPS, "frac_of_peak": gbps / HBM_PEAK_GBPS,
                      "algorithmic_bytes_per_step": nbytes, "experts_read": used,
                      "experts_read_primary_fanout": used_primary,
                      "ms_per_step_aux_fanout_equal_to_primary": ms_eq,
                      "aux_fanout_increment": ms / ms_eq - 1.0}), flush=True)


def bench_prefill(args):
    """Primary-only prefill of 4 prompts of 4096 tokens (32/8 heads of 128): the prompts' keys and values
    written to the paged cache and causal self-attention (dfa_prefill), then the auxiliary flow's first
    step at the last prompt position (dfa_decode_attn over the 4096 cached positions, both flows)."""
    import numpy as np
    import torch

    import dual_flow_shared_decode_amd as dfa
    import workloads as W
    from workloads.device import to_device

    cfg = W.PREFILL
    log("generating prefill inputs")
    case = W.make_prefill_case(cfg, W.SEEDS["prefill"])
    t = {name: to_device(getattr(case, name)) for name in ("q", "k", "v", "lens", "k_cache", "v_cache",
                                                            "block_table")}
    lmax = case.q.shape[1]
    o = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    pd = dfa.PrefillDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                         head_dim=cfg.head_dim, max_prompt_len=lmax, block_size=case.block_size,
                         max_blocks_per_seq=case.max_blocks_per_seq, num_blocks=case.k_cache.shape[0],
                         scale=cfg.scale)
    stream = torch.cuda.current_stream()
    last = to_device(np.stack([case.q[b, int(case.lens[b]) - 1] for b in range(cfg.batch)]))
    ad = dfa.AttnDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                      head_dim=cfg.head_dim, block_size=case.block_size, max_blocks_per_seq=case.max_blocks_per_seq,
                      num_blocks=case.k_cache.shape[0], max_ctx_len=int(case.lens.max()), num_flows=2, split_len=0,
                      scale=cfg.scale, q_dtype=dfa.DFA_BF16, kv_dtype=dfa.DFA_BF16)
    aws = torch.empty(max(dfa.dfa_decode_attn_workspace_size(ad) // 4, 4), device="cuda")
    o1 = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), device="cuda")
    o2 = torch.empty_like(o1)
    q2, a = to_device(case.q2), to_device(case.a)

    def prefill():
        dfa.dfa_prefill(pd, t["q"], t["k"], t["v"], t["lens"], t["k_cache"], t["v_cache"], t["block_table"], o, stream)

    def aux_step():
        dfa.dfa_decode_attn(ad, last, q2, a, t["k_cache"], t["v_cache"], t["block_table"], t["lens"], aws, o1, o2,
                            stream)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    warmup = max(args.warmup, 5)
    ms = timed(prefill, args.steps, warmup)
    aux_ms = timed(aux_step, args.steps, warmup)
    pairs = sum(int(n) * (int(n) + 1) // 2 for n in case.lens)  # (query, key) pairs per head
    flops = 4.0 * cfg.head_dim * cfg.num_q_heads * pairs  # scores and weighted values, 2 flops per product
    tflops = flops / (ms * 1e-3) / 1e12
    tokens = int(case.lens.sum())
    log(f"prefill {ms * 1e3:.1f} us for {tokens} prompt tokens: {tflops:.0f} TFLOP/s of causal attention "
        f"({100 * tflops / 2500:.0f}% of the 2.5 PFLOP/s bf16 peak); the auxiliary flow's first step over the "
        f"cache: {aux_ms * 1e3:.1f} us")
    print(json.dumps({"metric": "primary-only prefill (causal attention + cache write): prompt tokens/s + TFLOP/s",
                      "value": tokens / (ms * 1e-3), "unit": "prompt tokens/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
                      "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "prefill: 4 prompts of 4096 tokens, 32/8 heads of 128, causal, "
                                             "16-position paged cache", "batch": cfg.batch, "prompt_len": lmax},
                      "attention_tflops": tflops, "mfma_peak_tflops": 2500.0, "frac_of_peak": tflops / 2500.0,
                      "flops_per_step": flops, "aux_first_step_us": aux_ms * 1e3}), flush=True)


def bench_stack(args):
    """One token through 4 dual-flow layers of the c5 shape (batch 32, hidden 4096, 32/8 heads of 128, SwiGLU
    14336, 4096 cached positions) with RMSNorm and rotate-half rotary embeddings (dfa_decode_stack), launched
    eagerly and replayed from a HIP graph that holds the whole step. The layers hold equal values in
    separate buffers (one layer's draw copied): every layer reads its own 436 MB of weights and its own
    cache, as a deeper model would."""
    import torch

    import dual_flow_shared_decode_amd as dfa
    import workloads as W
    from workloads.device import to_device

    cfg = W.STACK
    lc = cfg.layer
    log(f"generating stack inputs ({cfg.layers} layers)")
    sc = W.make_stack_case(cfg.replace(layers=1), W.SEEDS["stack"], pad_nan=False)
    w0 = sc.layers[0]
    packed = {}
    for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        dev = to_device(w0[name])
        packed[name] = torch.empty_like(dev)
        dfa.dfa_pack_weight(dev, packed[name], w0[name].shape[0], w0[name].shape[1])
        del dev
    vecs = {name: to_device(w0[name].astype("float32")) for name in ("a", "b", "c", "n_attn", "n_mlp")}
    k0, v0 = to_device(sc.k_caches[0]), to_device(sc.v_caches[0])
    entries = []
    for li in range(cfg.layers):
        p = packed if li == 0 else {k: t.clone() for k, t in packed.items()}
        vv = vecs if li == 0 else {k: t.clone() for k, t in vecs.items()}
        lw = dfa.layer_weights(p["wq"], p["wk"], p["wv"], p["wo"], p["wg"], p["wu"], p["wd"], vv["a"], vv["b"], vv["c"])
        entries.append((lw, vv["n_attn"], vv["n_mlp"], k0.clone(), v0.clone()))
    del k0, v0
    layers = dfa.stack_layers(entries)
    desc = dfa.StackDesc(layer=dfa.LayerDesc(batch=lc.batch, hidden=lc.hidden, num_q_heads=lc.num_q_heads,
                                             num_kv_heads=lc.num_kv_heads, head_dim=lc.head_dim, mlp=lc.mlp,
                                             block_size=sc.block_size, max_blocks_per_seq=sc.max_blocks_per_seq,
                                             num_blocks=sc.k_caches[0].shape[0], max_ctx_len=lc.ctx + 1,
                                             scale=lc.scale, x_exact_bf16=1),
                         num_layers=cfg.layers, rope=dfa.DFA_ROPE_HALF, rope_max_pos=sc.cos.shape[0], rms_norm=1,
                         rms_eps=cfg.eps)
    cos, sin = to_device(sc.cos), to_device(sc.sin)
    x1, x2 = to_device(sc.x1), to_device(sc.x2)
    table, ctx = to_device(sc.block_table), to_device(sc.ctx_lens)
    ws = torch.empty(dfa.dfa_decode_stack_workspace_size(desc) // 4 + 64, device="cuda")
    out1 = torch.empty_like(x1)
    out2 = torch.empty_like(x2)

    def step():  # every step appends at the same position (the same values each time)
        dfa.dfa_decode_stack(desc, layers, cos, sin, x1, x2, table, ctx, out1, out2, ws)

    def timed(fn, steps):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    warmup = max(args.warmup, 50)
    for _ in range(warmup):
        step()
    ms = timed(step, args.steps)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(10):
        graph.replay()
    ms_graph = timed(graph.replay, args.steps)
    nbytes = cfg.layers * layer_bytes(lc)
    gbps = nbytes / (ms_graph * 1e-3) / 1e9
    log(f"stack of {cfg.layers} layers: {ms * 1e3:.1f} us per token eager, {ms_graph * 1e3:.1f} us replayed from a "
        f"graph ({ms_graph * 1e3 / cfg.layers:.1f} us per layer, {gbps:.0f} GB/s over {nbytes / 1e6:.0f} MB)")
    print(json.dumps({"metric": "dual-flow decode step through a layer stack: tokens/s (both flows) + HBM GB/s",
                      "value": 2 * lc.batch / (ms_graph * 1e-3), "unit": "tokens/s (both flows)", "n_gpus": 1,
                      "steps": args.steps, "warmup": warmup, "ms_per_step": ms_graph, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": f"stack: {cfg.layers} dual-flow layers of the c5 shape with RMSNorm and "
                                             "rotate-half rotary embeddings, batch 32, one token, HIP graph",
                                 "batch": lc.batch, "layers": cfg.layers},
                      "ms_per_step_eager": ms, "achieved_gbps": gbps, "hbm_peak_gbps": HBM_PEAK_GBPS,
                      "frac_of_peak": gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_step": nbytes}), flush=True)


def attn_measure(name, args, flows=2, one_flow=True, log_prefix=""):
    """Times dfa_decode_attn on attention workload `name`: K steps back to back between two HIP
    events, then K launches with per-dispatch events for the attention kernel alone, optionally the
    same with one flow. Returns the case and the figures."""
    import torch

    import dual_flow_shared_decode_amd as dfa
    import workloads as W
    from workloads.device import upload_attn_case

    cfg = W.ATTN_CONFIGS[name]
    log(f"{log_prefix}generating {cfg.name} inputs")
    case = W.make_attn_case(cfg, W.SEEDS[cfg.name], pad_nan=False)
    t = upload_attn_case(case)
    kv_set_bytes = (case.k_cache.nbytes + case.v_cache.nbytes)
    nsets = max(1, min(4, math.ceil((1 << 30) / kv_set_bytes)))
    sets = [(t["k_cache"], t["v_cache"])] + [(t["k_cache"].clone(), t["v_cache"].clone()) for _ in range(nsets - 1)]
    log(f"{log_prefix}{nsets} cache copies of {kv_set_bytes / 2**20:.0f} MiB rotated between steps")

    def make_desc(nf):
        return dfa.AttnDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                            head_dim=cfg.head_dim, block_size=case.block_size,
                            max_blocks_per_seq=case.max_blocks_per_seq, num_blocks=case.k_cache.shape[0],
                            max_ctx_len=case.max_ctx_len, num_flows=nf, split_len=args.split,
                            scale=cfg.scale, q_dtype=dfa.DFA_BF16, kv_dtype=dfa.DFA_BF16)

    stream = torch.cuda.current_stream()
    o1 = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)

    def runner(nf):
        d = make_desc(nf)
        ws = torch.zeros(max(dfa.dfa_decode_attn_workspace_size(d) // 4, 4), dtype=torch.float32, device="cuda")
        q2 = t["q2"] if nf == 2 else None
        a = t["a"] if nf == 2 else None
        out2 = o2 if nf == 2 else None

        def step(i, ev=None):
            k, v = sets[i % nsets]
            dfa.dfa_decode_attn_timed(d, t["q1"], q2, a, k, v, t["block_table"], t["ctx_lens"], ws, o1, out2,
                                      stream, *(ev or (None, None)))
        return d, step

    def timed(step, steps, warmup):
        for i in range(warmup):
            step(i)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for i in range(steps):
            step(warmup + i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        return start.elapsed_time(end) / steps, wall

    def kernel_ms(step, steps):
        """Durations (ms) of the attention kernel, from events recorded by each launch's dispatch."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in evs:  # the events must exist before a dispatch can record them
            e0.record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        for i, ev in enumerate(evs):
            step(i, ev)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    d_main, step_main = runner(flows)
    log(f"{log_prefix}{flows} flow(s), split length {dfa.dfa_decode_attn_split_len(d_main)}, "
        f"{dfa.dfa_decode_attn_num_splits(d_main)} splits; timing")
    ms, wall = timed(step_main, args.steps, args.warmup)
    kern_all = sorted(kernel_ms(step_main, args.steps))
    m = {"case": case, "cfg": cfg, "flows": flows, "ms": ms, "wall": wall, "kern_all": kern_all,
         "kern_ms": sum(kern_all) / len(kern_all), "split_len": dfa.dfa_decode_attn_split_len(d_main),
         "num_splits": dfa.dfa_decode_attn_num_splits(d_main), "nsets": nsets,
         "bytes": algorithmic_bytes(case, flows)}
    log(f"{log_prefix}{cfg.name}: {ms * 1e3:.1f} us/step ({wall:.3f} s wall for {args.steps} steps); attention "
        f"kernel {m['kern_ms'] * 1e3:.1f} us per launch; {m['bytes'] / (m['kern_ms'] * 1e-3) / 1e9:.0f} GB/s kernel")
    if one_flow and flows == 2:
        d1, step1 = runner(1)
        ms1, _ = timed(step1, args.steps, args.warmup)
        kern1 = sum(kernel_ms(step1, args.steps)) / args.steps
        m["ms_one_flow"] = ms1
        m["kern_ms_one_flow"] = kern1
        log(f"{log_prefix}one flow: {ms1 * 1e3:.1f} us/step, kernel {kern1 * 1e3:.1f} us -> aux increment "
            f"{100 * (ms / ms1 - 1):.1f}% (step), {100 * (m['kern_ms'] / kern1 - 1):.1f}% (kernel)")
    del sets, t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return m


def kernel_name_of(cfg, flows):
    rows = cfg.num_q_heads // cfg.num_kv_heads * flows
    if cfg.dtype != "bf16":
        return f"attn_f32_kernel<{cfg.head_dim}>"
    return (f"attn_bf16_kernel<{cfg.head_dim}, {8 if rows <= 8 else 16}, false, 1>" if rows <= 16
            else f"attn_bf16_kernel<{cfg.head_dim}, 16, false, 2>")


def summary_of(m):
    """The figures of one attention workload, as extra keys of the bench line."""
    kb = m["bytes"] / (m["kern_ms"] * 1e-3) / 1e9
    sb = m["bytes"] / (m["ms"] * 1e-3) / 1e9
    out = {"workload": m["cfg"].name, "ms_per_step": m["ms"], "kernel_avg_us": m["kern_ms"] * 1e3,
           "kernel": kernel_name_of(m["cfg"], m["flows"]), "algorithmic_bytes_per_launch": m["bytes"],
           "kernel_gbps": kb, "frac": kb / HBM_PEAK_GBPS, "step_gbps": sb, "step_frac": sb / HBM_PEAK_GBPS,
           "split_len": m["split_len"], "num_splits": m["num_splits"],
           "tokens_per_s_both_flows": 2 * m["cfg"].batch / (m["ms"] * 1e-3),
           "traffic": measured_traffic(m["cfg"].name, m["flows"])}
    if "ms_one_flow" in m:
        out["ms_per_step_one_flow"] = m["ms_one_flow"]
        out["aux_increment"] = m["ms"] / m["ms_one_flow"] - 1.0
        out["aux_increment_kernel"] = m["kern_ms"] / m["kern_ms_one_flow"] - 1.0
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4",
                    choices=["c2", "c3", "c4", "g16", "c5", "gemv", "head", "moe", "prefill", "stack"],
                    help="c4 (default): the largest attention workload, the headline; c2, c3: the other attention "
                         "workloads alone; g16: attention with 16 query heads per kv head (128/8 heads, 32 rows per kv head "
                         "with both flows), batch 8 x 16384 positions; c5: a whole layer step; gemv: the dual GEMV on the layer's four weight "
                         "streams; head: the dual output head and mixture sampling; "
                         "moe: the MoE FFN with router replay; prefill: the primary-only prefill and the first "
                         "auxiliary step; stack: 4 layers with RMSNorm and rotary embeddings in a HIP graph")
    ap.add_argument("--flows", type=int, default=2, choices=[1, 2],
                    help="flows of the timed attention (or gemv) steps (1: the single-flow run of the same "
                         "kernels, for counter comparisons)")
    ap.add_argument("--split", type=int, default=0, help="positions per split (0: library choice)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time the steps only (for profiler runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, copy a MIB-MiB buffer once (a known-size reference for HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); this "
              "library runs on a single GPU and sharding across GPUs is not part of it", file=sys.stderr)
        sys.exit(2)

    import torch

    import dual_flow_shared_decode_amd as dfa

    torch.cuda.set_device(0)
    other = {"c5": bench_layer, "gemv": bench_gemv, "head": bench_head, "moe": bench_moe, "prefill": bench_prefill,
             "stack": bench_stack}
    if args.config in other:
        other[args.config](args)
        return
    stream = torch.cuda.current_stream()
    m = attn_measure(args.config, args, flows=args.flows, one_flow=not args.no_extras)
    case, cfg = m["case"], m["cfg"]
    ms, kern_all, kern_ms = m["ms"], m["kern_all"], m["kern_ms"]

    def pct(v, q):  # nearest-rank percentile of a sorted list
        return v[min(len(v) - 1, max(0, int(math.ceil(q / 100 * len(v))) - 1))]
    step_bytes = kern_bytes = m["bytes"]
    step_gbps = step_bytes / (ms * 1e-3) / 1e9
    kern_gbps = kern_bytes / (kern_ms * 1e-3) / 1e9
    flow_tokens = args.flows * cfg.batch / (ms * 1e-3)
    rec = {"metric": METRIC, "value": flow_tokens,
           "unit": "tokens/s (both flows)" if args.flows == 2 else "tokens/s (one flow)", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{cfg.name}: dual-flow decode attention, batch {cfg.batch}, "
                                  f"{cfg.num_q_heads} query / {cfg.num_kv_heads} kv heads, head_dim {cfg.head_dim}, "
                                  f"context {int(case.ctx_lens.min())}-{int(case.ctx_lens.max())}, bf16 cache, "
                                  f"{'paged ' + str(case.block_size) if cfg.block_size else 'contiguous'}"
                                  f"{', 1% of keys x8' if cfg.name == 'c4' else ''}",
                      "batch": cfg.batch, "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                      "head_dim": cfg.head_dim, "ctx_total": int(case.ctx_lens.sum()), "num_flows": args.flows,
                      "split_len": m["split_len"], "num_splits": m["num_splits"], "cache_copies": m["nsets"]},
           "accumulate": "f32",
           "seq_tokens_per_s": cfg.batch / (ms * 1e-3),
           "achieved_gbps": step_gbps, "hbm_peak_gbps": HBM_PEAK_GBPS, "frac_of_peak": step_gbps / HBM_PEAK_GBPS,
           "algorithmic_bytes_per_step": step_bytes,
           "roofline": {"bound": "hbm", "kernel": kernel_name_of(cfg, args.flows), "achieved": kern_gbps,
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": kern_gbps / HBM_PEAK_GBPS,
                        "traffic": measured_traffic(cfg.name, args.flows), "algorithmic_bytes_per_launch": kern_bytes,
                        "avg_launch_us": kern_ms * 1e3, "median_launch_us": pct(kern_all, 50) * 1e3,
                        "p10_launch_us": pct(kern_all, 10) * 1e3, "p90_launch_us": pct(kern_all, 90) * 1e3}}
    if rec["roofline"]["traffic"]:
        rec["roofline"]["traffic_over_algorithmic"] = rec["roofline"]["traffic"] / kern_bytes
    t2, t1 = measured_traffic(cfg.name, 2), measured_traffic(cfg.name, 1)
    if t2 and t1:
        rec["traffic_two_flows_over_one_flow"] = t2 / t1

    copy_calibration(args, rec)
    if not args.no_extras:
        if "ms_one_flow" in m:
            rec["ms_per_step_one_flow"] = m["ms_one_flow"]
            rec["aux_increment"] = ms / m["ms_one_flow"] - 1.0
            rec["aux_increment_kernel"] = kern_ms / m["kern_ms_one_flow"] - 1.0
        buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
        sink = torch.empty(dfa.dfa_stream_read_sink_bytes() // 4, dtype=torch.int32, device="cuda")
        for _ in range(3):
            dfa.dfa_stream_read(buf, sink, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dfa.dfa_stream_read(buf, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ceil_gbps = buf.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        rec["stream_read_gbps"] = ceil_gbps
        rec["frac_of_stream_read"] = kern_gbps / ceil_gbps
        del buf
        log(f"stream-read ceiling {ceil_gbps:.0f} GB/s")
        # the other attention workloads, timed the same way
        rec["other_workloads"] = {}
        for name in ("c2", "c3", "c4", "g16"):
            if name == cfg.name:
                continue
            rec["other_workloads"][name] = summary_of(attn_measure(name, args, flows=2, one_flow=True,
                                                                   log_prefix="  "))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        rec["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
