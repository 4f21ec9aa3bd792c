"""Writes the oracle regression fixtures in this folder.

Calls only the seeded input generators and the CPU oracle. Re-run it only
when a change to the oracle's arithmetic is justified by the method's source
pages, and say which passage in the commit that changes the fixture.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W  # noqa: E402
from oracle import attention as A  # noqa: E402
from oracle import layer as LY  # noqa: E402

ATTN = W.AttnConfig("golden_attn", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="bf16",
                    ctx_lens=(3, 21), block_size=16, shuffle_blocks=True)
LAYER = W.C5.replace(batch=1, hidden=8, num_q_heads=2, num_kv_heads=1, head_dim=8, mlp=12, ctx=3,
                     capacity=16)
SEED = 7


def build():
    case = W.make_attn_case(ATTN, SEED)
    att = A.decode_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache, case.block_table,
                             case.ctx_lens, num_kv_heads=ATTN.num_kv_heads, scale=ATTN.scale,
                             block_size=case.block_size, num_flows=2)
    lc = W.make_layer_case(LAYER, SEED)
    lay = LY.dual_flow_layer(lc.x1, lc.x2, lc.w, lc.a, lc.b, lc.c, lc.k_cache, lc.v_cache, lc.block_table,
                             lc.ctx_lens, num_q_heads=LAYER.num_q_heads, num_kv_heads=LAYER.num_kv_heads,
                             head_dim=LAYER.head_dim, scale=LAYER.scale, block_size=lc.block_size)
    return {
        "attention": {"config": ATTN.name, "seed": SEED, "o1": att["o1"].tolist(), "o2": att["o2"].tolist()},
        "layer": {"config": "c5 at hidden 8, heads 2/1, head_dim 8, mlp 12, ctx 3", "seed": SEED,
                  "out1": lay["out1"].tolist(), "out2": lay["out2"].tolist(),
                  "k1_bits": lay["k1_bits"].astype(int).tolist(), "v1_bits": lay["v1_bits"].astype(int).tolist()},
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(build(), f, indent=1)
