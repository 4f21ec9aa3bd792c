"""Scalar brute force for tiny inputs -- test infrastructure only.

Pure-Python loops over every index, ``math.exp`` and ``math.fsum``; no numpy
arithmetic. It is written independently of ``attention`` and ``layer`` (its
own bf16 decoding through ``struct``, its own cache indexing and head mapping,
its own rounding) so that the vectorised oracle can be checked against it.
It follows the same definitions and sources as those modules.
"""
import math
import struct


def _bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _val(x, dtype) -> float:
    return _bf16(x) if dtype == "bf16" else float(x)


def _dot(u, v) -> float:
    return math.fsum(ui * vi for ui, vi in zip(u, v))


def _softmax_avg(q, keys, values, scale):
    """sum_t softmax_t(scale * q.k_t) v_t, one scalar at a time."""
    s = [scale * _dot(q, k) for k in keys]
    top = max(s)
    e = [math.exp(si - top) for si in s]
    tot = math.fsum(e)
    d = len(values[0])
    return [math.fsum(e[t] * values[t][j] for t in range(len(values))) / tot for j in range(d)]


def _kv_rows(k_cache, v_cache, table_row, length, g, block, kv_dtype):
    keys, values = [], []
    d = v_cache.shape[3]
    for t in range(length):
        blk = int(table_row[t // block])
        slot = t - (t // block) * block
        keys.append([_val(k_cache[blk, g, slot // 16, j // 8, slot % 16, j % 8], kv_dtype) for j in range(d)])
        values.append([_val(v_cache[blk, g, slot // 16, j, slot % 16], kv_dtype) for j in range(d)])
    return keys, values


def brute_attention(q1, q2, a, k_cache, v_cache, block_table, ctx_lens, *, num_kv_heads, scale,
                    block_size, num_flows=2, q_dtype="bf16", kv_dtype="bf16"):
    """Nested lists out[f][b][h][d] of both flows' attention outputs."""
    batch, hq, d = len(q1), len(q1[0]), len(q1[0][0])
    out = [[[None] * hq for _ in range(batch)] for _ in range(num_flows)]
    for b in range(batch):
        for h in range(hq):
            g = (h * num_kv_heads) // hq
            keys, values = _kv_rows(k_cache, v_cache, block_table[b], int(ctx_lens[b]), g,
                                    block_size, kv_dtype)
            p = [_val(q1[b][h][j], q_dtype) for j in range(d)]
            out[0][b][h] = _softmax_avg(p, keys, values, scale)
            if num_flows == 2:
                x = [_val(q2[b][h][j], q_dtype) + float(a[h][j]) * p[j] for j in range(d)]
                out[1][b][h] = _softmax_avg(x, keys, values, scale)
    return out


def _matvec(w_bits, x):
    """W x with W as bf16 bits [out, in]."""
    return [math.fsum(_bf16(w_bits[i, j]) * x[j] for j in range(len(x))) for i in range(w_bits.shape[0])]


def _round_bf16(x: float) -> int:
    """Nearest bf16 (ties to even) of a finite float, as bits."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    m, e = math.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    q = max(e - 1, -126) - 7  # exponent of the bf16 spacing around x
    y = math.ldexp(round(math.ldexp(x, -q)), q)  # round() is half-to-even
    return struct.unpack("<I", struct.pack("<f", y))[0] >> 16


def _silu(u: float) -> float:
    return u / (1.0 + math.exp(-u))


def brute_layer(x1, x2, w, a, b, c, k_cache, v_cache, block_table, ctx_lens, *, num_q_heads,
                num_kv_heads, head_dim, scale, block_size):
    """Per-sequence scalar evaluation of one dual-flow layer step: dict of nested lists."""
    res = {k: [] for k in ("out1", "out2", "k1_bits", "v1_bits", "o1", "o2")}
    d = head_dim
    for s in range(len(x1)):
        u1 = [float(v) for v in x1[s]]
        u2 = [float(v) for v in x2[s]]
        q1 = _matvec(w["wq"], u1)
        q2 = _matvec(w["wq"], u2)
        k1 = _matvec(w["wk"], u1)
        v1 = _matvec(w["wv"], u1)
        kb = [_round_bf16(v) for v in k1]
        vb = [_round_bf16(v) for v in v1]
        res["k1_bits"].append(kb)
        res["v1_bits"].append(vb)
        length = int(ctx_lens[s])
        o = [[], []]
        for h in range(num_q_heads):
            g = (h * num_kv_heads) // num_q_heads
            keys, values = _kv_rows(k_cache, v_cache, block_table[s], length, g, block_size, "bf16")
            keys.append([_bf16(kb[g * d + j]) for j in range(d)])  # this step's primary key
            values.append([_bf16(vb[g * d + j]) for j in range(d)])
            p = q1[h * d:(h + 1) * d]
            x = [q2[h * d + j] + float(a[h * d + j]) * p[j] for j in range(d)]
            o[0] += _softmax_avg(p, keys, values, scale)
            o[1] += _softmax_avg(x, keys, values, scale)
        res["o1"].append(o[0])
        res["o2"].append(o[1])
        hh = [[u1[i] + v for i, v in enumerate(_matvec(w["wo"], o[0]))],
              [u2[i] + v for i, v in enumerate(_matvec(w["wo"], o[1]))]]
        z = []
        for f in range(2):
            gate = _matvec(w["wg"], hh[f])
            up = _matvec(w["wu"], hh[f])
            z.append([_silu(gate[i]) * up[i] for i in range(len(gate))])
        z2c = [z[1][i] + float(b[i]) * z[0][i] for i in range(len(z[0]))]
        m1 = _matvec(w["wd"], z[0])
        m2 = _matvec(w["wd"], z2c)
        res["out1"].append([hh[0][i] + m1[i] for i in range(len(m1))])
        res["out2"].append([hh[1][i] + m2[i] + float(c[i]) * m1[i] for i in range(len(m1))])
    return res
