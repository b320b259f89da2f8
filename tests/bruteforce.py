"""Independent brute-force attention for pinning the oracle (tests only).

Pure Python over *contiguous* per-sequence K/V: no paging, no numpy, exact
summation with math.fsum. Written separately from the oracle so that a slip in
the oracle's gather, GQA mapping, scale or normalisation shows up as a
disagreement.
"""
import math


def attend_contiguous(q_heads, k_rows, v_rows, scale, num_kv_heads):
    """q_heads: [Hq][D] floats; k_rows, v_rows: [L][Hkv][D] floats.

    Query head j reads KV head floor(j * Hkv / Hq) (consecutive query heads
    share a KV head). Returns [Hq][D] floats.
    """
    hq = len(q_heads)
    out = []
    for j in range(hq):
        h = (j * num_kv_heads) // hq
        logits = [scale * math.fsum(a * b for a, b in zip(q_heads[j], k[h])) for k in k_rows]
        top = max(logits)
        expo = [math.exp(z - top) for z in logits]
        denom = math.fsum(expo)
        d = len(q_heads[j])
        out.append([math.fsum(expo[t] * v_rows[t][h][i] for t in range(len(v_rows))) / denom
                    for i in range(d)])
    return out
