"""Pure-Python brute force attention for tiny shapes (pins the oracle).

Written independently of ``oracle/``: plain loops, ``math.exp`` and
``math.fsum``, the head mapping and causal visibility spelled out inline.
Inputs are nested Python lists of floats.
"""

import math


def brute_attention(q, k, v, kv_len, qo_len, num_qo_heads, num_kv_heads,
                    causal, sm_scale):
    """q: [qo_len][Hq][d]; k, v: [kv_len][Hkv][d] (Python floats).

    Row i of the chunk is token kv_len - qo_len + i of the sequence; when
    causal it sees keys 0 .. that position.  Query head h reads KV head
    h // (Hq / Hkv).  Returns (O [qo][Hq][d], LSE [qo][Hq])."""
    group = num_qo_heads // num_kv_heads
    d = len(q[0][0])
    out_o, out_l = [], []
    for i in range(qo_len):
        pos = kv_len - qo_len + i
        last = pos if causal else kv_len - 1
        row_o, row_l = [], []
        for h in range(num_qo_heads):
            g = h // group
            scores = []
            for j in range(last + 1):
                scores.append(sm_scale * math.fsum(q[i][h][c] * k[j][g][c]
                                                   for c in range(d)))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = math.fsum(w)
            o = [math.fsum(w[j] * v[j][g][c] for j in range(len(w))) / tot
                 for c in range(d)]
            row_o.append(o)
            row_l.append(mx + math.log(tot))
        out_o.append(row_o)
        out_l.append(row_l)
    return out_o, out_l
