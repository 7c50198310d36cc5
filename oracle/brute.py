"""Pure-Python scalar brute force of the literal GQLA decode (test infrastructure only).

No numpy arithmetic: every dot product is ``math.fsum`` over explicit
products, every exponential is ``math.exp``.  Meant for tiny inputs
(a few heads, latent dims of ~8, contexts of ~100 tokens); it pins the numpy
oracle in ``gqla_ref`` (same definition, independent code).

Definition (GQLA pages, paperlayer.ai section 3 "Architecture" and
"Two equivalent decoding paths"; readings as in ``gqla_ref``):

  k_t[G]  = c_t W_UK[G],  v_t[G] = c_t W_UV[G]
  s_t     = (q_nope . k_t[G] + q_rope . k_rope_t) / sqrt(d_nope + d_R)
  out     = sum_t exp(s_t - m) v_t[G] / sum_t exp(s_t - m),  t <= L - s_q + i
"""
from __future__ import annotations

import math


def _row_times_matrix(row, mat):
    """row (len r) @ mat (r x n), exact-sum per column."""
    n = len(mat[0])
    return [math.fsum(row[a] * mat[a][j] for a in range(len(row))) for j in range(n)]


def decode(q_nope, q_rope, pages, block_table, seqlens, w_uk, w_uv,
           h_q, g, r, d_R, d_nope, d_v, s_q, bs):
    """Nested lists in, nested lists out: (out[b][i][h][j], lse[b][i][h])."""
    hpg = h_q // g
    scale = 1.0 / math.sqrt(d_nope + d_R)
    out, lse = [], []
    for b in range(len(seqlens)):
        L = int(seqlens[b])
        lat = []
        for t in range(L):
            page = int(block_table[b][t // bs])
            lat.append([float(x) for x in pages[page][t % bs]])
        ob, lb = [], []
        for i in range(s_q):
            oi, li = [], []
            n = L - s_q + i + 1
            for h in range(h_q):
                G = h // hpg
                scores, vals = [], []
                for t in range(n):
                    c = lat[t][:r]
                    kr = lat[t][r:r + d_R]
                    k = _row_times_matrix(c, w_uk[G])
                    v = _row_times_matrix(c, w_uv[G])
                    dot = math.fsum([q_nope[b][i][h][j] * k[j] for j in range(d_nope)]
                                    + [q_rope[b][i][h][j] * kr[j] for j in range(d_R)])
                    scores.append(dot * scale)
                    vals.append(v)
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                z = math.fsum(e)
                oi.append([math.fsum(e[t] * vals[t][j] for t in range(n)) / z for j in range(d_v)])
                li.append(m + math.log(z))
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return out, lse
