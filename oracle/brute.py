"""Pure-Python masked attention for tiny inputs (pins the vectorized oracle).

TEST INFRASTRUCTURE ONLY.  Loops over heads, queries and keys with
``math.exp`` and no array library, following the same definition as
``oracle.attention`` (Tessera paper, sections 1 and 2.2): only (i, j) whose
logical block M[h][i // B_Q][j // B_KV] is active enter the softmax; a query
with no active key outputs zeros; scores are scaled by 1/sqrt(d).
"""

import math


def attention(Q, K, V, M, BQ, BKV):
    """Q, K, V: nested lists [H][N][d] of floats; M: nested [H][nQB][nKB]."""
    H = len(Q)
    out = []
    for h in range(H):
        N = len(Q[h])
        d = len(Q[h][0])
        scale = 1.0 / math.sqrt(d)
        rows = []
        for i in range(N):
            act = [j for j in range(N) if M[h][i // BQ][j // BKV]]
            if not act:
                rows.append([0.0] * d)
                continue
            s = {}
            for j in act:
                acc = 0.0
                for t in range(d):
                    acc += Q[h][i][t] * K[h][j][t]
                s[j] = acc * scale
            mx = max(s.values())
            w = {j: math.exp(s[j] - mx) for j in act}
            den = sum(w.values())
            o = [0.0] * d
            for j in act:
                for t in range(d):
                    o[t] += w[j] * V[h][j][t]
            rows.append([x / den for x in o])
        out.append(rows)
    return out
