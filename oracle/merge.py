"""Split-K partial softmax states and their merge, in float64.

TEST INFRASTRUCTURE ONLY.

Tessera paper, section 4.3 "Split-K": one query tile's K/V reduction is
partitioned across several workers; each writes its maximum score m, scaled
exponential sum l and unnormalized output accumulator O; a later step rescales
the partial states to a common maximum, merges them and normalizes.  Section
4.2 ("Refined") names the same state (running maximum, scaled exponential sum,
output accumulator) for sequential K/V traversal.

For one query q and a key subset S:
    m_S = max_{j in S} s_j,  l_S = sum_{j in S} exp(s_j - m_S),
    O_S = sum_{j in S} exp(s_j - m_S) v_j,       s_j = q . k_j / sqrt(d)
An empty subset has m = -inf, l = 0, O = 0.  Merge over a partition {S_p}:
    m* = max_p m_p,  w_p = exp(m_p - m*) (0 for an empty part),
    o = (sum_p w_p O_p) / (sum_p w_p l_p);  o = 0 if every part is empty.
"""

import math

import numpy as np


def partial_state(q, K, V, scale=None):
    """q: [d], K/V: [n, d] float64 (n may be 0). Returns (m, l, O)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64).reshape(-1, q.shape[0])
    V = np.asarray(V, dtype=np.float64)
    assert V.ndim == 2 and V.shape[0] == K.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[0])
    if K.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(V.shape[1])
    s = (K @ q) * scale
    m = float(s.max())
    w = np.exp(s - m)
    return m, float(w.sum()), w @ V


def merge(parts, dv):
    """parts: iterable of (m, l, O). Returns the normalized output row [dv]."""
    parts = [p for p in parts if p[1] > 0.0]
    if not parts:
        return np.zeros(dv)
    mstar = max(p[0] for p in parts)
    num = np.zeros(dv)
    den = 0.0
    for m, l, O in parts:
        w = math.exp(m - mstar)
        num += w * np.asarray(O, dtype=np.float64)
        den += w * l
    return num / den
