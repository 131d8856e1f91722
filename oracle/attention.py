"""Dense masked attention in float64: the definition of the BSA forward output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed (Tessera paper, section 1 "Introduction" and section 2.2
"The Cost of Logical-to-Physical Coupling"): a logical mask M over blocks of
B_Q query tokens by B_KV key/value tokens marks which blocks are active; the
attention computes only the active blocks, i.e. the interactions E(M).  The
Coarsened mapping (section 4.2) states that normalization and the weighted
sum of values include only the effective entries in E(M).  Written per head
h and query i < N:

    A_i = { j < N : M[h, i // B_Q, j // B_KV] != 0 }
    o_i = 0                                                   if A_i is empty
    o_i = sum_{j in A_i} softmax_{A_i}(q_i . k_j / sqrt(d))_j v_j   otherwise

Parity pins: tests/test_oracle_pins.py (brute force, dense special case,
empty rows, block-diagonal, support, row-stochastic, shift invariance, block
permutation).
"""

import math

import numpy as np


def _f64(x):
    """Upcast a torch tensor or array-like to a float64 numpy array."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def mask_grid_shape(N, BQ, BKV):
    """Logical mask grid (ceil(N/B_Q), ceil(N/B_KV)); the last block is ragged."""
    return (-(-N // BQ), -(-N // BKV))


def token_mask(Mh, BQ, BKV, N, rows=None):
    """Expand one head's logical mask to token level: bool [len(rows), N].

    Entry (i, j) is True iff the logical block containing (i, j) is active.
    """
    Mh = np.asarray(Mh) != 0
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    qb = rows // BQ
    kb = np.arange(N) // BKV
    return Mh[qb][:, kb]


def _rows_attention(q, K, V, allowed, scale):
    """softmax over allowed entries of (q K^T * scale), times V; empty rows -> 0.

    q: [r, d], K/V: [N, d] float64, allowed: bool [r, N].
    """
    s = (q @ K.T) * scale
    s = np.where(allowed, s, -np.inf)
    has = allowed.any(axis=1)
    mx = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.exp(s - mx[:, None])  # exp(-inf) = 0 for masked entries
    p = np.where(allowed, p, 0.0)
    den = p.sum(axis=1)
    out = p @ V
    out[has] /= den[has, None]
    out[~has] = 0.0
    return out


def attention(Q, K, V, M, BQ, BKV, chunk=1024):
    """Masked attention for every head and row.

    Q, K, V: [H, N, d] (any float dtype; upcast to float64).
    M: [H, ceil(N/B_Q), ceil(N/B_KV)] with nonzero = active.
    Returns float64 [H, N, d].
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    M = np.asarray(M)
    H, N, d = Q.shape
    assert M.shape == (H,) + mask_grid_shape(N, BQ, BKV), M.shape
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((H, N, d), dtype=np.float64)
    for h in range(H):
        for r0 in range(0, N, chunk):
            rows = np.arange(r0, min(N, r0 + chunk))
            allowed = token_mask(M[h], BQ, BKV, N, rows)
            out[h, rows] = _rows_attention(Q[h, rows], K[h], V[h], allowed, scale)
    return out


def attention_rows(Q, K, V, M, BQ, BKV, head_rows):
    """Masked attention for selected (head, rows) only, by the same definition.

    head_rows: dict {h: array of row indices}.  Returns {h: float64 [r, d]}.
    Only the key/value rows of active blocks are gathered, so this runs at
    full problem sizes where the dense per-head product would not fit.
    """
    M = np.asarray(M)
    N = Q.shape[1]
    d = Q.shape[2]
    scale = 1.0 / math.sqrt(d)
    res = {}
    for h, rows in head_rows.items():
        rows = np.asarray(rows)
        Kh = _f64(K[h])
        Vh = _f64(V[h])
        qh = _f64(Q[h])[rows]
        out = np.zeros((len(rows), d), dtype=np.float64)
        # group rows by query block so the active key set is gathered once
        qbs = rows // BQ
        for qb in np.unique(qbs):
            sel = np.nonzero(qbs == qb)[0]
            cols = np.nonzero(M[h, qb])[0]
            if cols.size == 0:
                continue  # A_i empty: output row stays 0
            j = (cols[:, None] * BKV + np.arange(BKV)[None, :]).reshape(-1)
            j = j[j < N]
            allowed = np.ones((sel.size, j.size), dtype=bool)
            out[sel] = _rows_attention(qh[sel], Kh[j], Vh[j], allowed, scale)
        res[h] = out
    return res
