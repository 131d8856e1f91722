"""Enumeration of E(M), the (head, query, key) interactions a mask specifies.

TEST INFRASTRUCTURE ONLY.

Tessera paper, section 2.2: every physical plan must preserve E(M), the set of
specified interactions; section 4.2 describes Direct (T = B), Coarsened (one
tile over several logical regions, inactive entries masked by membership
metadata) and Refined (smaller tiles; the worked example splits a 128x128
block into four 64x64 tiles, block-CSR column c becoming K/V tiles 2c and
2c+1).  Whatever the plan, each effective pair must be computed exactly once
and no other pair may enter the softmax.

* ``token_pairs``  E(M) as a boolean [H, N, N] array (small N only).
* ``cells``        E(M) at the granularity of cells of cq x ckv tokens, where
  cq divides B_Q and ckv divides B_KV, so each cell lies inside one logical
  block: the expected number of times a plan covers each cell (1 if its block
  is active, else 0).  Cells are aligned from token 0 and clipped at N.
"""

import numpy as np


def token_pairs(M, BQ, BKV, N):
    M = np.asarray(M) != 0
    qb = np.arange(N) // BQ
    kb = np.arange(N) // BKV
    return M[:, qb][:, :, kb]


def cells(M, BQ, BKV, N, cq, ckv):
    if BQ % cq or BKV % ckv:
        raise ValueError("cell size must divide the logical block size")
    M = (np.asarray(M) != 0).astype(np.uint8)
    nq = -(-N // cq)
    nk = -(-N // ckv)
    qb = (np.arange(nq) * cq) // BQ
    kb = (np.arange(nk) * ckv) // BKV
    return M[:, qb][:, :, kb]


def effective_pairs(M, BQ, BKV, N):
    """|E(M)|: number of effective (head, query, key) pairs, clipped at N."""
    M = np.asarray(M) != 0
    nQB, nKB = M.shape[1], M.shape[2]
    qsz = np.minimum(BQ, N - np.arange(nQB) * BQ)
    ksz = np.minimum(BKV, N - np.arange(nKB) * BKV)
    return int(np.einsum("hab,a,b->", M.astype(np.int64), qsz, ksz))
