"""Scalar mask statistics and active-block runs, by their definitions.

TEST INFRASTRUCTURE ONLY.

* Active-block run (Tessera paper, section 4.3 "Grouping and traversal"): a
  maximal sequence of consecutive active K/V blocks within one query-block
  row.  The paper's example: columns {2, 3, 4, 9} form runs [2, 4] and [9, 9].
* Density (section 5.1 and section 7.1 "Workloads"): the fraction of logical
  blocks that are active.
* Active-block-run coverage (section 5.1): the fraction of active blocks that
  belong to runs of length at least two; zero for an empty mask.

Both statistics are taken over the whole request (all heads); a ragged last
block counts as one block.
"""

import numpy as np


def runs(cols):
    """Maximal runs of consecutive integers in a sorted list of column indices."""
    out = []
    for c in cols:
        c = int(c)
        if out and c == out[-1][1] + 1:
            out[-1][1] = c
        else:
            out.append([c, c])
    return [tuple(r) for r in out]


def row_nnz(M):
    """Active blocks per query-block row: int64 [H, nQB]."""
    return (np.asarray(M) != 0).sum(axis=-1).astype(np.int64)


def density(M):
    M = np.asarray(M) != 0
    return float(M.sum()) / float(M.size) if M.size else 0.0


def blocks_in_long_runs(M):
    """Number of active blocks that lie in runs of length >= 2 (per row runs)."""
    M = np.asarray(M) != 0
    total = 0
    for row in M.reshape(-1, M.shape[-1]):
        for a, b in runs(np.nonzero(row)[0]):
            if b > a:
                total += b - a + 1
    return total


def blocks_in_long_runs_neighbour(M):
    """Same count as ``blocks_in_long_runs``, for large masks.

    An active block lies in a run of length >= 2 exactly when its left or its
    right neighbour in the same query-block row is active.
    """
    M = np.asarray(M) != 0
    left = np.zeros_like(M)
    right = np.zeros_like(M)
    left[..., 1:] = M[..., :-1]
    right[..., :-1] = M[..., 1:]
    return int((M & (left | right)).sum())


def run_coverage(M, large=False):
    M = np.asarray(M) != 0
    act = int(M.sum())
    if act == 0:
        return 0.0
    n = blocks_in_long_runs_neighbour(M) if large else blocks_in_long_runs(M)
    return n / act
