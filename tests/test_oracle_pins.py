"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (dropped scale, a
transposed mask index, a wrong sign in the max shift, a missing empty-row
rule, a key-block addressing error) fails at least one of them:

P1  brute force: pure-Python loops equal the vectorized oracle (ragged N,
    non-square blocks both ways).
P2  all-active mask = textbook attention (torch SDPA in float64 on the CPU).
P3  a query row with no active block outputs exactly 0.
P4  block-diagonal mask = independent dense attention per diagonal slice.
P5  one-hot V turns O into the probability matrix: its support equals E(M)
    and non-empty rows sum to 1.
P6  constant V = c gives O = c on every non-empty row.
P7  merging split-K partial states over any partition of the keys equals the
    unsplit result; empty partials are ignored.
P8  adding a vector u to every key leaves O unchanged (per-row score shift).
P9  permuting whole K/V blocks together with their mask columns leaves O
    unchanged.
P10 active-block runs and run coverage match the paper's worked example.
P11 the cell enumeration of E(M) matches the paper's refinement example.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import brute, coverage, merge, stats

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask(H, N, BQ, BKV, p, seed):
    nq, nk = oatt.mask_grid_shape(N, BQ, BKV)
    M = (np.random.default_rng(seed).random((H, nq, nk)) < p).astype(np.uint8)
    return M


@pytest.mark.parametrize("N,BQ,BKV", [(48, 16, 8), (50, 16, 8), (48, 8, 16), (50, 8, 16), (50, 16, 16)])
def test_p1_brute_force(N, BQ, BKV):
    H, d = 2, 8
    Q, K, V = _rand((H, N, d), 1), _rand((H, N, d), 2), _rand((H, N, d), 3)
    M = _mask(H, N, BQ, BKV, 0.4, N + BQ)
    M[0, 1] = 0  # an empty query-block row
    ref = np.array(brute.attention(Q.tolist(), K.tolist(), V.tolist(), M.tolist(), BQ, BKV))
    out = oatt.attention(Q, K, V, M, BQ, BKV, chunk=7)
    assert np.abs(out - ref).max() <= 1e-12
    rows = {0: np.array([0, 5, 17, N - 1]), 1: np.arange(N)}
    got = oatt.attention_rows(Q, K, V, M, BQ, BKV, rows)
    for h, r in rows.items():
        assert np.abs(got[h] - ref[h][r]).max() <= 1e-12


@pytest.mark.parametrize("N,B", [(64, (16, 16)), (70, (16, 32)), (96, (32, 8))])
def test_p2_all_active_equals_dense(N, B):
    H, d = 3, 16
    Q, K, V = _rand((H, N, d), 4), _rand((H, N, d), 5), _rand((H, N, d), 6)
    M = np.ones((H,) + oatt.mask_grid_shape(N, *B), dtype=np.uint8)
    out = oatt.attention(Q, K, V, M, *B)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V)).numpy()
    assert np.abs(out - ref).max() <= 1e-12


def test_p3_empty_rows_exact_zero():
    H, N, d, BQ, BKV = 2, 100, 8, 16, 32
    Q, K, V = _rand((H, N, d), 7), _rand((H, N, d), 8), _rand((H, N, d), 9)
    M = _mask(H, N, BQ, BKV, 0.5, 10)
    M[0, 2] = 0
    M[1, -1] = 0  # ragged last query block (rows 96..99)
    M[1, 0] = 0
    out = oatt.attention(Q, K, V, M, BQ, BKV)
    assert (out[0, 32:48] == 0.0).all()
    assert (out[1, 96:100] == 0.0).all()
    assert (out[1, 0:16] == 0.0).all()
    nz = stats.row_nnz(M) > 0
    for h in range(H):
        for qb in np.nonzero(nz[h])[0]:
            assert np.abs(out[h, qb * BQ:min(N, (qb + 1) * BQ)]).sum(axis=1).min() > 0


def test_p4_block_diagonal():
    H, N, d, b = 2, 80, 8, 16
    Q, K, V = _rand((H, N, d), 11), _rand((H, N, d), 12), _rand((H, N, d), 13)
    M = np.zeros((H, 5, 5), dtype=np.uint8)
    for i in range(5):
        M[:, i, i] = 1
    out = oatt.attention(Q, K, V, M, b, b)
    for s in range(5):
        sl = slice(s * b, (s + 1) * b)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[:, sl]), torch.from_numpy(K[:, sl]), torch.from_numpy(V[:, sl])).numpy()
        assert np.abs(out[:, sl] - ref).max() <= 1e-12


@pytest.mark.parametrize("N,BQ,BKV", [(40, 8, 16), (37, 16, 8)])
def test_p5_support_equals_E(N, BQ, BKV):
    H = 2
    d = N  # V = one-hot rows: O becomes the probability matrix
    Q, K = _rand((H, N, 8), 14), _rand((H, N, 8), 15)
    V = np.broadcast_to(np.eye(N), (H, N, N)).copy()
    M = _mask(H, N, BQ, BKV, 0.45, 16)
    M[1, 0] = 0
    # a different d for Q/K than for V: scale must follow the Q/K width
    out = np.stack([oatt._rows_attention(Q[h], K[h], V[h], oatt.token_mask(M[h], BQ, BKV, N),
                                         1 / math.sqrt(8)) for h in range(H)])
    E = coverage.token_pairs(M, BQ, BKV, N)
    assert ((out > 0) == E).all()
    rs = out.sum(axis=2)
    has = E.any(axis=2)
    assert np.abs(rs[has] - 1).max() <= 1e-12 and (rs[~has] == 0).all()


def test_p6_row_stochastic():
    H, N, d, BQ, BKV = 2, 90, 8, 32, 16
    Q, K = _rand((H, N, d), 17), _rand((H, N, d), 18)
    V = np.full((H, N, d), 2.5)
    M = _mask(H, N, BQ, BKV, 0.3, 19)
    M[0, 1] = 0
    out = oatt.attention(Q, K, V, M, BQ, BKV)
    has = coverage.token_pairs(M, BQ, BKV, N).any(axis=2)
    assert np.abs(out[has] - 2.5).max() <= 1e-12
    assert (out[~has] == 0).all()


def test_p7_merge_identity():
    rng = np.random.default_rng(20)
    d, n = 16, 50
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d))
    s = K @ q / math.sqrt(d)
    p = np.exp(s - s.max())
    ref = (p / p.sum()) @ V
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, n), size=trial + 1, replace=False))
        perm = rng.permutation(n)
        parts = [merge.partial_state(q, K[idx], V[idx]) for idx in np.split(perm, cuts)]
        parts.append(merge.partial_state(q, K[:0], V[:0]))  # an empty partition
        assert np.abs(merge.merge(parts, d) - ref).max() <= 1e-12
    assert (merge.merge([merge.partial_state(q, K[:0], V[:0])], d) == 0).all()


def test_p8_key_shift_invariance():
    H, N, d, BQ, BKV = 2, 64, 8, 16, 16
    Q, K, V = _rand((H, N, d), 21), _rand((H, N, d), 22), _rand((H, N, d), 23)
    M = _mask(H, N, BQ, BKV, 0.5, 24)
    u = _rand((H, 1, d), 25) * 4
    a = oatt.attention(Q, K, V, M, BQ, BKV)
    b = oatt.attention(Q, K + u, V, M, BQ, BKV)
    assert np.abs(a - b).max() <= 1e-10


def test_p9_block_permutation():
    H, N, d, BQ, BKV = 2, 96, 8, 32, 16
    Q, K, V = _rand((H, N, d), 26), _rand((H, N, d), 27), _rand((H, N, d), 28)
    M = _mask(H, N, BQ, BKV, 0.5, 29)
    perm = np.random.default_rng(30).permutation(N // BKV)
    tok = (perm[:, None] * BKV + np.arange(BKV)).reshape(-1)
    a = oatt.attention(Q, K, V, M, BQ, BKV)
    b = oatt.attention(Q, K[:, tok], V[:, tok], M[:, :, perm], BQ, BKV)
    assert np.abs(a - b).max() <= 1e-12


def test_p10_runs_worked_example():
    g = json.load(open(os.path.join(GOLD, "runs_example.json")))
    assert stats.runs(g["row_cols"]) == [tuple(r) for r in g["runs"]]
    M = np.zeros((1, 1, 12), dtype=np.uint8)
    M[0, 0, g["row_cols"]] = 1
    assert stats.run_coverage(M) == g["run_coverage"]
    assert stats.run_coverage(M, large=True) == g["run_coverage"]
    assert stats.run_coverage(np.zeros((2, 3, 4), np.uint8)) == g["empty_mask_run_coverage"]
    assert stats.density(M) == 4 / 12


def test_p10_run_counts_agree_on_random_masks():
    for seed in range(20):
        M = _mask(2, 200, 16, 8, 0.1 + 0.04 * seed, seed)
        assert stats.blocks_in_long_runs(M) == stats.blocks_in_long_runs_neighbour(M)


def test_p11_refinement_worked_example():
    g = json.load(open(os.path.join(GOLD, "refine_example.json")))
    (BQ, BKV), (TQ, TKV), N = g["block"], g["tile"], g["N"]
    nq, nk = oatt.mask_grid_shape(N, BQ, BKV)
    M = np.zeros((1, nq, nk), dtype=np.uint8)
    for a, b in g["logical_active"]:
        M[0, a, b] = 1
    C = coverage.cells(M, BQ, BKV, N, TQ, TKV)[0]
    for r in range(C.shape[0]):
        want = g["tile_rows_cols"].get(str(r), [])
        assert list(np.nonzero(C[r])[0]) == want
    # the four 64x64 tiles of each active block cover exactly its token pairs
    E = coverage.token_pairs(M, BQ, BKV, N)[0]
    tok = np.kron(C, np.ones((TQ, TKV), dtype=np.uint8))[:N, :N].astype(bool)
    assert (tok == E).all()


def test_effective_pairs_ragged():
    N, BQ, BKV = 100, 32, 16
    M = _mask(3, N, BQ, BKV, 0.5, 31)
    assert coverage.effective_pairs(M, BQ, BKV, N) == int(coverage.token_pairs(M, BQ, BKV, N).sum())
