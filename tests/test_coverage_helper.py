"""CPU check of the cell-coverage expansion that the full-size GPU coverage
tests rely on (tests/bsa_testutil.cell_counts_by_head).

Tile lists are built here by hand from the mapping definitions (Tessera
paper, section 4.2: Direct keeps each active block as one tile; Coarsened
merges c_Q x c_KV blocks into one tile with membership bits; Refined splits a
block into smaller tiles, the 128x128 -> four 64x64 example) and must expand
to exactly the oracle's cell coverage; a dropped, duplicated or spurious tile
must be detected.
"""

import numpy as np
import pytest

from oracle import coverage
from workloads import gen

from bsa_testutil import cell_counts_by_head


class FakePlan:
    def __init__(self, H, info, tiles, batch=1):
        self.H = H
        self.batch = batch
        self.info = info
        self._tiles = tuple(np.asarray(t) for t in tiles)

    def export_tiles(self):
        return self._tiles


def _info(TQ, TKV, cQ=1, cKV=1):
    return dict(tile_q=TQ, tile_kv=TKV, coarsen_q=cQ, coarsen_kv=cKV)


def _direct(M):
    h, a, b = np.nonzero(M)
    return (h.astype(np.int32), a.astype(np.int32), b.astype(np.int32), np.ones(h.size, np.uint32))


def _coarsened(M, cQ, cKV):
    H, nq, nk = M.shape
    out = [[], [], [], []]
    for h in range(H):
        for tq in range(-(-nq // cQ)):
            for tk in range(-(-nk // cKV)):
                bits = 0
                for a in range(cQ):
                    for b in range(cKV):
                        qa, kb = tq * cQ + a, tk * cKV + b
                        if qa < nq and kb < nk and M[h, qa, kb]:
                            bits |= 1 << (a * cKV + b)
                if bits:
                    for lst, v in zip(out, (h, tq, tk, bits)):
                        lst.append(v)
    return (np.array(out[0], np.int32), np.array(out[1], np.int32), np.array(out[2], np.int32),
            np.array(out[3], np.uint32))


def _refined(M, rQ, rKV, N, TQ, TKV):
    out = [[], [], []]
    for h, a, b in zip(*np.nonzero(M)):
        for i in range(rQ):
            for j in range(rKV):
                qt, kt = a * rQ + i, b * rKV + j
                if qt * TQ < N and kt * TKV < N:
                    out[0].append(h)
                    out[1].append(qt)
                    out[2].append(kt)
    n = len(out[0])
    return (np.array(out[0], np.int32), np.array(out[1], np.int32), np.array(out[2], np.int32),
            np.ones(n, np.uint32))


def _expand(plan, block, N):
    return np.stack([c for _, c in cell_counts_by_head(plan, block, N)])


CASES = [
    # (N, B, T, kind)
    (777, (64, 64), (64, 64), "direct"),
    (777, (64, 32), (128, 64), "coarse"),
    (1000, (32, 128), (64, 64), "mixed"),     # Q coarsened x2, K/V refined x2
    (777, (128, 128), (64, 64), "refine"),
]


@pytest.mark.parametrize("N,block,T,kind", CASES)
def test_expansion_matches_oracle(N, block, T, kind):
    H = 3
    M = gen.mask_iid_diag(H, N, *block, 0.3, seed=N + T[0], empty_rows={1: [0]})
    BQ, BKV = block
    TQ, TKV = T
    if kind == "direct":
        tiles, info = _direct(M), _info(TQ, TKV)
    elif kind == "coarse":
        tiles, info = _coarsened(M, TQ // BQ, TKV // BKV), _info(TQ, TKV, TQ // BQ, TKV // BKV)
    elif kind == "refine":
        tiles, info = _refined(M, BQ // TQ, BKV // TKV, N, TQ, TKV), _info(TQ, TKV)
    else:
        # Q coarsened (TQ = 2 BQ), K/V refined (TKV = BKV / 2): coarsen rows,
        # then split each K/V block column into two tile columns
        h, tq, tk, bits = _coarsened(M, TQ // BQ, 1)
        r = BKV // TKV
        tiles = (np.repeat(h, r), np.repeat(tq, r),
                 (tk[:, None] * r + np.arange(r)[None, :]).reshape(-1).astype(np.int32), np.repeat(bits, r))
        keep = tiles[2].astype(np.int64) * TKV < N
        tiles = tuple(t[keep] for t in tiles)
        info = _info(TQ, TKV, TQ // BQ, 1)
    cq, ckv = min(BQ, TQ), min(BKV, TKV)
    want = coverage.cells(M, BQ, BKV, N, cq, ckv)
    got = _expand(FakePlan(H, info, tiles), block, N)
    assert np.array_equal(got, want)
    # the same tiles as one head per batch entry: heads are counted over
    # batch x H, not H alone
    assert np.array_equal(_expand(FakePlan(1, info, tiles, batch=H), block, N), want)
    # a dropped tile, a duplicated tile and a tile on an inactive block are
    # all detected
    drop = tuple(t[1:] for t in tiles)
    assert not np.array_equal(_expand(FakePlan(H, info, drop), block, N), want)
    dup = tuple(np.concatenate([t, t[:1]]) for t in tiles)
    assert not np.array_equal(_expand(FakePlan(H, info, dup), block, N), want)
    hz, az, bz = np.argwhere(want == 0)[0]
    cQ, cKV = info["coarsen_q"], info["coarsen_kv"]
    extra = (np.array([hz], np.int32), np.array([az // cQ], np.int32), np.array([bz // cKV], np.int32),
             np.array([1 << ((az % cQ) * cKV + bz % cKV)], np.uint32))
    spur = tuple(np.concatenate([t, e]) for t, e in zip(tiles, extra))
    assert not np.array_equal(_expand(FakePlan(H, info, spur), block, N), want)


def test_bits_outside_grid_rejected():
    # a coarsened tile at the ragged edge with a membership bit for a block
    # row that does not exist
    N, block = 200, (64, 64)            # 4 x 4 blocks; tiles of 2 x 1 blocks
    M = np.ones((1, 4, 4), np.uint8)
    tiles = _coarsened(M, 2, 1)
    h, tq, tk, bits = tiles
    bad = (np.append(h, 0).astype(np.int32), np.append(tq, 2).astype(np.int32),
           np.append(tk, 0).astype(np.int32), np.append(bits, 3).astype(np.uint32))
    with pytest.raises(AssertionError):
        _expand(FakePlan(1, _info(128, 64, 2, 1), bad), block, N)
