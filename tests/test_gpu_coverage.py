"""Tile coverage of the table-selected plans at the full workload sizes,
bit-exact against the oracle's enumeration of E(M).

Every plan must preserve E(M), the interactions the logical mask specifies
(Tessera paper, section 2.2), whether it keeps blocks (Direct), merges them
with membership bits (Coarsened) or splits them (Refined; section 4.2 and its
128x128 -> four 64x64 example).  The plan's exported tiles (head, query tile,
K/V tile, membership bits) are expanded to the cells they cover and the
multiplicity of every cell is compared with the oracle's: 1 for a cell of an
active block, 0 otherwise, so a missing, duplicated or spurious tile fails.

* medium (8 x 8192, B = (128, 128)): token level, against
  ``oracle.coverage.token_pairs``;
* wan720p (40 x 75,600, B = (64, 64), ragged last block), hunyuan
  (24 x 115,200, B = (128, 32)) and eight requests of the request stream (two
  per block geometry, heads with empty query-block rows among them): cell
  level, against ``oracle.coverage.cells``.

Plans come from the regime table with their own split rule, as the benchmark
times them; the masks need no Q/K/V.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import coverage
from workloads import gen

from bsa_testutil import cell_counts_by_head

pytestmark = pytest.mark.gpu


def _plan(M, block, H, N, d=128):
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(torch.device("cuda"))
    p = bsa.plan(Md, block, H, N, d)
    torch.cuda.synchronize()
    return p


def _check_cells(M, block, N, label):
    H = M.shape[0]
    p = _plan(M, block, H, N)
    info = p.info
    try:
        n_heads = 0
        for h, cnt in cell_counts_by_head(p, block, N):
            cq, ckv = min(block[0], info["tile_q"]), min(block[1], info["tile_kv"])
            want = coverage.cells(M[h:h + 1], block[0], block[1], N, cq, ckv)[0]
            bad = np.argwhere(cnt != want)
            assert bad.size == 0, (f"{label}: head {h} cell {tuple(bad[0])} covered "
                                   f"{cnt[tuple(bad[0])]} times, oracle {want[tuple(bad[0])]}")
            n_heads += 1
        assert n_heads == H
    finally:
        p.destroy()
    print(f"{label}: plan {info['plan_id']} T=({info['tile_q']},{info['tile_kv']}) "
          f"coarsen ({info['coarsen_q']},{info['coarsen_kv']}) refine "
          f"({info['refine_q']},{info['refine_kv']}) split {info['split_items']}: "
          f"coverage exact on {H} heads", flush=True)
    return info


def test_medium_token_level():
    BQ, BKV, M = gen.mask_for(2)
    H, N = M.shape[0], 8192
    p = _plan(M, (BQ, BKV), H, N)
    info = p.info
    try:
        cq, ckv = min(BQ, info["tile_q"]), min(BKV, info["tile_kv"])
        for h, cnt in cell_counts_by_head(p, (BQ, BKV), N):
            c8 = np.minimum(cnt, 2).astype(np.uint8)
            tok = np.repeat(np.repeat(c8, cq, axis=0)[:N], ckv, axis=1)[:, :N]
            want = coverage.token_pairs(M[h:h + 1], BQ, BKV, N)[0]
            assert np.array_equal(tok, want.astype(np.uint8)), f"medium head {h}: token coverage"
    finally:
        p.destroy()


@pytest.mark.parametrize("c", [3, 4])
def test_fullsize_cells(c):
    BQ, BKV, M = gen.mask_for(c)
    _check_cells(M, (BQ, BKV), gen.CONFIGS[c]["N"], gen.CONFIGS[c]["name"])


# two requests of each block geometry: (128,128) 0, 1; (128,32) 2, 3;
# (64,64) 6, 10; (32,128) 7, 12
@pytest.mark.parametrize("r", [0, 1, 2, 3, 6, 10, 7, 12])
def test_stream_request_cells(r):
    BQ, BKV, M, _ = gen.request_c5(r)
    empty = int(((M != 0).sum(-1) == 0).sum())
    _check_cells(M, (BQ, BKV), gen.CONFIGS[5]["N"], f"stream request {r} B=({BQ},{BKV}) "
                 f"{empty} empty query-block rows")
