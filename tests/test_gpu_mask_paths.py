"""The three mask-state paths agree bit for bit: a mask at a 16-byte aligned
address goes through the single-launch kernel (small masks) or the 16-byte
row kernels (large masks), the same mask one byte past an aligned address
through the byte-per-lane kernels.  Block-CSR and statistics must be
identical, and the CSR must equal the oracle's enumeration.  Row lengths are
chosen so rows straddle 16-byte chunks and the mask's last chunk ends inside
the buffer."""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import stats as ostats
from workloads import gen

pytestmark = pytest.mark.gpu

KEYS = ("nnz_blocks", "max_row_nnz", "long_run_blocks", "density", "run_coverage", "row_skew")


def _plan_at(M, block, H, N, offset):
    """Plan of mask M placed `offset` bytes past a 256-byte aligned address."""
    flat = np.ascontiguousarray(M).reshape(-1)
    buf = torch.zeros(flat.size + 64, dtype=torch.uint8, device="cuda")
    view = buf[offset:offset + flat.size]
    view.copy_(torch.from_numpy(flat).to("cuda"))
    m = view.view(M.shape)
    assert (m.data_ptr() % 16 == 0) == (offset % 16 == 0)
    p = bsa.plan(m, block, H, N, 128)
    torch.cuda.synchronize()
    return p


# (block, N, H): small masks (single launch when aligned) and large ones with
# row lengths 625, 469 and 3600 bytes, and 2240 rows of 8 bytes (two rows per
# 16-byte chunk) (aligned: 16-byte kernels)
@pytest.mark.parametrize("block,N,H", [((64, 64), 1024, 3), ((128, 32), 777, 5), ((32, 128), 5000, 5),
                                       ((64, 64), 40000, 3), ((32, 128), 60000, 2), ((128, 32), 115200, 1),
                                       ((32, 128), 1000, 70)])
def test_mask_paths_agree(block, N, H):
    M, _, _, _ = gen.random_case(H, N, 8, *block, p=0.3, seed=4242 + N, empty_rows={0: [1, 2]},
                                 dense_heads=(H - 1,) if H > 1 else ())
    Mb = np.asarray(M) != 0
    rows = Mb.reshape(-1, Mb.shape[-1])
    exp_rp = np.concatenate([[0], np.cumsum(rows.sum(axis=1))])
    exp_cols = np.concatenate([np.nonzero(r)[0] for r in rows])
    res = []
    for off in (0, 1):
        p = _plan_at(M, block, H, N, off)
        rp, cols = p.export_csr()
        info = p.info
        p.destroy()
        assert (rp == exp_rp).all(), f"row_ptr, offset {off}"
        assert (cols == exp_cols).all(), f"cols, offset {off}"
        assert info["density"] == pytest.approx(ostats.density(M), abs=1e-12)
        assert info["run_coverage"] == pytest.approx(ostats.run_coverage(M, large=M.size > 10**6), abs=1e-12)
        res.append({k: info[k] for k in KEYS})
    assert res[0] == res[1]
