"""The seeded generators produce the workload shapes and densities stated for
each benchmark configuration (Tessera paper, section 7.1: video masks with
9-12% default mean density; per-config ranges as configured)."""

import numpy as np
import pytest

from oracle import stats
from workloads import gen


def test_c1_c2_structure():
    BQ, BKV, M = gen.mask_for(1)
    assert M.shape == (1, 16, 16) and (np.diag(M[0]) == 1).all()
    assert 0.45 < stats.density(M) < 0.65
    BQ, BKV, M = gen.mask_for(2)
    assert M.shape == (8, 64, 64) and (BQ, BKV) == (128, 128)
    assert (M[6] == 1).all()
    assert (M[7, 0] == 0).all() and (M[7, 63] == 0).all()
    assert all((np.diag(M[h]) == 1).all() for h in range(6))
    for h in range(6):
        assert 0.17 < stats.density(M[h]) < 0.26


def test_c3_spatiotemporal_density():
    BQ, BKV, M = gen.mask_for(3)
    assert M.shape == (40, 1182, 1182)
    dh = [stats.density(M[h]) for h in range(40)]
    assert min(dh) > 0.095 and max(dh) < 0.165  # ties in the radius overshoot slightly
    assert stats.row_nnz(M).min() > 0


def test_c4_clustered_density_and_runs():
    BQ, BKV, M = gen.mask_for(4)
    assert M.shape == (24, 900, 3600) and (BQ, BKV) == (128, 32)
    dh = np.array([stats.density(M[h]) for h in range(24)])
    assert dh.min() >= 0.049 and dh.max() <= 0.301
    assert stats.run_coverage(M, large=True) > 0.5


def test_c5_requests():
    seen = set()
    for r in range(6):
        BQ, BKV, M, seeds = gen.request_c5(r)
        assert (BQ, BKV) in gen.GEOMETRIES_C5
        assert M.shape == (24, -(-115200 // BQ), -(-115200 // BKV))
        dh = np.array([stats.density(M[h]) for h in range(24)])
        assert dh.max() <= 0.501
        seen.add((BQ, BKV))
    assert len(seen) >= 2


def test_qkv_deterministic_bf16():
    import torch
    a = gen.qkv(2, 100, 16, (1, 2, 3))
    b = gen.qkv(2, 100, 16, (1, 2, 3))
    assert all(x.dtype == torch.bfloat16 and x.shape == (2, 100, 16) for x in a)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[0], a[1])
    assert abs(float(a[0].float().std()) - 1.0) < 0.05
