"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (regime-table plan selection, the plan's own split rule).

The oracle cannot compute every row at these sizes, so each case checks:
* sampled rows against ``oracle.attention_rows`` (the first, second-to-last
  and last query block of every head, the ragged tail, and 256 seeded random
  rows per head), to max |err| <= 1e-2 and mean |err| <= 1e-3;
* properties that hold at any size on the WHOLE output: no NaN (O starts
  NaN-filled, so an unwritten row fails), rows of empty query blocks are
  exactly zero, and |o| <= max |v| of the head (a convex combination).
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import MAX_ERR, MEAN_ERR

pytestmark = pytest.mark.gpu


def _sample_rows(N, BQ, H, seed, per_head=256):
    rng = np.random.default_rng(seed)
    nqb = -(-N // BQ)
    fixed = np.concatenate([np.arange(0, min(BQ, N)),
                            np.arange(max(0, (nqb - 2) * BQ), N)])
    rows = {}
    for h in range(H):
        r = np.unique(np.concatenate([fixed, rng.integers(0, N, per_head)]))
        rows[h] = r
    return rows


def _check_case(M, q, k, v, block, label, heads=None):
    H, N, d = q.shape
    dev = torch.device("cuda")
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    p = bsa.plan(Md, block, H, N, d)
    out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    bsa.run(p, qd, kd, vd, out)
    torch.cuda.synchronize()
    info = p.info
    p.destroy()
    # whole-output properties
    assert not torch.isnan(out).any().item(), f"{label}: NaN (unwritten or invalid rows)"
    vmax = vd.float().abs().amax(dim=(1, 2))
    omax = out.float().abs().amax(dim=(1, 2))
    assert bool((omax <= vmax * 1.02 + 1e-6).all()), f"{label}: |o| exceeds max |v|"
    empty = torch.from_numpy((np.asarray(M) != 0).sum(-1) == 0).to(dev)  # [H, nQB]
    if bool(empty.any()):
        rowblk = torch.arange(N, device=dev) // block[0]
        erows = empty[:, rowblk]  # [H, N]
        assert bool((out[erows].float() == 0).all()), f"{label}: empty rows not zero"
    # sampled rows against the oracle
    rows = _sample_rows(N, block[0], H, seed=N + block[0] + 7 * block[1])
    if heads is not None:
        rows = {h: rows[h] for h in heads}
    ref = oatt.attention_rows(q, k, v, M, block[0], block[1], rows)
    errs = []
    for h, r in rows.items():
        o = out[h, torch.from_numpy(r).to(dev)].float().cpu().numpy().astype(np.float64)
        errs.append(np.abs(o - ref[h]))
    e = np.concatenate(errs)
    assert e.max() <= MAX_ERR and e.mean() <= MEAN_ERR, \
        f"{label}: plan {info['plan_id']} max {e.max():.3e} mean {e.mean():.3e}"
    print(f"{label}: plan {info['plan_id']} T=({info['tile_q']},{info['tile_kv']}) split "
          f"{info['split_items']} max|err| {e.max():.2e} mean|err| {e.mean():.2e}", flush=True)


@pytest.mark.parametrize("c", [3, 4])
def test_fullsize_config(c):
    cfg = gen.config(c)
    _check_case(cfg["mask"], cfg["q"], cfg["k"], cfg["v"], (cfg["BQ"], cfg["BKV"]),
                f"config {c}")


@pytest.mark.parametrize("r", [0, 2, 6, 7])  # one request of each geometry
def test_fullsize_stream_request(r):
    cfg = gen.config(5, r)
    _check_case(cfg["mask"], cfg["q"], cfg["k"], cfg["v"], (cfg["BQ"], cfg["BKV"]),
                f"stream request {r} B=({cfg['BQ']},{cfg['BKV']})", heads=range(0, 24, 3))
