"""Helpers shared by the GPU tests: run the library on a case, compare with the
oracle, expand exported tiles to cell coverage."""

import numpy as np
import torch

import dynamic_block_sparse_bsa_amd as bsa

MAX_ERR = 1e-2   # max |GPU - oracle| on bf16-rounded inputs, fp32 accumulation
MEAN_ERR = 1e-3  # mean |GPU - oracle|


def gpu_run(M, q, k, v, block, force_plan=-1, force_split=-1, workspace_limit=0):
    H, N, d = q.shape
    dev = torch.device("cuda")
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev)
    p = bsa.plan(Md, block, H, N, d, force_plan=force_plan, force_split=force_split,
                 workspace_limit=workspace_limit)
    out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    bsa.run(p, q.to(dev), k.to(dev), v.to(dev), out)
    torch.cuda.synchronize()
    return p, out


def assert_close(out, ref, where=""):
    o = out.float().cpu().numpy().astype(np.float64) if isinstance(out, torch.Tensor) else out
    assert not np.isnan(o).any(), f"NaN in output {where}"
    err = np.abs(o - ref)
    assert err.max() <= MAX_ERR, f"max err {err.max():.3e} {where}"
    assert err.mean() <= MEAN_ERR, f"mean err {err.mean():.3e} {where}"
    return float(err.max()), float(err.mean())


def tile_cells(p, block, N):
    """Multiplicity with which the plan's exported tiles cover each cell."""
    info = p.info
    TQ, TKV = info["tile_q"], info["tile_kv"]
    cQ, cKV = info["coarsen_q"], info["coarsen_kv"]
    BQ, BKV = block
    cq, ckv = min(BQ, TQ), min(BKV, TKV)
    nq, nk = -(-N // cq), -(-N // ckv)
    head, qt, kt, bits = p.export_tiles()
    cov = np.zeros((p.H * p.batch, nq, nk), dtype=np.int64)  # every (batch entry, head)
    for a in range(cQ):
        for b in range(cKV):
            sel = ((bits >> np.uint32(a * cKV + b)) & 1).astype(bool)
            r = qt[sel].astype(np.int64) * cQ + a
            c = kt[sel].astype(np.int64) * cKV + b
            ok = (r < nq) & (c < nk)
            assert ok.all(), "membership bit set outside the mask grid"
            np.add.at(cov, (head[sel], r, c), 1)
    return cov, cq, ckv


def cell_counts_by_head(p, block, N):
    """Per head h, the multiplicity with which the plan's exported tiles cover
    each cell of min(B_Q, T_Q) x min(B_KV, T_KV) tokens: yields (h, counts
    [nq, nk] int64).  Tiles are grouped by head first, so memory stays at one
    head's cell grid at full workload sizes."""
    info = p.info
    TQ, TKV = info["tile_q"], info["tile_kv"]
    cQ, cKV = info["coarsen_q"], info["coarsen_kv"]
    BQ, BKV = block
    cq, ckv = min(BQ, TQ), min(BKV, TKV)
    nq, nk = -(-N // cq), -(-N // ckv)
    head, qt, kt, bits = p.export_tiles()
    order = np.argsort(head, kind="stable")
    head, qt, kt, bits = head[order], qt[order], kt[order], bits[order]
    bounds = np.searchsorted(head, np.arange(p.H * p.batch + 1))
    assert bounds[-1] == head.size, "tile with a head index out of range"
    for h in range(p.H * p.batch):
        s, e = bounds[h], bounds[h + 1]
        q_h = qt[s:e].astype(np.int64)
        k_h = kt[s:e].astype(np.int64)
        b_h = bits[s:e]
        cnt = np.zeros(nq * nk, dtype=np.int64)
        for a in range(cQ):
            for b in range(cKV):
                sel = ((b_h >> np.uint32(a * cKV + b)) & 1).astype(bool)
                r = q_h[sel] * cQ + a
                c = k_h[sel] * cKV + b
                assert ((r >= 0) & (r < nq) & (c >= 0) & (c < nk)).all(), \
                    "membership bit set outside the mask grid"
                cnt += np.bincount(r * nk + c, minlength=nq * nk)
        yield h, cnt.reshape(nq, nk)
