"""GPU: task organizations (grouping, traversal order, K/V partitions).

Tessera paper, section 3 (task organization: grouping, traversal order,
number of K/V reduction partitions) and section 4.3 ("Grouping and
traversal", "Split-K").  For every catalog plan whose tiles neither coarsen
nor merge logical blocks on the query side (so a query tile's tile-list row
is its logical row of the shared block-CSR), the exported task list is
checked against the organization's definition:

* every query tile's row of n entries is cut into p = ceil(n / split)
  contiguous partitions of ceil(n / p) entries (one task when split == 0 or
  n <= split; rows without entries still get one empty task);
* split partitions own distinct, consecutive workspace slots, unsplit tasks
  none;
* query-tile order lists tasks by (head, query tile, begin); longest-first
  order lists the same tasks by non-increasing length; signature order lists
  them by head, and within a head by non-decreasing band of the median column
  of the query tile's row (8192 / H bands over the row's columns).

Two of the masks are large enough (more than 8192 query tiles for every
uncoarsened tile shape) that the task builder walks several chunks of its
counting sort, the third fits one chunk; sampled output rows of each
longest-first plan are checked against the oracle.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import MAX_ERR, MEAN_ERR

pytestmark = pytest.mark.gpu


def _expected_tasks(rp, H, nqb, nqt_head, refine_q, split, split_min):
    out = []
    for h in range(H):
        for qt in range(nqt_head):
            i = h * nqb + qt // refine_q
            b, e = int(rp[i]), int(rp[i + 1])
            n = e - b
            p = -(-n // split) if (split > 0 and n > split_min) else 1
            ch = -(-n // p)
            for j in range(p):
                out.append((h, qt, min(e, b + j * ch), min(e, b + (j + 1) * ch), p > 1))
    return out


def _expected_stream(rp, H, nqb, nqt_head, refine_q, G):
    """Stream organization: the concatenated entries (W) cut into
    Ge = min(G, W) ranges [ceil(kW/Ge), ceil((k+1)W/Ge)); a tile becomes one
    task per range it overlaps (an empty tile: one task at its position)."""
    rows = []
    for h in range(H):
        for qt in range(nqt_head):
            i = h * nqb + qt // refine_q
            rows.append((h, qt, int(rp[i]), int(rp[i + 1])))
    W = sum(e - b for _, _, b, e in rows)
    Ge = min(G, W) if W > 0 else 1
    out, P = [], 0
    for h, qt, b, e in rows:
        n = e - b
        if n == 0:
            out.append((h, qt, b, b, False))
            continue
        w0, w1 = min(Ge - 1, P * Ge // W), min(Ge - 1, (P + n - 1) * Ge // W)
        for w in range(w0, w1 + 1):
            cb, ce = -(-w * W // Ge), -(-(w + 1) * W // Ge)
            out.append((h, qt, b + max(P, cb) - P, b + min(P + n, ce) - P, w1 > w0))
        P += n
    return out, W, Ge


# (block, N, H, uncoarsened catalog entries that must be checked)
CASES = [((64, 64), 70000, 8, 2), ((128, 128), 9000, 6, 6), ((128, 32), 90000, 12, 7)]


@pytest.mark.parametrize("block,N,H,min_checked", CASES)
def test_task_organizations(block, N, H, min_checked):
    d = 128
    M = gen.mask_clustered(H, N, *block, seed=4242 + N, rho=(0.05, 0.45), p_empty_head=0.25)
    nqb = M.shape[1]
    dev = torch.device("cuda")
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev)
    q = k = v = None
    checked = 0
    for e in bsa.catalog():
        if not bsa.eligible(e["id"], H, N, d, block):
            continue
        p = bsa.plan(Md, block, H, N, d, force_plan=e["id"])
        info = p.info
        if info["coarsen_q"] != 1 or info["coarsen_kv"] != 1:
            p.destroy()
            continue
        rp, cols = p.export_csr()
        head, qt, beg, end, slot = p.export_tasks()
        nqt_head = -(-N // info["tile_q"])
        label_pre = f"{e['name']} B={block} N={N}: split threshold"
        exp = _expected_tasks(rp, H, nqb, nqt_head, info["refine_q"], info["split_items"],
                              info["split_threshold"])
        if info["split_items"] > 0:
            # the balance rule keeps rows of up to twice the mean length whole
            mean = -(-int(rp[-1]) * info["refine_q"] // (H * nqt_head))
            assert info["split_threshold"] == max(info["split_items"], 2 * mean), label_pre
        got = list(zip(head.tolist(), qt.tolist(), beg.tolist(), end.tolist(), (slot >= 0).tolist()))
        label = f"{e['name']} B={block} N={N}"
        assert sorted(got) == sorted(exp), f"{label}: task multiset"
        if e["order"] == 0 and e["xcd_remap"] == 0:
            assert got == exp, f"{label}: query-tile order"
        if e["order"] == 1:
            ln = end - beg
            assert (np.diff(ln) <= 0).all(), f"{label}: not longest first"
        if e["order"] == 2:
            nkt = M.shape[2]  # uncoarsened: the tile list is the block-CSR
            bph = max(1, 8192 // H)
            key = []
            for h_, q_ in zip(head.tolist(), qt.tolist()):
                i = h_ * nqb + q_ // info["refine_q"]
                b_, e_ = int(rp[i]), int(rp[i + 1])
                sig = int(cols[(b_ + e_ - 1) // 2]) if e_ > b_ else 0
                key.append(min(8191, h_ * bph + min(bph - 1, sig * bph // max(nkt, 1))))
            assert (np.diff(np.array(key)) >= 0).all(), f"{label}: not in signature order"
        # split slots: distinct, consecutive per query tile in partition order
        s = slot[slot >= 0]
        assert len(np.unique(s)) == len(s), f"{label}: shared slot"
        o = np.lexsort((beg, qt, head))
        same = (head[o][1:] == head[o][:-1]) & (qt[o][1:] == qt[o][:-1])
        assert (np.diff(slot[o])[same] == 1).all(), f"{label}: slots not consecutive per query tile"
        assert (slot[o][1:][same] >= 0).all(), f"{label}: split tile with an unslotted part"
        if e["order"] == 1:
            if q is None:
                q, k, v = gen.qkv(H, N, d, (11, 12, 13))
                qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
                rng = np.random.default_rng(N)
                rows = {h: np.unique(np.concatenate([rng.integers(0, N, 96), [N - 1]]))
                        for h in range(H)}
                ref = oatt.attention_rows(q, k, v, M, block[0], block[1], rows)
            out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
            bsa.run(p, qd, kd, vd, out)
            torch.cuda.synchronize()
            assert not torch.isnan(out).any().item(), f"{label}: unwritten rows"
            err = np.concatenate([np.abs(out[h, torch.from_numpy(r).to(dev)].float().cpu().numpy()
                                         .astype(np.float64) - ref[h]) for h, r in rows.items()])
            assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR, \
                f"{label}: max {err.max():.3e} mean {err.mean():.3e}"
        p.destroy()
        checked += 1
    assert checked >= min_checked


@pytest.mark.parametrize("block,N,H", [c[:3] for c in CASES] + [((64, 64), 3000, 1)])
def test_stream_organization(block, N, H):
    """force_split = SPLIT_STREAM: tasks are the tiles' intersections with G
    equal entry ranges (G = the plan's grid), in tile order; every range holds
    floor or ceil of W/G entries; sampled rows match the oracle."""
    d = 128
    M = gen.mask_clustered(H, N, *block, seed=777 + N, rho=(0.05, 0.45), p_empty_head=0.25)
    nqb = M.shape[1]
    dev = torch.device("cuda")
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev)
    q, k, v = gen.qkv(H, N, d, (21, 22, 23))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    rng = np.random.default_rng(N + 1)
    rows = {h: np.unique(np.concatenate([rng.integers(0, N, 64), [0, N - 1]])) for h in range(H)}
    ref = oatt.attention_rows(q, k, v, M, block[0], block[1], rows)
    checked = 0
    for e in bsa.catalog():
        if e["order"] != 0 or e["xcd_remap"] != 0 or e["split"] != 2 or not bsa.eligible(e["id"], H, N, d, block):
            continue
        p = bsa.plan(Md, block, H, N, d, force_plan=e["id"], force_split=bsa.SPLIT_STREAM)
        info = p.info
        label = f"{e['name']} B={block} N={N} H={H}"
        out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
        bsa.run(p, qd, kd, vd, out)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item(), f"{label}: unwritten rows"
        err = np.concatenate([np.abs(out[h, torch.from_numpy(r).to(dev)].float().cpu().numpy()
                                     .astype(np.float64) - ref[h]) for h, r in rows.items()])
        assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR, f"{label}: max {err.max():.3e} mean {err.mean():.3e}"
        if info["coarsen_q"] == 1 and info["coarsen_kv"] == 1:
            rp, _ = p.export_csr()
            head, qt, beg, end, slot = p.export_tasks()
            nqt_head = -(-N // info["tile_q"])
            exp, W, Ge = _expected_stream(rp, H, nqb, nqt_head, info["refine_q"], info["grid"])
            got = list(zip(head.tolist(), qt.tolist(), beg.tolist(), end.tolist(), (slot >= 0).tolist()))
            assert got == exp, f"{label}: stream tasks"
            s = slot[slot >= 0]
            assert len(np.unique(s)) == len(s), f"{label}: shared slot"
            # range sizes: each range is floor or ceil of W / Ge entries
            sizes = [-(-(w + 1) * W // Ge) - -(-w * W // Ge) for w in range(Ge)]
            assert min(sizes) >= W // Ge and max(sizes) <= -(-W // Ge)
        p.destroy()
        checked += 1
    assert checked >= 3
