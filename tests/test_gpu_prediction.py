"""Speculative task lists for repeated request keys: the task builder of the
entry a key selected last time is queued before the statistics reach the
host and used when the selection agrees.  Both paths must give the same task
set and oracle-correct outputs, and the plan reports which one it took."""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import assert_close

pytestmark = pytest.mark.gpu


def _predictable(e, block):
    # uncoarsened in both dimensions (the task builder walks the block-CSR)
    return e["tile_q"] <= block[0] and e["tile_kv"] <= block[1]


def _run(M, q, k, v, block, force_plan=-1):
    H, N, d = q.shape
    dev = torch.device("cuda")
    p = bsa.plan(torch.from_numpy(np.ascontiguousarray(M)).to(dev), block, H, N, d, force_plan=force_plan)
    out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    bsa.run(p, q.to(dev), k.to(dev), v.to(dev), out)
    torch.cuda.synchronize()
    return p, out


def _task_set(p):
    return sorted(zip(*[a.tolist() for a in p.export_tasks()]))


def test_forced_entry_repeats_use_the_speculative_list():
    """Same key (forced uncoarsened entry), masks of changing density: from
    the second request on the task list is the speculative one, equal as a
    set to a fresh build, and every output matches the oracle."""
    H, N, d, block = 2, 2003, 64, (64, 64)
    cat = bsa.catalog()
    pid = next(e["id"] for e in cat if e["name"] == "T64x32_d64_splitk_xcd128")
    seen = []
    for i, rho in enumerate((0.2, 0.2, 0.5, 0.05)):
        M, q, k, v = gen.random_case(H, N, d, *block, p=rho, seed=8100 + i, empty_rows={0: [3]},
                                     dense_heads=(1,) if i == 2 else ())
        p, out = _run(M, q, k, v, block, force_plan=pid)
        info = p.info
        assert info["plan_id"] == pid
        seen.append(info["tasks_predicted"])
        assert_close(out, oatt.attention(q, k, v, M, *block), f"request {i}")
        if i == 1:
            # the same request again, built after the selection: same task set
            spec = _task_set(p)
            p.destroy()
            fresh_key = bsa.plan(torch.from_numpy(M).cuda(), block, H, N, d, force_plan=pid,
                                 force_split=-1, workspace_limit=1 << 40)  # a key not seen before
            assert fresh_key.info["tasks_predicted"] == 0
            assert _task_set(fresh_key) == spec
            fresh_key.destroy()
        else:
            p.destroy()
    assert seen[1:] == [1, 1, 1]


def test_table_selection_sequence():
    """Table-selected plans over a sequence of densities: a request takes the
    speculative list exactly when the previous request of the key chose the
    same uncoarsened entry; outputs always match the oracle."""
    H, N, d, block = 2, 1999, 128, (128, 128)
    cat = {e["id"]: e for e in bsa.catalog()}
    prev = None
    for i, rho in enumerate((0.1, 0.1, 0.45, 0.45, 0.1)):
        M, q, k, v = gen.random_case(H, N, d, *block, p=rho, seed=8200 + i)
        p, out = _run(M, q, k, v, block)
        info = p.info
        expect = int(prev is not None and prev == info["plan_id"] and _predictable(cat[prev], block))
        assert info["tasks_predicted"] == expect, (i, prev, info["plan_id"])
        assert_close(out, oatt.attention(q, k, v, M, *block), f"request {i}")
        prev = info["plan_id"]
        p.destroy()


@pytest.mark.parametrize("layout,batch", [("NHD", 2), ("HND", 3)])
def test_speculative_list_with_batch_and_layout(layout, batch):
    """Repeats of a batched request in either layout (forced uncoarsened
    entry, so the key's selection repeats): from the second request on the
    list is speculative and the outputs match the oracle head by head."""
    H, N, d, block = 2, 1501, 128, (64, 64)
    Ht = batch * H
    pid = next(e["id"] for e in bsa.catalog() if e["name"] == "T64x64_d128_splitk_xcd")
    dev = torch.device("cuda")
    flags = []
    for i in range(3):
        M, q, k, v = gen.random_case(Ht, N, d, *block, p=0.25 + 0.1 * i, seed=8300 + 10 * batch + i,
                                     empty_rows={Ht - 1: [0]})
        ref = oatt.attention(q, k, v, M, *block)
        to = (lambda x: x.to(dev).view(batch, H, N, d).permute(0, 2, 1, 3).contiguous()) if layout == "NHD" \
            else (lambda x: x.to(dev).view(batch, H, N, d).contiguous())
        qd, kd, vd = to(q), to(k), to(v)
        Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev).view(batch, H, *M.shape[1:])
        p = bsa.plan(Md, block, H, N, d, force_plan=pid, batch=batch, layout=layout)
        out = bsa.run(p, qd, kd, vd)
        torch.cuda.synchronize()
        if layout == "NHD":
            out = out.permute(0, 2, 1, 3)
        assert_close(out.reshape(Ht, N, d), ref, f"{layout} batch {batch} request {i}")
        flags.append(p.info["tasks_predicted"])
        p.destroy()
    assert flags[1:] == [1, 1]


def test_speculative_list_for_a_large_mask():
    """Large mask (the multi-kernel mask state, the speculative builder
    queued behind the scan): repeats take the speculative list, sampled rows
    match the oracle, and the task set equals a fresh build's."""
    H, N, d, block = 4, 20011, 64, (64, 64)
    pid = next(e["id"] for e in bsa.catalog() if e["name"] == "T64x32_d64_nosplit_lpt")
    rng = np.random.default_rng(8400)
    dev = torch.device("cuda")
    flags, sets = [], []
    for i in range(3):
        M, q, k, v = gen.random_case(H, N, d, *block, p=0.08 + 0.04 * i, seed=8400 + i)
        assert M.size > 32768  # not the single-launch mask state
        p = bsa.plan(torch.from_numpy(np.ascontiguousarray(M)).to(dev), block, H, N, d, force_plan=pid)
        out = bsa.run(p, q.to(dev), k.to(dev), v.to(dev))
        torch.cuda.synchronize()
        rows = {h: np.sort(rng.choice(N, 64, replace=False)) for h in range(H)}
        ref = oatt.attention_rows(q, k, v, M, *block, rows)
        o = out.float().cpu().numpy()
        for h, r in rows.items():
            assert_close(o[h, r], ref[h], f"request {i} head {h}")
        flags.append(p.info["tasks_predicted"])
        if i == 2:
            sets.append(_task_set(p))
            fresh = bsa.plan(torch.from_numpy(np.ascontiguousarray(M)).to(dev), block, H, N, d, force_plan=pid,
                             workspace_limit=1 << 40)
            assert fresh.info["tasks_predicted"] == 0
            sets.append(_task_set(fresh))
            fresh.destroy()
        p.destroy()
    assert flags[1:] == [1, 1]
    assert sets[0] == sets[1]
