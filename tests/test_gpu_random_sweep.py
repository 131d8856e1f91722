"""GPU parity on a seeded random sweep of requests.

Each case draws a head dim (32, 64, 128, 256), a logical block geometry
(B_Q, B_KV each a power of two from 16 to 256), a ragged length N, a head
count, a batch size and a layout (HND or NHD), a mask family (i.i.d. blocks
with the diagonal, some heads all active or with empty rows; or clustered
top-k with empty rows) and density, and then either the table's plan or a
random eligible catalog plan with a random split mode (none, the plan's
rule, partitions of 1, 2 or 5 entries, or the stream organization).  The
whole output is compared with the fp64 oracle (Tessera paper, section 2.2:
masked attention over E(M); empty rows are zero), and the plan's exported
tiles must cover E(M) exactly (section 4.2), whatever mapping and
organization the draw produced.  Cases with no eligible plan must be refused
as unsupported.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from oracle import coverage
from workloads import gen

from bsa_testutil import assert_close, tile_cells

pytestmark = pytest.mark.gpu

NCASES = 400
SPLITS = (-1, 0, 1, 2, 5, bsa.SPLIT_STREAM)


def _draw(i):
    rng = np.random.default_rng(880000 + i)
    d = int(rng.choice([32, 64, 128, 256]))
    block = (int(2 ** rng.integers(4, 9)), int(2 ** rng.integers(4, 9)))
    N = int(rng.integers(1, 2500))
    H = int(rng.integers(1, 4))
    batch = int(rng.integers(1, 3))
    layout = str(rng.choice(["HND", "NHD"]))
    seed = 881000 + 10 * i
    Ht = batch * H
    if rng.random() < 0.5:
        rows = {Ht - 1: [0]} if rng.random() < 0.5 else None
        M = gen.mask_iid_diag(Ht, N, *block, float(rng.uniform(0.02, 0.6)), seed,
                              dense_heads=(0,) if rng.random() < 0.3 else (), empty_rows=rows)
    else:
        lo = float(rng.uniform(0.02, 0.4))
        M = gen.mask_clustered(Ht, N, *block, seed, rho=(lo, min(1.0, 2 * lo)), p_empty_head=0.3)
    return rng, d, block, N, H, batch, layout, M, seed


def _to_layout(x, batch, H, layout):
    x = x.view(batch, H, *x.shape[1:])
    return (x.permute(0, 2, 1, 3) if layout == "NHD" else x).contiguous()


def _from_layout(x, layout):
    if layout == "NHD":
        x = x.permute(0, 2, 1, 3)
    return x.reshape(-1, x.shape[2], x.shape[3])


@pytest.mark.parametrize("i", range(NCASES))
def test_random_request(i):
    rng, d, block, N, H, batch, layout, M, seed = _draw(i)
    Ht = batch * H
    label = f"case {i}: d={d} B={block} N={N} H={H} batch={batch} {layout}"
    eligible = [e["id"] for e in bsa.catalog() if bsa.eligible(e["id"], H, N, d, block, batch=batch, layout=layout)]
    dev = torch.device("cuda")
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev).view(batch, H, *M.shape[1:])
    if not eligible:
        with pytest.raises(bsa.BsaError):
            bsa.plan(Md, block, H, N, d, batch=batch, layout=layout)
        return
    force = -1 if rng.random() < 0.4 else int(rng.choice(eligible))
    fs = int(rng.choice(SPLITS))
    label += f" plan {force} split {fs}"
    q, k, v = gen.qkv(Ht, N, d, (seed + 1, seed + 2, seed + 3))
    ref = oatt.attention(q, k, v, M, *block)
    qd, kd, vd = (_to_layout(t.to(dev), batch, H, layout) for t in (q, k, v))
    p = bsa.plan(Md, block, H, N, d, force_plan=force, force_split=fs, batch=batch, layout=layout)
    out = torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    bsa.run(p, qd, kd, vd, out)
    torch.cuda.synchronize()
    label += f" -> {p.info['plan_id']}"
    assert_close(_from_layout(out, layout), ref, label)
    cov, cq, ckv = tile_cells(p, block, N)
    assert (cov == coverage.cells(M, *block, N, cq, ckv)).all(), f"{label}: coverage"
    p.destroy()
