"""GPU parity for batch > 1 and the NHD layout (Tessera paper, section 4.4:
the request's tensor properties include the layout; section 5.1: batch size
is a request dimension).

Every (batch entry, head) pair is an independent head: the oracle computes
each on its own, in [head][N][d] order, and the test moves the data into and
out of the requested layout with torch permutes (data movement only).
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import assert_close

pytestmark = pytest.mark.gpu

CASES = [  # layout, batch, heads per entry, N, block, head dim
    ("NHD", 1, 3, 777, (64, 64), 128),
    ("NHD", 2, 3, 1000, (128, 32), 128),
    ("NHD", 3, 2, 1024, (32, 128), 128),
    ("HND", 2, 3, 777, (128, 128), 128),
    ("HND", 3, 1, 1500, (64, 32), 128),
    ("NHD", 2, 3, 777, (64, 64), 32),     # rows of H*d = 96 elements
    ("NHD", 2, 2, 1000, (128, 32), 256),  # rows of 512 elements
]


def _to_layout(x, batch, H, layout):
    """[batch*H][N][d] -> the layout's shape (contiguous)."""
    x = x.view(batch, H, *x.shape[1:])
    return (x.permute(0, 2, 1, 3) if layout == "NHD" else x).contiguous()


def _from_layout(x, layout):
    """The layout's [batch][...] -> [batch*H][N][d]."""
    if layout == "NHD":
        x = x.permute(0, 2, 1, 3)
    return x.reshape(-1, x.shape[2], x.shape[3])


@pytest.mark.parametrize("layout,batch,H,N,block,d", CASES)
def test_layout_and_batch_all_plans(layout, batch, H, N, block, d):
    Ht = batch * H
    seed = 700 + 13 * batch + N + block[0]
    M, q, k, v = gen.random_case(Ht, N, d, *block, p=0.3, seed=seed, empty_rows={Ht - 1: [0]},
                                 dense_heads=(0,))
    ref = oatt.attention(q, k, v, M, *block)
    dev = torch.device("cuda")
    qd, kd, vd = (_to_layout(t.to(dev), batch, H, layout) for t in (q, k, v))
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev).view(batch, H, *M.shape[1:])
    plans = [e["id"] for e in bsa.catalog() if bsa.eligible(e["id"], H, N, d, block, batch=batch, layout=layout)]
    assert len(plans) >= (6 if d == 128 else 1)
    for pid in plans:
        for fs in (-1, 1, bsa.SPLIT_STREAM):
            p = bsa.plan(Md, block, H, N, d, force_plan=pid, force_split=fs, batch=batch, layout=layout)
            out = torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device=dev)
            bsa.run(p, qd, kd, vd, out)
            torch.cuda.synchronize()
            assert_close(_from_layout(out, layout), ref, f"{layout} batch {batch} d {d} plan {pid} split {fs}")
            p.destroy()


def test_layouts_agree_bitwise():
    """The same request in HND and NHD runs the same arithmetic: identical
    outputs after the permute, for the table's own plan choice."""
    batch, H, N, d, block = 2, 4, 3000, 128, (64, 64)
    M, q, k, v = gen.random_case(batch * H, N, d, *block, p=0.2, seed=77)
    dev = torch.device("cuda")
    Md = torch.from_numpy(M).to(dev)
    outs = {}
    for layout in ("HND", "NHD"):
        qd, kd, vd = (_to_layout(t.to(dev), batch, H, layout) for t in (q, k, v))
        p = bsa.plan(Md, block, H, N, d, batch=batch, layout=layout)
        outs[layout] = _from_layout(bsa.run(p, qd, kd, vd), layout)
        torch.cuda.synchronize()
        p.destroy()
    assert torch.equal(outs["HND"], outs["NHD"])
