"""A decision-tree plan table on the GPU (Tessera paper, section 5.1: the
second-stage regime boundaries may be thresholds learned by a decision tree
whose leaves are the regimes).

The shipped profiling records are compiled with a tree partition into `rule`
lines, the text artifact is loaded through bsa_table_load, and requests of
profiled keys are planned on the GPU: the regime the library reports must be
a tree leaf (a `rule` line), the plan must be that leaf's first eligible
plan (the host lookup on the same statistics, bsa_select), and the output
must match the fp64 oracle.
"""

import json
import os

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from dynamic_block_sparse_bsa_amd import profile_table as pt
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tree_table(tmp_path_factory):
    tables = os.path.join(os.path.dirname(pt.__file__), "tables")
    with open(os.path.join(tables, "gfx950_v2_records.json")) as f:
        recs = json.load(f)
    for r in recs:
        r["block"] = tuple(r["block"])
        r["latency"] = {int(k): v for k, v in r["latency"].items()}
    text = pt.compile_table(recs, "vtree-test", ("tree", 3))
    path = tmp_path_factory.mktemp("tree") / "tree.txt"
    path.write_text(text)
    heads = [ln.split(" : ")[0] for ln in text.splitlines() if ln.startswith(("regime ", "rule "))]
    bsa.table_load(str(path))
    yield heads
    bsa.table_load(None)


@pytest.mark.parametrize("block,N,p", [((128, 128), 4096, 0.25), ((64, 64), 3000, 0.1), ((128, 32), 2048, 0.3)])
def test_request_through_a_tree_leaf(tree_table, block, N, p):
    heads = tree_table
    assert bsa.table_version() == "vtree-test"
    H, d = 4, 128
    M, q, k, v = gen.random_case(H, N, d, *block, p=p, seed=7100 + N, empty_rows={1: [0]})
    dev = torch.device("cuda")
    plan = bsa.plan(torch.from_numpy(M).to(dev), block, H, N, d)
    info = plan.info
    out = bsa.run(plan, q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    plan.destroy()
    assert info["regime"] >= 0 and heads[info["regime"]].startswith("rule "), heads[info["regime"]]
    # the host lookup on the statistics the GPU reported selects the same plan and leaf
    pid, reg = bsa.select(H, N, d, block, info["density"], info["run_coverage"], info["row_skew"])
    assert (pid, reg) == (info["plan_id"], info["regime"])
    assert_close(out, oatt.attention(q, k, v, M, *block), f"tree leaf {heads[reg]}")
