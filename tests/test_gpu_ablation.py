"""The selection-quality ablation harness on the GPU (Tessera paper, section
7.4 and Table 7: Direct mapping A0, exhaustive online probing A1, the plan
table A2), on three held-out cases (one at head dim 256): the harness runs end to end, its summary
is consistent with its rows, and the plan the table selects for each case
(A2) reproduces the fp64 oracle's output through the library."""

import numpy as np
import pytest

import dynamic_block_sparse_bsa_amd as bsa
from dynamic_block_sparse_bsa_amd import ablation
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import assert_close, gpu_run

pytestmark = pytest.mark.gpu


def test_quick_ablation_and_selected_plan_against_oracle():
    cases, make_mask = ablation.heldout(quick=True)
    cases = [cases[0], cases[2], cases[6]]  # keys (64, 64) and (128, 32) at d = 128, (128, 32) at d = 256
    assert (cases[2]["d"], cases[2]["block"]) == (256, (128, 32))
    rows = ablation.run(cases, make_mask, reps=2, warmup=1, log=lambda s: print(s, flush=True))
    s = ablation.summarize(rows)
    assert s["cases"] == 3
    reg = [r["k_a2"] / r["k_best"] for r in rows]
    assert min(reg) >= 1.0 and s["selection_regret"]["max"] == pytest.approx(max(reg))
    assert s["A2_output_vs_reference"]["max_abs_err"] <= 1e-2
    for c, r in zip(cases, rows):
        assert r["fastest"] in r["latency"] and r["selected"] in r["latency"]
        H, N, d, block = c["H"], c["N"], c["d"], tuple(c["block"])
        M = make_mask(c)
        q, k, v = gen.qkv(H, N, d, (c["seed"] + 1, c["seed"] + 2, c["seed"] + 3))
        p, out = gpu_run(M, q, k, v, block)  # the table's selection, as A2
        names = {e["id"]: e["name"] for e in bsa.catalog()}
        assert names[p.info["plan_id"]] == r["selected"]
        p.destroy()
        assert_close(out, oatt.attention(q, k, v, np.asarray(M), *block), f"A2 {r['selected']}")
