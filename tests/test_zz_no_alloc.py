"""The entry point that allocates nothing, bsa_attention_noalloc, against the
existing path bsa_plan_create + bsa_run (same request, same inputs), through
the C ABI: two calls in a row on one device, the second with a smaller input
(the scratch keeps the first call's contents), each within the parity bar of
the oracle and of the existing path's output, for the table's plans and for
every plan of the XCD organizations (per-XCD task queues); a request whose
block-CSR does not fit the fixed scratch is refused with BSA_ERR_UNSUPPORTED
and leaves O untouched.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import assert_close, gpu_run

pytestmark = pytest.mark.gpu


def _noalloc(M, q, k, v, block):
    H, N, d = q.shape
    dev = torch.device("cuda")
    Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    bsa.attention_noalloc(Md, block, H, N, d, qd, kd, vd, out)
    torch.cuda.synchronize()
    return out


# (H, N, d, block, seed): the first call is the larger; both take split-K
# plans from the table at these sizes
CASES = [(8, 4096, 128, (128, 128), 31), (3, 1000, 64, (64, 32), 32)]


def test_two_calls_match_plan_and_run():
    for H, N, d, block, seed in CASES:
        M, q, k, v = gen.random_case(H, N, d, *block, p=0.3, seed=seed, empty_rows={1: [0, 2]},
                                     dense_heads=(H - 1,))
        ref = oatt.attention(q, k, v, M, *block)
        p, want = gpu_run(M, q, k, v, block)
        p.destroy()
        got = _noalloc(M, q, k, v, block)
        where = f"H={H} N={N} d={d} B={block}"
        assert_close(want, ref, "plan+run " + where)
        assert_close(got, ref, "noalloc " + where)
        diff = (got.float() - want.float()).abs()
        assert diff.max().item() <= 1e-2 and diff.mean().item() <= 1e-3, where
        print(f"{where}: noalloc vs plan+run max {diff.max().item():.2e}", flush=True)


def test_oversized_request_refused():
    # an all-active mask of 8 x 2048 x 2048 blocks: 33.5M block-CSR columns
    # (134 MB) cannot fit the 128 MiB scratch
    H, N, d, block = 8, 65536, 64, (32, 32)
    dev = torch.device("cuda")
    Md = torch.ones((H, N // 32, N // 32), dtype=torch.uint8, device=dev)
    q = torch.zeros((H, N, d), dtype=torch.bfloat16, device=dev)
    out = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    with pytest.raises(bsa.BsaError) as ei:
        bsa.attention_noalloc(Md, block, H, N, d, q, q, q, out)
    assert "BSA_ERR_UNSUPPORTED" in str(ei.value) and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(out).all().item()
    # the scratch still serves a request that fits afterwards
    test_two_calls_match_plan_and_run()


def test_xcd_queue_plans():
    """The XCD organizations dispatch through per-XCD task queues whose words
    are carved from the scratch as well: every such plan, two calls in a row
    (the second smaller; fewer tasks than one round of eight runs when the
    run is 128), against plan + run with the same plan and the oracle."""
    sizes = [(4, 4096, 128, (128, 32), 51), (2, 1500, 128, (128, 32), 52)]
    data = []
    for H, N, d, block, seed in sizes:
        M, q, k, v = gen.random_case(H, N, d, *block, p=0.25, seed=seed, empty_rows={0: [1]})
        data.append((M, q, k, v, oatt.attention(q, k, v, M, *block)))
    H0, N0, d0, b0, _ = sizes[0]
    ids = [e["id"] for e in bsa.catalog() if e["xcd_remap"] > 0 and bsa.eligible(e["id"], H0, N0, d0, b0)]
    assert len(ids) >= 4
    for pid in ids:
        for (H, N, d, block, _), (M, q, k, v, ref) in zip(sizes, data):
            where = f"plan {pid} H={H} N={N} d={d} B={block}"
            p, want = gpu_run(M, q, k, v, block, force_plan=pid)
            assert p.info["plan_id"] == pid, where
            p.destroy()
            dev = torch.device("cuda")
            Md = torch.from_numpy(np.ascontiguousarray(M)).to(dev)
            got = torch.full((H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
            torch.cuda.synchronize()
            bsa.attention_noalloc(Md, block, H, N, d, q.to(dev), k.to(dev), v.to(dev), got, force_plan=pid)
            torch.cuda.synchronize()
            assert_close(got, ref, "noalloc " + where)
            diff = (got.float() - want.float()).abs()
            assert diff.max().item() <= 1e-2 and diff.mean().item() <= 1e-3, where
