"""GPU: the plan cache for warm exact repeats (Tessera paper, section 7.4:
repeats of a request reuse its prepared plan state).

A repeat must be recognized only when the request (geometry and options) and
every mask byte match; whatever the cache returns must produce the oracle's
output for the mask actually passed.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import assert_close

pytestmark = pytest.mark.gpu


def _run(p, q, k, v):
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    bsa.run(p, q, k, v, out)
    torch.cuda.synchronize()
    return out


def test_plan_cache_exact_repeats():
    dev = torch.device("cuda")
    H, N, d, block = 3, 1500, 128, (64, 64)
    M, q, k, v = gen.random_case(H, N, d, *block, p=0.3, seed=31, empty_rows={1: [0]})
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cache = bsa.PlanCache(capacity=2)
    try:
        a = torch.from_numpy(M).to(dev)
        p1, hit = cache.get(a, block, H, N, d)
        assert not hit
        assert_close(_run(p1, qd, kd, vd), oatt.attention(q, k, v, M, *block), "first request")
        # the same mask in another buffer: a repeat, the same prepared plan
        b = a.clone()
        p2, hit = cache.get(b, block, H, N, d)
        assert hit and p2.handle.value == p1.handle.value
        assert_close(_run(p2, qd, kd, vd), oatt.attention(q, k, v, M, *block), "repeat")
        # one byte changed (the last block of the last head): not a repeat
        M2 = M.copy()
        M2[-1, -1, -1] ^= 1
        c = torch.from_numpy(M2).to(dev)
        p3, hit = cache.get(c, block, H, N, d)
        assert not hit
        assert_close(_run(p3, qd, kd, vd), oatt.attention(q, k, v, M2, *block), "changed mask")
        # other options with the same mask: not a repeat
        _, hit = cache.get(b, block, H, N, d, force_split=2)
        assert not hit
        # capacity 2: the first mask's plan was evicted (least recently used)
        _, hit = cache.get(a, block, H, N, d)
        assert not hit
        # and the changed mask's plan too (M2 was used before the force_split one)
        p5, hit = cache.get(c, block, H, N, d)
        assert not hit
        assert_close(_run(p5, qd, kd, vd), oatt.attention(q, k, v, M2, *block), "changed mask again")
        p6, hit = cache.get(c, block, H, N, d)
        assert hit and p6.handle.value == p5.handle.value
    finally:
        cache.destroy()


def test_plan_cache_ragged_and_unaligned_mask():
    """Mask bytes not a multiple of 16 and a mask that starts at an odd offset
    (the byte-wise comparison path)."""
    dev = torch.device("cuda")
    H, N, d, block = 2, 777, 64, (64, 32)
    M, q, k, v = gen.random_case(H, N, d, *block, p=0.4, seed=5)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    flat = torch.zeros(M.size + 1, dtype=torch.uint8, device=dev)
    flat[1:] = torch.from_numpy(M.reshape(-1)).to(dev)
    odd = flat[1:].view(M.shape)  # data pointer one byte past an aligned allocation
    assert odd.data_ptr() % 16 == 1
    cache = bsa.PlanCache(capacity=4)
    try:
        p1, hit = cache.get(torch.from_numpy(M).to(dev), block, H, N, d)
        assert not hit
        p2, hit = cache.get(odd, block, H, N, d)
        assert hit and p2.handle.value == p1.handle.value
        flat[-1] ^= 1  # last byte differs
        p3, hit = cache.get(odd, block, H, N, d)
        assert not hit
        M3 = M.copy()
        M3.reshape(-1)[-1] ^= 1
        assert_close(_run(p3, qd, kd, vd), oatt.attention(q, k, v, M3, *block), "unaligned changed mask")
    finally:
        cache.destroy()


def _xcd_plan(name):
    return next(e["id"] for e in bsa.catalog() if e["name"] == name)


@pytest.mark.parametrize("force_split,plan", [(-1, None), (1, None), (-2, None),
                                              (-1, "T128x64_d128_splitk_sim_xcd"), (1, "T128x32_d128_splitk_xcd")])
def test_plan_cache_run_speculative(force_split, plan):
    """bsa_plan_cache_run: the most recently used candidate runs behind the
    comparison, guarded by its verdict.  Every output must match the oracle
    for the mask passed, whether that candidate matched (hit), another one
    did (hit on an older entry) or none did (miss, new plan); force_split=1
    makes every split-K path (and its merge) part of the guarded run.  With
    an XCD organization forced, the guarded runs also go through the per-XCD
    task queues, which are reset before every launch: a guarded run that must
    do nothing leaves them empty, and the next run must still cover every
    task."""
    dev = torch.device("cuda")
    H, N, d, block = 2, 1300, 128, (64, 64)
    masks = []
    for s in range(3):
        M, q, k, v = gen.random_case(H, N, d, *block, p=0.25 + 0.1 * s, seed=400 + s, empty_rows={0: [1]})
        masks.append(M)
    q, k, v = gen.qkv(H, N, d, (41, 42, 43))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    refs = [oatt.attention(q, k, v, M, *block) for M in masks]
    cache = bsa.PlanCache(capacity=3)

    def go(i, want_hit):
        out = torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device=dev)
        o, hit = cache.run(torch.from_numpy(masks[i]).to(dev), block, H, N, d, qd, kd, vd, out,
                           force_split=force_split, force_plan=_xcd_plan(plan) if plan else -1)
        torch.cuda.synchronize()
        assert hit == want_hit, (i, hit)
        assert_close(o, refs[i], f"mask {i} hit {hit}")

    try:
        go(0, False)  # miss: plan and run
        go(0, True)   # repeat: the speculated candidate matches
        go(1, False)  # differs from the speculated candidate: guarded run does nothing, new plan
        go(2, False)
        go(0, True)   # candidate 0 (mask 2) differs, an older one matches
        go(0, True)
        go(1, True)
    finally:
        cache.destroy()
