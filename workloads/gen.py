"""Generators for the five benchmark workloads and for test variants.

Seeds: workload c uses 1000*c + {0: mask, 1: Q, 2: K, 3: V}; request r of the
request stream uses 5000 + 10*r + {0, 1, 2, 3}.  Q, K and V are drawn per head
as float32 N(0, 1) from NumPy's PCG64 and rounded to bfloat16 (round to
nearest even, torch's ``.to(torch.bfloat16)``).  Token order is frame-major,
n = t*(Y*X) + y*X + x; a logical block takes the coordinates of its centre
token.

Mask families (uint8 [H, ceil(N/B_Q), ceil(N/B_KV)], nonzero = active):
* ``mask_iid_diag``        i.i.d. Bernoulli blocks plus the blocks that hold
                           a token pair (i, i)
* ``mask_spatiotemporal``  a temporal window of +-1 frame intersected with a
                           spatial neighbourhood whose radius is set per head
                           to hit a target density, plus i.i.d. random blocks
* ``mask_clustered``       top-k per query-block row of inner products of
                           low-rank cluster centroids; clusters are assigned
                           over contiguous segments, which produces runs
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

CONFIGS = {
    1: dict(name="tiny", H=1, N=1024, d=64, BQ=64, BKV=64),
    2: dict(name="medium", H=8, N=8192, d=128, BQ=128, BKV=128),
    3: dict(name="wan720p", H=40, N=75600, d=128, BQ=64, BKV=64, frames=21, Y=45, X=80),
    4: dict(name="hunyuan", H=24, N=115200, d=128, BQ=128, BKV=32, frames=30, Y=48, X=80),
    5: dict(name="stream", H=24, N=115200, d=128, frames=30, Y=48, X=80, requests=50),
}
GEOMETRIES_C5 = [(64, 64), (128, 128), (128, 32), (32, 128)]


def grid(N, BQ, BKV):
    return (-(-N // BQ), -(-N // BKV))


def _rng(seed, *extra):
    return np.random.Generator(np.random.PCG64([int(seed)] + [int(e) for e in extra]))


def mask_iid_diag(H, N, BQ, BKV, p, seed, dense_heads=(), empty_rows=None):
    """i.i.d. Bernoulli(p) blocks OR diagonal blocks.

    dense_heads: heads made all-active.  empty_rows: {head: [query-block rows]}
    whose blocks are all cleared (diagonal included).
    """
    nq, nk = grid(N, BQ, BKV)
    rng = _rng(seed)
    M = (rng.random((H, nq, nk)) < p).astype(np.uint8)
    # diagonal: blocks (a, b) that contain some token pair (i, i)
    i = np.arange(N)
    M[:, i // BQ, i // BKV] = 1
    for h in dense_heads:
        M[h] = 1
    for h, rows in (empty_rows or {}).items():
        M[h, list(rows)] = 0
    return M


def _block_centres(N, B, frames, Y, X):
    """(t, y, x) float coordinates of each block's centre token."""
    start = np.arange(-(-N // B)) * B
    end = np.minimum(start + B, N)
    c = (start + end - 1) / 2.0
    per = Y * X
    t = np.floor(c / per)
    rem = c - t * per
    y = np.floor(rem / X)
    x = rem - y * X
    return t, y, x


def mask_spatiotemporal(H, N, B, frames, Y, X, seed, rho=(0.10, 0.15), p_rand=0.03,
                        window=1):
    """Temporal window (|dt| <= window) AND spatial radius r_h, OR random blocks.

    For each head a target density rho_h ~ U[rho] is drawn; r_h is the smallest
    radius (in units of max(|dy|/Y, |dx|/X)) whose mask reaches rho_h, found as
    an order statistic of the pair distances (equivalent to a bisection on r).
    """
    n = -(-N // B)
    t, y, x = _block_centres(N, B, frames, Y, X)
    dt = np.abs(t[:, None] - t[None, :])
    dist = np.maximum(np.abs(y[:, None] - y[None, :]) / Y, np.abs(x[:, None] - x[None, :]) / X)
    inwin = dt <= window
    rng = _rng(seed)
    M = np.zeros((H, n, n), dtype=np.uint8)
    for h in range(H):
        target = rng.uniform(*rho)
        rand = rng.random((n, n)) < p_rand
        cand = np.sort(dist[inwin & ~rand])
        k = int(round(target * n * n)) - int(rand.sum())
        r = cand[min(k, cand.size) - 1] if k > 0 and cand.size else -1.0
        M[h] = (rand | (inwin & (dist <= r))).astype(np.uint8)
    return M


def _segment_clusters(rng, nblocks, mean_len, nclusters):
    """Cluster id per block, constant over contiguous segments."""
    out = np.empty(nblocks, dtype=np.int64)
    i = 0
    lam = max(mean_len - 1.0, 0.0)
    while i < nblocks:
        ln = 1 + int(rng.poisson(lam))
        out[i:i + ln] = rng.integers(nclusters)
        i += ln
    return out


def mask_clustered(H, N, BQ, BKV, seed, rho=(0.05, 0.30), nclusters=16, rank=8,
                   noise=0.3, seg_tokens=512, p_empty_head=0.0, empty_rows=(1, 4)):
    """Top-k per query-block row of <c_q, c_k> over low-rank cluster centroids.

    Per head: nclusters centres z ~ N(0, I_rank); query and key/value blocks
    get clusters over contiguous segments (mean span seg_tokens tokens);
    centroid = z[cluster] + noise * eps; k = round(rho_h * nKB), rho_h ~ U[rho].
    With probability p_empty_head a head clears 1-4 seeded query-block rows.
    """
    nq, nk = grid(N, BQ, BKV)
    rng = _rng(seed)
    M = np.zeros((H, nq, nk), dtype=np.uint8)
    for h in range(H):
        z = rng.standard_normal((nclusters, rank))
        cq = _segment_clusters(rng, nq, seg_tokens / BQ, nclusters)
        ck = _segment_clusters(rng, nk, seg_tokens / BKV, nclusters)
        eq = z[cq] + noise * rng.standard_normal((nq, rank))
        ek = z[ck] + noise * rng.standard_normal((nk, rank))
        score = eq @ ek.T
        rho_h = rng.uniform(*rho)
        k = min(nk, max(1, int(round(rho_h * nk))))
        top = np.argpartition(-score, k - 1, axis=1)[:, :k]
        np.put_along_axis(M[h], top, 1, axis=1)
        if p_empty_head > 0 and rng.random() < p_empty_head:
            cnt = int(rng.integers(empty_rows[0], empty_rows[1] + 1))
            rows = rng.choice(nq, size=min(cnt, nq), replace=False)
            M[h, rows] = 0
    return M


def qkv(H, N, d, seeds, threads=8, std=(1.0, 1.0, 1.0)):
    """bf16 CPU tensors Q, K, V [H, N, d]; element ~ N(0, std^2) float32 then
    RNE (std per tensor; the default is the workloads' N(0, 1))."""
    import torch

    out = []
    for s, sd in zip(seeds, std):
        t = torch.empty((H, N, d), dtype=torch.bfloat16)

        def fill(h, s=s, t=t, sd=sd):
            a = _rng(s, h).standard_normal((N, d), dtype=np.float32)
            if sd != 1.0:
                a *= np.float32(sd)
            t[h] = torch.from_numpy(a).to(torch.bfloat16)

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(H)))
        out.append(t)
    return tuple(out)


def qkv_device(shape, seeds, device, std=1.0):
    """bf16 device tensors Q, K, V of the given shape, element ~ N(0, std^2)
    float32 from torch's generator on `device` seeded per tensor, rounded to
    bfloat16 (RNE).  For sizes whose host generation would take minutes; the
    oracle reads the same values back from the device."""
    import torch

    out = []
    for s_ in seeds:
        g = torch.Generator(device=device)
        g.manual_seed(int(s_))
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out.append(t.to(torch.bfloat16))
    return tuple(out)


def mask_for(c, r=0):
    """(BQ, BKV, mask) for workload c (request r for the request stream)."""
    cfg = CONFIGS[c]
    base = 1000 * c
    if c == 1:
        return 64, 64, mask_iid_diag(1, 1024, 64, 64, 0.5, base)
    if c == 2:
        return 128, 128, mask_iid_diag(8, 8192, 128, 128, 0.20, base, dense_heads=(6,),
                                       empty_rows={7: (0, 63)})
    if c == 3:
        return 64, 64, mask_spatiotemporal(cfg["H"], cfg["N"], 64, cfg["frames"], cfg["Y"],
                                           cfg["X"], base)
    if c == 4:
        return 128, 32, mask_clustered(cfg["H"], cfg["N"], 128, 32, base)
    if c == 5:
        return request_c5(r)[:3]
    raise ValueError(c)


def request_c5(r):
    """Request r of the 50-request stream: (BQ, BKV, mask, seeds)."""
    cfg = CONFIGS[5]
    base = 5000 + 10 * r
    rng = _rng(base)
    BQ, BKV = GEOMETRIES_C5[int(rng.integers(len(GEOMETRIES_C5)))]
    M = mask_clustered(cfg["H"], cfg["N"], BQ, BKV, base, rho=(0.02, 0.50), p_empty_head=0.25)
    return BQ, BKV, M, (base + 1, base + 2, base + 3)


def config(c, r=0, with_qkv=True):
    """Workload c as a dict: H, N, d, BQ, BKV, mask and (optionally) q, k, v."""
    cfg = dict(CONFIGS[c])
    BQ, BKV, M = mask_for(c, r)
    cfg.update(BQ=BQ, BKV=BKV, mask=M)
    if with_qkv:
        seeds = (5000 + 10 * r + 1, 5000 + 10 * r + 2, 5000 + 10 * r + 3) if c == 5 else \
            (1000 * c + 1, 1000 * c + 2, 1000 * c + 3)
        cfg["q"], cfg["k"], cfg["v"] = qkv(cfg["H"], cfg["N"], cfg["d"], seeds)
    return cfg


def random_case(H, N, d, BQ, BKV, p, seed, empty_rows=None, dense_heads=(), std=(1.0, 1.0, 1.0)):
    """Small test case: i.i.d. mask plus diagonal, Q/K/V from the same seeds."""
    M = mask_iid_diag(H, N, BQ, BKV, p, seed, dense_heads=dense_heads, empty_rows=empty_rows)
    q, k, v = qkv(H, N, d, (seed + 1, seed + 2, seed + 3), std=std)
    return M, q, k, v


__all__ = ["CONFIGS", "GEOMETRIES_C5", "config", "qkv", "qkv_device", "mask_iid_diag",
           "mask_spatiotemporal", "mask_clustered", "request_c5", "random_case", "mask_for"]
