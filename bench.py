"""Benchmark: block-sparse attention request latency and active-block TFLOP/s.

One step = one complete BSA request on the GPU: plan creation (mask state,
statistics transfer, regime lookup, launch preparation) + the attention
kernels (+ split-K merge) + stream synchronization, with mask, Q, K and V
already resident in HBM.  Active-block FLOPs are 4*d*|E(M)|: the per-tile
accounting of the Tessera paper (section 2.3: QK^T and PV each cost 2*d flops
per query/key pair) over the effective (query, key) pairs only, clipped at N.

Default workload: the hunyuan-like layer (24 heads, N=115,200, d=128,
B=(128,32), clustered top-k mask at 5-30% density per head), the largest
workload that fits one GPU.  --config 1|2|3|5 runs the others.  --config 5 is
the request stream: timed step i is request i mod 50 of the stream, in order
(mask and geometry re-drawn per request; one Q/K/V set, whose values do not
change the work), so --steps 50 times the whole stream once; the warmup steps
run requests 0 .. W-1 before it.

CPU baseline: the fp64 oracle as it stands.  For the tiny and medium
workloads whole heads are timed; for the others a whole head does not fit the
budget, so seeded random query blocks (every row of each) are timed with the
oracle's row routine and the active-block flop rate of that sample is
extrapolated to the request (labelled "extrapolated").

Prints one JSON line.  Single GPU only.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BSA request latency (ms, incl. planning) + active-block TFLOP/s, bf16 d=128"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
WORKLOAD = {1: "tiny", 2: "medium", 3: "wan720p", 4: "hunyuan", 5: "stream"}


def effective_pairs(M, BQ, BKV, N):
    """|E(M)| per head: active blocks weighted by their clipped token extents."""
    import numpy as np
    M = np.asarray(M) != 0
    qsz = np.minimum(BQ, N - np.arange(M.shape[1]) * BQ).astype(np.int64)
    ksz = np.minimum(BKV, N - np.arange(M.shape[2]) * BKV).astype(np.int64)
    per_head = (M.astype(np.int64) * qsz[:, None] * ksz[None, :]).sum(axis=(1, 2))
    return int(per_head.sum()), per_head


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("attn_fwd.h", "attn_kernels.hip"):
        with open(os.path.join(ROOT, "dynamic_block_sparse_bsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary
    (profiles/attn_fwd_<workload>_traffic.txt), if it was taken on the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                kv[parts[0]] = parts[1]
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(cfg, budget_s, whole_heads):
    """Time the fp64 oracle, as it stands, on a bounded sample of the workload.

    whole_heads: whole-head evaluations in order (cycling) until the budget is
    spent.  Otherwise: seeded random query blocks, all rows of each, through
    the oracle's row routine (it gathers only the active keys), batched per
    head; the rate of the sample (active-block flops / wall time) is
    extrapolated to the whole request."""
    import numpy as np
    from oracle import attention as oatt
    cores = _blas_threads()
    M, BQ, BKV, N, H, d = cfg["mask"], cfg["BQ"], cfg["BKV"], cfg["N"], cfg["H"], cfg["d"]
    total_pairs, per_head = effective_pairs(M, BQ, BKV, N)
    Mb = np.asarray(M) != 0
    ksz = np.minimum(BKV, N - np.arange(Mb.shape[2]) * BKV).astype(np.int64)
    t0 = time.perf_counter()
    n, flops = 0, 0.0
    if whole_heads:
        while True:
            h = n % H
            oatt.attention(cfg["q"][h:h + 1], cfg["k"][h:h + 1], cfg["v"][h:h + 1], M[h:h + 1], BQ, BKV)
            flops += 4.0 * d * float(per_head[h])
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        sample = f"fp64 oracle, {n} whole-head evaluations (heads 0..{min(n, H) - 1} of {H}, cycling)"
    else:
        rng = np.random.default_rng(12345)
        nqb = Mb.shape[1]
        blocks_per_call = 4
        while True:
            h = int(rng.integers(H))
            qbs = rng.choice(nqb, size=min(blocks_per_call, nqb), replace=False)
            rows = np.concatenate([np.arange(qb * BQ, min(N, (qb + 1) * BQ)) for qb in qbs])
            oatt.attention_rows(cfg["q"], cfg["k"], cfg["v"], M, BQ, BKV, {h: rows})
            for qb in qbs:
                nrow = min(N, (qb + 1) * BQ) - qb * BQ
                flops += 4.0 * d * nrow * float((Mb[h, qb] * ksz).sum())
            n += len(qbs)
            if time.perf_counter() - t0 >= budget_s:
                break
        sample = (f"fp64 oracle row routine on {n} seeded random query blocks ({n * BQ} rows) of "
                  f"{H * nqb}; rate extrapolated to the request")
    dt = time.perf_counter() - t0
    rate = flops / dt
    req_flops = 4.0 * d * total_pairs
    return {"value": float(rate / 1e12), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{sample}, {dt:.1f} s; active-block flops / wall time",
            "extrapolated": not whole_heads,
            "request_s": float(req_flops / rate),
            "cpu_model": _cpu_model(), "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; for --config 5 the whole stream, --requests)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--requests", type=int, default=50, help="stream length for --config 5")
    ap.add_argument("--force-plan", type=int, default=-1)
    ap.add_argument("--force-split", type=int, default=-1)
    ap.add_argument("--layout", default="HND", choices=["HND", "NHD"],
                    help="tensor layout of Q, K, V and O ([H][N][d] or [N][H][d])")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (5 times): the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(heads would shard across GPUs without communication); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 5}), flush=True)
        return

    import dynamic_block_sparse_bsa_amd as bsa
    from workloads import gen

    dev = torch.device("cuda:0")
    cfg = gen.config(args.config)
    H, N, d = cfg["H"], cfg["N"], cfg["d"]
    q, k, v = (t.to(dev) for t in (cfg["q"], cfg["k"], cfg["v"]))
    if args.layout == "NHD":
        q, k, v = (t.permute(1, 0, 2).contiguous() for t in (q, k, v))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    # requests: (mask on device, block, flops)
    reqs = []
    nreq = args.requests if args.config == 5 else 1
    if args.steps is None:
        args.steps = nreq if args.config == 5 else 20
    for r in range(nreq):
        if args.config == 5:
            BQ, BKV, M, _ = gen.request_c5(r)
        else:
            BQ, BKV, M = cfg["BQ"], cfg["BKV"], cfg["mask"]
        pairs, _ = effective_pairs(M, BQ, BKV, N)
        reqs.append((torch.from_numpy(M).to(dev), (BQ, BKV), 4.0 * d * pairs, pairs))
    torch.cuda.synchronize()

    def request(i, want_info=False):
        Md, block, _, _ = reqs[i % len(reqs)]
        p = bsa.plan(Md, block, H, N, d, force_plan=args.force_plan, force_split=args.force_split,
                     layout=args.layout)
        # returns once the request's last kernel has completed (HIP event wait)
        _, a_ms, m_ms = bsa.run_timed(p, q, k, v, out)
        info = p.info if want_info else None
        p.destroy()
        return a_ms, m_ms, info

    for i in range(args.warmup):
        request(i)
    torch.cuda.synchronize()
    req_ms, attn_ms, merge_ms, infos = [], [], [], []
    flops_total = 0.0
    # timed step i runs request i (mod the stream length): the stream is timed
    # in order from its first request
    t_start = time.perf_counter()
    for i in range(args.steps):
        t0 = time.perf_counter()
        a_ms, m_ms, info = request(i, want_info=(i == args.steps - 1))
        req_ms.append((time.perf_counter() - t0) * 1e3)
        attn_ms.append(a_ms)
        merge_ms.append(m_ms)
        infos.append(info)
        flops_total += reqs[i % len(reqs)][2]
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t_start

    ms_per_step = total_s * 1e3 / args.steps
    med_req = statistics.median(req_ms)
    attn_avg = statistics.mean(attn_ms)
    merge_avg = statistics.mean(merge_ms)
    # kernel-side rate: the attention kernel's algorithmic flops / its duration
    attn_flops = [reqs[i % len(reqs)][2] for i in range(args.steps)]
    achieved = sum(attn_flops) / (sum(attn_ms) * 1e-3) / 1e12
    workload = WORKLOAD[args.config]
    info = infos[-1]
    cat = {e["id"]: e for e in bsa.catalog()}
    Md, block, flops0, pairs0 = reqs[0]
    if args.config == 5:
        wl = f"{workload}: {len(reqs)} requests, H={H} N={N} d={d}, B re-drawn per request"
    else:
        wl = f"{workload}: H={H} N={N} d={d} B=({block[0]},{block[1]})"
    if args.layout != "HND":
        wl += f", layout {args.layout}"
    planning = [r - a - m for r, a, m in zip(req_ms, attn_ms, merge_ms)]
    traffic = load_traffic(workload) if args.layout == "HND" else None
    res = {
        "metric": METRIC,
        "value": flops_total / total_s / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "heads": H, "seq_len": N, "head_dim": d,
                   "density": round(info["density"], 4), "active_pairs": pairs0,
                   "active_gflop": round(flops0 / 1e9, 3)},
        "request_ms_median": med_req,
        "request_ms_p95": float(np.percentile(req_ms, 95)),
        "attn_kernel_ms": attn_avg,
        "merge_kernel_ms": merge_avg,
        "planning_ms_median": statistics.median(planning),
        "planning_share": statistics.median(planning) / med_req,
        "plan": cat[info["plan_id"]]["name"],
        "regime": info["regime"],
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
        # the attention kernel's measured HBM bytes per launch (from the
        # committed counter summary) over its event-timed duration
        "hbm": None if traffic is None else {
            "achieved": traffic / (attn_avg * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": traffic / (attn_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS},
    }
    if args.config == 5:
        res["stream"] = {"requests_timed": args.steps, "stream_length": len(reqs),
                         "whole_stream_ms": sum(req_ms[:len(reqs)]) if args.steps >= len(reqs) else None}
    if args.no_cpu:
        res["cpu_baseline"] = None
    else:
        if args.config == 5:
            BQ0, BKV0, M0, _ = gen.request_c5(0)
            ccfg = dict(cfg, BQ=BQ0, BKV=BKV0, mask=M0)
        else:
            ccfg = cfg
        res["cpu_baseline"] = cpu_baseline(ccfg, args.cpu_budget, whole_heads=args.config in (1, 2))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
