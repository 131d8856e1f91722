"""Benchmark: block-sparse attention request latency and active-block TFLOP/s.

One step = one complete BSA request on the GPU: plan creation (mask state,
statistics transfer, regime lookup, launch preparation) + the attention
kernels + stream synchronization, with mask, Q, K and V already resident in
HBM.  Active-block FLOPs are 4*d*|E(M)| (the pages' per-tile accounting over
effective (query, key) pairs only, clipped at N).

Default workload: the medium request (8 heads, N=8192, d=128, B=(128,128),
20% i.i.d. + diagonal, one all-active head, one head with two empty query-block
rows).  --config 3|4|5 runs the other workloads (not the default line).

Prints one JSON line (rank 0).  Single GPU only.
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
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_GBS = 8000.0


def effective_pairs(M, BQ, BKV, N):
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
    """HBM bytes per attention launch from committed rocprofv3 PMC runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, budget_s=12.0):
    """Time the fp64 oracle (as it stands) on a bounded sample: whole heads, in
    order, until the budget is spent."""
    import numpy as np

    from oracle import attention as oatt
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    M, BQ, BKV, N = cfg["mask"], cfg["BQ"], cfg["BKV"], cfg["N"]
    _, per_head = effective_pairs(M, BQ, BKV, N)
    t0 = time.perf_counter()
    heads = 0
    for h in range(cfg["H"]):
        oatt.attention(cfg["q"][h:h + 1], cfg["k"][h:h + 1], cfg["v"][h:h + 1], M[h:h + 1], BQ, BKV)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * cfg["d"] * float(per_head[:heads].sum())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle on heads 0..{heads - 1} of {cfg['H']} (all rows), "
                      f"{dt:.1f} s, active-block flops / wall time",
            "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--force-plan", type=int, default=-1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(heads would shard across GPUs without communication); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    from workloads import gen

    dev = torch.device("cuda:0")
    cfg = gen.config(args.config)
    H, N, d, BQ, BKV = cfg["H"], cfg["N"], cfg["d"], cfg["BQ"], cfg["BKV"]
    pairs, _ = effective_pairs(cfg["mask"], BQ, BKV, N)
    flops = 4.0 * d * pairs
    Md = torch.from_numpy(cfg["mask"]).to(dev)
    q, k, v = (t.to(dev) for t in (cfg["q"], cfg["k"], cfg["v"]))
    out = torch.empty((H, N, d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def request():
        p = bsa.plan(Md, (BQ, BKV), H, N, d, force_plan=args.force_plan)
        _, a_ms, m_ms = bsa.run_timed(p, q, k, v, out)
        torch.cuda.synchronize()
        info = p.info
        p.destroy()
        return a_ms, m_ms, info

    for _ in range(args.warmup):
        request()
    torch.cuda.synchronize()
    req_ms, attn_ms, merge_ms = [], [], []
    info = None
    t_start = time.perf_counter()
    for _ in range(args.steps):
        t0 = time.perf_counter()
        a_ms, m_ms, info = request()
        req_ms.append((time.perf_counter() - t0) * 1e3)
        attn_ms.append(a_ms)
        merge_ms.append(m_ms)
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t_start

    ms_per_step = total_s * 1e3 / args.steps
    med_req = statistics.median(req_ms)
    attn_avg = statistics.mean(attn_ms)
    merge_avg = statistics.mean(merge_ms)
    achieved = flops / (attn_avg * 1e-3) / 1e12
    workload = {1: "tiny", 2: "medium", 3: "wan720p", 4: "hunyuan", 5: "stream-r0"}[args.config]
    traffic = load_traffic(workload)
    cat = {e["id"]: e for e in bsa.catalog()}
    res = {
        "metric": METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
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
        "config": {"workload": f"{workload}: H={H} N={N} d={d} B=({BQ},{BKV})",
                   "global_batch": H, "seq_len": N, "parallelism": "none",
                   "density": round(info["density"], 4), "active_pairs": pairs,
                   "active_gflop": round(flops / 1e9, 3)},
        "request_ms_median": med_req,
        "request_ms_p95": float(np.percentile(req_ms, 95)),
        "attn_kernel_ms": attn_avg,
        "merge_kernel_ms": merge_avg,
        "planning_ms": med_req - attn_avg - merge_avg,
        "planning_share": (med_req - attn_avg - merge_avg) / med_req,
        "plan": cat[info["plan_id"]]["name"],
        "regime": info["regime"],
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
    }
    if args.no_cpu:
        res["cpu_baseline"] = None
    else:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
