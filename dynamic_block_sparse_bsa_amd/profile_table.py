"""Offline plan-table compilation for gfx950 (run on the MI355X).

    python -m dynamic_block_sparse_bsa_amd.profile_table [--out PATH] [--quick]

Tessera paper, section 5.1 "Offline Plan-Table Compilation":
  1. every profiling case (a mask with its request parameters) is run with
     every eligible catalog plan; each output is validated against a
     masked-attention reference and the median kernel latency L[M, P] of the
     valid plans is recorded;
  2. cases are grouped in two stages: by the request key (architecture,
     logical geometry, tensor properties), then by bucketed request
     dimensions and mask statistics (density, active-block-run coverage);
     each group is a performance regime;
  3. each regime ranks the plans that are valid on every one of its cases by
     geometric-mean latency; the ranking ends with the key's base plan;
  4. catalog, plan table and feature schema ship together as one versioned
     artifact (the text table, stamped with the catalog hash).

The profiling corpus is synthetic (the pages' corpus of video-model masks is
not available): clustered top-k masks (per-head densities spread around the
target, some heads with empty rows), spatiotemporal window masks, i.i.d.
masks, and i.i.d. masks with one all-active head and one head with empty
rows, over a range of densities, drawn with seeds disjoint from the
benchmark's.  Validation uses a float32 masked-attention reference computed
with torch on the GPU for a sample of rows; a plan whose output deviates by
more than the parity tolerance on any case is invalid for that case.
"""

import argparse
import json
import math
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# feature schema: bucket k of a feature holds bounds[k-1] <= x < bounds[k]
BOUNDS = {
    # head count: with many heads the task list spans far more K/V than the
    # caches hold, and organizations that keep neighbouring tiles together win
    "H": [16.0],
    "N": [12288.0, 49152.0],
    "density": [0.08, 0.2, 0.35],
    "run_coverage": [0.5],
    "row_skew": [2.0],
}
TOL_MAX, TOL_MEAN = 1e-2, 1e-3
TOP = 6  # plans kept per regime ranking, before the base plan


def bucket(bounds, x):
    k = 0
    while k < len(bounds) and x >= bounds[k]:
        k += 1
    return k


def corpus(quick=False):
    """Profiling cases: (key, H, N, family, density target, seed).  Seeds start
    at 900000, disjoint from the benchmark workloads' (1000*c, 5000 + 10*r)."""
    keys = [((64, 64), 128), ((128, 128), 128), ((128, 32), 128), ((32, 128), 128), ((64, 64), 64)]
    if quick:
        sizes, dens = [(4, 8192), (2, 65536)], [0.1, 0.3]
        big, big_dens = [(24, 32768)], [0.1]
    else:
        sizes = [(8, 8192), (8, 16384), (8, 32768), (4, 75600), (4, 115200)]
        dens = [0.03, 0.06, 0.1, 0.14, 0.2, 0.28, 0.4, 0.5]
        # many heads at long sequences (the second head-count bucket)
        big, big_dens = [(24, 75600), (32, 115200)], [0.06, 0.14, 0.22]
    families = ["clustered", "window", "iid_mixed", "iid"]
    cases = []
    seed = 900000
    for block, d in keys:
        for grid, rhos in ((sizes, dens), (big, big_dens)):
            for H, N in grid:
                if d == 64 and N > 32768:
                    continue
                for i, rho in enumerate(rhos):
                    fam = families[(i + N) % 4]
                    if fam == "window" and block[0] != block[1]:
                        fam = "clustered"
                    cases.append(dict(block=block, d=d, H=H, N=N, family=fam, rho=rho, seed=seed))
                    seed += 1
    return cases


def make_mask(c):
    import numpy as np

    from workloads import gen
    BQ, BKV = c["block"]
    H, N, rho, seed = c["H"], c["N"], c["rho"], c["seed"]
    if c["family"] == "clustered":
        # per-head densities spread around the target, some heads with empty rows
        return gen.mask_clustered(H, N, BQ, BKV, seed, rho=(0.4 * rho, min(1.0, 1.6 * rho)),
                                  p_empty_head=0.25)
    if c["family"] == "window":
        # frame-major layout of 40x64 tokens per frame
        frames = -(-N // 2560)
        return gen.mask_spatiotemporal(H, N, BQ, frames, 40, 64, seed, rho=(rho, rho),
                                       p_rand=min(0.03, rho / 3))
    if c["family"] == "iid_mixed":
        # one all-active head and one head with two empty query-block rows
        nq = -(-N // BQ)
        return gen.mask_iid_diag(H, N, BQ, BKV, rho, seed, dense_heads=(H - 2,),
                                 empty_rows={H - 1: (0, nq - 1)})
    return gen.mask_iid_diag(H, N, BQ, BKV, rho, seed)


def reference_rows(q, k, v, M, block, rows):
    """float32 masked attention on the GPU for the given (head, rows)."""
    import torch
    BQ, BKV = block
    H, N, d = q.shape
    out = {}
    scale = 1.0 / math.sqrt(d)
    Mt = torch.as_tensor(M, device=q.device)
    for h, r in rows.items():
        r = torch.as_tensor(r, device=q.device, dtype=torch.long)
        qs = q[h, r].float()
        s = (qs @ k[h].float().T.contiguous()) * scale        # [r, N]
        allowed = Mt[h][r // BQ][:, torch.arange(N, device=q.device) // BKV] != 0
        s = s.masked_fill(~allowed, float("-inf"))
        has = allowed.any(dim=1)
        mx = torch.where(has, s.max(dim=1).values, torch.zeros_like(s[:, 0]))
        p = torch.exp(s - mx[:, None])
        o = (p @ v[h].float()) / p.sum(dim=1).clamp_min(1e-30)[:, None]
        o[~has] = 0
        out[h] = o
    return out


def profile(cases, reps=5, warmup=3, log=print):
    import numpy as np
    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    from workloads import gen
    dev = torch.device("cuda")
    cat = bsa.catalog()
    records = []
    for ci, c in enumerate(cases):
        H, N, d = c["H"], c["N"], c["d"]
        BQ, BKV = c["block"]
        M = make_mask(c)
        q, k, v = (t.to(dev) for t in gen.qkv(H, N, d, (c["seed"] + 1, c["seed"] + 2, c["seed"] + 3)))
        Md = torch.from_numpy(M).to(dev)
        rng = np.random.default_rng(c["seed"])
        rows = {h: np.unique(rng.integers(0, N, 48)) for h in range(min(H, 2))}
        ref = reference_rows(q, k, v, M, (BQ, BKV), rows)
        out = torch.empty_like(q)
        lat = {}
        stats = None
        for e in cat:
            if not bsa.eligible(e["id"], H, N, d, (BQ, BKV)):
                continue
            try:
                p = bsa.plan(Md, (BQ, BKV), H, N, d, force_plan=e["id"])
            except bsa.BsaError:
                continue
            info = p.info
            stats = (info["density"], info["run_coverage"], info["row_skew"])
            ts = []
            nw, nr = (1, 3) if H >= 16 else (warmup, reps)  # many-head cases run 10-100 ms
            for i in range(nw + nr):
                _, a_ms, m_ms = bsa.run_timed(p, q, k, v, out)
                if i >= nw:
                    ts.append(a_ms + m_ms)
            torch.cuda.synchronize()
            ok = True
            for h, r in rows.items():
                o = out[h, torch.as_tensor(r, device=dev)].float()
                err = (o - ref[h]).abs()
                if not bool(torch.isfinite(o).all()) or err.max().item() > TOL_MAX or err.mean().item() > TOL_MEAN:
                    ok = False
            p.destroy()
            if ok:
                lat[e["id"]] = statistics.median(ts)
        rec = dict(c, density=stats[0] if stats else 0.0, run_coverage=stats[1] if stats else 0.0,
                   row_skew=stats[2] if stats else 0.0, latency=lat)
        records.append(rec)
        best = min(lat, key=lat.get) if lat else None
        log(f"case {ci + 1}/{len(cases)} B={c['block']} d={d} H={H} N={N} {c['family']} "
            f"density={rec['density']:.3f} runcov={rec['run_coverage']:.2f} skew={rec['row_skew']:.2f} "
            f"valid={len(lat)} "
            f"best={cat[best]['name'] if best is not None else '-'} {lat.get(best, 0):.3f} ms")
        del q, k, v, out, Md
        torch.cuda.empty_cache()
    return records


def compile_table(records, version):
    """Two-stage regime partition and geometric-mean ranking."""
    import dynamic_block_sparse_bsa_amd as bsa
    cat = bsa.catalog()
    names = {e["id"]: e["name"] for e in cat}
    groups = {}
    for r in records:
        key = (r["block"][0], r["block"][1], r["d"])
        reg = (bucket(BOUNDS["H"], r["H"]), bucket(BOUNDS["N"], r["N"]),
               bucket(BOUNDS["density"], r["density"]), bucket(BOUNDS["run_coverage"], r["run_coverage"]),
               bucket(BOUNDS["row_skew"], r["row_skew"]))
        groups.setdefault(key, {}).setdefault(reg, []).append(r)
    lines = [f"bsa-plan-table {version}", "arch gfx950", f"catalog {bsa.catalog_hash()}"]
    for f in ("H", "N", "density", "run_coverage", "row_skew"):
        if BOUNDS[f]:
            lines.append(f"bounds {f} " + " ".join(repr(float(x)) for x in BOUNDS[f]))
    def emit(key, fields, rs):
        common = set.intersection(*[set(r["latency"]) for r in rs]) if rs else set()
        if not common:
            return
        gm = {pid: math.exp(sum(math.log(r["latency"][pid]) for r in rs) / len(rs)) for pid in common}
        ranking = sorted(common, key=lambda pid: (gm[pid], pid))[:TOP]
        base = bsa.base_plan(rs[0]["H"], rs[0]["N"], key[2], (key[0], key[1]))
        if ranking[-1] != base:
            ranking.append(base)  # every ranking ends with the key's base plan
        lines.append(f"# {len(rs)} cases; best GM {gm[ranking[0]]:.4f} ms")
        lines.append("regime %d %d %d %s : %s" % (key[0], key[1], key[2], " ".join(fields),
                                                  " ".join(names[p] for p in ranking)))

    for key in sorted(groups):
        # regimes: request-dimension and mask-statistic buckets
        for reg in sorted(groups[key]):
            hb = str(reg[0]) if BOUNDS["H"] else "*"
            emit(key, [hb] + [str(x) for x in reg[1:]], groups[key][reg])
        # coarser regimes after them (the lookup takes the first match): the
        # same request-dimension buckets with any mask statistics, then any
        # request of the key; a request misses only for a key never profiled
        coarse = {}
        for reg, rs in groups[key].items():
            coarse.setdefault(reg[:2], []).extend(rs)
        for (h, n) in sorted(coarse):
            emit(key, [str(h) if BOUNDS["H"] else "*", str(n), "*", "*", "*"], coarse[(h, n)])
        emit(key, ["*"] * 5, [r for rs in groups[key].values() for r in rs])
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "tables", "gfx950_v1.txt"))
    ap.add_argument("--quick", action="store_true", help="small corpus (smoke test of the tool)")
    ap.add_argument("--version", default=None)
    ap.add_argument("--records", default=None, help="also write the profiling records (JSON) here")
    ap.add_argument("--from-records", default=None, help="compile from saved records (no GPU)")
    a = ap.parse_args()
    t0 = time.time()
    if a.from_records:
        with open(a.from_records) as f:
            recs = json.load(f)
        for r in recs:
            r["block"] = tuple(r["block"])
            r["latency"] = {int(k): v for k, v in r["latency"].items()}
    else:
        recs = profile(corpus(a.quick), log=lambda s: print(s, flush=True))
        if a.records:
            with open(a.records, "w") as f:
                json.dump(recs, f)
    version = a.version or time.strftime("v1-%Y%m%d", time.gmtime())
    text = ("# Plan table for gfx950 (MI355X), compiled by profile_table.py from %d synthetic\n"
            "# profiling cases in %.0f s.  Format: see csrc/catalog.cpp.\n" % (len(recs), time.time() - t0))
    text += compile_table(recs, version)
    with open(a.out, "w") as f:
        f.write(text)
    print(f"wrote {a.out}: {text.count(chr(10) + 'regime')} regimes", flush=True)


if __name__ == "__main__":
    main()
