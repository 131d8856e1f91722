"""Offline plan-table compilation for gfx950 (run on the MI355X).

    python -m dynamic_block_sparse_bsa_amd.profile_table [--out PATH] [--quick]

Tessera paper, section 5.1 "Offline Plan-Table Compilation":
  1. every profiling case (a mask with its request parameters) is run with
     every eligible catalog plan; each output is validated against a
     masked-attention reference and the median kernel latency L[M, P] of the
     valid plans is recorded (here in two or more sessions, on separate
     boxes, combined per case by geometric mean: combine_sessions);
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
benchmark's.  Validation of every plan on every case: the output is filled
with NaN before the plan runs and must come back finite everywhere; the rows
of query blocks without an active block must be exactly zero; every element
must lie within max|V| (each output row is a convex combination of V rows);
and sampled rows of every head (16 random rows plus the first and last) must
match a float32 masked-attention reference computed with torch on the GPU
within the parity tolerance.  A plan failing any check is invalid for that
case.
"""

import argparse
import json
import math
import os
import re
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
    "N": [16384.0, 65536.0],
    "density": [0.1, 0.25],
    # run coverage and row skew are left to the decision-tree partition
    "run_coverage": [],
    "row_skew": [],
}
TOL_MAX, TOL_MEAN = 1e-2, 1e-3
TOP = 6  # plans kept per regime ranking, before the base plan
MIN_CASES = 8  # a regime's ranking rests on at least this many cases


def bucket(bounds, x):
    k = 0
    while k < len(bounds) and x >= bounds[k]:
        k += 1
    return k


# request keys of the corpus: (B_Q, B_KV), head dim, largest N profiled
KEYS = [((64, 64), 128, None), ((128, 128), 128, None), ((128, 32), 128, None), ((32, 128), 128, None),
        ((64, 64), 64, 40960), ((16, 16), 128, 49152), ((32, 16), 128, 49152),
        ((64, 64), 32, 75600), ((128, 32), 256, 49152)]
# two (H, N) sizes in every (head-count bucket, length bucket) cell
SIZES = [(8, 8192), (4, 12288), (8, 16384), (4, 40960), (4, 75600), (2, 115200),
         (24, 8192), (32, 12288), (24, 16384), (16, 49152), (24, 75600), (16, 115200)]
# four target densities in every density bucket
DENSITIES = [0.03, 0.05, 0.07, 0.09, 0.11, 0.15, 0.19, 0.23, 0.28, 0.35, 0.42, 0.5]


def combine_sessions(records):
    """Records of several profiling sessions (and shards) as one record per
    case.  Records with the same seed are the same case measured in separate
    sessions: a plan keeps the geometric mean of its latencies and stays valid
    only if every session validated it.  Timings of one plan on one case vary
    by a few percent from box to box, enough to reorder near-equal plans, so
    rankings rest on every session measured.  Records of distinct seeds (the
    shards of one session) pass through unchanged; the result is in seed
    order and records how many sessions each case combines."""
    by_seed = {}
    for r in records:
        by_seed.setdefault(r["seed"], []).append(r)
    out = []
    for seed in sorted(by_seed):
        rs = by_seed[seed]
        if len(rs) == 1:
            out.append(dict(rs[0], sessions=rs[0].get("sessions", 1)))
            continue
        common = set.intersection(*[set(r["latency"]) for r in rs])
        lat = {p: math.exp(sum(math.log(r["latency"][p]) for r in rs) / len(rs)) for p in sorted(common)}
        n = sum(r.get("sessions", 1) for r in rs)
        out.append(dict(rs[0], latency=lat, sessions=n))
    return out


def corpus(quick=False):
    """Profiling cases: (key, H, N, family, density target, seed).  Every
    (head-count, length, density) bucket of a key gets two sizes times four
    densities, so each fixed-interval regime rests on 8 cases; the mask
    family rotates over the cases.  Seeds start at 920000, disjoint from the
    benchmark workloads' (1000*c, 5000 + 10*r) and the held-out ablation
    cases' (950000...)."""
    sizes, dens = (SIZES[:1] + SIZES[6:7], DENSITIES[::4]) if quick else (SIZES, DENSITIES)
    families = ["clustered", "window", "iid_mixed", "iid"]
    cases = []
    seed = 920000
    for block, d, nmax in KEYS:
        for si, (H, N) in enumerate(sizes):
            if nmax is not None and N > nmax:
                continue
            for i, rho in enumerate(dens):
                fam = families[(i + si) % 4]
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


def profile(cases, reps=5, warmup=3, log=print, plans=None, save=None, done=()):
    """plans: optional regular expression; only catalog entries whose names
    match it are profiled (to add new entries to existing records).  save:
    called with the records so far after every case; done: records of an
    earlier, interrupted run whose cases (by seed) are not profiled again."""
    import numpy as np
    import torch

    import dynamic_block_sparse_bsa_amd as bsa
    from workloads import gen
    dev = torch.device("cuda")
    cat = bsa.catalog()
    records = list(done)
    seen = {r["seed"] for r in records}
    for ci, c in enumerate(cases):
        if c["seed"] in seen:
            continue
        H, N, d = c["H"], c["N"], c["d"]
        BQ, BKV = c["block"]
        M = make_mask(c)
        q, k, v = (t.to(dev) for t in gen.qkv(H, N, d, (c["seed"] + 1, c["seed"] + 2, c["seed"] + 3)))
        Md = torch.from_numpy(M).to(dev)
        rng = np.random.default_rng(c["seed"])
        rows = {h: np.unique(np.concatenate([rng.integers(0, N, 16), [0, N - 1]])) for h in range(H)}
        ref = reference_rows(q, k, v, M, (BQ, BKV), rows)
        # token rows whose query block has no active block: exactly zero
        empty_tok = (~Md.bool().any(dim=2))[:, torch.arange(N, device=dev) // BQ]
        vmax = v.abs().amax().float().item()
        out = torch.empty_like(q)
        lat = {}
        stats = None
        for e in cat:
            if plans and not re.search(plans, e["name"]):
                continue
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
            out.fill_(float("nan"))
            for i in range(nw + nr):
                _, a_ms, m_ms = bsa.run_timed(p, q, k, v, out)
                if i >= nw:
                    ts.append(a_ms + m_ms)
            torch.cuda.synchronize()
            ok = bool(torch.isfinite(out).all())
            if ok and bool(empty_tok.any()):
                ok = float(out[empty_tok].abs().amax()) == 0.0
            if ok:
                ok = float(out.abs().amax()) <= vmax * (1.0 + 1e-2)
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
        del q, k, v, out, Md, empty_tok
        torch.cuda.empty_cache()
        if save:
            save(records)
    return records


def _ranking(bsa, key, rs):
    """Plans valid on every case of rs ranked by geometric-mean latency (top
    TOP), ending with the key's base plan; None when no plan is common."""
    common = set.intersection(*[set(r["latency"]) for r in rs]) if rs else set()
    if not common:
        return None, None
    gm = {pid: math.exp(sum(math.log(r["latency"][pid]) for r in rs) / len(rs)) for pid in common}
    ranking = sorted(common, key=lambda pid: (gm[pid], pid))[:TOP]
    base = bsa.base_plan(rs[0]["H"], rs[0]["N"], key[2], (key[0], key[1]))
    if ranking[-1] != base:
        ranking.append(base)  # every ranking ends with the key's base plan
    return ranking, gm[ranking[0]]


# ---- decision-tree partition of a key's cases -------------------------------
# Section 5.1 of the Tessera paper allows the second-stage boundaries to be
# thresholds learned by a decision tree whose leaves are the regimes, with the
# depth chosen by cross-validation over corpus folds that keep masks of one
# source together and at least 32 cases per leaf.  The split criterion here
# is the quantity the table serves: a leaf picks the plan with the lowest
# geometric-mean latency over its cases, and a split is taken when it lowers
# the summed log selection regret (latency of the leaf's plan over the
# case's fastest valid plan) of its cases.

FEATURES = ("H", "N", "density", "run_coverage", "row_skew")
MIN_LEAF = 32
MAX_DEPTH = 4


def fit_tree(rs, depth, min_leaf=None):
    """Greedy regret-minimizing tree over FEATURES.  Returns nested dicts:
    {"idx": case indices} for a leaf, plus "f", "thr", "lo", "hi" for a split
    (lo: feature < thr, hi: feature >= thr)."""
    import numpy as np
    min_leaf = MIN_LEAF if min_leaf is None else min_leaf
    pids = sorted(set().union(*[set(r["latency"]) for r in rs]))
    L = np.full((len(rs), len(pids)), np.inf)
    for i, r in enumerate(rs):
        for j, pid in enumerate(pids):
            if pid in r["latency"]:
                L[i, j] = math.log(r["latency"][pid])
    best = L.min(axis=1)
    X = np.array([[float(r[f]) for f in FEATURES] for r in rs])

    def leaf_cost(idx):
        return float(L[idx].sum(axis=0).min() - best[idx].sum())

    def best_split(idx):
        n = len(idx)
        found = (math.inf, None)
        for f in range(len(FEATURES)):
            order = idx[np.argsort(X[idx, f], kind="stable")]
            xs = X[order, f]
            fin = np.isfinite(L[order])
            cs = np.cumsum(np.where(fin, L[order], 0.0), axis=0)
            bad = np.cumsum(~fin, axis=0)
            cb = np.cumsum(best[order])
            for k in range(min_leaf, n - min_leaf + 1):
                if xs[k - 1] == xs[k]:
                    continue
                left = np.where(bad[k - 1] == 0, cs[k - 1], np.inf).min() - cb[k - 1]
                right = np.where(bad[-1] - bad[k - 1] == 0, cs[-1] - cs[k - 1], np.inf).min() - (cb[-1] - cb[k - 1])
                if left + right < found[0]:
                    found = (float(left + right), (f, float((xs[k - 1] + xs[k]) / 2)))
        return found

    def grow(idx, dep):
        node = {"idx": idx}
        if dep == 0 or len(idx) < 2 * min_leaf:
            return node
        c, split = best_split(idx)
        if split is None or not c < leaf_cost(idx) - 1e-9:
            return node
        f, thr = split
        node.update(f=f, thr=thr, lo=grow(idx[X[idx, f] < thr], dep - 1), hi=grow(idx[X[idx, f] >= thr], dep - 1))
        return node

    return grow(np.arange(len(rs)), depth)


def tree_leaves(node, path=()):
    """(tests, case indices) per leaf; a test is (feature name, op, threshold)."""
    if "f" not in node:
        return [(list(path), node["idx"])]
    f, thr = FEATURES[node["f"]], node["thr"]
    return tree_leaves(node["lo"], path + ((f, "<", thr),)) + tree_leaves(node["hi"], path + ((f, ">=", thr),))


def compile_table(records, version, partition="intervals"):
    """Two-stage regime partition and geometric-mean ranking.  partition:
    "intervals" (the fixed BOUNDS buckets, then coarser buckets) or
    ("tree", depth) (decision-tree leaves per request key)."""
    import dynamic_block_sparse_bsa_amd as bsa
    cat = bsa.catalog()
    names = {e["id"]: e["name"] for e in cat}
    keyed = {}
    for r in records:
        if r["latency"]:
            keyed.setdefault((r["block"][0], r["block"][1], r["d"]), []).append(r)
    lines = [f"bsa-plan-table {version}", "arch gfx950", f"catalog {bsa.catalog_hash()}"]

    def emit(key, head, rs, min_cases=MIN_CASES):
        if len(rs) < min_cases:
            return  # too few cases: requests fall through to a coarser regime
        ranking, best = _ranking(bsa, key, rs)
        if ranking is None:
            return
        lines.append(f"# {len(rs)} cases; best GM {best:.4f} ms")
        lines.append(" ".join([head[0], str(key[0]), str(key[1]), str(key[2])] + ([head[1]] if head[1] else [])
                              + [":"] + [names[p] for p in ranking]))

    if partition != "intervals":
        depth = partition[1]
        lines.append(f"# partition: decision tree per key, depth <= {depth}, >= {MIN_LEAF} cases per leaf")
        for key in sorted(keyed):
            rs = keyed[key]
            for tests, idx in tree_leaves(fit_tree(rs, depth)):
                emit(key, ("rule", " ".join(f"{f}{op}{thr!r}" for f, op, thr in tests)), [rs[i] for i in idx])
            emit(key, ("regime", " ".join(["*"] * 5)), rs, min_cases=1)
        return "\n".join(lines) + "\n"

    for f in ("H", "N", "density", "run_coverage", "row_skew"):
        if BOUNDS[f]:
            lines.append(f"bounds {f} " + " ".join(repr(float(x)) for x in BOUNDS[f]))
    for key in sorted(keyed):
        groups = {}
        for r in keyed[key]:
            reg = (bucket(BOUNDS["H"], r["H"]), bucket(BOUNDS["N"], r["N"]),
                   bucket(BOUNDS["density"], r["density"]), bucket(BOUNDS["run_coverage"], r["run_coverage"]),
                   bucket(BOUNDS["row_skew"], r["row_skew"]))
            groups.setdefault(reg, []).append(r)
        # regimes: request-dimension and mask-statistic buckets
        for reg in sorted(groups):
            hb = str(reg[0]) if BOUNDS["H"] else "*"
            emit(key, ("regime", " ".join([hb] + [str(x) for x in reg[1:]])), groups[reg])
        # coarser regimes after them (the lookup takes the first match): the
        # same request-dimension buckets with any mask statistics, then any
        # request of the key; a request misses only for a key never profiled
        coarse = {}
        for reg, rs in groups.items():
            coarse.setdefault(reg[:2], []).extend(rs)
        for (h, n) in sorted(coarse):
            emit(key, ("regime", " ".join([str(h) if BOUNDS["H"] else "*", str(n), "*", "*", "*"])),
                 coarse[(h, n)])
        emit(key, ("regime", " ".join(["*"] * 5)), keyed[key], min_cases=1)
    return "\n".join(lines) + "\n"


def table_rankings(text):
    """Rankings (catalog ids) of a table's regimes in file order (the regime
    index that bsa_select reports)."""
    import dynamic_block_sparse_bsa_amd as bsa
    ids = {e["name"]: e["id"] for e in bsa.catalog()}
    return [[ids[n] for n in ln.split(":", 1)[1].split()] for ln in text.splitlines()
            if ln.startswith(("regime ", "rule "))]


def selection_regret(text, cases):
    """Per case: latency of the plan the table selects (its regime's first
    plan valid on the case, else the base plan) over the case's fastest
    valid plan.  Uses the library's own lookup on the loaded table."""
    import tempfile

    import dynamic_block_sparse_bsa_amd as bsa
    rankings = table_rankings(text)
    with tempfile.NamedTemporaryFile("w", suffix=".txt", delete=False) as f:
        f.write(text)
        path = f.name
    out = []
    try:
        bsa.table_load(path)
        for r in cases:
            lat = r["latency"]
            if not lat:
                continue
            block, H, N, d = tuple(r["block"]), r["H"], r["N"], r["d"]
            _, reg = bsa.select(H, N, d, block, r["density"], r["run_coverage"], r["row_skew"])
            cand = (rankings[reg] if reg >= 0 else []) + [bsa.base_plan(H, N, d, block)]
            sel = next((p for p in cand if p in lat), None)
            out.append((lat[sel] if sel is not None else max(lat.values())) / min(lat.values()))
    finally:
        bsa.table_load(None)
        os.unlink(path)
    return out


def cross_validate(records, partitions):
    """Leave-one-source-out cross-validation: the mask generator family is
    the source, so every fold holds out all masks of one generator.  Returns
    {partition: GM selection regret over all held-out cases}."""
    fams = sorted(set(r["family"] for r in records))
    res = {}
    for part in partitions:
        regrets = []
        for fam in fams:
            train = [r for r in records if r["family"] != fam]
            test = [r for r in records if r["family"] == fam]
            regrets += selection_regret(compile_table(train, "cv", part), test)
        res[part] = math.exp(sum(math.log(x) for x in regrets) / len(regrets))
    return res


def choose_partition(records, log=print):
    """The fixed intervals or the tree depth with the lowest cross-validated
    regret (ties go to the simpler partition)."""
    parts = ["intervals"] + [("tree", dep) for dep in range(MAX_DEPTH + 1)]
    cv = cross_validate(records, parts)
    for p in parts:
        log(f"cv {p}: GM regret {cv[p]:.4f}")
    best = min(parts, key=lambda p: (round(cv[p], 4), parts.index(p)))
    return best, cv


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "tables", "gfx950_v2.txt"))
    ap.add_argument("--quick", action="store_true", help="small corpus (smoke test of the tool)")
    ap.add_argument("--version", default=None)
    ap.add_argument("--records", default=None, help="also write the profiling records (JSON) here")
    ap.add_argument("--from-records", default=None, nargs="+",
                    help="compile from saved records (no GPU); several files are merged by "
                         "combine_sessions (shards concatenate, sessions of one case combine)")
    ap.add_argument("--shard", default=None, help="i/n: profile every n-th case starting at i")
    ap.add_argument("--plans", default=None, help="profile only catalog entries matching this regex")
    ap.add_argument("--partition", default="auto",
                    help="intervals | tree:<depth> | auto (cross-validated choice)")
    a = ap.parse_args()
    t0 = time.time()
    if a.from_records:
        recs = []
        for path in a.from_records:
            with open(path) as f:
                recs.extend(json.load(f))
        for r in recs:
            r["block"] = tuple(r["block"])
            r["latency"] = {int(k): v for k, v in r["latency"].items()}
        recs = combine_sessions(recs)
        if a.records:  # the combined records, as shipped beside the table
            with open(a.records, "w") as f:
                json.dump([dict(r, latency={str(k): v for k, v in r["latency"].items()}) for r in recs], f)
    else:
        cases = corpus(a.quick)
        if a.shard:
            i, n = (int(x) for x in a.shard.split("/"))
            cases = cases[i::n]
        done = []
        if a.records and os.path.exists(a.records):
            with open(a.records) as f:
                done = json.load(f)  # resume an interrupted run

        def save(rs):
            if a.records:
                with open(a.records + ".tmp", "w") as f:
                    json.dump(rs, f)
                os.replace(a.records + ".tmp", a.records)

        recs = profile(cases, log=lambda s: print(s, flush=True), plans=a.plans, save=save, done=done)
        save(recs)
    version = a.version or time.strftime("v1-%Y%m%d", time.gmtime())
    cvtext = ""
    if a.partition == "auto":
        part, cv = choose_partition(recs, log=lambda s: print(s, flush=True))
        cvtext = "".join("# leave-one-source-out GM regret, %s: %.4f\n"
                         % ("fixed intervals" if p == "intervals" else f"tree of depth <= {p[1]}", v)
                         for p, v in cv.items())
    elif a.partition == "intervals":
        part = "intervals"
    else:
        part = ("tree", int(a.partition.split(":")[1]))
    how = ("compiled from saved records" if a.from_records
           else "profiled and compiled in %.0f s" % (time.time() - t0))
    ns = sorted({r.get("sessions", 1) for r in recs})
    if ns != [1]:
        how += " (%s profiling sessions per case, latencies combined by geometric mean)" % "-".join(
            str(n) for n in sorted({ns[0], ns[-1]}))
    text = ("# Plan table for gfx950 (MI355X): %d synthetic profiling cases, %s by\n"
            "# profile_table.py.  Format: see csrc/catalog.cpp.\n" % (len(recs), how))
    text += cvtext + compile_table(recs, version, part)
    with open(a.out, "w") as f:
        f.write(text)
    print(f"wrote {a.out}: {text.count(chr(10) + 'regime')} regimes", flush=True)


if __name__ == "__main__":
    main()
