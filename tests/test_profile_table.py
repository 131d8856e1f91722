"""CPU checks of the offline plan-table compiler (paper section 5.1): regime
partition by request key and feature buckets, geometric-mean ranking over the
plans valid on every case of a regime, the base plan at the end of every
ranking, and a versioned artifact the library accepts.  No GPU: the records
are synthetic latency tables."""

import math

import pytest

import dynamic_block_sparse_bsa_amd as bsa
from dynamic_block_sparse_bsa_amd import profile_table as pt


def _ids(block, d=128, H=8, N=8192):
    return [e["id"] for e in bsa.catalog() if bsa.eligible(e["id"], H, N, d, block)]


def _rec(block, N, density, runcov, skew, lat, H=8, d=128):
    return dict(block=block, d=d, H=H, N=N, family="iid", rho=density, seed=0, density=density,
                run_coverage=runcov, row_skew=skew, latency=lat)


def test_bucket_bounds():
    assert pt.bucket([0.1, 0.2], 0.05) == 0
    assert pt.bucket([0.1, 0.2], 0.1) == 1  # bucket k holds bounds[k-1] <= x < bounds[k]
    assert pt.bucket([0.1, 0.2], 0.5) == 2
    assert pt.bucket([], 3.0) == 0


def test_geometric_mean_ranking_and_validity(tmp_path, monkeypatch):
    monkeypatch.setattr(pt, "MIN_CASES", 1)  # two cases make a regime here
    ids = _ids((128, 128))
    a, b, c = ids[0], ids[3], ids[6]
    # plan a: GM sqrt(1*4) = 2; plan b: GM sqrt(2*2) = 2.0 + tie-break by id; plan c: 1.5 but
    # invalid on the second case (missing) -> excluded from the regime's ranking
    recs = [_rec((128, 128), 8192, 0.3, 0.6, 1.2, {a: 1.0, b: 2.0, c: 1.5}),
            _rec((128, 128), 8192, 0.31, 0.7, 1.3, {a: 4.0, b: 2.1})]
    text = pt.compile_table(recs, "vtest")
    lines = [ln for ln in text.splitlines() if ln.startswith("regime")]
    # both cases fall in one regime; then the coarser regimes of the key
    assert len(lines) == 3
    assert lines[1].split(" : ")[0].split()[6:] == ["*", "*", "*"]
    assert lines[2].split(" : ")[0].split()[4:] == ["*"] * 5
    names = {e["id"]: e["name"] for e in bsa.catalog()}
    ranking = lines[0].split(" : ")[1].split()
    gm_a, gm_b = math.sqrt(1.0 * 4.0), math.sqrt(2.0 * 2.1)
    assert gm_a < gm_b
    assert ranking[0] == names[a] and ranking[1] == names[b]
    assert names[c] not in ranking[:2]
    assert ranking[-1] == names[bsa.base_plan(8, 8192, 128, (128, 128))]
    # regime fields: key, buckets of H, N, density, run coverage, row skew
    f = lines[0].split(" : ")[0].split()
    assert f[1:4] == ["128", "128", "128"] and f[4] == str(pt.bucket(pt.BOUNDS["H"], 8))
    assert f[5:] == [str(pt.bucket(pt.BOUNDS["N"], 8192)), str(pt.bucket(pt.BOUNDS["density"], 0.3)),
                     str(pt.bucket(pt.BOUNDS["run_coverage"], 0.6)),
                     str(pt.bucket(pt.BOUNDS["row_skew"], 1.2))]
    # the artifact loads and the lookup returns the regime's top plan
    path = tmp_path / "t.txt"
    path.write_text(text)
    bsa.table_load(str(path))
    try:
        assert bsa.table_version() == "vtest"
        pid, reg = bsa.select(8, 8192, 128, (128, 128), 0.3, 0.6, 1.2)
        assert reg == 0 and pid == a
        pid, reg = bsa.select(8, 8192, 128, (128, 128), 0.05, 0.6, 1.2)  # other density bucket
        assert reg == 1 and pid == a  # the coarser regime of the same request dimensions
        pid, reg = bsa.select(8, 8192, 128, (64, 64), 0.3, 0.6, 1.2)  # key never profiled
        assert reg == -1 and pid == bsa.base_plan(8, 8192, 128, (64, 64))
    finally:
        bsa.table_load(None)


def test_cases_split_by_key_and_buckets(monkeypatch):
    monkeypatch.setattr(pt, "MIN_CASES", 1)
    i128, i64 = _ids((128, 128)), _ids((64, 64))
    recs = [_rec((128, 128), 8192, 0.3, 0.6, 1.0, {i128[0]: 1.0}),
            _rec((128, 128), 8192, 0.05, 0.6, 3.0, {i128[1]: 1.0}),   # density bucket differs
            _rec((128, 128), 100000, 0.3, 0.6, 1.0, {i128[2]: 1.0}),  # N bucket differs
            _rec((128, 128), 8192, 0.3, 0.6, 1.0, {i128[3]: 1.0}, H=40),  # head-count bucket differs
            _rec((64, 64), 8192, 0.3, 0.6, 1.0, {i64[0]: 1.0})]       # key differs
    text = pt.compile_table(recs, "v2")
    fine = [ln for ln in text.splitlines() if ln.startswith("regime") and "*" not in ln]
    assert len(fine) == 5


def test_regimes_rest_on_min_cases():
    """A fixed-interval regime is emitted only with at least MIN_CASES cases;
    fewer fall through to the coarser regimes (the key-wide one always
    exists)."""
    ids = _ids((128, 128))
    few = [_rec((128, 128), 8192, 0.3, 0.6, 1.0, {ids[0]: 1.0, ids[1]: 2.0}) for _ in range(pt.MIN_CASES - 1)]
    text = pt.compile_table(few, "vmin")
    heads = [ln.split(" : ")[0].split()[4:] for ln in text.splitlines() if ln.startswith("regime")]
    assert heads == [["*"] * 5]
    enough = few + [_rec((128, 128), 8192, 0.31, 0.6, 1.0, {ids[0]: 1.0, ids[1]: 2.0})]
    text = pt.compile_table(enough, "vmin")
    heads = [ln.split(" : ")[0].split()[4:] for ln in text.splitlines() if ln.startswith("regime")]
    assert len(heads) == 3 and "*" not in heads[0]


def test_corpus_fills_every_interval_regime():
    """Every (head-count, length, density) bucket of a key's profiled sizes
    holds 2 sizes x 4 densities = 8 cases, or 4 where the key's length limit
    keeps only one of the two sizes."""
    import collections
    cells = collections.Counter()
    for c in pt.corpus():
        cells[(c["block"], c["d"], pt.bucket(pt.BOUNDS["H"], c["H"]), pt.bucket(pt.BOUNDS["N"], c["N"]),
               pt.bucket(pt.BOUNDS["density"], c["rho"]))] += 1
    limits = {(b, d): n for b, d, n in pt.KEYS}
    for (b, d, hb, nb, db), n in cells.items():
        sizes = [s for s in pt.SIZES if pt.bucket(pt.BOUNDS["H"], s[0]) == hb and
                 pt.bucket(pt.BOUNDS["N"], s[1]) == nb and (limits[(b, d)] is None or s[1] <= limits[(b, d)])]
        assert n == 4 * len(sizes) and len(sizes) >= 1, (b, d, hb, nb, db)


def test_corpus_seeds_disjoint_from_workloads():
    cases = pt.corpus()
    seeds = {c["seed"] for c in cases}
    assert len(seeds) == len(cases) and min(seeds) >= 900000
    # the benchmark workloads draw from 1000*c (+0..3) and 5000 + 10*r (+0..3)
    assert not seeds & ({1000 * c + k for c in range(1, 6) for k in range(4)} |
                        {5000 + 10 * r + k for r in range(50) for k in range(4)})
    assert {c["family"] for c in cases} == {"clustered", "window", "iid", "iid_mixed"}
    assert all(bsa.base_plan(c["H"], c["N"], c["d"], c["block"]) >= 0 for c in cases)


@pytest.mark.parametrize("fam", ["clustered", "window", "iid", "iid_mixed"])
def test_corpus_masks_have_requested_shape(fam):
    block = (64, 64)
    c = dict(block=block, d=128, H=4, N=4096, family=fam, rho=0.2, seed=900001)
    M = pt.make_mask(c)
    assert M.shape == (4, 64, 64) and M.dtype.name == "uint8"
    assert 0.02 < (M != 0).mean() < 0.6


def test_ablation_summary_metrics():
    from dynamic_block_sparse_bsa_amd import ablation
    rows = [dict(k_a0=2.0, k_a2=1.0, k_best=1.0, a0_cold_ms=3.0, a1_cold_ms=30.0, a2_cold_ms=2.0,
                 a0_warm_ms=2.5, a2_warm_ms=1.5),
            dict(k_a0=1.0, k_a2=1.1, k_best=1.0, a0_cold_ms=2.0, a1_cold_ms=20.0, a2_cold_ms=2.2,
                 a0_warm_ms=1.2, a2_warm_ms=1.3),
            dict(k_a0=1.0, k_a2=1.01, k_best=1.0, a0_cold_ms=2.0, a1_cold_ms=10.0, a2_cold_ms=2.0,
                 a0_warm_ms=1.0, a2_warm_ms=1.0)]
    s = ablation.summarize(rows)
    assert s["cases"] == 3
    assert s["selection_regret"]["max"] == pytest.approx(1.1)
    assert s["selection_regret"]["within_3pct_share"] == pytest.approx(2 / 3)
    # A2 vs A0 kernel speedups 2.0 (win), 1/1.1 (loss), 1/1.01 (tie, inside the 3% band)
    assert s["A2_vs_A0_kernel_wins_ties_losses"] == [1, 1, 1]
    assert s["kernel_speedup_over_direct_gm"]["A2_table"] == pytest.approx((2.0 / 1.1 / 1.01) ** (1 / 3))
    assert s["cold_request_speedup_gm"]["A2_over_A1"] == pytest.approx((15 * (20 / 2.2) * 5) ** (1 / 3))
    assert s["selection_regret"]["p99"] == pytest.approx(1.1)
    assert "four_pass_speedup_gm" not in s  # no A1 repeats recorded


def test_ablation_four_pass_and_organization():
    from dynamic_block_sparse_bsa_amd import ablation
    rows = [dict(k_a0=2.0, k_a2=1.0, k_best=1.0, a0_cold_ms=4.0, a1_cold_ms=40.0, a2_cold_ms=4.0,
                 a0_warm_ms=2.0, a1_warm_ms=3.0, a2_warm_ms=1.0, k_o0=1.5, k_o2=0.9),
            dict(k_a0=1.0, k_a2=1.0, k_best=1.0, a0_cold_ms=2.0, a1_cold_ms=20.0, a2_cold_ms=2.0,
                 a0_warm_ms=1.0, a1_warm_ms=1.5, a2_warm_ms=1.0, k_o0=None, k_o2=1.0)]
    s = ablation.summarize(rows)
    # four passes: (cold + 3 warm) / 4 per variant
    a2 = [(4 + 3) / 4, (2 + 3) / 4]
    a1 = [(40 + 9) / 4, (20 + 4.5) / 4]
    assert s["four_pass_speedup_gm"]["A2_over_A1"] == pytest.approx((a1[0] / a2[0] * a1[1] / a2[1]) ** 0.5)
    assert s["warm_repeat_speedup_gm"]["A2_over_A1"] == pytest.approx((3.0 * 1.5) ** 0.5)
    o = s["organization_at_fixed_mapping"]
    assert o["cases"] == 1  # the case without a base organization is left out
    assert o["O1_over_O0_gm"] == pytest.approx(1.5) and o["O2_over_O0_gm"] == pytest.approx(1.5 / 0.9)
    assert o["O1_regret_vs_O2_gm"] == pytest.approx(1 / 0.9)
    assert o["O1_vs_O0_wins_ties_losses"] == [1, 0, 0]
    assert "plan_cache_repeat" not in s


def test_ablation_plan_cache_repeats():
    from dynamic_block_sparse_bsa_amd import ablation
    rows = [dict(k_a0=2.0, k_a2=1.0, k_best=1.0, a0_cold_ms=4.0, a1_cold_ms=40.0, a2_cold_ms=4.0,
                 a0_warm_ms=2.0, a2_warm_ms=1.0, a2_cached_ms=1.25),
            dict(k_a0=1.0, k_a2=1.0, k_best=1.0, a0_cold_ms=2.0, a1_cold_ms=20.0, a2_cold_ms=3.0,
                 a0_warm_ms=1.0, a2_warm_ms=1.0, a2_cached_ms=1.05),
            dict(k_a0=1.0, k_a2=1.0, k_best=1.0, a0_cold_ms=2.0, a1_cold_ms=20.0, a2_cold_ms=2.0,
                 a0_warm_ms=1.0, a2_warm_ms=1.0, a2_cached_ms=1.1)]
    c = ablation.summarize(rows)["plan_cache_repeat"]
    assert c["A2_over_A0_gm"] == pytest.approx((2.0 / 1.25 / 1.05 / 1.1) ** (1 / 3))
    assert c["cold_over_cached_gm"] == pytest.approx((4.0 / 1.25 * 3.0 / 1.05 * 2.0 / 1.1) ** (1 / 3))
    assert c["median_check_ms"] == pytest.approx(0.1)  # median of 0.25, 0.05, 0.1


def test_sessions_combine_by_geometric_mean():
    """Records of one case from two sessions become one record: latencies
    combine by geometric mean, a plan invalid in either session is dropped,
    and shards of distinct cases pass through in seed order."""
    a = dict(seed=7, block=(64, 64), latency={1: 1.0, 2: 4.0, 3: 2.0})
    b = dict(seed=7, block=(64, 64), latency={1: 4.0, 2: 1.0})
    c = dict(seed=5, block=(64, 64), latency={1: 3.0})
    out = pt.combine_sessions([a, c, b])
    assert [r["seed"] for r in out] == [5, 7]
    assert out[0]["latency"] == {1: 3.0} and out[0]["sessions"] == 1
    assert out[1]["sessions"] == 2
    assert set(out[1]["latency"]) == {1, 2}
    assert out[1]["latency"][1] == pytest.approx(2.0) and out[1]["latency"][2] == pytest.approx(2.0)
    # already-combined records count their sessions
    assert pt.combine_sessions([out[1], dict(a)])[0]["sessions"] == 3


def test_builtin_table_recompiles_from_its_records():
    """The shipped table is exactly what the compiler makes of the shipped
    profiling records (same catalog, same bounds, same rankings)."""
    import json
    import os
    tables = os.path.join(os.path.dirname(pt.__file__), "tables")
    with open(os.path.join(tables, "gfx950_v2_records.json")) as f:
        recs = json.load(f)
    for r in recs:
        r["block"] = tuple(r["block"])
        r["latency"] = {int(k): v for k, v in r["latency"].items()}
    with open(os.path.join(tables, "gfx950_v2.txt")) as f:
        text = f.read()
    # the partition the shipped table was compiled with is the cross-validated choice
    part, _ = pt.choose_partition(recs, log=lambda s: None)
    if part == "intervals":
        assert "\nrule " not in text
    else:
        assert f"depth <= {part[1]}," in text
    keep = ("regime", "rule", "bounds", "catalog")
    shipped = [ln for ln in text.splitlines() if ln.startswith(keep)]
    fresh = [ln for ln in pt.compile_table(recs, "x", part).splitlines() if ln.startswith(keep)]
    assert fresh == shipped


def _two_regime_records(threshold, n_per_family=40, fams=("clustered", "window", "iid_mixed", "iid")):
    """Synthetic records of key (128, 128): below `threshold` density plan a
    is fastest, above it plan b; densities spread evenly over [0.02, 0.5]."""
    ids = _ids((128, 128))
    a, b = ids[0], ids[3]
    recs = []
    for fi, fam in enumerate(fams):
        for i in range(n_per_family):
            dens = 0.02 + 0.48 * (i + fi / len(fams)) / n_per_family
            lat = {a: 1.0, b: 1.3} if dens < threshold else {a: 1.4, b: 1.0}
            r = _rec((128, 128), 8192, dens, 0.6, 1.2, lat)
            r["family"] = fam
            recs.append(r)
    return recs, a, b


def test_tree_learns_density_threshold(tmp_path):
    recs, a, b = _two_regime_records(0.27)
    tree = pt.fit_tree(recs, 2)
    assert tree["f"] == pt.FEATURES.index("density")
    below = max(r["density"] for r in recs if r["density"] < 0.27)
    above = min(r["density"] for r in recs if r["density"] >= 0.27)
    assert below < tree["thr"] < above
    # both leaves are pure: no further split lowers the regret
    assert "f" not in tree["lo"] and "f" not in tree["hi"]
    leaves = pt.tree_leaves(tree)
    assert [len(idx) for _, idx in leaves] == [sum(r["density"] < 0.27 for r in recs),
                                               sum(r["density"] >= 0.27 for r in recs)]
    assert pt.fit_tree(recs, 0).keys() == {"idx"}
    # the compiled table holds one rule per leaf; the library's lookup routes by the threshold
    text = pt.compile_table(recs, "vtree", ("tree", 2))
    rules = [ln for ln in text.splitlines() if ln.startswith("rule ")]
    assert len(rules) == 2 and "density<" in rules[0] and "density>=" in rules[1]
    path = tmp_path / "tree.txt"
    path.write_text(text)
    bsa.table_load(str(path))
    try:
        assert bsa.select(8, 8192, 128, (128, 128), 0.1, 0.6, 1.2) == (a, 0)
        assert bsa.select(8, 8192, 128, (128, 128), 0.4, 0.6, 1.2) == (b, 1)
        assert pt.selection_regret(text, recs) == [1.0] * len(recs)
    finally:
        bsa.table_load(None)


def test_tree_keeps_min_leaf_cases():
    # 12 of 48 cases below the threshold: a leaf of them would hold fewer than 32 cases
    recs, a, b = _two_regime_records(0.14, n_per_family=12)
    assert sum(r["density"] < 0.14 for r in recs) < pt.MIN_LEAF
    tree = pt.fit_tree(recs, 3)
    for _, idx in pt.tree_leaves(tree):
        assert len(idx) >= pt.MIN_LEAF or len(pt.tree_leaves(tree)) == 1
    assert len(pt.tree_leaves(tree)) == 1  # 48 cases cannot make two leaves of 32


def test_cross_validation_prefers_tree_off_the_fixed_bounds():
    # 0.27 lies inside the fixed density bucket [0.25, inf): the intervals mix both regimes
    recs, _, _ = _two_regime_records(0.27)
    cv = pt.cross_validate(recs, ["intervals", ("tree", 0), ("tree", 1)])
    assert cv[("tree", 1)] < cv["intervals"] and cv[("tree", 1)] < cv[("tree", 0)]
    assert cv[("tree", 1)] < 1.01
    part, _ = pt.choose_partition(recs, log=lambda s: None)
    assert part[0] == "tree" and part[1] >= 1


def test_leave_one_source_out_folds():
    """Every fold holds out all cases of one generator family: a plan that is
    fastest only on one family's masks cannot be learned for that family."""
    ids = _ids((128, 128))
    a, b = ids[0], ids[3]
    recs = []
    for fam in ("clustered", "window", "iid_mixed", "iid"):
        for i in range(40):
            lat = {a: 1.0, b: 2.0} if fam != "iid" else {a: 2.0, b: 1.0}
            r = _rec((128, 128), 8192, 0.02 + 0.01 * i, 0.6, 1.2, lat)
            r["family"] = fam
            recs.append(r)
    cv = pt.cross_validate(recs, [("tree", 2)])
    # the iid fold trains on a-favoring families only: regret 2 on its 40 cases, 1 elsewhere
    assert cv[("tree", 2)] == pytest.approx(2.0 ** (40 / 160))
