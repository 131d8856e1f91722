"""CPU-only checks of the C-ABI library: it loads, exports every symbol the
header declares, and its host-side selection logic behaves (no GPU calls)."""

import os
import re

import pytest

import dynamic_block_sparse_bsa_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_symbols():
    txt = open(os.path.join(ROOT, "include", "bsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(bsa_\w+)\s*\(", txt, re.M)))


def test_library_exports_header_symbols():
    lib = bsa._load()
    syms = _header_symbols()
    assert len(syms) >= 15
    for s in syms:
        assert hasattr(lib, s), s


def test_catalog_and_hash():
    """The native catalog: 39 entries over 15 kernel tile shapes (33 entries
    at d = 64 and 128, where the pages' catalogs hold 14-26 entries per
    architecture, plus one per shape at d = 32 and 256), every shape with the
    default organization that base plans use, every entry a distinct
    (shape, organization)."""
    cat = bsa.catalog()
    shapes = {(e["tile_q"], e["tile_kv"], e["d"]) for e in cat}
    orgs = {(e["split"], e["xcd_remap"], e["order"]) for e in cat}
    assert len(cat) == 39 and len(shapes) == 15
    assert orgs <= {(2, 0, 0), (0, 0, 0), (2, 16, 0), (2, 128, 0), (2, 0, 1), (3, 0, 1), (4, 0, 1), (0, 0, 1),
                    (2, 16, 2)}
    for sh in shapes:
        assert any((e["tile_q"], e["tile_kv"], e["d"]) == sh and (e["split"], e["xcd_remap"], e["order"]) == (2, 0, 0)
                   for e in cat), sh
    assert len({(e["tile_q"], e["tile_kv"], e["d"], e["split"], e["xcd_remap"], e["order"]) for e in cat}) == 39
    per_d = {d: sum(1 for e in cat if e["d"] == d) for d in (32, 64, 128, 256)}
    assert per_d == {32: 4, 64: 11, 128: 22, 256: 2}
    names = [e["name"] for e in cat]
    assert len(set(names)) == len(names)
    assert re.fullmatch(r"[0-9a-f]{16}", bsa.catalog_hash())


def test_base_plan_direct_or_smallest_refined():
    cat = {e["id"]: e for e in bsa.catalog()}
    e = cat[bsa.base_plan(8, 8192, 128, (128, 128))]
    assert (e["tile_q"], e["tile_kv"]) == (128, 128)  # Direct when the catalog has T = B
    assert e["split"] == 2 and e["xcd_remap"] == 0 and e["order"] == 0  # default organization
    e = cat[bsa.base_plan(24, 115200, 128, (32, 128))]
    assert e["tile_q"] * e["tile_kv"] == min(
        c["tile_q"] * c["tile_kv"] for c in cat.values()
        if bsa.eligible(c["id"], 24, 115200, 128, (32, 128)))


def test_lookup_miss_returns_base_plan(tmp_path):
    empty = tmp_path / "empty.txt"
    empty.write_text(f"bsa-plan-table empty\narch gfx950\ncatalog {bsa.catalog_hash()}\n")
    bsa.table_load(str(empty))
    try:
        for block in ((128, 128), (32, 128), (128, 32), (64, 64)):
            pid, reg = bsa.select(8, 8192, 128, block, 0.3, 0.5)
            assert reg == -1 and pid == bsa.base_plan(8, 8192, 128, block)
    finally:
        bsa.table_load(None)


def test_builtin_table_is_versioned_and_covers_workload_keys():
    assert bsa.table_version().startswith("v2")
    for H, N, d, block, dens, rc, sk in ((8, 8192, 128, (128, 128), 0.31, 0.5, 3.2),
                                         (40, 75600, 128, (64, 64), 0.13, 0.9, 1.3),
                                         (24, 115200, 128, (128, 32), 0.17, 0.86, 1.7),
                                         (24, 115200, 128, (32, 128), 0.2, 0.9, 1.5)):
        pid, reg = bsa.select(H, N, d, block, dens, rc, sk)
        assert reg >= 0, (block, N)
        assert bsa.eligible(pid, H, N, d, block)


def test_eligibility_rules():
    cat = bsa.catalog()
    by = {(e["tile_q"], e["tile_kv"], e["d"], e["split"], e["xcd_remap"]): e["id"] for e in cat
          if e["order"] == 0}
    # B_Q = 16 only inside coarsened query tiles (a wave's rows then span two
    # logical rows, resolved per lane), within 32 membership bits
    assert bsa.eligible(by[(64, 64, 128, 2, 0)], 1, 1024, 128, (16, 64))      # 4 x 1 blocks
    assert bsa.eligible(by[(128, 64, 128, 2, 0)], 1, 1024, 128, (16, 16))     # 8 x 4 blocks
    assert not bsa.eligible(by[(128, 128, 128, 2, 0)], 1, 1024, 128, (16, 16))  # 8 x 8 > 32 bits
    assert bsa.eligible(by[(64, 64, 128, 2, 0)], 1, 1024, 128, (32, 64))
    assert not bsa.eligible(by[(64, 64, 128, 2, 0)], 1, 1024, 64, (64, 64))  # head dim
    assert bsa.eligible(by[(128, 32, 128, 2, 0)], 1, 1024, 128, (64, 128))  # mixed map
    # head dims 32 and 256 (request property x, Tessera section 4.4)
    assert bsa.eligible(by[(64, 64, 32, 2, 0)], 1, 1024, 32, (64, 64))
    assert not bsa.eligible(by[(64, 64, 32, 2, 0)], 1, 1024, 64, (64, 64))
    assert bsa.eligible(by[(64, 32, 256, 2, 0)], 1, 1024, 256, (64, 64))
    assert bsa.eligible(by[(128, 32, 256, 2, 0)], 1, 1024, 256, (128, 32))
    assert not bsa.eligible(by[(128, 32, 256, 2, 0)], 1, 1024, 128, (128, 32))
    for d in (32, 256):
        for block in ((64, 64), (128, 128), (128, 32), (32, 128)):
            e = {c["id"]: c for c in cat}[bsa.base_plan(4, 4096, d, block)]
            assert e["d"] == d and (e["split"], e["xcd_remap"], e["order"]) == (2, 0, 0)


def test_unsupported_request_errors():
    with pytest.raises(bsa.BsaError) as ei:
        bsa.select(1, 1024, 96, (64, 64), 0.1, 0.1)
    assert "UNSUPPORTED" in str(ei.value)


def test_table_load_rejects_bad_tables(tmp_path):
    bad = tmp_path / "t.txt"
    bad.write_text("bsa-plan-table x\narch gfx942\ncatalog 0\n")
    with pytest.raises(bsa.BsaError) as ei:
        bsa.table_load(str(bad))
    assert "TABLE" in str(ei.value)
    bad.write_text(f"bsa-plan-table x\narch gfx950\ncatalog {'0' * 16}\n")
    with pytest.raises(bsa.BsaError):
        bsa.table_load(str(bad))
    good = tmp_path / "g.txt"
    name = bsa.catalog()[3]["name"]
    good.write_text(f"bsa-plan-table test1\narch gfx950\ncatalog {bsa.catalog_hash()}\n"
                    f"bounds density 0.2\nregime 128 128 128 * * 1 * * : {name}\n")
    bsa.table_load(str(good))
    try:
        assert bsa.table_version() == "test1"
        pid, reg = bsa.select(8, 8192, 128, (128, 128), 0.3, 0.5)
        assert reg == 0
        # the ranking's plan (T=64x64) is eligible for B=128x128 (refined)
        assert pid == 3
        pid, reg = bsa.select(8, 8192, 128, (128, 128), 0.1, 0.5)
        assert reg == -1  # density bucket 0: lookup miss -> base plan
    finally:
        bsa.table_load(None)
    assert bsa.table_version() != "test1"


def test_table_rules_parse_and_route(tmp_path):
    """Decision-tree leaves in the table text: threshold tests on the regime
    features, every test of a rule must hold, first match in file order."""
    names = {e["id"]: e["name"] for e in bsa.catalog()}
    ids = [e["id"] for e in bsa.catalog() if bsa.eligible(e["id"], 8, 8192, 128, (64, 64))]
    a, b, c = ids[0], ids[1], ids[2]
    head = f"bsa-plan-table vrules\narch gfx950\ncatalog {bsa.catalog_hash()}\n"
    text = head + (f"rule 64 64 128 N<20000 density<0.25 : {names[a]}\n"
                   f"rule 64 64 128 N<20000 density>=0.25 : {names[b]}\n"
                   f"rule 64 64 128 H>=16 row_skew>=2.5 : {names[c]}\n")
    p = tmp_path / "rules.txt"
    p.write_text(text)
    bsa.table_load(str(p))
    try:
        assert bsa.select(8, 8192, 128, (64, 64), 0.1, 0.5, 1.0) == (a, 0)
        assert bsa.select(8, 8192, 128, (64, 64), 0.25, 0.5, 1.0) == (b, 1)
        assert bsa.select(32, 40000, 128, (64, 64), 0.25, 0.5, 3.0) == (c, 2)
        # no rule matches: the key's base plan, regime -1
        assert bsa.select(8, 40000, 128, (64, 64), 0.25, 0.5, 3.0) == (bsa.base_plan(8, 40000, 128, (64, 64)), -1)
    finally:
        bsa.table_load(None)
    for bad in (f"rule 64 64 128 density<<0.2 : {names[a]}\n", f"rule 64 64 128 depth<3 : {names[a]}\n",
                f"rule 64 64 128 density=0.2 : {names[a]}\n", f"rule 64 64 128 density<0.2 {names[a]}\n",
                f"rule 64 * 128 : {names[a]}\n"):
        p.write_text(head + bad)
        with pytest.raises(bsa.BsaError):
            bsa.table_load(str(p))
    assert bsa.table_version() != "vrules"


def _create_status(**kw):
    """bsa_plan_create on a request that host-side validation must reject
    (the mask pointer is never dereferenced)."""
    import ctypes
    args = dict(H=4, N=1024, d=128, block=(64, 64), mask_ptr=16, batch=1, layout="HND")
    args.update(kw)
    req = bsa._request(args["H"], args["N"], args["d"], args["block"], args["mask_ptr"], batch=args["batch"],
                       layout=args["layout"])
    if "raw_layout" in kw:
        req.layout = kw["raw_layout"]
    h = ctypes.c_void_p()
    L = bsa._load()
    st = L.bsa_plan_create(ctypes.byref(req), None, ctypes.byref(h))
    return L.bsa_status_string(st).decode()


def test_layout_and_batch_validation():
    assert _create_status(raw_layout=2) == "BSA_ERR_UNSUPPORTED"
    assert _create_status(batch=-1) == "BSA_ERR_INVALID_ARG"
    assert _create_status(H=1 << 16, batch=1 << 15) == "BSA_ERR_UNSUPPORTED"  # batch * H >= 2^31
    # NHD rows of one head are H*d elements apart: N * H * d * 2 bytes must stay below 2^31
    assert _create_status(H=64, N=131072, layout="NHD") == "BSA_ERR_UNSUPPORTED"
    assert _create_status(mask_ptr=None, layout="NHD") == "BSA_ERR_INVALID_ARG"
    # block geometries outside the documented ranges are refused before any
    # launch (the mask pointer is never read)
    assert _create_status(block=(8, 64)) == "BSA_ERR_UNSUPPORTED"
    assert _create_status(block=(512, 64)) == "BSA_ERR_UNSUPPORTED"
    assert _create_status(block=(64, 8)) == "BSA_ERR_UNSUPPORTED"
    assert _create_status(block=(48, 64)) == "BSA_ERR_UNSUPPORTED"
    assert _create_status(d=96) == "BSA_ERR_UNSUPPORTED"
    assert _create_status(d=512) == "BSA_ERR_UNSUPPORTED"
    with pytest.raises(bsa.BsaError):
        bsa.tensor_shapes(4, 1024, 128, layout="HDN")


def test_batch_folds_into_heads_for_selection():
    """Every (batch entry, head) pair is one head of the request: the regime
    lookup and eligibility see batch * H heads, for either layout."""
    for block in ((64, 64), (128, 128)):
        for dens in (0.05, 0.3):
            want = bsa.select(32, 75600, 128, block, dens, 0.5, 1.5)
            assert bsa.select(8, 75600, 128, block, dens, 0.5, 1.5, batch=4) == want
            assert bsa.select(8, 75600, 128, block, dens, 0.5, 1.5, batch=4, layout="NHD") == want
    assert bsa.base_plan(2, 4096, 64, (64, 64), batch=3) == bsa.base_plan(6, 4096, 64, (64, 64))
    ids = [e["id"] for e in bsa.catalog()]
    assert [bsa.eligible(i, 4, 2048, 128, (64, 64), layout="NHD") for i in ids] == \
        [bsa.eligible(i, 4, 2048, 128, (64, 64)) for i in ids]
    assert bsa.tensor_shapes(4, 100, 64, batch=2, layout="NHD") == [(2, 100, 4, 64)]
    assert bsa.tensor_shapes(4, 100, 64) == [(1, 4, 100, 64), (4, 100, 64)]
