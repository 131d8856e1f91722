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
    cat = bsa.catalog()
    assert 14 <= len(cat) <= 40
    names = [e["name"] for e in cat]
    assert len(set(names)) == len(names)
    assert re.fullmatch(r"[0-9a-f]{16}", bsa.catalog_hash())


def test_base_plan_direct_or_smallest_refined():
    cat = {e["id"]: e for e in bsa.catalog()}
    pid, reg = bsa.select(8, 8192, 128, (128, 128), 0.3, 0.5)
    e = cat[pid]
    assert (e["tile_q"], e["tile_kv"]) == (128, 128)  # Direct when the catalog has T = B
    pid, reg = bsa.select(24, 115200, 128, (32, 128), 0.1, 0.5)
    e = cat[pid]
    assert e["tile_q"] * e["tile_kv"] == min(
        c["tile_q"] * c["tile_kv"] for c in cat.values()
        if bsa.eligible(c["id"], 24, 115200, 128, (32, 128)))


def test_eligibility_rules():
    cat = bsa.catalog()
    by = {(e["tile_q"], e["tile_kv"], e["d"], e["split"], e["xcd_remap"]): e["id"] for e in cat}
    # coarsening B_Q = 16 into a 64-row tile would split a wave across logical rows
    assert not bsa.eligible(by[(64, 64, 128, 1, 0)], 1, 1024, 128, (16, 64))
    assert bsa.eligible(by[(64, 64, 128, 1, 0)], 1, 1024, 128, (32, 64))
    assert not bsa.eligible(by[(64, 64, 128, 1, 0)], 1, 1024, 64, (64, 64))  # head dim
    assert bsa.eligible(by[(128, 32, 128, 1, 0)], 1, 1024, 128, (64, 128))  # mixed map


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
                    f"bounds density 0.2\nregime 128 128 128 * * 1 * : {name}\n")
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
