"""The attention kernels' asm-issued LDS reads are never touched in flight
(static check of the shipped gfx950 code, see lds_wait_check.py), and the
checker itself catches the mistakes it exists for."""

import os

import pytest

import lds_wait_check as chk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SO = os.path.join(ROOT, "dynamic_block_sparse_bsa_amd", "libbsa.so")


def test_checker_flags_use_before_wait():
    prog = ["ds_read_b128 v[0:3], v10", "v_mov_b32_e32 v20, v1", "s_waitcnt lgkmcnt(0)"]
    h = chk.check_function(prog)
    assert len(h) == 1 and h[0][2] == ("v", 1)


def test_checker_counts_waits_in_order():
    prog = ["ds_read_b128 v[0:3], v10", "ds_read_b128 v[4:7], v11", "s_waitcnt lgkmcnt(1)",
            "v_mov_b32_e32 v20, v1",   # first read retired: fine
            "v_mov_b32_e32 v21, v5",   # second still in flight: hazard
            "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v22, v6"]
    h = chk.check_function(prog)
    assert [x[2] for x in h] == [("v", 5)]


def test_checker_agpr_and_overwrite():
    prog = ["ds_read_b64_tr_b16 a[4:5], v3 offset:8192", "v_accvgpr_write_b32 a5, v0",
            "s_waitcnt lgkmcnt(0)"]
    assert [x[2] for x in chk.check_function(prog)] == [("a", 5)]


def test_checker_scalar_loads_do_not_retire_lds_reads():
    # lgkmcnt(1) with an older LDS read and a younger scalar load in flight:
    # the scalar load may have completed first, so the read is still pending
    prog = ["ds_read_b128 v[0:3], v10", "s_load_dword s4, s[0:1], 0x0", "s_waitcnt lgkmcnt(1)",
            "v_mov_b32_e32 v20, v2", "s_waitcnt lgkmcnt(0)"]
    assert [x[2] for x in chk.check_function(prog)] == [("v", 2)]


def test_checker_address_register_may_change():
    # the address operand is consumed at issue; only the destination is live
    prog = ["ds_read_b128 v[0:3], v10", "v_add_u32_e32 v10, 64, v10", "s_waitcnt lgkmcnt(0)"]
    assert chk.check_function(prog) == []


def test_checker_writes_have_no_destination():
    prog = ["ds_write_b128 v10, v[0:3]", "v_mov_b32_e32 v1, 0", "s_waitcnt lgkmcnt(0)"]
    assert chk.check_function(prog) == []


needs_lib = pytest.mark.skipif(not (os.path.exists(SO) and chk.tools_available()),
                               reason="libbsa.so not built or ROCm LLVM tools missing")


@needs_lib
def test_attention_kernels_have_no_lds_hazard():
    res, n_reads, n_funcs = chk.attention_hazards(SO)
    assert n_funcs >= 13 and n_reads > 1000, (n_funcs, n_reads)
    assert res == {}, {k: v[:3] for k, v in res.items()}


@needs_lib
def test_removing_a_wait_in_real_code_is_caught():
    """Delete, in a real attention kernel, the first lgkmcnt wait that follows
    a transposed V read: the checker must then report its consumer."""
    for co in chk.gfx950_code_objects(SO):
        funcs = chk.functions(chk.disassemble(co))
        name = next((n for n in funcs if "attn_fwd_kernel" in n), None)
        if name is None:
            continue
        ins = funcs[name]
        first_tr = next(i for i, x in enumerate(ins) if x.startswith("ds_read_b64_tr_b16"))
        wait = next(i for i in range(first_tr, len(ins))
                    if ins[i].startswith("s_waitcnt") and "lgkmcnt" in ins[i])
        broken = ins[:wait] + ins[wait + 1:]
        assert chk.check_function(ins) == []
        assert chk.check_function(broken) != []
        return
    pytest.fail("no attention kernel found in the library")
