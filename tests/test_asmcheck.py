"""The static load/wait check of the kernels' gfx950 assembly, on small
hand-written snippets whose verdict is known."""

import textwrap

from moe_grouped_precision_amd import asmcheck


def _check(tmp_path, body):
    src = tmp_path / "k.s"
    src.write_text("kern:\n" + textwrap.dedent(body) + "\ts_endpgm\n")
    return asmcheck.check(str(src))


def test_read_before_wait_is_found(tmp_path):
    f = _check(tmp_path, """
        global_load_dwordx4 v[0:3], v10, s[2:3]
        v_add_f32_e32 v4, v0, v1
    """)
    assert any("reads VGPR v0" in x for x in f)


def test_covering_wait_clears_it(tmp_path):
    f = _check(tmp_path, """
        global_load_dwordx4 v[0:3], v10, s[2:3]
        global_load_dwordx4 v[4:7], v10, s[2:3]
        s_waitcnt vmcnt(1)
        v_add_f32_e32 v8, v0, v1
    """)
    assert f == []


def test_wait_that_leaves_the_load_pending(tmp_path):
    # loads complete in issue order: vmcnt(1) after two loads leaves the newer one
    f = _check(tmp_path, """
        global_load_dwordx4 v[0:3], v10, s[2:3]
        global_load_dwordx4 v[4:7], v10, s[2:3]
        s_waitcnt vmcnt(1)
        v_add_f32_e32 v8, v4, v1
    """)
    assert any("reads VGPR v4" in x for x in f)


def test_overwrite_of_a_pending_destination(tmp_path):
    f = _check(tmp_path, """
        global_load_dword v5, v10, s[2:3]
        v_mov_b32_e32 v5, 0
    """)
    assert any("overwrites VGPR v5" in x for x in f)


def test_lds_dma_has_no_register_destination(tmp_path):
    f = _check(tmp_path, """
        global_load_lds_dwordx4 v10, s[2:3]
        v_add_u32_e32 v10, 16, v10
    """)
    assert f == []


def test_valu_written_sgpr_needs_five_wait_states(tmp_path):
    bad = _check(tmp_path, """
        v_readfirstlane_b32 s2, v0
        v_readfirstlane_b32 s3, v1
        global_load_dwordx4 v[4:7], v10, s[2:3]
        s_waitcnt vmcnt(0)
    """)
    assert any("SGPR" in x for x in bad)
    good = _check(tmp_path, """
        v_readfirstlane_b32 s2, v0
        v_readfirstlane_b32 s3, v1
        s_nop 4
        global_load_dwordx4 v[4:7], v10, s[2:3]
        s_waitcnt vmcnt(0)
    """)
    assert good == []


def test_pending_load_carried_around_a_loop(tmp_path):
    # the load issued at the bottom of the loop is read at the top of the next
    # iteration before any wait
    f = _check(tmp_path, """
        s_mov_b32 s4, 8
    .Lloop:
        v_add_f32_e32 v8, v0, v1
        global_load_dwordx4 v[0:3], v10, s[2:3]
        s_sub_u32 s4, s4, 1
        s_cbranch_scc1 .Lloop
        s_waitcnt vmcnt(0)
    """)
    assert any("reads VGPR v0" in x for x in f)


def test_pending_load_across_a_branch_merge(tmp_path):
    f = _check(tmp_path, """
        s_cbranch_scc1 .Lskip
        global_load_dword v5, v10, s[2:3]
    .Lskip:
        v_add_u32_e32 v6, v5, v5
        s_waitcnt vmcnt(0)
    """)
    assert any("reads VGPR v5" in x for x in f)


def test_long_branch_target_is_followed(tmp_path):
    # a kernel too large for short branches jumps through s_getpc/s_setpc; the
    # target's code must be checked with the state the branch carries
    f = _check(tmp_path, """
        global_load_dwordx4 v[0:3], v10, s[2:3]
        s_getpc_b64 s[8:9]
    .Lpost_getpc0:
        s_add_u32 s8, s8, (.LBB0_2-.Lpost_getpc0)&4294967295
        s_addc_u32 s9, s9, (.LBB0_2-.Lpost_getpc0)>>32
        s_setpc_b64 s[8:9]
    .LBB0_1:
        s_nop 0
    .LBB0_2:
        v_mov_b64_e32 v[20:21], v[0:1]
    """)
    assert any("reads VGPR v0" in x for x in f)


def test_unreachable_code_is_reported(tmp_path):
    # code the parsed control-flow graph cannot reach would escape the check
    f = _check(tmp_path, """
        s_branch .LBB0_2
    .LBB0_1:
        v_mov_b32_e32 v1, v2
    .LBB0_2:
        s_nop 0
    """)
    assert any("unreachable" in x for x in f)
