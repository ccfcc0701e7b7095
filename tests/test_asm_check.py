"""The assembly check that guards the inline-asm LDS transpose reads: it must
flag a use of a read's destination before the covering wait, and accept the
pipelined pattern the kernels use (several reads in flight, partial waits)."""
from decode_fmha_fwd_amd.asm_check import check_text


def _asm(*lines):
    """A kernel body: entries ending in ':' are block labels (column 0)."""
    out = ["kern:"]
    for l in lines:
        out.append(l if l.endswith(":") else "\t" + l)
    return "\n".join(out) + "\n"


READ = [";;#ASMSTART", "ds_read_b64_tr_b16 v[0:1], v10 offset:64", ";;#ASMEND"]
READ2 = [";;#ASMSTART", "ds_read_b64_tr_b16 v[2:3], v10 offset:128", ";;#ASMEND"]


def test_copy_before_wait_is_flagged():
    r = check_text(_asm(*READ, "v_mov_b64_e32 v[102:103], v[0:1]",
                        ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND"))
    assert r.reads == 1 and len(r.problems) == 1 and "v_mov_b64" in r.problems[0]


def test_use_after_wait_is_fine():
    r = check_text(_asm(*READ, "v_add_u32_e32 v5, v6, v7",
                        ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND",
                        "v_mfma_f32_16x16x16_bf16 v[20:23], v[0:1], v[4:5], v[20:23]"))
    assert r.reads == 1 and r.problems == []


def test_partial_wait_counts_later_reads():
    # lgkmcnt(1) with one LDS op issued after the first read: the first is done,
    # the second is not
    ok = check_text(_asm(*READ, *READ2, "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v9, v0",
                         "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v9, v2"))
    assert ok.problems == []
    bad = check_text(_asm(*READ, *READ2, "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v9, v3",
                          "s_waitcnt lgkmcnt(0)"))
    assert len(bad.problems) == 1 and "v[2, 3]" in bad.problems[0]


def test_write_to_destination_and_scalar_loads():
    waw = check_text(_asm(*READ, "v_mov_b32_e32 v1, 0", "s_waitcnt lgkmcnt(0)"))
    assert len(waw.problems) == 1
    # a scalar load issued after the read may return first: lgkmcnt(1) does not cover it
    smem = check_text(_asm(*READ, "s_load_dword s4, s[0:1], 0x0", "s_waitcnt lgkmcnt(1)",
                           "v_mov_b32_e32 v9, v0", "s_waitcnt lgkmcnt(0)"))
    assert len(smem.problems) == 1
    # ... nor does a pending scalar load issued before it
    before = check_text(_asm("s_load_dword s4, s[0:1], 0x0", *READ, "s_waitcnt lgkmcnt(1)",
                             "v_mov_b32_e32 v9, v0", "s_waitcnt lgkmcnt(0)"))
    assert len(before.problems) == 1


def test_scalar_load_between_reads_does_not_void_a_partial_wait():
    # READ, scalar load, READ2, lgkmcnt(1): one LDS read follows READ, so READ
    # is complete (a pending scalar load only raises the counter); READ2 is not
    ok = check_text(_asm(*READ, "s_load_dword s4, s[0:1], 0x0", *READ2, "s_waitcnt lgkmcnt(1)",
                         "v_mov_b32_e32 v9, v0", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v9, v2"))
    assert ok.problems == []
    bad = check_text(_asm(*READ, "s_load_dword s4, s[0:1], 0x0", *READ2, "s_waitcnt lgkmcnt(1)",
                          "v_mov_b32_e32 v9, v2", "s_waitcnt lgkmcnt(0)"))
    assert len(bad.problems) == 1


def test_use_on_a_branch_path_before_the_wait_is_flagged():
    r = check_text(_asm(*READ, "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)",
                        ".LBB0_2:", "v_mov_b32_e32 v9, v0", "s_waitcnt lgkmcnt(0)"))
    assert len(r.problems) == 1 and "v_mov_b32_e32 v9, v0" in r.problems[0]


def test_wait_on_every_path_after_a_branch_is_fine():
    # the kernels issue copies under uniform branches while LDS reads are in
    # flight; every path then reaches the wait before the use
    r = check_text(_asm(*READ, "s_cbranch_scc0 .LBB0_2", "global_load_lds_dwordx4 v[4:5], off",
                        ".LBB0_2:", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v9, v0"))
    assert r.problems == []


def test_join_keeps_the_fewest_later_lds_ops():
    # on the taken path one more LDS op follows the read; on the other none, so
    # lgkmcnt(1) at the join does not cover the read
    r = check_text(_asm(*READ, "s_cbranch_scc0 .LBB0_2", "ds_read_b32 v20, v21",
                        ".LBB0_2:", "s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v9, v0",
                        "s_waitcnt lgkmcnt(0)"))
    assert len(r.problems) == 1


def test_read_pending_around_a_loop_is_flagged():
    # a read issued at the bottom of a loop and used at its top without a wait
    r = check_text(_asm(".LBB0_1:", "v_mov_b32_e32 v9, v0", *READ, "s_cbranch_scc1 .LBB0_1",
                        "s_waitcnt lgkmcnt(0)"))
    assert len(r.problems) == 1


def test_compiler_managed_reads_are_not_tracked():
    # a transpose read outside an inline-asm region is the compiler's to wait for
    r = check_text(_asm("ds_read_b64_tr_b16 v[0:1], v10", "v_mov_b32_e32 v9, v0"))
    assert r.reads == 0 and r.problems == []
