"""The build-time check of inline-assembly loads, on small hand-written device-assembly fixtures.

An inline-assembly load's registers must not be read or written before the s_waitcnt vmcnt(N) that
retires it, on any path through the control-flow graph (attention_causal_gqa_amd/asm_guard.py).
"""
from attention_causal_gqa_amd.asm_guard import hazards

LOAD = ";;#ASMSTART\n\tglobal_load_dwordx4 v[50:53], v[34:35], off\n;;#ASMEND\n"


def k(body):
    return "k:\n" + body


def test_use_in_another_block_before_the_wait_is_reported():
    # the branch skips the wait: the use in the join block may see stale data
    asm = k(LOAD + "\ts_cbranch_scc1 .LBB0_2\n; %bb.1:\n\ts_waitcnt vmcnt(0)\n"
            ".LBB0_2:\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n")
    assert hazards(asm) == ["k: v_mov_b32_e32 v1, v50"]
    # a wait on both paths
    ok = k(LOAD + "\ts_cbranch_scc1 .LBB0_2\n; %bb.1:\n\ts_waitcnt vmcnt(0)\n\ts_branch .LBB0_3\n"
           ".LBB0_2:\n\ts_waitcnt vmcnt(0)\n.LBB0_3:\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n")
    assert hazards(ok) == []


def test_a_write_to_an_in_flight_register_is_reported():
    asm = k(LOAD + "\ts_branch .LBB0_1\n.LBB0_1:\n\tv_mov_b32_e32 v51, 0\n\ts_waitcnt vmcnt(0)\n\ts_endpgm\n")
    assert hazards(asm) == ["k: v_mov_b32_e32 v51, 0"]


def test_younger_operations_retire_the_load_through_vmcnt():
    # two younger loads on every path: vmcnt(2) retires the asm load
    asm = k(LOAD + "\tglobal_load_dword v9, v[2:3], off\n\ts_cbranch_scc1 .LBB0_2\n; %bb.1:\n"
            "\tglobal_load_dword v10, v[2:3], off\n\ts_branch .LBB0_3\n"
            ".LBB0_2:\n\tglobal_load_dword v11, v[2:3], off\n"
            ".LBB0_3:\n\ts_waitcnt vmcnt(2)\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n")
    assert hazards(asm) == []
    # one path issues only one younger load: vmcnt(2) leaves the asm load in flight there
    short = asm.replace("\tglobal_load_dword v11, v[2:3], off\n", "")
    assert hazards(short) == ["k: v_mov_b32_e32 v1, v50"]


def test_flag_the_compiler_sets_and_tests_again_prunes_the_path_that_cannot_run():
    # the compiler's lowering of "if (c) { wait } ... if (!c) { wait }": a flag
    # set to -1 or 0 and tested through VCC
    body = (LOAD + "\ts_mov_b64 s[16:17], -1\n\ts_cbranch_scc1 .LBB0_2\n; %bb.1:\n"
            "\ts_waitcnt vmcnt(0)\n\ts_mov_b64 s[16:17], 0\n"
            ".LBB0_2:\n\ts_andn2_b64 vcc, exec, s[16:17]\n\ts_cbranch_vccnz .LBB0_4\n; %bb.3:\n"
            "\ts_waitcnt vmcnt(0)\n.LBB0_4:\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n")
    assert hazards(k(body)) == []
    # without the second wait the path through the skipped first wait is real
    assert hazards(k(body.replace("; %bb.3:\n\ts_waitcnt vmcnt(0)\n", "; %bb.3:\n"))) == \
        ["k: v_mov_b32_e32 v1, v50"]


def test_a_comparison_recomputed_on_the_same_operands_prunes_the_other_side():
    body = ("\tv_mov_b64_e32 v[4:5], s[6:7]\n\tv_cmp_lt_i64_e64 s[12:13], s[8:9], v[4:5]\n" + LOAD +
            "\ts_and_b64 vcc, exec, s[12:13]\n\ts_cbranch_vccz .LBB0_2\n; %bb.1:\n\ts_waitcnt vmcnt(0)\n"
            ".LBB0_2:\n\tv_cmp_ge_i64_e32 vcc, s[8:9], v[4:5]\n\ts_cbranch_vccnz .LBB0_4\n; %bb.3:\n"
            "\tv_mov_b32_e32 v1, v50\n.LBB0_4:\n\ts_endpgm\n")
    assert hazards(k(body)) == []
    # an operand redefined between the two comparisons: no longer the same condition
    changed = body.replace(".LBB0_2:\n", ".LBB0_2:\n\ts_add_u32 s8, s8, 1\n")
    assert hazards(k(changed)) == ["k: v_mov_b32_e32 v1, v50"]


def test_copy_of_a_register_refilled_for_the_next_iteration_is_reported():
    loop = (LOAD + ".LBB0_1:\n\ts_waitcnt vmcnt(0)\n\tv_add_f32_e32 v1, v50, v1\n" + LOAD +
            "{copy}\ts_cbranch_scc1 .LBB0_1\n; %bb.2:\n\ts_waitcnt vmcnt(0)\n\ts_endpgm\n")
    assert hazards(k(loop.format(copy=""))) == []
    assert hazards(k(loop.format(copy="\tv_mov_b64_e32 v[60:61], v[50:51]\n"))) == \
        ["k: v_mov_b64_e32 v[60:61], v[50:51]"]


def test_facts_about_values_a_loop_redefines_do_not_cross_its_header():
    # before the loop s2 < 4; inside, s2 grows, so the use on the s2 >= 4 side
    # (no wait) is reachable in a later iteration
    asm = k("\ts_cmp_lt_i32 s2, 4\n\ts_cbranch_scc0 .LBB0_9\n.LBB0_1:\n" + LOAD +
            "\ts_cmp_lt_i32 s2, 4\n\ts_cbranch_scc1 .LBB0_3\n; %bb.2:\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n"
            ".LBB0_3:\n\ts_waitcnt vmcnt(0)\n\ts_add_i32 s2, s2, 1\n\ts_branch .LBB0_1\n"
            ".LBB0_9:\n\ts_endpgm\n")
    assert hazards(asm) == ["k: v_mov_b32_e32 v1, v50"]
    # a loop that leaves s2 alone keeps the fact: the s2 >= 4 side never runs
    fixed = asm.replace("\ts_add_i32 s2, s2, 1\n", "\ts_add_i32 s3, s3, 1\n")
    assert hazards(fixed) == []


def test_memory_operation_under_a_possibly_empty_exec_does_not_count_as_issued():
    asm = k(LOAD + "\tv_cmp_gt_u32_e32 vcc, 4, v0\n\ts_and_saveexec_b64 s[0:1], vcc\n"
            "\tglobal_store_dword v[2:3], v1, off\n\ts_or_b64 exec, exec, s[0:1]\n"
            "\ts_waitcnt vmcnt(1)\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n")
    assert hazards(asm) == ["k: v_mov_b32_e32 v1, v50"]
    # with every lane known active (uniform code), the store counts
    uniform = k(LOAD + "\tglobal_store_dword v[2:3], v1, off\n\ts_waitcnt vmcnt(1)\n"
                "\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n")
    assert hazards(uniform) == []


def test_only_functions_with_inline_assembly_are_checked_and_allowlist_applies():
    plain = "f:\n\tglobal_load_dwordx4 v[50:53], v[34:35], off\n\tv_mov_b32_e32 v1, v50\n\ts_endpgm\n"
    assert hazards(plain) == []
    asm = k(LOAD + "\tv_mov_b32_e32 v1, v50\n\ts_waitcnt vmcnt(0)\n\ts_endpgm\n")
    assert hazards(asm) == ["k: v_mov_b32_e32 v1, v50"]
    assert hazards(asm, allowed=["k: v_mov_b32_e32 v1, v50"]) == []


def test_a_load_under_two_conditions_and_an_exit_on_one_of_them():
    # if (c && j == 0) load; if (!c) use (no wait): the load and the use
    # never meet, since the load implies c
    body = ("\tv_mov_b64_e32 v[4:5], s[6:7]\n\tv_cmp_lt_i64_e64 s[12:13], s[8:9], v[4:5]\n"
            "\ts_cmp_eq_u32 s10, 0\n\ts_cselect_b64 s[14:15], -1, 0\n"
            "{both}\ts_andn2_b64 vcc, exec, s[14:15]\n\ts_cbranch_vccnz .LBB0_2\n; %bb.1:\n" + LOAD +
            ".LBB0_2:\n\ts_andn2_b64 vcc, exec, s[12:13]\n\ts_cbranch_vccnz .LBB0_4\n; %bb.3:\n"
            "\ts_waitcnt vmcnt(0)\n\ts_branch .LBB0_5\n.LBB0_4:\n\tv_mov_b32_e32 v1, v50\n.LBB0_5:\n\ts_endpgm\n")
    assert hazards(k(body.format(both="\ts_and_b64 s[14:15], s[12:13], s[14:15]\n"))) == []
    # the load under j == 0 alone: with !c it is still in flight at the use
    assert hazards(k(body.format(both=""))) == ["k: v_mov_b32_e32 v1, v50"]


def test_a_uniform_copy_made_on_two_paths_keeps_its_value_through_joins_and_the_loop():
    # v[4:5] holds s[6:7] on both paths into the loop (s6 differs between
    # them); a flag keeps the paths apart until inside the loop, where they
    # join.  The loop never writes s[6:7] or v[4:5], so the comparison against
    # v[4:5] names one value in every iteration and the recomputed comparison
    # prunes the use on the side without the wait.
    asm = k("\ts_cbranch_scc1 .LBB0_1\n; %bb.0:\n\ts_add_u32 s6, s6, 1\n\tv_mov_b64_e32 v[4:5], s[6:7]\n"
            "\ts_mov_b64 s[20:21], -1\n\ts_branch .LBB0_2\n"
            ".LBB0_1:\n\tv_mov_b64_e32 v[4:5], s[6:7]\n\ts_mov_b64 s[20:21], 0\n"
            ".LBB0_2:\n\ts_and_b64 vcc, exec, s[20:21]\n\ts_cbranch_vccz .LBB0_3\n; %bb.a:\n\ts_nop 0\n"
            ".LBB0_3:\n\ts_mov_b64 s[20:21], 0\n\ts_branch .LBB0_4\n"
            ".LBB0_4:\n\tv_cmp_lt_i64_e64 s[12:13], s[8:9], v[4:5]\n" + LOAD +
            "\ts_and_b64 vcc, exec, s[12:13]\n\ts_cbranch_vccz .LBB0_6\n; %bb.5:\n\ts_waitcnt vmcnt(0)\n"
            ".LBB0_6:\n\tv_cmp_ge_i64_e32 vcc, s[8:9], v[4:5]\n\ts_cbranch_vccnz .LBB0_8\n; %bb.7:\n"
            "\tv_mov_b32_e32 v1, v50\n.LBB0_8:\n\ts_waitcnt vmcnt(0)\n\ts_add_i32 s2, s2, -1\n"
            "\ts_cmp_lg_u32 s2, 0\n\ts_cbranch_scc1 .LBB0_2\n; %bb.9:\n\ts_endpgm\n")
    assert hazards(asm) == []
    # s6 written inside the loop: the check names v[4:5]'s value after the
    # version of s[6:7] it was copied from, and a name the loop redefines does
    # not survive its header, so the use is reported (a conservative answer)
    assert hazards(asm.replace("\ts_add_i32 s2, s2, -1\n", "\ts_add_i32 s2, s2, -1\n\ts_add_u32 s6, s6, 1\n")) == \
        ["k: v_mov_b32_e32 v1, v50"]
    # v[4:5] refilled inside the loop from another register: a new value
    # between the two comparisons is caught as before
    assert hazards(asm.replace("\ts_cbranch_vccz .LBB0_6\n; %bb.5:", "\tv_mov_b64_e32 v[4:5], s[16:17]\n"
                               "\ts_cbranch_vccz .LBB0_6\n; %bb.5:")) == ["k: v_mov_b32_e32 v1, v50"]


def test_an_execz_branch_under_the_whole_wave_mask_is_not_taken():
    # the structurizer's "skip the arm if no lane is left in it" test: under
    # the whole wave's mask the skip cannot happen, so the wait in the arm
    # always runs before the write
    tail = ("\ts_cbranch_execz .LBB0_2\n; %bb.1:\n\ts_waitcnt vmcnt(0)\n"
            ".LBB0_2:\n\ts_or_b64 exec, exec, s[0:1]\n\tv_mov_b32_e32 v51, 0\n\ts_endpgm\n")
    assert hazards(k(LOAD + "\ts_mov_b64 s[0:1], 0\n" + tail)) == []
    # under a mask that may be empty (s_and_saveexec of a lane condition) the
    # arm, and its wait, may be skipped: the write is reported
    masked = LOAD + "\tv_cmp_gt_u32_e32 vcc, 4, v0\n\ts_and_saveexec_b64 s[0:1], vcc\n" + tail
    assert hazards(k(masked)) == ["k: v_mov_b32_e32 v51, 0"]
