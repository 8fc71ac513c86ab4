"""The build's path checks over the generated gfx950 assembly.  From every MFMA,
every path (fall-through and branch targets) must keep reads of its result at
least 8 wait states away, except the accumulator of the next MFMA on the same
registers and interlocked v_accvgpr_read of an AGPR result (CPU only)."""
import pytest

from ssd_chunked_scan_amd import _build

HDR = "k:\n"


def _asm(*lines):
    return HDR + "\n".join("\t" + l if not l.endswith(":") else l for l in lines) + "\n"


def test_rejects_short_straight_line_read():
    asm = _asm("v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
               "s_nop 3",
               "v_mul_f32_e32 v20, v1, v21")
    with pytest.raises(RuntimeError):
        _build.check_mfma_result_reads(asm, "t")


def test_rejects_read_in_taken_branch_target():
    # the fall-through path is long enough, the taken branch is not
    asm = _asm("v_mfma_f32_16x16x32_bf16 v[62:65], v[194:197], v[34:37], 0",
               "s_cbranch_vccnz .LBB0_2",
               "s_nop 15",
               "v_mul_f32_e32 v3, v63, v189",
               ".LBB0_2:",
               "v_mul_f32_e32 v3, v63, v189")
    with pytest.raises(RuntimeError):
        _build.check_mfma_result_reads(asm, "t")


def test_accepts_safe_forms():
    asm = _asm("v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
               "v_mfma_f32_16x16x32_bf16 v[0:3], v[12:15], v[16:19], v[0:3]",   # chain
               "s_nop 7",
               "v_mul_f32_e32 v20, v1, v21",                                    # 8 wait states
               "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], 0",
               "v_accvgpr_read_b32 v30, a0",                                    # interlocked
               "s_endpgm")
    assert _build.check_mfma_result_reads(asm, "t") == 3


def test_rejects_result_used_as_a_operand_too_soon():
    asm = _asm("v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
               "v_mfma_f32_16x16x32_bf16 v[20:23], v[0:3], v[8:11], 0")
    with pytest.raises(RuntimeError):
        _build.check_mfma_result_reads(asm, "t")


def test_counted_barrier_wait_accepts_newer_plain_loads():
    asm = _asm("global_load_lds_dwordx4 v[0:1], off",
               "global_load_dwordx4 v[2:5], v[6:7], off",
               "global_load_dwordx4 v[8:11], v[6:7], off offset:64",
               "s_waitcnt vmcnt(2) lgkmcnt(0)",
               "s_barrier")
    assert _build.check_counted_barrier_waits(asm, "t") == 1


def test_counted_barrier_wait_rejects_lds_load_in_flight():
    asm = _asm("global_load_dwordx4 v[2:5], v[6:7], off",
               "global_load_lds_dwordx4 v[0:1], off",
               "global_load_dwordx4 v[8:11], v[6:7], off offset:64",
               "s_waitcnt vmcnt(2) lgkmcnt(0)",
               "s_barrier")
    with pytest.raises(RuntimeError):
        _build.check_counted_barrier_waits(asm, "t")


def test_counted_barrier_wait_rejects_label_in_window():
    asm = _asm("global_load_dwordx4 v[2:5], v[6:7], off",
               ".LBB0_3:",
               "global_load_dwordx4 v[8:11], v[6:7], off offset:64",
               "s_waitcnt vmcnt(2) lgkmcnt(0)",
               "s_barrier")
    with pytest.raises(RuntimeError):
        _build.check_counted_barrier_waits(asm, "t")


# look-ahead waits (vmem_lds_sync_lookahead): the marker comment precedes the
# wait, and exactly the K newest vector-memory operations must be
# direct-to-LDS loads on straight-line code

def test_lookahead_wait_accepts_newest_lds_loads():
    asm = _asm("global_load_dwordx4 v[2:5], v[6:7], off",
               "global_load_lds_dwordx4 v[0:1], off",
               "s_mov_b32 m0, s6",
               "global_load_lds_dwordx4 v[8:9], off",
               "; ssd lookahead wait 1",
               "s_waitcnt vmcnt(2) lgkmcnt(0)",
               "s_barrier")
    assert _build.check_counted_barrier_waits(asm, "t") == 1


def test_lookahead_wait_rejects_plain_load_in_flight():
    asm = _asm("global_load_lds_dwordx4 v[0:1], off",
               "global_load_dwordx4 v[2:5], v[6:7], off",
               "; ssd lookahead wait 0",
               "s_waitcnt vmcnt(2) lgkmcnt(0)",
               "s_barrier")
    with pytest.raises(RuntimeError):
        _build.check_counted_barrier_waits(asm, "t")


def test_lookahead_wait_rejects_branch_in_window():
    asm = _asm("global_load_lds_dwordx4 v[0:1], off",
               "s_cbranch_scc1 .LBB0_4",
               "global_load_lds_dwordx4 v[8:9], off",
               "; ssd lookahead wait 2",
               "s_waitcnt vmcnt(2) lgkmcnt(0)",
               "s_barrier")
    with pytest.raises(RuntimeError):
        _build.check_counted_barrier_waits(asm, "t")


def test_marker_does_not_count_as_a_wait_state():
    asm = _asm("v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
               "s_nop 6",
               "; ssd lookahead wait 0",
               "v_mul_f32_e32 v20, v1, v21")
    with pytest.raises(RuntimeError):
        _build.check_mfma_result_reads(asm, "t")


def test_fp32_mfma_needs_eleven_wait_states():
    """The fp32 MFMA's result is read after 8 wait states: enough for the bf16
    op, not for this one."""
    asm = "\n".join([
        "k:",
        "v_mfma_f32_16x16x4_f32 v[0:3], v4, v5, v[0:3]",
        "s_nop 7",
        "v_add_f32_e32 v6, v0, v1",
        "s_endpgm",
    ])
    with pytest.raises(RuntimeError, match="after only 8"):
        _build.check_mfma_result_reads(asm, "t")
    ok = asm.replace("s_nop 7", "s_nop 7\ns_nop 2")
    assert _build.check_mfma_result_reads(ok, "t") == 1


def test_barrier_wait_at_vmcnt_max_waits_for_no_vector_memory():
    """s_waitcnt vmcnt(63) (the field's maximum) leaves every vector-memory
    operation in flight on purpose: it is not a counted wait."""
    asm = "\n".join([
        "k:",
        "global_load_lds_dwordx4 v1, s[0:1]",
        "s_waitcnt vmcnt(63) expcnt(7) lgkmcnt(0)",
        "s_barrier",
        "s_endpgm",
    ])
    _build.check_counted_barrier_waits(asm, "t")
