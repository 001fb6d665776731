"""The device-assembly scan that the library build runs: it must report a
select that takes its condition from a carry flag (the signature of a vector
compare whose copy into SCC was dropped) and stay quiet on compares, on the
carry-save idiom of wide integer arithmetic and across block boundaries."""

from scaled_fp8_casting_amd.build import scan_device_asm

# min(n - e0, 8192) with the v_cmp result never copied into SCC: the
# selects read the borrow of the 64-bit subtraction.
DROPPED_COPY = """
	s_sub_u32 s12, s12, s56
	s_subb_u32 s13, s13, s57
	v_cmp_lt_i64_e32 vcc, s[12:13], v[52:53]
	s_cselect_b32 s45, s13, 0
	s_cselect_b32 s44, s12, 0x2000
	s_cbranch_vccz .LBB2_87
"""

# the same with the copy in place: s_and_b64 sets SCC from vcc
WITH_COPY = """
	s_sub_u32 s38, s38, s28
	s_subb_u32 s39, s39, s29
	v_cmp_lt_i64_e32 vcc, s[38:39], v[6:7]
	s_and_b64 s[28:29], vcc, exec
	v_cmp_gt_i64_e32 vcc, s[38:39], v[8:9]
	s_cselect_b32 s29, s39, 0
	s_cselect_b32 s28, s38, 0x1000
"""

CARRY_SAVE = """
	s_add_u32 s30, s4, s5
	s_cselect_b64 s[4:5], -1, 0
	s_cmp_lg_u64 s[4:5], 0
	s_addc_u32 s7, s7, s23
"""

ACROSS_LABEL = """
	s_add_u32 s4, s4, 1
.LBB0_3:
	s_cselect_b32 s5, 1, 0
"""

BRANCH_ON_CARRY = """
	s_add_u32 s4, s4, s6
	; a comment line
	s_cbranch_scc1 .LBB0_9
"""


def test_reports_dropped_copy():
    found = scan_device_asm(DROPPED_COPY)
    assert [f[1].split()[0] for f in found] == ["s_cselect_b32", "s_cselect_b32"]
    assert all("s_subb_u32" in f[2] for f in found)


def test_reports_branch_on_carry():
    assert len(scan_device_asm(BRANCH_ON_CARRY)) == 1


def test_quiet_on_correct_code():
    assert scan_device_asm(WITH_COPY) == []
    assert scan_device_asm(CARRY_SAVE) == []
    assert scan_device_asm(ACROSS_LABEL) == []
