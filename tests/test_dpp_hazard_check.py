"""The build-time check for the VALU-write -> DPP-read hazard (CPU only).

The NSPLIT readout writes its DPP instructions in inline asm and places the
required wait states by hand; the build checks the generated assembly with
this checker.  Here it is pinned on small listings with a known answer, and
run over the listings of the current build when they exist."""
import glob
import os

import pytest

from mamba_selective_scan_06_amd import build as hipbuild
from mamba_selective_scan_06_amd.dpp_hazard_check import check_lines

DPP = [";;#ASMSTART", "\tv_fmac_f32_dpp v7, v5, v8 row_newbcast:3 row_mask:0xf bank_mask:0xf", ";;#ASMEND"]


@pytest.mark.parametrize("before,n_bad", [
    (["\tv_lshlrev_b32_e32 v5, 16, v3", "\ts_nop 1"], 0),               # two wait states from s_nop 1
    (["\tv_lshlrev_b32_e32 v5, 16, v3", "\ts_nop 0"], 1),               # one is not enough
    (["\tv_lshlrev_b32_e32 v5, 16, v3"], 1),                           # back to back
    (["\tv_lshlrev_b32_e32 v5, 16, v3", "\tv_mul_f32_e32 v9, v1, v2"], 1),
    (["\tv_lshlrev_b32_e32 v5, 16, v3", "\tv_mul_f32_e32 v9, v1, v2", "\tv_add_f32_e32 v9, v1, v2"], 0),
    (["\tv_lshlrev_b64 v[4:5], 16, v[2:3]"], 1),                       # register ranges
    (["\tv_lshlrev_b32_e32 v6, 16, v3"], 0),                           # another register
    (["\tv_mul_f32_e32 v9, v1, v2", "\tv_mul_f32_e32 v9, v1, v2", ".LBB0_3:"], 1),  # a path may enter
    ([".LBB0_3:", "\ts_nop 1"], 0),
    (["\tds_read_b32 v5, v2", "\ts_waitcnt lgkmcnt(0)"], 0),           # not a VALU write
    (["\tv_lshlrev_b32_e32 v5, 16, v3", ";;#ASMEND", ";;#ASMSTART"], 1),  # across asm blocks
])
def test_checker_on_listings(before, n_bad):
    assert len(check_lines(before + DPP)) == n_bad


def test_compiler_generated_dpp_is_left_to_the_compiler():
    listing = ["\tv_lshlrev_b32_e32 v5, 16, v3", "\tv_mul_f32_dpp v7, v5, v8 row_newbcast:3 bound_ctrl:1"]
    assert check_lines(listing) == []


def test_built_listings_are_clean():
    listings = glob.glob(os.path.join(hipbuild.OBJ, "nsplit_*.s"))
    if not listings:
        pytest.skip("no build listings here (run the build first)")
    for path in listings:
        with open(path) as f:
            assert check_lines(f.read().split("\n"), path) == []
