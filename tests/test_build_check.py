"""Host-side check of the build: a GEMM kernel that spills registers fails the build
(every GEMM kernel is sized to its register budget; scratch traffic in the MFMA loop or
the epilogue is a regression)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_spill_in_a_gemm_kernel_fails_the_build():
    from combine_top_router_amd import build as b
    bad = ("remark: Function Name: _ZN3moe12_GLOBAL__N_18k_bwd_daILb0EEEvNS_7BwdArgsENS_6MxArgsEi\n"
           "remark:     VGPRs: 256\nremark:     ScratchSize [bytes/lane]: 8\n")
    with pytest.raises(RuntimeError, match="spills 8 bytes"):
        b._check_no_spill("gemm_fw320.hip", bad)
    with pytest.raises(RuntimeError, match="spills 8 bytes"):
        b._check_no_spill("gemm_fw256.hip", bad.replace("k_bwd_daILb0E", "k_bwd_daILb1E"))
    # no spill: accepted
    b._check_no_spill("gemm_fw256.hip", bad.replace("ScratchSize [bytes/lane]: 8", "ScratchSize [bytes/lane]: 0"))


def test_every_gemm_source_is_checked():
    from combine_top_router_amd import build as b
    gemm = [s for s in b.SOURCES if s.startswith("gemm") and s != "gemm_f32.hip"]
    assert sorted(gemm) == sorted(b.GEMM_SOURCES)
