"""Host-side check of the build: a register-staged GEMM kernel that spills must fail the
build (its inline-asm loads' destinations must never be spilled or reused in flight)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_spill_in_a_register_staged_kernel_fails_the_build():
    from combine_top_router_amd import build as b
    bad = ("remark: Function Name: _ZN3moe12_GLOBAL__N_18k_bwd_daILb0EEEvNS_7BwdArgsENS_6MxArgsEi\n"
           "remark:     VGPRs: 128\nremark:     ScratchSize [bytes/lane]: 8\n")
    with pytest.raises(RuntimeError, match="spills 8 bytes"):
        b._check_no_spill("gemm.hip", bad)
    # no spill, or a spill in a kernel with direct-to-LDS loads only: accepted
    b._check_no_spill("gemm.hip", bad.replace("ScratchSize [bytes/lane]: 8", "ScratchSize [bytes/lane]: 0"))
    b._check_no_spill("gemm.hip", bad.replace("k_bwd_daILb0E", "k_bwd_daILb1E"))
