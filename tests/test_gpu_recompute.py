"""Activation checkpointing (recompute = 1): the forward keeps nothing for the backward
(no saved buffer is allocated or passed) and the backward recomputes G|U and A with the
forward's own gate/up GEMM.  The kernels are deterministic, so every output must equal
the outputs of the saved-activation path bit for bit; that path's parity with the
oracle is tested elsewhere, so this also holds the recompute path to the oracle.  Each
precision mode (bf16, fp8_bwd, mxfp8, MXFP8 forward with a bf16 backward), both weight
modes, a local share, a skewed layer, forced 320-row tiles, and the full Qwen3-30B-A3B layer
and 235B-A22B share (bf16 and fp8_bwd)."""
import numpy as np
import pytest

import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import inputs, run_layer  # noqa: E402

CASES = {
    "tiny_bf16": wl.CONFIGS["tiny_bf16"],
    "ragged_bf16_share": wl.MoeConfig("ragged_bf16_share", 700, 192, 320, 10, 3, 4, 5, 6),
    "skew_bf16": wl.MoeConfig("skew_bf16", 1024, 256, 192, 64, 4, 0, 64, 16, routing="zipf"),
    # every bf16 row-tiled GEMM, the recomputed gate/up one included, on 320-row tiles
    "tall_bf16_share": wl.MoeConfig("tall_bf16_share", 1280, 320, 192, 8, 2, 2, 5, 12, row_tile=320),
    "ragged_fp8bwd": wl.MoeConfig("ragged_fp8bwd", 700, 256, 192, 6, 2, 0, 6, 8, bwd="mxfp8"),
    # fp8_bwd with about 1000 rows per expert (four or more row tiles): the saved path takes
    # the weights' codes from the forward GEMMs' B stages, the recompute path from the row
    # quantiser, so equality pins those codes byte for byte; H = 384 leaves the down GEMM a
    # half-empty last column tile, and 320-row tiles run the gate/up GEMM's 320-row build
    "ragged_fp8bwd_h384": wl.MoeConfig("ragged_fp8bwd_h384", 2400, 384, 192, 7, 3, 1, 5, 9, bwd="mxfp8"),
    "tall_fp8bwd_share": wl.MoeConfig("tall_fp8bwd_share", 4800, 256, 320, 8, 2, 2, 5, 10, bwd="mxfp8",
                                      row_tile=320),
    "ragged_mxfp8_share": wl.MoeConfig("ragged_mxfp8_share", 500, 256, 256, 10, 3, 4, 5, 13, bwd="mxfp8",
                                       fwd="mxfp8"),
    # MXFP8 forward with the bf16 backward: the recompute runs the fp8 gate/up chain
    "ragged_mxfp8_fwd_only": wl.MoeConfig("ragged_mxfp8_fwd_only", 300, 256, 128, 5, 2, 0, 5, 15, fwd="mxfp8"),
}
KEYS = ("y", "dx", "dw_gate", "dw_up", "dw_down", "d_topk_w", "d_logits", "topk_idx", "row_src")


def _check_equal(cfg, fuse):
    inp = inputs(cfg)
    ref = run_layer(cfg, inp, fuse_gather=fuse, recompute=0)
    got = run_layer(cfg, inp, fuse_gather=fuse, recompute=1)
    for key in KEYS:
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("fuse", [True, False], ids=["fused_gather", "xp"])
def test_recompute_equals_saved_path(name, fuse):
    print(f"[recompute] {name} fuse={fuse}", flush=True)
    _check_equal(CASES[name], fuse)


@pytest.mark.parametrize("name", ["qwen3_30b", "qwen3_235b_ep8", "qwen3_235b_ep8_fp8bwd"])
def test_recompute_full_size(name):
    # 30B: every bf16 row-tiled GEMM on 320-row tiles; the 235B share: the (recomputed)
    # gate/up GEMM on 320-row tiles, dA' and dX' on 256-row ones (both tables, one launch);
    # in fp8_bwd the forward GEMMs' weight codes against the row quantiser's
    cfg = wl.CONFIGS[name]
    print(f"[recompute-full] {cfg.name}", flush=True)
    _check_equal(cfg, True)
