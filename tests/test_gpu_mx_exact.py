"""MXFP8 GEMMs on exactly representable operands, against the unquantised oracle.

The layer tests hold the MXFP8 paths to the oracle's MXFP8 forward and backward within
4e-2, the quantisation budget, which would hide a GEMM-level defect of a few percent.
Here every operand of the GEMM under test lies on the MX grid of every block that could
hold it: all its values are E4M3 values of one binade ([256, 416] * 2^X, 3 mantissa
bits), so each 32-element block, along either axis and at any alignment, has the scale
2^X and quantises without loss (the quantiser's own rule, pinned on the CPU).  The
MXFP8 GEMM must then give the unquantised product up to its fp32 sums and the bf16
rounding of its result: within 5e-3 of the fp64 oracle (one bf16 rounding is 2^-9 per
element at most).

The backward reads the saved G|U and A rows, which the test writes between moe_fwd and
moe_bwd (layout: G|U [R_cap, 2I] bf16 at offset 0 of `saved`, A [R_cap, I] after it at
the next multiple of 256 bytes), choosing them so that dG and dU are exact too:
* G = 0, U = 2: sigmoid(0) = 1/2, so dU = 0 and dG = dA' (top-1 routing: w = 1);
* G = 64, U = 0: sigmoid(64) = 1 in fp32 and fp64, so dG = 0 and dU = 64 dA'.
W_down is 2^j times a 0/1 matrix with one 1 per row, so dA' = Q(dY') Q(W_down)^T is a
power-of-two multiple of columns of dY', on the grid again.  Then B2 (dW_down), B3 (dX)
and B4 (dW_gate or dW_up) each contract exactly quantisable operands over a real K.

The mxfp8 forward: with on-grid X, W_gate and W_up, the gate/up GEMM is exact-operand
(G and U read back from `saved`); with W_gate = 64 times a 0/1 matrix (G = 64 x[pi(i)] >=
64, silu(G) = G in fp32 and fp64) and W_up picking a constant column of X (U = 1), A = G
is on the grid and the down GEMM is exact-operand (y of top-1 routing = Yp).
"""
import numpy as np
import pytest

import workloads as wl
from oracle import moe as om

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import BF16_TOL, rel, to_dev  # noqa: E402

EXACT_TOL = 5e-3
BINADE = np.array([256.0, 288.0, 320.0, 352.0, 384.0, 416.0])   # E4M3 0x78 .. 0x7D


def grid(rng, shape, X, signed=True):
    """Values of one E4M3 binade times 2^X: every MX block of them is exact."""
    v = rng.choice(BINADE, size=shape) * 2.0 ** X
    if signed:
        v = v * np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    return v


def perm01(rng, rows, cols, scale):
    """[rows, cols] with one entry `scale` per row, in distinct columns (rows <= cols)."""
    m = np.zeros((rows, cols))
    m[np.arange(rows), rng.permutation(cols)[:rows]] = scale
    return m


def _layer(cfg):
    from combine_top_router_amd.layer import MoeLayer
    import combine_top_router_amd.lib as L
    return MoeLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local, L.MOE_BF16,
                    L.MOE_BWD_MXFP8 if cfg.bwd == "mxfp8" else L.MOE_BWD_SAME, cfg.renorm,
                    fwd=L.MOE_FWD_MXFP8 if cfg.fwd == "mxfp8" else L.MOE_FWD_SAME)


def _saved_views(layer, cfg):
    R_cap, I = layer.R_cap, cfg.I
    gu_bytes = R_cap * 2 * I * 2
    off_a = (gu_bytes + 255) // 256 * 256
    gu = layer.saved[:gu_bytes].view(torch.bfloat16).view(R_cap, 2 * I)
    a = layer.saved[off_a:off_a + R_cap * I * 2].view(torch.bfloat16).view(R_cap, I)
    return gu, a


def _bwd_case(which):
    cfg = wl.MoeConfig(f"exact_bwd_{which}", 300, 256, 128, 4, 1, 0, 4, 41 if which == "gate" else 42,
                       bwd="mxfp8")
    inp = dict(wl.make_inputs(cfg))
    rng = np.random.default_rng(cfg.seed)
    inp["x"] = grid(rng, (cfg.T, cfg.H), -8)
    inp["dy"] = grid(rng, (cfg.T, cfg.H), -8)
    inp["w_gate"] = grid(rng, (cfg.e_local, cfg.H, cfg.I), -12)
    inp["w_up"] = grid(rng, (cfg.e_local, cfg.H, cfg.I), -12)
    inp["w_down"] = np.stack([perm01(rng, cfg.I, cfg.H, 0.5) for _ in range(cfg.e_local)])
    return cfg, inp, rng


@pytest.mark.parametrize("which", ["gate", "up"])
def test_mx_backward_gemms_on_exact_operands(which):
    cfg, inp, rng = _bwd_case(which)
    print(f"[mx-exact-bwd] {which}", flush=True)
    layer = _layer(cfg)
    dt = torch.bfloat16
    x, wg, wu, wd = (to_dev(inp[n], dt) for n in ("x", "w_gate", "w_up", "w_down"))
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"])).cuda()
    layer.forward(logits, x, wg, wu, wd)
    torch.cuda.synchronize()
    idx, w = om.route_topk(inp["logits"], 1)
    assert np.all(w == 1.0)
    ix = om.build_index(idx, 0, cfg.e_local)
    R = int(ix["offsets"][-1])
    assert np.array_equal(layer.row_src[:R].cpu().numpy(), ix["row_src"])
    G = np.full((R, cfg.I), 0.0 if which == "gate" else 64.0)
    U = np.full((R, cfg.I), 2.0 if which == "gate" else 0.0)
    A = grid(rng, (R, cfg.I), -6)
    gu, a = _saved_views(layer, cfg)
    gu[:R, :cfg.I] = to_dev(G, dt)
    gu[:R, cfg.I:] = to_dev(U, dt)
    a[:R] = to_dev(A, dt)
    g = layer.backward(to_dev(inp["dy"], dt))
    torch.cuda.synchronize()
    ref = om.layer_backward(inp, 1, 0, cfg.e_local, idx, w, {"G": G, "U": U, "A": A, "index": ix})
    live, dead = ("dw_gate", "dw_up") if which == "gate" else ("dw_up", "dw_gate")
    for key in ("dx", live, "dw_down", "d_topk_w"):
        err = rel(g[key].float().cpu().numpy(), ref[key])
        print(f"  {key}: {err:.3e}", flush=True)
        assert err < EXACT_TOL, (key, err)
    assert not g[dead].float().abs().sum().item()
    assert not np.abs(ref[dead]).sum()


def test_mx_b1_on_grid_d_topk_w_matches_unquantised():
    """fp8_bwd with top-2 routing (weights not powers of two): dY' and W_down on the grid
    of their row blocks along H make B1 exact-operand, so d_topk_w = <dA', a> must match
    the unquantised oracle (a is the forward's saved A: bf16 here, fp64 there)."""
    cfg = wl.MoeConfig("exact_b1", 400, 256, 192, 6, 2, 0, 6, 43, bwd="mxfp8")
    inp = dict(wl.make_inputs(cfg))
    rng = np.random.default_rng(43)
    inp["dy"] = grid(rng, (cfg.T, cfg.H), -8)
    inp["w_down"] = grid(rng, (cfg.e_local, cfg.I, cfg.H), -11)
    from gpu_util import run_layer, oracle_full
    out = run_layer(cfg, inp)
    ref = oracle_full(cfg, inp)
    err = rel(out["d_topk_w"], ref["d_topk_w"])
    print(f"  d_topk_w vs unquantised: {err:.3e}", flush=True)
    assert err < BF16_TOL, err


def _fwd_run(cfg, inp):
    layer = _layer(cfg)
    dt = torch.bfloat16
    x, wg, wu, wd = (to_dev(inp[n], dt) for n in ("x", "w_gate", "w_up", "w_down"))
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"])).cuda()
    y = layer.forward(logits, x, wg, wu, wd)
    torch.cuda.synchronize()
    return layer, y.float().cpu().numpy()


def test_mxfp8_gate_up_gemm_on_exact_operands():
    cfg = wl.MoeConfig("exact_k1", 300, 256, 256, 5, 2, 0, 5, 44, bwd="mxfp8", fwd="mxfp8")
    inp = dict(wl.make_inputs(cfg))
    rng = np.random.default_rng(44)
    inp["x"] = grid(rng, (cfg.T, cfg.H), -8)
    inp["w_gate"] = grid(rng, (cfg.e_local, cfg.H, cfg.I), -13)
    inp["w_up"] = grid(rng, (cfg.e_local, cfg.H, cfg.I), -13)
    layer, _ = _fwd_run(cfg, inp)
    idx, w = om.route_topk(inp["logits"], cfg.k)
    _, saved = om.layer_forward(inp, cfg.k, 0, cfg.e_local, idx, w)
    R = int(saved["index"]["offsets"][-1])
    gu, _ = _saved_views(layer, cfg)
    gu = gu[:R].float().cpu().numpy()
    for name, got, want in (("G", gu[:, :cfg.I], saved["G"]), ("U", gu[:, cfg.I:], saved["U"])):
        err = rel(got, want)
        print(f"  {name}: {err:.3e}", flush=True)
        assert err < EXACT_TOL, (name, err)


def test_mxfp8_down_gemm_on_exact_operands():
    cfg = wl.MoeConfig("exact_k2", 300, 256, 128, 5, 1, 0, 5, 45, bwd="mxfp8", fwd="mxfp8")
    inp = dict(wl.make_inputs(cfg))
    rng = np.random.default_rng(45)
    x = grid(rng, (cfg.T, cfg.H), -8, signed=False)          # in [1, 1.625]
    h0 = 7
    x[:, h0] = 1.0                                            # a constant column
    inp["x"] = x
    # G[:, i] = 64 x[:, pi(i)] (>= 64): one 64 per column of W_gate, in distinct rows != h0
    wg = np.zeros((cfg.e_local, cfg.H, cfg.I))
    for e in range(cfg.e_local):
        rows = rng.permutation(np.delete(np.arange(cfg.H), h0))[:cfg.I]
        wg[e, rows, np.arange(cfg.I)] = 64.0
    inp["w_gate"] = wg
    wu = np.zeros((cfg.e_local, cfg.H, cfg.I))
    wu[:, h0, :] = 1.0                                        # U = x[:, h0] = 1
    inp["w_up"] = wu
    inp["w_down"] = grid(rng, (cfg.e_local, cfg.I, cfg.H), -12)
    layer, y = _fwd_run(cfg, inp)
    idx, w = om.route_topk(inp["logits"], 1)
    Y, saved = om.layer_forward(inp, 1, 0, cfg.e_local, idx, w)
    assert np.all(saved["G"] >= 64.0) and np.array_equal(saved["A"], saved["G"])
    err = rel(y, Y)
    print(f"  y: {err:.3e}", flush=True)
    assert err < EXACT_TOL, err
