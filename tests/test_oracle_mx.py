"""Pins of the oracle's MXFP8 quantizer (E4M3 elements, e8m0 scale per 32) against the
OCP 8-bit floating point / Microscaling definitions: code table facts, exhaustive
round trips, ties-to-even, the half-ulp bound, the scale rule and group boundaries."""
import numpy as np
import pytest

from oracle import mx
from oracle import moe as om
import workloads as wl


def test_e4m3_code_facts():
    # OCP E4M3 (FN): bias 7, 3 mantissa bits, max normal 1.75*2^8, min normal 2^-6,
    # min subnormal 2^-9, 0x7F/0xFF are NaN.
    d = mx.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x3C) == 1.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))


def test_exhaustive_round_trip_of_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = mx.e4m3_decode(codes)
    assert np.array_equal(mx.e4m3_round(vals), vals)
    enc = mx.e4m3_encode(np.where(codes & 0x80, -1.0, 1.0) * np.abs(vals))
    assert np.array_equal(enc, codes.astype(np.uint8))
    # 253 distinct non-negative... values are strictly monotone in the code
    pos = mx.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(pos) > 0)


def test_ties_go_to_even_mantissa():
    pos = mx.e4m3_decode(np.arange(0, 0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    r = mx.e4m3_round(mids)
    codes = mx.e4m3_encode(r)
    assert np.all((codes & 1) == 0)
    assert np.all((r == pos[:-1]) | (r == pos[1:]))


def test_half_ulp_bound_on_random_values():
    rng = np.random.default_rng(0)
    v = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-6, 0, 20000))
    v = v[np.abs(v) >= 2.0 ** -6]
    r = mx.e4m3_round(v)
    _, ex = np.frexp(np.abs(v))
    ulp = np.exp2(ex - 1 - 3.0)
    assert np.all(np.abs(r - v) <= ulp / 2)


def test_scale_rule():
    X = mx.e8m0_exponent(np.array([448.0, 448.0 * 2 ** 5, 448.0 * 2 ** 5 * (1 + 2 ** -20), 1.0, 0.0, 1.75]))
    assert list(X) == [0, 5, 6, -8, 0, -8]
    blk = np.zeros((1, 32)); blk[0, 3] = 448.0 * 4; blk[0, 7] = -1.0
    codes, scale, deq = mx.quantize_blocks(blk)
    assert scale[0] == 127 + 2 and codes[0, 3] == 0x7E and deq[0, 3] == 448.0 * 4
    assert deq[0, 7] == -1.0
    z = mx.quantize_blocks(np.zeros((2, 32)))
    assert np.all(z[1] == 127) and not z[2].any()


def test_values_on_the_block_grid_survive_exactly():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7E, size=(8, 32))
    sgn = np.where(rng.integers(0, 2, size=(8, 32)) == 1, -1.0, 1.0)
    X = rng.integers(-20, 20, size=(8, 1))
    m = sgn * mx.e4m3_decode(codes) * np.exp2(X)
    m[:, 0] = 448.0 * np.exp2(X[:, 0])      # pin the block amax to the top of the range
    assert np.array_equal(mx.qdq_rows(m), m)


def test_column_blocks_do_not_cross_groups():
    rng = np.random.default_rng(2)
    m = np.concatenate([rng.standard_normal((40, 64)) * 1e-3, rng.standard_normal((30, 64)) * 1e3])
    off = np.array([0, 40, 70])
    q = mx.qdq_cols_grouped(m, off)
    rel = np.abs(q - m) / np.abs(m)
    assert rel.max() < 2 ** -3          # no small value of group 0 is flushed by group 1
    # the short last block of group 0 (rows 32..39) is quantised on its own
    q2 = mx.qdq_cols_grouped(m[32:40], np.array([0, 8]))
    assert np.array_equal(q[32:40], q2)


def test_mx_backward_is_close_to_exact_backward():
    cfg = wl.CONFIGS["tiny_bf16"].replace(bwd="mxfp8")
    inp = wl.make_inputs(cfg)
    idx, w = om.route_topk(inp["logits"], cfg.k)
    Y, saved = om.layer_forward(inp, cfg.k, 0, cfg.e_local, idx, w)
    g = om.layer_backward(inp, cfg.k, 0, cfg.e_local, idx, w, saved)
    gq = mx.layer_backward_mx(inp, cfg.k, 0, cfg.e_local, idx, w, saved)
    for key in ("dx", "dw_gate", "dw_up", "dw_down", "d_topk_w"):
        rel = np.linalg.norm(gq[key] - g[key]) / np.linalg.norm(g[key])
        assert 1e-3 < rel < 8e-2, (key, rel)


def _on_grid_rows(rng, n, K, xlo=-9, xhi=-5):
    """[n, K] values on the MX grid of their own 32-element row blocks: each block has
    a random exponent X, E4M3 grid values times 2^X, and its amax pinned to 448 * 2^X,
    so row-wise quantisation returns them unchanged.  Neighbouring rows get unrelated
    exponents, so the same values are off the grid of column blocks."""
    codes = rng.integers(0, 0x7E, size=(n, K))
    sgn = np.where(rng.integers(0, 2, size=(n, K)) == 1, -1.0, 1.0)
    X = rng.integers(xlo, xhi, size=(n, K // 32))
    m = sgn * mx.e4m3_decode(codes) * np.repeat(np.exp2(X), 32, axis=1)
    m[:, ::32] = 448.0 * np.exp2(X)
    return m


def _mx_fwd_case(seed, grid):
    """Tiny layer (E = 4, k = 2) whose X rows are on their row-block grid and whose
    W_gate, W_up, W_down columns are on their column-block grid (grid=True).

    E4M3 keeps 3 mantissa bits at every scale down to 2^-15 below a block's maximum,
    so the block axis only shows on values that far below their block's largest:
    token rows are scaled by 2^-8, 1 or 2^8 (A's rows then span 2^32), which a
    column block of A cannot hold but a row block can."""
    cfg = wl.MoeConfig("mxf", 48, 64, 64, 4, 2, 0, 4, seed, bwd="mxfp8")
    inp = wl.make_inputs(cfg)
    if grid:
        rng = np.random.default_rng(seed)
        inp["x"] = _on_grid_rows(rng, 48, 64) * np.exp2(8.0 * rng.integers(-1, 2, size=(48, 1)))
        for w in ("w_gate", "w_up", "w_down"):
            inp[w] = np.stack([_on_grid_rows(rng, 64, 64, -12, -8).T for _ in range(4)])
    idx, w = om.route_topk(inp["logits"], cfg.k)
    return cfg, inp, idx, w


def test_mx_forward_quantises_along_the_contraction_axes():
    # X and the weights lie on the grid of the blocks the mxfp8 forward uses (X rows
    # along H, weight columns along H or I), so the gate/up GEMM is exact: G and U
    # equal the exact oracle's.  Quantising along the other axis would change them.
    cfg, inp, idx, w = _mx_fwd_case(31, grid=True)
    _, sx = om.layer_forward(inp, cfg.k, 0, cfg.e_local, idx, w)
    _, sq = mx.layer_forward_mx(inp, cfg.k, 0, cfg.e_local, idx, w)
    assert np.array_equal(sx["index"]["row_src"], sq["index"]["row_src"])
    assert np.allclose(sq["G"], sx["G"], rtol=1e-12, atol=1e-12)
    assert np.allclose(sq["U"], sx["U"], rtol=1e-12, atol=1e-12)
    assert not np.allclose(mx.qdq_rows(inp["w_gate"][0]), inp["w_gate"][0])   # the wrong axis is lossy
    assert not np.allclose(mx.qdq_cols_grouped(inp["x"], np.array([0, 48])), inp["x"])
    # W_down is exact too, so only A's row-wise quantisation (along I) remains in Yp
    wf = w.reshape(-1)
    ri = sx["index"]["row_src"]
    off = sx["index"]["offsets"]
    for e in range(cfg.e_local):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        ref = wf[ri[lo:hi]][:, None] * (mx.qdq_rows(sx["A"][lo:hi]) @ inp["w_down"][e])
        assert np.allclose(sq["Yp"][lo:hi], ref, rtol=1e-12, atol=1e-12)
        exact = sx["Yp"][lo:hi]
        rowrel = lambda a: np.max(np.linalg.norm(a - ref, axis=1) / np.linalg.norm(ref, axis=1))
        assert rowrel(exact) > 1e-3                                                    # A's quantisation is seen
        wrong = wf[ri[lo:hi]][:, None] * (mx.qdq_cols_grouped(sx["A"][lo:hi], np.array([0, hi - lo]))
                                          @ inp["w_down"][e])
        assert rowrel(wrong) > 1e-1                                                    # and its axis matters


def test_mx_forward_is_close_to_exact_forward():
    # Gaussian data: each E4M3 quantisation adds a relative error of a few percent at
    # most (3 mantissa bits), and the results stay within that of the exact forward.
    cfg, inp, idx, w = _mx_fwd_case(32, grid=False)
    Y, sx = om.layer_forward(inp, cfg.k, 0, cfg.e_local, idx, w)
    Yq, sq = mx.layer_forward_mx(inp, cfg.k, 0, cfg.e_local, idx, w)
    for a, b in ((Yq, Y), (sq["G"], sx["G"]), (sq["U"], sx["U"]), (sq["A"], sx["A"])):
        rel = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert 1e-3 < rel < 8e-2, rel
    # combine: Y is the sum of each token's weighted rows
    Ysum = np.zeros_like(Yq)
    np.add.at(Ysum, sq["index"]["row_src"] // cfg.k, sq["Yp"])
    assert np.allclose(Ysum, Yq)


def test_mx_forward_power_of_two_equivariance():
    # MX quantisation commutes with scaling by a power of two (the block exponent moves,
    # the codes stay): 4 W_up and W_down / 2 give exactly 2 Y.
    cfg, inp, idx, w = _mx_fwd_case(33, grid=False)
    Y, _ = mx.layer_forward_mx(inp, cfg.k, 0, cfg.e_local, idx, w)
    inp2 = dict(inp, w_up=inp["w_up"] * 4.0, w_down=inp["w_down"] * 0.5)
    Y2, _ = mx.layer_forward_mx(inp2, cfg.k, 0, cfg.e_local, idx, w)
    assert np.array_equal(Y2, 2.0 * Y)
