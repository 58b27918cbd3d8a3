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
