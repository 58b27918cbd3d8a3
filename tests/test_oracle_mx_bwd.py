"""Pins of the oracle's MXFP8 backward: where each of its eight quantisation points sits.

The reading (oracle/mx.py docstring): blocks of 32 lie along each backward GEMM's
contraction axis, row-wise for B1 (dY' and W_down along H) and B3 (dG, dU, W_gate, W_up
along I), column-wise in group-aware 32-row blocks for B2 (A and w*dY') and B4 (Xp, dG,
dU); B1 quantises the unweighted dY' (NVIDIA article, "which optimisations does dropless
MoE need": group-aware MXFP8 quantisation for the MXFP8 grouped GEMMs).

Every property below follows from that reading and from the quantiser's own facts (pinned
in test_oracle_mx.py): values on the grid of their block survive quantisation exactly,
and quantisation commutes with scaling a whole block by a power of two.  Each test also
moves single quantisation points of the oracle (its BWD_POINTS table) to another axis,
another block alignment or another operand, and checks that the property then fails, so
a moved point cannot go unnoticed.
"""
import numpy as np
import pytest

from oracle import moe as om
from oracle import mx
import workloads as wl


# ---- mutants: one quantisation point moved ----
def _cols_whole(dye, we):                      # B1's dY' in column blocks over the expert's rows
    return mx.qdq_cols_grouped(dye, np.array([0, dye.shape[0]]))


def _b1_weighted(dye, we):                     # B1 quantising w * dY' instead of dY'
    return mx.qdq_rows(we[:, None] * dye) / we[:, None]


def _w_other_axis(w):                          # a weight quantised along its other axis
    return mx.qdq_rows(w.T).T


def _act_rows(m, seg):                         # a column-wise operand quantised row-wise
    return mx.qdq_rows(m)


def _act_cols(m, seg):                         # a row-wise operand quantised column-wise
    return mx.qdq_cols_grouped(m, seg)


def _act_end_aligned(m, seg):                  # column blocks aligned at the group's last row
    return mx.qdq_cols_grouped(m[::-1], seg)[::-1]


def _b2_rows(dye, we, seg):
    return mx.qdq_rows(we[:, None] * dye)


def _b2_unweighted(dye, we, seg):              # B2 quantising dY' and weighting after
    return we[:, None] * mx.qdq_cols_grouped(dye, seg)


def _b2_end_aligned(dye, we, seg):
    return mx.qdq_cols_grouped((we[:, None] * dye)[::-1], seg)[::-1]


def _grid_blocks(rng, shape, xlo, xhi):
    """Values on the MX grid of 32-element blocks along the last axis: E4M3 values times
    2^X per block, with one element of each block at 256 * 2^X and none above 416 * 2^X,
    so the block's scale is 2^X (the smallest with amax <= 448 * 2^X) and stays so when
    the values move by an fp64 rounding.  Returns an array of `shape`."""
    *lead, K = shape
    codes = rng.integers(0, 0x7E, size=shape)
    sgn = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    X = rng.integers(xlo, xhi, size=(*lead, K // 32))
    m = sgn * mx.e4m3_decode(codes) * np.repeat(np.exp2(X), 32, axis=-1)
    m[..., ::32] = 256.0 * np.exp2(X)
    return m


def _layer(seed, T=96, H=64, I=64, E=3, k=2):
    cfg = wl.MoeConfig("mxb", T, H, I, E, k, 0, E, seed, bwd="mxfp8")
    inp = dict(wl.make_inputs(cfg))
    idx, w = om.route_topk(inp["logits"], k)
    _, saved = om.layer_forward(inp, k, 0, E, idx, w)
    return cfg, inp, idx, w, saved


def _bwd(cfg, inp, idx, w, saved, points=None):
    return mx.layer_backward_mx(inp, cfg.k, 0, cfg.e_local, idx, w, saved, points)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _rowrel(a, b):
    """Largest relative error of one row (token rows here span 2^16 in size)."""
    a = a.reshape(a.shape[0], -1); b = b.reshape(b.shape[0], -1)
    nb = np.linalg.norm(b, axis=1)
    keep = nb > 0
    return float(np.max(np.linalg.norm(a - b, axis=1)[keep] / nb[keep]))


def test_layer_has_ragged_groups():
    # the cases below rely on expert groups that are not multiples of 32 rows
    cfg, _, _, _, saved = _layer(5)
    counts = saved["index"]["counts"]
    assert np.all(counts % 32 != 0) and np.all(counts > 32)


# ---- B1: dY' and W_down row-wise along H, dY' unweighted ----
def test_b1_on_grid_operands_are_exact():
    cfg, inp, idx, w, saved = _layer(5)
    rng = np.random.default_rng(50)
    # dY rows on their own 32-column grid, token rows 2^-8 / 1 / 2^8 apart so that
    # column blocks (which mix tokens) cannot hold them
    inp["dy"] = _grid_blocks(rng, (cfg.T, cfg.H), -9, -5) * np.exp2(8.0 * rng.integers(-1, 2, size=(cfg.T, 1)))
    # W_down [I, H] rows on their grid along H, rows 2^-8 / 1 / 2^8 apart: its column
    # blocks (along I) span more than E4M3's 2^15 of relative range and cannot hold them
    s_i = rng.integers(-1, 2, size=cfg.I)
    inp["w_down"] = np.stack([_grid_blocks(rng, (cfg.I, cfg.H), -12, -4) * np.exp2(8.0 * s_i)[:, None]
                              for _ in range(cfg.e_local)])
    assert not np.allclose(_w_other_axis(inp["w_down"][0]), inp["w_down"][0])
    # saved A columns scaled the other way, so every i weighs alike in d_w = <dA', a>
    saved = dict(saved, A=saved["A"] * np.exp2(-8.0 * s_i))
    ref = om.layer_backward(inp, cfg.k, 0, cfg.e_local, idx, w, saved)
    got = _bwd(cfg, inp, idx, w, saved)
    # B1 is then exact: d_w = <dA', a> equals the unquantised one
    assert np.allclose(got["d_topk_w"], ref["d_topk_w"], rtol=1e-12, atol=1e-12 * np.abs(ref["d_topk_w"]).max())
    for pts in ({"b1_dy": _cols_whole}, {"b1_dy": _b1_weighted}, {"b1_wd": _w_other_axis}):
        bad = _bwd(cfg, inp, idx, w, saved, pts)
        assert _rowrel(bad["d_topk_w"], ref["d_topk_w"]) > 1e-3, pts


# ---- B2: A and w dY' column-wise, group-aware ----
def test_b2_on_grid_operands_are_exact():
    # top-1 routing: every token has one row, so dY can be chosen row by row
    cfg = wl.MoeConfig("mxb2", 150, 64, 64, 3, 1, 0, 3, 7, bwd="mxfp8")
    inp = dict(wl.make_inputs(cfg))
    idx, _ = om.route_topk(inp["logits"], 1)
    rng = np.random.default_rng(70)
    w = rng.uniform(0.25, 1.0, size=(cfg.T, 1))          # any weights, not powers of two
    ix = om.build_index(idx, 0, cfg.e_local)
    off, rs = ix["offsets"], ix["row_src"]
    assert np.all(np.diff(off) % 32 != 0)
    R = int(off[-1])
    A = np.zeros((R, cfg.I))
    M = np.zeros((R, cfg.H))                             # the intended w * dY'
    for e in range(cfg.e_local):
        lo, hi = int(off[e]), int(off[e + 1])
        for r0 in range(lo, hi, 32):                     # group-aware blocks from the first row
            n = min(32, hi - r0)
            # element 0 of each column block (the one at 256 * 2^X) is the block's first
            # row, which a short last block keeps too
            # neighbouring blocks 2^16 apart (a block of other rows would mix them), A's and
            # M's the opposite way so that every block adds alike to A^T M
            sb = np.exp2(8.0 * (1 - 2 * (((r0 - lo) // 32) % 2)))
            A[r0:r0 + n] = _grid_blocks(rng, (cfg.I, 32), -10, -2).T[:n] * sb
            M[r0:r0 + n] = _grid_blocks(rng, (cfg.H, 32), -10, -2).T[:n] / sb
    # columns 2^-8 / 1 / 2^8 apart: row blocks (which mix columns) span more than E4M3's
    # 2^15 of relative range and cannot hold them; column blocks scale as a whole
    A *= np.exp2(8.0 * rng.integers(-1, 2, size=cfg.I))
    M *= np.exp2(8.0 * rng.integers(-1, 2, size=cfg.H))
    dy = np.zeros((cfg.T, cfg.H))
    dy[rs // cfg.k] = M / w[rs // cfg.k]
    inp["dy"] = dy
    saved = {"G": rng.standard_normal((R, cfg.I)), "U": rng.standard_normal((R, cfg.I)), "A": A, "index": ix}
    ref = om.layer_backward(inp, 1, 0, cfg.e_local, idx, w, saved)
    got = mx.layer_backward_mx(inp, 1, 0, cfg.e_local, idx, w, saved)
    assert np.allclose(got["dw_down"], ref["dw_down"], rtol=1e-12, atol=0)

    def worst(bad):   # largest relative error of one row (i) or one column (h) of some dW_down[e]
        return max(max(_rowrel(bad[e], ref["dw_down"][e]), _rowrel(bad[e].T, ref["dw_down"][e].T))
                   for e in range(cfg.e_local))

    for pts in ({"b2_a": _act_rows}, {"b2_a": _act_end_aligned}, {"b2_dy": _b2_rows},
                {"b2_dy": _b2_unweighted}, {"b2_dy": _b2_end_aligned}):
        bad = mx.layer_backward_mx(inp, 1, 0, cfg.e_local, idx, w, saved, pts)
        assert worst(bad["dw_down"]) > 1e-3, pts


# ---- row-wise points: scaling one token's dY row touches that token only ----
def _token_row_local(cfg, inp, idx, w, saved, t, points=None):
    base = _bwd(cfg, inp, idx, w, saved, points)
    inp2 = dict(inp)
    inp2["dy"] = inp["dy"].copy()
    inp2["dy"][t] *= 256.0
    new = _bwd(cfg, inp2, idx, w, saved, points)
    others = np.arange(cfg.T) != t
    return (np.array_equal(new["dx"][others], base["dx"][others])
            and np.array_equal(new["d_topk_w"][others], base["d_topk_w"][others])
            and np.array_equal(new["dx"][t], 256.0 * base["dx"][t])
            and np.array_equal(new["d_topk_w"][t], 256.0 * base["d_topk_w"][t]))


def test_token_row_scaling_stays_in_its_row():
    cfg, inp, idx, w, saved = _layer(5)
    for t in (3, 50):
        assert _token_row_local(cfg, inp, idx, w, saved, t)
        for pts in ({"b1_dy": _cols_whole}, {"b3_dgu": _act_cols}):
            assert not _token_row_local(cfg, inp, idx, w, saved, t, pts), pts


# ---- weight rows: W_gate / W_up rows (along I) and W_down rows (along H) ----
def test_weight_row_scaling_stays_in_its_row():
    cfg, inp, idx, w, saved = _layer(5)
    e, h, i = 1, 37, 21

    def gate_local(points=None):
        base = _bwd(cfg, inp, idx, w, saved, points)
        inp2 = dict(inp, w_gate=inp["w_gate"].copy())
        inp2["w_gate"][e, h] *= 256.0
        new = _bwd(cfg, inp2, idx, w, saved, points)
        cols = np.arange(cfg.H) != h
        # only dX column h moves (saved G, U are fixed, so W_gate enters through B3 alone)
        return np.array_equal(new["dx"][:, cols], base["dx"][:, cols]) and not np.array_equal(new["dx"], base["dx"])

    def down_local(points=None):
        base = _bwd(cfg, inp, idx, w, saved, points)
        inp2 = dict(inp, w_down=inp["w_down"].copy())
        inp2["w_down"][e, i] *= 256.0
        new = _bwd(cfg, inp2, idx, w, saved, points)
        cols = np.arange(cfg.I) != i
        # dA' column i moves; B4's column blocks keep every other column of dG, dU as it was
        return (np.array_equal(new["dw_gate"][e][:, cols], base["dw_gate"][e][:, cols])
                and np.array_equal(new["dw_up"][e][:, cols], base["dw_up"][e][:, cols])
                and not np.array_equal(new["dw_gate"][e], base["dw_gate"][e]))

    assert gate_local()
    assert not gate_local({"b3_w": _w_other_axis})
    assert down_local()
    assert not down_local({"b1_wd": _w_other_axis})
    assert not down_local({"b4_dgu": _act_rows})


# ---- column-wise points: separate group-aware blocks add up, one block does not ----
def _rows_of_expert(saved, cfg, e):
    ix = saved["index"]
    lo, hi = int(ix["offsets"][e]), int(ix["offsets"][e + 1])
    return lo, hi, ix["row_src"][lo:hi] // cfg.k


def _pairs(lo, hi, tok):
    """Two row pairs inside expert rows [lo, hi): `apart` lies in two different blocks
    counted from the first row but one block counted from the last; `same` lies in one
    block counted from the first row but two counted from the last."""
    n = hi - lo
    tail = n % 32
    assert 1 <= tail and n > 32
    apart = (31, 32)                      # blocks 0 and 1 from the first row
    # from the last row, blocks start at lo + tail + 32 j: rows tail - 1 and tail differ
    same = (tail - 1, tail)
    assert (apart[0] - tail) // 32 == (apart[1] - tail) // 32   # one block from the last row
    return [tok[r] for r in apart], [tok[r] for r in same]


def _additive(f, inp, key, toks, e, scale=256.0):
    """f(inp) -> output; is f's expert-e output additive over scaling the two rows?"""
    def mod(ts):
        d = dict(inp)
        d[key] = inp[key].copy()
        for t in ts:
            d[key][t] *= scale
        return f(d)[e]
    b, one, two, both = mod([]), mod(toks[:1]), mod(toks[1:]), mod(toks)
    return np.allclose(both - b, (one - b) + (two - b), rtol=0, atol=1e-12 * np.abs(both).max())


def test_column_blocks_are_group_aware():
    cfg, inp, idx, w, saved = _layer(5)
    e = 1
    lo, hi, tok = _rows_of_expert(saved, cfg, e)
    # each chosen token has exactly one row in expert e (k distinct experts per token)
    apart, same = _pairs(lo, hi, tok)

    def check(key, out, points=None):
        f = lambda d: _bwd(cfg, d, idx, w, saved, points)[out]
        return _additive(f, inp, key, apart, e) and not _additive(f, inp, key, same, e)

    # B4: x enters the backward only through B4's Xp (saved G, U, A fixed)
    assert check("x", "dw_gate") and check("x", "dw_up")
    for pts in ({"b4_x": _act_rows}, {"b4_x": _act_end_aligned}):
        assert not check("x", "dw_gate", pts), pts
    # B4: dG, dU rows scale with the token's dY row (B1 is row-wise), quantised column-wise
    assert check("dy", "dw_gate") and check("dy", "dw_up")
    for pts in ({"b4_dgu": _act_rows}, {"b4_dgu": _act_end_aligned}):
        assert not check("dy", "dw_gate", pts), pts
    # B2: w dY' column-wise
    assert check("dy", "dw_down")
    for pts in ({"b2_dy": _b2_rows}, {"b2_dy": _b2_end_aligned}):
        assert not check("dy", "dw_down", pts), pts


def test_column_blocks_of_a_are_group_aware():
    cfg, inp, idx, w, saved = _layer(5)
    e = 2
    ix = saved["index"]
    lo, hi = int(ix["offsets"][e]), int(ix["offsets"][e + 1])
    tail = (hi - lo) % 32
    apart, same = (lo + 31, lo + 32), (lo + tail - 1, lo + tail)

    def check(rows, points=None):
        def f(A):
            s = dict(saved, A=A)
            return _bwd(cfg, inp, idx, w, s, points)["dw_down"][e]
        def mod(rs):
            A = saved["A"].copy()
            A[list(rs)] *= 256.0
            return f(A)
        b, one, two, both = mod([]), mod(rows[:1]), mod(rows[1:]), mod(rows)
        return np.allclose(both - b, (one - b) + (two - b), rtol=0, atol=1e-12 * np.abs(both).max())

    assert check(apart) and not check(same)
    for pts in ({"b2_a": _act_rows}, {"b2_a": _act_end_aligned}):
        assert not (check(apart, pts) and not check(same, pts)), pts
