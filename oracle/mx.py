"""fp64 oracle of the MXFP8 GEMMs: E4M3 elements with one e8m0 scale per 32.

The pages name the formats only: MXFP8 block scaling for the expert GEMMs and a
group-aware MXFP8 quantisation (NVIDIA article, "Optimization 1" and its list of
Transformer Engine building blocks), and an fp8_bwd mode with a bf16 forward and an
fp8 backward, and an mxfp8 mode that runs the expert GEMMs in MXFP8 (Prime Mega
MoE pages: precision bf16, mxfp8, fp8 or fp8_bwd).  The element and scale encodings are the OCP
Microscaling (MX) v1.0 ones: E4M3 "FN" (bias 7, max 448, no infinities, 0x7F/0xFF
NaN) and E8M0 (2^(code-127)).

Readings:
* Scale rule: X = the smallest integer with amax <= 448 * 2^X (so x / 2^X never
  saturates), clamped to [-127, 127]; an all-zero block takes X = 0 (code 127).
* Element rounding: x / 2^X rounded to the nearest E4M3 value, ties to even; the
  code's sign bit is the sign bit of x.
* Blocks lie along each backward GEMM's contraction axis.  Row-wise: 32 consecutive
  columns of a row (dY' and W_down along H; dG, dU, W_gate and W_up along I).
  Column-wise and group-aware: 32 consecutive rows of one expert's group, the first
  block starting at the expert's first row, a short last block padded with zeros
  (A and w*dY' for dW_down; X and dG, dU for dW_gate, dW_up).
* B1 quantises the unweighted dY' and applies w after the GEMM; B2 quantises w*dY'.
  dG and dU are quantised from their unrounded values.  Outputs stay unquantised.
* mxfp8 forward: the two forward GEMMs take MXFP8 operands along their contraction
  axes: the gate/up GEMM quantises the rows of X along H and W_gate, W_up in blocks
  of 32 consecutive rows (h) of each column; the down GEMM quantises the rows of A
  along I and W_down in blocks of 32 consecutive rows (i) of each column.  A is
  quantised from its unrounded value and the routing weight applies after the GEMM.
  G, U and A (what the backward reads) are the unquantised results of these GEMMs.
"""
from __future__ import annotations

import numpy as np

from .moe import build_index, sigmoid, silu, _f64

E4M3_MAX = 448.0
BLOCK = 32

__all__ = ["e4m3_decode", "e4m3_round", "e4m3_encode", "e8m0_exponent", "quantize_blocks",
           "qdq_rows", "qdq_cols_grouped", "layer_forward_mx", "layer_backward_mx", "BWD_POINTS"]


def e4m3_decode(code):
    """Value of an E4M3 (FN) code; 0x7F and 0xFF (NaN) are returned as nan."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_round(v):
    """Nearest E4M3 value to v (|v| <= 448), ties to even, as fp64."""
    v = _f64(v)
    a = np.abs(v)
    _, ex = np.frexp(a)                  # a = m * 2^ex, m in [0.5, 1)
    e = ex - 1                           # floor(log2 a) for a > 0
    quantum = np.where(a >= 2.0 ** -6, np.exp2(np.maximum(e, -6) - 3.0), 2.0 ** -9)
    return np.rint(v / quantum) * quantum


def e4m3_encode(v):
    """E4M3 code of a value already on the E4M3 grid (|v| <= 448); sign from signbit."""
    v = _f64(v)
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = ex - 1
    normal = a >= 2.0 ** -6
    mant_n = np.where(normal, a / np.exp2(np.where(normal, e, 0)) * 8.0 - 8.0, 0.0)
    code_n = ((e + 7) << 3) + mant_n.astype(np.int64)
    code_s = (a / 2.0 ** -9).astype(np.int64)
    return (sign | np.where(normal, code_n, code_s)).astype(np.uint8)


def e8m0_exponent(amax):
    """Smallest X with amax <= 448 * 2^X, clamped to [-127, 127]; 0 for amax == 0."""
    a = _f64(amax)
    _, ex = np.frexp(np.where(a > 0, a / E4M3_MAX, 1.0))
    X = ex - 1                                          # 2^X <= a/448 < 2^(X+1)
    X = np.where(a > np.ldexp(E4M3_MAX, X), X + 1, X)   # exact comparison
    X = np.where(a > np.ldexp(E4M3_MAX, X), X + 1, X)
    X = np.where(a == 0, 0, X)
    return np.clip(X, -127, 127).astype(np.int64)


def quantize_blocks(blocks):
    """Quantise an array [..., 32] block by block along the last axis.

    Returns (codes uint8 [..., 32], scale codes uint8 [...], dequantised fp64)."""
    b = _f64(blocks)
    X = e8m0_exponent(np.max(np.abs(b), axis=-1))
    scaled = b / np.exp2(X)[..., None]
    q = e4m3_round(scaled)
    codes = e4m3_encode(np.where(q == 0, np.copysign(0.0, scaled), q))
    deq = q * np.exp2(X)[..., None]
    return codes, (X + 127).astype(np.uint8), deq


def qdq_rows(m):
    """Row-wise MX quantize-dequantize of a matrix [M, K] (K % 32 == 0)."""
    m = _f64(m)
    M, K = m.shape
    _, _, deq = quantize_blocks(m.reshape(M, K // BLOCK, BLOCK))
    return deq.reshape(M, K)


def qdq_cols_grouped(m, offsets):
    """Column-wise MX quantize-dequantize of a ragged [R, N] matrix: 32-row blocks
    that start at each group's first row; a short last block is padded with zeros."""
    m = _f64(m)
    out = np.zeros_like(m)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(lo, hi, BLOCK):
            r1 = min(r0 + BLOCK, hi)
            blk = np.zeros((BLOCK, m.shape[1]))
            blk[: r1 - r0] = m[r0:r1]
            _, _, deq = quantize_blocks(blk.T)          # [N, 32]
            out[r0:r1] = deq.T[: r1 - r0]
    return out


def layer_forward_mx(inp: dict, k: int, e_begin: int, e_local: int, topk_idx, topk_w, index=None):
    """The forward with the four forward-GEMM operands quantize-dequantized to MXFP8
    (module docstring, mxfp8 forward); fp64 everywhere else.  Returns Y [T,H] and the
    saved rows (G, U, A, Yp) in the same form as the plain oracle's forward."""
    if index is None:
        index = build_index(topk_idx, e_begin, e_local)
    x = _f64(inp["x"])
    T, H = x.shape
    I = inp["w_gate"].shape[2]
    R = index["row_src"].shape[0]
    wflat = _f64(topk_w).reshape(-1)
    G = np.zeros((R, I)); U = np.zeros((R, I)); A = np.zeros((R, I)); Yp = np.zeros((R, H))
    Y = np.zeros((T, H))
    for e in range(e_local):
        lo, hi = int(index["offsets"][e]), int(index["offsets"][e + 1])
        if hi == lo:
            continue
        rows = index["row_src"][lo:hi]
        tok = rows // k
        # gate/up GEMM: Q(X rows along H) against Q(W columns along H)
        qx = qdq_rows(x[tok])
        g = qx @ qdq_cols_grouped(inp["w_gate"][e], np.array([0, H]))
        u = qx @ qdq_cols_grouped(inp["w_up"][e], np.array([0, H]))
        a = silu(g) * u
        # down GEMM: Q(A rows along I) against Q(W_down columns along I), then w
        yp = wflat[rows][:, None] * (qdq_rows(a) @ qdq_cols_grouped(inp["w_down"][e], np.array([0, I])))
        G[lo:hi], U[lo:hi], A[lo:hi], Yp[lo:hi] = g, u, a, yp
        Y[tok] += yp                                  # tokens are distinct within one expert
    return Y, {"G": G, "U": U, "A": A, "Yp": Yp, "index": index}


def _b1_dy(dye, we):
    """B1's dY' operand: the unweighted gathered rows, row-wise along H."""
    return qdq_rows(dye)


def _b2_dy(dye, we, seg):
    """B2's dY' operand: w * dY', column-wise in group-aware 32-row blocks."""
    return qdq_cols_grouped(we[:, None] * dye, seg)


def _rows_w(w):
    """A weight matrix quantised row-wise (W_down [I, H] along H for B1; W_gate and
    W_up [H, I] along I for B3)."""
    return qdq_rows(w)


def _rows_act(m, seg):
    """An activation operand quantised row-wise (dG and dU along I for B3)."""
    return qdq_rows(m)


def _cols_act(m, seg):
    """An activation operand quantised column-wise in group-aware 32-row blocks (A for
    B2; Xp, dG and dU for B4)."""
    return qdq_cols_grouped(m, seg)


# The eight quantisation points of the MXFP8 backward (module docstring, "Blocks lie along
# each backward GEMM's contraction axis" and "B1 quantises the unweighted dY'").  Each entry
# is the quantise-dequantise applied at that point.  layer_backward_mx takes the table as
# an argument only so that the tests can move one point at a time and show that a pin fails.
BWD_POINTS = {
    "b1_dy": _b1_dy,        # (dY' rows, w) -> Q_rows(dY')
    "b1_wd": _rows_w,       # W_down [I, H] -> Q along H
    "b2_a": _cols_act,      # (A, seg) -> Q_cols(A)
    "b2_dy": _b2_dy,        # (dY' rows, w, seg) -> Q_cols(w dY')
    "b3_dgu": _rows_act,    # (dG or dU, seg) -> Q along I
    "b3_w": _rows_w,        # W_gate / W_up [H, I] -> Q along I
    "b4_x": _cols_act,      # (Xp, seg) -> Q_cols(Xp)
    "b4_dgu": _cols_act,    # (dG or dU, seg) -> Q_cols
}


def layer_backward_mx(inp: dict, k: int, e_begin: int, e_local: int, topk_idx, topk_w, saved, points=None):
    """The backward with the eight backward-GEMM operands quantize-dequantized to
    MXFP8 at the points listed in the module docstring (the table BWD_POINTS, which
    `points` may override entry by entry); fp64 everywhere else."""
    q = dict(BWD_POINTS, **(points or {}))
    index = saved["index"]
    x = _f64(inp["x"]); dy = _f64(inp["dy"])
    T, H = x.shape
    I = inp["w_gate"].shape[2]
    wflat = _f64(topk_w).reshape(-1)
    dX = np.zeros((T, H))
    dWg = np.zeros((e_local, H, I)); dWu = np.zeros((e_local, H, I)); dWd = np.zeros((e_local, I, H))
    d_topk_w = np.zeros(T * k)
    for e in range(e_local):
        lo, hi = int(index["offsets"][e]), int(index["offsets"][e + 1])
        if hi == lo:
            continue
        rows = index["row_src"][lo:hi]
        tok = rows // k
        we = wflat[rows]
        g, u, a = saved["G"][lo:hi], saved["U"][lo:hi], saved["A"][lo:hi]
        wg = _f64(inp["w_gate"][e]); wu = _f64(inp["w_up"][e]); wd = _f64(inp["w_down"][e])
        xe, dye = x[tok], dy[tok]
        seg = np.array([0, hi - lo])
        # B1: dA' = Q(dY') Q(Wd)^T, both row-wise along H; w applies after the GEMM
        dap = q["b1_dy"](dye, we) @ q["b1_wd"](wd).T
        d_w = np.sum(dap * a, axis=1)
        da = we[:, None] * dap
        s = sigmoid(g)
        du = da * g * s
        dg = da * u * s * (1.0 + g * (1.0 - s))
        # B2: dWd = Q_col(A)^T Q_col(w dY')
        dWd[e] = q["b2_a"](a, seg).T @ q["b2_dy"](dye, we, seg)
        # B3: dXp = Q(dG) Q(Wg)^T + Q(dU) Q(Wu)^T, row-wise along I
        dxe = q["b3_dgu"](dg, seg) @ q["b3_w"](wg).T + q["b3_dgu"](du, seg) @ q["b3_w"](wu).T
        # B4: dWg = Q_col(X)^T Q_col(dG), dWu = Q_col(X)^T Q_col(dU)
        qx = q["b4_x"](xe, seg)
        dWg[e] = qx.T @ q["b4_dgu"](dg, seg)
        dWu[e] = qx.T @ q["b4_dgu"](du, seg)
        dX[tok] += dxe
        d_topk_w[rows] = d_w
    return {"dx": dX, "dw_gate": dWg, "dw_up": dWu, "dw_down": dWd,
            "d_topk_w": d_topk_w.reshape(T, k)}
