"""fp64 oracle of the dropless MoE layer: route, index, forward, backward.

Readings (the pages name the steps but print no formula):

* Routing -- NVIDIA article, "What makes MoE training hard" (a learned router picks
  the top-K experts), Prime Mega MoE pages ("128 experts, top-8 routing").
  The k largest fp32 logits are selected, ties going to the lower expert id, slots
  ordered by logit descending; weights are the softmax over the k selected logits
  (renorm=1, equal to softmax -> top-k -> renormalise) or the full softmax over all
  E logits evaluated at the selected experts (renorm=0).
* Permutation -- NVIDIA article, "Optimization 2" (dispatch permutes tokens by
  expert).  Rows are ordered expert-major, token-ascending: a stable sort of the
  flattened (token, slot) ids by local expert.  Slots routed to experts outside
  [e_begin, e_begin+e_local) are not local: they get no row (row_of = -1).
* Expert MLP -- Prime Mega MoE pages (two expert linear layers with SwiGLU between
  them): a = silu(x Wg) * (x Wu), y = a Wd; silu(g) = g / (1 + exp(-g)).
* Combine -- NVIDIA article, "Optimization 2" and Figure 3 (combine accumulates the
  per-expert outputs in token order): Y[t] = sum over local slots of w * y.  A token
  with no local slot gets Y = 0 (the partial sum another rank would complete).
* Backward -- the chain rule of the forward above (dA', d_w, SwiGLU backward, dX,
  dW_gate, dW_up, dW_down) and of the softmax weights (router backward).
* Router GEMM -- NVIDIA article, "Optimization 2" (fused router kernels assign each
  token to its experts): the plainest learned router is one linear map without bias,
  logits = X W_r with W_r [H, E] (every expert, not only the local ones), followed by
  the routing above.  Its backward: dX gains d_logits W_r^T, dW_r = X^T d_logits.

Everything is evaluated in fp64 from the (bf16- or fp32-valued) inputs, with no
intermediate rounding.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "route_topk", "build_index", "silu", "layer_forward", "layer_backward",
    "router_backward", "router_logits", "router_gemm_backward", "brute_force", "token_sample",
    "expert_sample",
]


def route_topk(logits: np.ndarray, k: int, renorm: int = 1):
    """Top-k experts per token and their softmax weights.

    Returns (topk_idx int32 [T,k], topk_w float64 [T,k]).  Selection compares the
    fp32 logits themselves (fp64 logits, used by finite-difference checks, are compared
    as given); a stable sort of -logits keeps the lower id first on ties.
    """
    L = np.asarray(logits)
    if L.dtype != np.float64:
        L = L.astype(np.float32)          # the layer's logits are fp32
    T, E = L.shape
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx, axis=1).astype(np.float64)
    if renorm:
        z = np.exp(sel - sel[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    else:
        full = L.astype(np.float64)
        z = np.exp(full - full.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, idx, axis=1)
    return idx, w


def build_index(topk_idx: np.ndarray, e_begin: int, e_local: int):
    """Stable expert-major permutation of the local (token, slot) pairs.

    Returns dict with counts [e_local], offsets [e_local+1], row_src [R] (row ->
    t*k+j) and row_of [T*k] (slot -> row, or -1 for a non-local slot).
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    local = (flat >= e_begin) & (flat < e_begin + e_local)
    slots = np.nonzero(local)[0]                     # ascending slot ids
    le = flat[slots] - e_begin
    order = np.argsort(le, kind="stable")            # expert-major, slot-ascending
    row_src = slots[order].astype(np.int32)
    counts = np.bincount(le, minlength=e_local).astype(np.int32)
    offsets = np.zeros(e_local + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_of = np.full(flat.shape[0], -1, dtype=np.int32)
    row_of[row_src] = np.arange(row_src.shape[0], dtype=np.int32)
    return {"counts": counts, "offsets": offsets, "row_src": row_src, "row_of": row_of}


def silu(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def sigmoid(g):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _expert_rows(index, e):
    return index["row_src"][index["offsets"][e]:index["offsets"][e + 1]]


def _expert_fwd(xe, wg, wu, wd, we):
    g = xe @ wg
    u = xe @ wu
    a = silu(g) * u
    yp = we[:, None] * (a @ wd)
    return g, u, a, yp


def _expert_bwd(xe, dye, g, u, a, wg, wu, wd, we):
    dap = dye @ wd.T                                  # dA' = dY' Wd^T
    d_w = np.sum(dap * a, axis=1)                     # d loss / d w for each row
    da = we[:, None] * dap
    s = sigmoid(g)
    du = da * g * s                                   # d/du of silu(g) u
    dg = da * u * s * (1.0 + g * (1.0 - s))           # d/dg of silu(g) u
    dxe = dg @ wg.T + du @ wu.T
    dwg = xe.T @ dg
    dwu = xe.T @ du
    dwd = a.T @ (we[:, None] * dye)
    return d_w, dg, du, dxe, dwg, dwu, dwd


def layer_forward(inp: dict, k: int, e_begin: int, e_local: int, topk_idx, topk_w, index=None):
    """Y [T,H] and the per-row saved tensors (G, U, A, Yp over rows in row order)."""
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
        lo, hi = index["offsets"][e], index["offsets"][e + 1]
        if hi == lo:
            continue
        rows = _expert_rows(index, e)
        tok = rows // k
        g, u, a, yp = _expert_fwd(x[tok], _f64(inp["w_gate"][e]), _f64(inp["w_up"][e]),
                                  _f64(inp["w_down"][e]), wflat[rows])
        G[lo:hi], U[lo:hi], A[lo:hi], Yp[lo:hi] = g, u, a, yp
        Y[tok] += yp                                  # tokens are distinct within one expert
    return Y, {"G": G, "U": U, "A": A, "Yp": Yp, "index": index}


def layer_backward(inp: dict, k: int, e_begin: int, e_local: int, topk_idx, topk_w, saved):
    """dX [T,H], dW_gate/dW_up [El,H,I], dW_down [El,I,H], d_topk_w [T,k]."""
    index = saved["index"]
    x = _f64(inp["x"]); dy = _f64(inp["dy"])
    T, H = x.shape
    I = inp["w_gate"].shape[2]
    wflat = _f64(topk_w).reshape(-1)
    dX = np.zeros((T, H))
    dWg = np.zeros((e_local, H, I)); dWu = np.zeros((e_local, H, I)); dWd = np.zeros((e_local, I, H))
    d_topk_w = np.zeros(T * k)
    for e in range(e_local):
        lo, hi = index["offsets"][e], index["offsets"][e + 1]
        if hi == lo:
            continue
        rows = _expert_rows(index, e)
        tok = rows // k
        d_w, dg, du, dxe, dwg, dwu, dwd = _expert_bwd(
            x[tok], dy[tok], saved["G"][lo:hi], saved["U"][lo:hi], saved["A"][lo:hi],
            _f64(inp["w_gate"][e]), _f64(inp["w_up"][e]), _f64(inp["w_down"][e]), wflat[rows])
        dX[tok] += dxe
        dWg[e], dWu[e], dWd[e] = dwg, dwu, dwd
        d_topk_w[rows] = d_w
    return {"dx": dX, "dw_gate": dWg, "dw_up": dWu, "dw_down": dWd,
            "d_topk_w": d_topk_w.reshape(T, k)}


def router_backward(logits, topk_idx, topk_w, d_topk_w, renorm: int = 1):
    """d loss / d logits [T,E] through the softmax weights (the selection itself is
    piecewise constant and has no gradient)."""
    L = _f64(logits)
    T, E = L.shape
    w = _f64(topk_w); dw = _f64(d_topk_w)
    out = np.zeros((T, E))
    if renorm:
        s = np.sum(w * dw, axis=1, keepdims=True)
        np.put_along_axis(out, np.asarray(topk_idx, dtype=np.int64), w * (dw - s), axis=1)
    else:
        z = np.exp(L - L.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        gsel = np.zeros((T, E))
        np.put_along_axis(gsel, np.asarray(topk_idx, dtype=np.int64), dw, axis=1)
        s = np.sum(w * dw, axis=1, keepdims=True)     # w_j = p[S_j]
        out = p * (gsel - s)
    return out


def router_logits(x, w_r):
    """Router GEMM: logits [T,E] = x [T,H] W_r [H,E] (fp64)."""
    return _f64(x) @ _f64(w_r)


def router_gemm_backward(x, w_r, d_logits):
    """Backward of the router GEMM: (d loss/d x [T,H], d loss/d W_r [H,E]) for the
    upstream d_logits [T,E]."""
    dl = _f64(d_logits)
    return dl @ _f64(w_r).T, _f64(x).T @ dl


def brute_force(inp: dict, k: int, e_begin: int, e_local: int, topk_idx, topk_w):
    """Per-token loop over its top-k experts, with no permutation and no offsets.

    Returns Y, dX, dW_gate, dW_up, dW_down, d_topk_w (fp64).  Meant for tiny inputs.
    """
    x = _f64(inp["x"]); dy = _f64(inp["dy"])
    T, H = x.shape
    I = inp["w_gate"].shape[2]
    Y = np.zeros((T, H)); dX = np.zeros((T, H))
    dWg = np.zeros((e_local, H, I)); dWu = np.zeros((e_local, H, I)); dWd = np.zeros((e_local, I, H))
    d_topk_w = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j]) - e_begin
            if e < 0 or e >= e_local:
                continue
            wg = _f64(inp["w_gate"][e]); wu = _f64(inp["w_up"][e]); wd = _f64(inp["w_down"][e])
            w = float(topk_w[t, j])
            g = x[t] @ wg
            u = x[t] @ wu
            sg = sigmoid(g)
            a = g * sg * u
            Y[t] += w * (a @ wd)
            dap = wd @ dy[t]
            d_topk_w[t, j] = float(dap @ a)
            da = w * dap
            du = da * g * sg
            dg = da * u * sg * (1.0 + g * (1.0 - sg))
            dX[t] += wg @ dg + wu @ du
            dWg[e] += np.outer(x[t], dg)
            dWu[e] += np.outer(x[t], du)
            dWd[e] += np.outer(a, w * dy[t])
    return {"y": Y, "dx": dX, "dw_gate": dWg, "dw_up": dWu, "dw_down": dWd, "d_topk_w": d_topk_w}


def token_sample(inp: dict, k: int, e_begin: int, e_local: int, topk_idx, topk_w, tokens):
    """Y, dX and d_topk_w for a subset of tokens only (each from its own slots)."""
    x = _f64(inp["x"]); dy = _f64(inp["dy"])
    tokens = np.asarray(tokens, dtype=np.int64)
    H = x.shape[1]
    n = tokens.shape[0]
    Y = np.zeros((n, H)); dX = np.zeros((n, H)); dtw = np.zeros((n, k))
    idx = np.asarray(topk_idx)[tokens]
    w = _f64(topk_w)[tokens]
    for e in range(e_local):
        pos_t, pos_j = np.nonzero(idx == e_begin + e)
        if pos_t.size == 0:
            continue
        xe = x[tokens[pos_t]]
        g, u, a, yp = _expert_fwd(xe, _f64(inp["w_gate"][e]), _f64(inp["w_up"][e]),
                                  _f64(inp["w_down"][e]), w[pos_t, pos_j])
        np.add.at(Y, pos_t, yp)
        d_w, dg, du, dxe, *_ = _expert_bwd(xe, dy[tokens[pos_t]], g, u, a, _f64(inp["w_gate"][e]),
                                           _f64(inp["w_up"][e]), _f64(inp["w_down"][e]),
                                           w[pos_t, pos_j])
        np.add.at(dX, pos_t, dxe)
        dtw[pos_t, pos_j] = d_w
    return {"y": Y, "dx": dX, "d_topk_w": dtw}


def expert_sample(inp: dict, k: int, index: dict, topk_w, experts):
    """dW_gate, dW_up, dW_down of a subset of local experts (each needs all its rows)."""
    x = _f64(inp["x"]); dy = _f64(inp["dy"])
    wflat = _f64(topk_w).reshape(-1)
    out = {}
    for e in experts:
        rows = _expert_rows(index, e)
        H = x.shape[1]; I = inp["w_gate"].shape[2]
        if rows.size == 0:
            out[e] = (np.zeros((H, I)), np.zeros((H, I)), np.zeros((I, H)))
            continue
        tok = rows // k
        wg = _f64(inp["w_gate"][e]); wu = _f64(inp["w_up"][e]); wd = _f64(inp["w_down"][e])
        g, u, a, _ = _expert_fwd(x[tok], wg, wu, wd, wflat[rows])
        _, _, _, _, dwg, dwu, dwd = _expert_bwd(x[tok], dy[tok], g, u, a, wg, wu, wd, wflat[rows])
        out[e] = (dwg, dwu, dwd)
    return out
