"""Pins of the oracle's routing and permutation against brute force and invariants."""
import math

import numpy as np
import pytest

from oracle import moe as om
import workloads as wl


def _brute_topk(row, k):
    """Repeated arg-max in pure Python: the largest remaining logit, lower id on ties."""
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.append(best)
    return taken


@pytest.mark.parametrize("k,E", [(2, 8), (8, 128), (3, 5), (5, 5)])
def test_topk_matches_repeated_argmax_with_ties(k, E):
    rng = np.random.default_rng(11)
    # few distinct values: many ties at every rank
    L = rng.integers(-3, 3, size=(40, E)).astype(np.float32) * np.float32(0.5)
    idx, w = om.route_topk(L, k)
    for t in range(L.shape[0]):
        assert list(idx[t]) == _brute_topk([float(v) for v in L[t]], k)


def test_topk_weights_closed_form_renorm():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((16, 12)).astype(np.float32)
    idx, w = om.route_topk(L, 4, renorm=1)
    for t in range(16):
        z = [math.exp(float(L[t, e])) for e in idx[t]]
        for j in range(4):
            assert abs(w[t, j] - z[j] / sum(z)) < 1e-15
    assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_weights_closed_form_full_softmax():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((10, 9)).astype(np.float32)
    idx, w = om.route_topk(L, 3, renorm=0)
    for t in range(10):
        den = sum(math.exp(float(v)) for v in L[t])
        for j in range(3):
            assert abs(w[t, j] - math.exp(float(L[t, idx[t, j]])) / den) < 1e-15


def test_k_equals_E_selects_all_and_renorm_is_full_softmax():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((7, 6)).astype(np.float32)
    i1, w1 = om.route_topk(L, 6, renorm=1)
    i0, w0 = om.route_topk(L, 6, renorm=0)
    assert np.array_equal(np.sort(i1, axis=1), np.tile(np.arange(6), (7, 1)))
    assert np.allclose(w1, w0, rtol=1e-14, atol=0)


def _brute_index(idx, e_begin, e_local):
    T, k = idx.shape
    groups = [[] for _ in range(e_local)]
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j]) - e_begin
            if 0 <= e < e_local:
                groups[e].append(t * k + j)
    row_src = [s for g in groups for s in g]
    return [len(g) for g in groups], row_src


@pytest.mark.parametrize("e_begin,e_local", [(0, 8), (2, 3), (7, 1), (0, 1)])
def test_index_matches_brute_force(e_begin, e_local):
    rng = np.random.default_rng(9)
    L = rng.standard_normal((50, 8)).astype(np.float32)
    idx, _ = om.route_topk(L, 3)
    ix = om.build_index(idx, e_begin, e_local)
    counts, row_src = _brute_index(idx, e_begin, e_local)
    assert list(ix["counts"]) == counts
    assert list(ix["row_src"]) == row_src
    assert ix["offsets"][0] == 0 and list(np.diff(ix["offsets"])) == counts
    R = len(row_src)
    assert np.array_equal(ix["row_of"][ix["row_src"]], np.arange(R))
    assert np.sum(ix["row_of"] >= 0) == R
    for s in range(idx.size):
        e = int(idx.reshape(-1)[s])
        assert (ix["row_of"][s] >= 0) == (e_begin <= e < e_begin + e_local)


def test_counts_sum_to_T_times_k_and_segments_token_ascending():
    cfg = wl.CONFIGS["qwen3_30b"]
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    idx, _ = om.route_topk(inp["logits"], cfg.k)
    ix = om.build_index(idx, 0, cfg.E)
    assert int(ix["counts"].sum()) == cfg.T * cfg.k
    for e in range(cfg.E):
        seg = ix["row_src"][ix["offsets"][e]:ix["offsets"][e + 1]]
        assert np.all(np.diff(seg // cfg.k) > 0)
        assert np.all(idx.reshape(-1)[seg] == e)


def test_skewed_workload_has_empty_experts_and_zipf_head():
    cfg = wl.CONFIGS["skew_zipf"]
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    idx, _ = om.route_topk(inp["logits"], cfg.k)
    ix = om.build_index(idx, 0, cfg.E)
    c = ix["counts"]
    assert int(c.sum()) == cfg.T * cfg.k
    assert int(np.sum(c == 0)) == 8
    assert c.max() > 10000          # the rank-1 expert takes most tokens
    assert np.sort(c)[8] > 0        # every other expert gets some


def test_round_trip_permute_unpermute_is_multiplicity():
    """Gathering rows with row_src and summing them back with row_of gives n_t * x[t]."""
    rng = np.random.default_rng(2)
    T, k, E = 40, 3, 6
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, 5))
    idx, _ = om.route_topk(L, k)
    for e_begin, e_local in [(0, 6), (1, 2)]:
        ix = om.build_index(idx, e_begin, e_local)
        xp = x[ix["row_src"] // k]
        back = np.zeros_like(x)
        n = np.zeros(T)
        for s, r in enumerate(ix["row_of"]):
            if r >= 0:
                back[s // k] += xp[r]
                n[s // k] += 1
        assert np.array_equal(back, n[:, None] * x)


def _router_case(seed=5):
    """Tiny fp64 layer whose logits come from a router GEMM x W_r (E = 8, k = 2)."""
    cfg = wl.CONFIGS["tiny_f32"].replace(seed=seed)
    inp = wl.make_inputs(cfg)
    inp = {kk: np.asarray(v, dtype=np.float64) for kk, v in inp.items()}
    rng = np.random.default_rng(seed)
    w_r = rng.standard_normal((cfg.H, cfg.E)) / np.sqrt(cfg.H)
    return cfg, inp, w_r


def _router_loss(cfg, inp, w_r, x=None):
    """<dY, Y> with logits = x W_r feeding the routing; x also feeds the experts."""
    x = inp["x"] if x is None else x
    lg = om.router_logits(x, w_r)
    idx, w = om.route_topk(lg, cfg.k, cfg.renorm)
    Y, _ = om.layer_forward(dict(inp, x=x), cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    return float(np.sum(inp["dy"] * Y)), lg


def _router_grads(cfg, inp, w_r):
    lg = om.router_logits(inp["x"], w_r)
    idx, w = om.route_topk(lg, cfg.k, cfg.renorm)
    Y, saved = om.layer_forward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    g = om.layer_backward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, saved)
    dl = om.router_backward(lg, idx, w, g["d_topk_w"], cfg.renorm)
    dx_r, dw_r = om.router_gemm_backward(inp["x"], w_r, dl)
    return lg, dl, g, dx_r, dw_r


def _margin(lg, k):
    s = np.sort(lg, axis=1)[:, ::-1]
    return float(np.min(s[:, k - 1] - s[:, k]))


def test_router_gemm_backward_by_finite_differences():
    # the whole chain logits = x W_r -> top-k softmax -> layer: central differences of
    # <dY, Y> on W_r entries, and on x entries where x feeds both the router and the
    # experts (dX = the experts' dX + d_logits W_r^T)
    cfg, inp, w_r = _router_case()
    lg, dl, g, dx_r, dw_r = _router_grads(cfg, inp, w_r)
    rng = np.random.default_rng(9)
    h = 1e-6
    checked = 0
    for _ in range(12):
        pos = (int(rng.integers(0, cfg.H)), int(rng.integers(0, cfg.E)))
        wp = w_r.copy(); wp[pos] += h
        wm = w_r.copy(); wm[pos] -= h
        (lp, lgp), (lm, lgm) = _router_loss(cfg, inp, wp), _router_loss(cfg, inp, wm)
        if min(_margin(lgp, cfg.k), _margin(lgm, cfg.k)) < 1e-4:
            continue      # the selection would change inside the difference
        fd = (lp - lm) / (2 * h)
        assert abs(fd - dw_r[pos]) <= 1e-5 * max(1.0, abs(fd)), (pos, fd, dw_r[pos])
        checked += 1
    dx = g["dx"] + dx_r
    for _ in range(12):
        pos = (int(rng.integers(0, cfg.T)), int(rng.integers(0, cfg.H)))
        xp = inp["x"].copy(); xp[pos] += h
        xm = inp["x"].copy(); xm[pos] -= h
        (lp, lgp), (lm, lgm) = _router_loss(cfg, inp, w_r, xp), _router_loss(cfg, inp, w_r, xm)
        if min(_margin(lgp, cfg.k), _margin(lgm, cfg.k)) < 1e-4:
            continue
        fd = (lp - lm) / (2 * h)
        assert abs(fd - dx[pos]) <= 1e-5 * max(1.0, abs(fd)), (pos, fd, dx[pos])
        checked += 1
    assert checked >= 16
    # the router's own share of dX is not negligible, so a dropped term would show
    assert np.linalg.norm(dx_r) > 1e-2 * np.linalg.norm(g["dx"])


def test_router_gemm_euler_identities():
    # logits are linear in W_r and in x (for the router path): <dW_r, W_r> = <dx_r, x> =
    # <d_logits, logits>
    cfg, inp, w_r = _router_case(6)
    lg, dl, g, dx_r, dw_r = _router_grads(cfg, inp, w_r)
    ref = float(np.sum(dl * lg))
    assert abs(ref) > 1e-3
    assert abs(float(np.sum(dw_r * w_r)) - ref) <= 1e-10 * max(1.0, abs(ref))
    assert abs(float(np.sum(dx_r * inp["x"])) - ref) <= 1e-10 * max(1.0, abs(ref))
