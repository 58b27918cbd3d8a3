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
