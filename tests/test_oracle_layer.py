"""Pins of the oracle's forward and backward: brute force, closed forms, a dense special
case, finite differences, Euler identities and a second opinion from torch autograd."""
import math

import numpy as np
import pytest

from oracle import moe as om
import workloads as wl


def _run(cfg, inp=None):
    inp = inp or wl.make_inputs(cfg)
    idx, w = om.route_topk(inp["logits"], cfg.k, cfg.renorm)
    Y, saved = om.layer_forward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    g = om.layer_backward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, saved)
    return inp, idx, w, Y, saved, g


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


TINY = [wl.CONFIGS["tiny_f32"], wl.CONFIGS["tiny_bf16"],
        wl.CONFIGS["tiny_bf16"].replace(e_begin=3, e_local=4),
        wl.CONFIGS["tiny_f32"].replace(renorm=0)]


@pytest.mark.parametrize("cfg", TINY, ids=lambda c: f"{c.name}-eb{c.e_begin}-el{c.e_local}-rn{c.renorm}")
def test_grouped_matches_per_token_brute_force(cfg):
    inp, idx, w, Y, saved, g = _run(cfg)
    bf = om.brute_force(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    assert _rel(Y, bf["y"]) < 1e-13
    for key in ("dx", "dw_gate", "dw_up", "dw_down", "d_topk_w"):
        assert _rel(g[key], bf[key]) < 1e-13, key


def test_swiglu_closed_form_with_diagonal_weights():
    """H = I with diagonal W_gate = a_e, W_up = b_e and W_down = c_e * identity:
    y[t] = sum_j w_j c_e silu(a_e x) (b_e x), element by element."""
    T, H, E, k = 12, 6, 4, 2
    rng = np.random.default_rng(1)
    x = rng.standard_normal((T, H))
    a = [0.5, -1.25, 2.0, 0.75]; b = [1.5, 0.25, -0.5, 2.5]; c = [1.0, -2.0, 0.5, 3.0]
    inp = {"x": x, "dy": np.zeros((T, H)),
           "w_gate": np.stack([np.eye(H) * a[e] for e in range(E)]),
           "w_up": np.stack([np.eye(H) * b[e] for e in range(E)]),
           "w_down": np.stack([np.eye(H) * c[e] for e in range(E)])}
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = om.route_topk(L, k)
    Y, _ = om.layer_forward(inp, k, 0, E, idx, w)
    for t in range(T):
        for h in range(H):
            ref = 0.0
            for j in range(k):
                e = int(idx[t, j])
                gv = a[e] * x[t, h]
                ref += w[t, j] * c[e] * (gv / (1.0 + math.exp(-gv))) * (b[e] * x[t, h])
            assert abs(Y[t, h] - ref) <= 1e-14 * max(1.0, abs(ref))


def test_single_expert_top1_is_dense_swiglu_mlp():
    cfg = wl.CONFIGS["tiny_f32"].replace(E=1, k=1, e_local=1)
    inp = wl.make_inputs(cfg)
    idx, w = om.route_topk(inp["logits"], 1)
    assert np.all(w == 1.0)
    Y, _ = om.layer_forward(inp, 1, 0, 1, idx, w)
    X = inp["x"].astype(np.float64)
    G = X @ inp["w_gate"][0].astype(np.float64)
    U = X @ inp["w_up"][0].astype(np.float64)
    ref = (G / (1 + np.exp(-G)) * U) @ inp["w_down"][0].astype(np.float64)
    assert _rel(Y, ref) < 1e-13


def test_token_permutation_and_expert_relabelling():
    cfg = wl.CONFIGS["tiny_f32"]
    inp = wl.make_inputs(cfg)
    _, idx, w, Y, _, g = _run(cfg, inp)
    perm = np.random.default_rng(0).permutation(cfg.T)
    inp_p = dict(inp, x=inp["x"][perm], dy=inp["dy"][perm], logits=inp["logits"][perm])
    _, _, _, Yp, _, gp = _run(cfg, inp_p)
    assert _rel(Yp, Y[perm]) < 1e-14 and _rel(gp["dx"], g["dx"][perm]) < 1e-14
    relabel = np.random.default_rng(1).permutation(cfg.E)      # new id of old expert e
    inv = np.argsort(relabel)
    inp_r = dict(inp, logits=inp["logits"][:, inv], w_gate=inp["w_gate"][inv],
                 w_up=inp["w_up"][inv], w_down=inp["w_down"][inv])
    _, _, _, Yr, _, gr = _run(cfg, inp_r)
    assert _rel(Yr, Y) < 1e-14 and _rel(gr["dw_down"], g["dw_down"][inv]) < 1e-14


def test_euler_identities():
    """Y is linear in W_down, in W_up and in the routing weights, so
    <dWd, Wd> = <dWu, Wu> = sum w * d_topk_w = <dY, Y>."""
    for cfg in (wl.CONFIGS["tiny_f32"], wl.CONFIGS["tiny_bf16"].replace(e_begin=2, e_local=5)):
        inp, idx, w, Y, saved, g = _run(cfg)
        ref = float(np.sum(inp["dy"].astype(np.float64) * Y))
        for v in (np.sum(g["dw_down"] * inp["w_down"]), np.sum(g["dw_up"] * inp["w_up"]),
                  np.sum(w * g["d_topk_w"])):
            assert abs(float(v) - ref) <= 1e-12 * max(1.0, abs(ref))


def test_empty_expert_gradients_are_zero():
    cfg = wl.CONFIGS["tiny_f32"]
    inp = wl.make_inputs(cfg)
    inp["logits"][:, 5] = -1e4
    _, idx, w, Y, saved, g = _run(cfg, inp)
    assert saved["index"]["counts"][5] == 0
    assert not g["dw_gate"][5].any() and not g["dw_up"][5].any() and not g["dw_down"][5].any()


def test_router_backward_properties():
    cfg = wl.CONFIGS["tiny_f32"]
    for renorm in (1, 0):
        c = cfg.replace(renorm=renorm)
        inp, idx, w, Y, saved, g = _run(c)
        dL = om.router_backward(inp["logits"], idx, w, g["d_topk_w"], renorm)
        assert np.max(np.abs(dL.sum(axis=1))) < 1e-14
        if renorm:
            mask = np.ones_like(dL, dtype=bool)
            np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
            assert not dL[mask].any()


def _loss(inp, cfg, logits=None):
    lg = inp["logits"] if logits is None else logits
    idx, w = om.route_topk(lg, cfg.k, cfg.renorm)
    Y, _ = om.layer_forward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    return float(np.sum(np.asarray(inp["dy"], dtype=np.float64) * Y))


@pytest.mark.parametrize("cfg", [wl.CONFIGS["tiny_f32"], wl.CONFIGS["tiny_f32"].replace(renorm=0, e_begin=2, e_local=5)],
                         ids=["full", "renorm0-share"])
def test_finite_differences(cfg):
    inp = wl.make_inputs(cfg)
    inp = {kk: np.asarray(v, dtype=np.float64) if kk != "logits" else v for kk, v in inp.items()}
    idx, w = om.route_topk(inp["logits"], cfg.k, cfg.renorm)
    Y, saved = om.layer_forward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    g = om.layer_backward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, saved)
    rng = np.random.default_rng(7)
    h = 1e-5
    for name, grad in (("x", g["dx"]), ("w_gate", g["dw_gate"]), ("w_up", g["dw_up"]),
                       ("w_down", g["dw_down"])):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in inp[name].shape)
            p = {kk: v.copy() if kk == name else v for kk, v in inp.items()}
            p[name][pos] += h
            lp = _loss(p, cfg)
            p[name][pos] -= 2 * h
            lm = _loss(p, cfg)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    # logits: the softmax weights are smooth; skip coordinates near the k-th boundary
    dL = om.router_backward(inp["logits"], idx, w, g["d_topk_w"], cfg.renorm)
    L64 = inp["logits"].astype(np.float64)
    checked = 0
    for _ in range(200):
        t = int(rng.integers(0, cfg.T)); e = int(rng.integers(0, cfg.E))
        srt = np.sort(L64[t])[::-1]
        if abs(srt[cfg.k - 1] - srt[cfg.k]) < 1e-3:
            continue
        hh = 1e-4
        lp_ = L64.copy(); lp_[t, e] += hh
        lm_ = L64.copy(); lm_[t, e] -= hh
        # evaluate the same selection with fp64 logits: the routing keys only change by hh
        fd = (_loss(inp, cfg, lp_) - _loss(inp, cfg, lm_)) / (2 * hh)
        assert abs(fd - dL[t, e]) <= 1e-6 * max(1.0, abs(fd)), (t, e, fd, dL[t, e])
        checked += 1
        if checked >= 12:
            break
    assert checked >= 12


def test_torch_autograd_second_opinion():
    torch = pytest.importorskip("torch")
    cfg = wl.CONFIGS["tiny_f32"].replace(e_begin=1, e_local=6)
    inp = wl.make_inputs(cfg)
    idx, w = om.route_topk(inp["logits"], cfg.k)
    Y, saved = om.layer_forward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    g = om.layer_backward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, saved)
    dt = torch.float64
    x = torch.tensor(inp["x"], dtype=dt, requires_grad=True)
    Wg = torch.tensor(inp["w_gate"], dtype=dt, requires_grad=True)
    Wu = torch.tensor(inp["w_up"], dtype=dt, requires_grad=True)
    Wd = torch.tensor(inp["w_down"], dtype=dt, requires_grad=True)
    L = torch.tensor(inp["logits"], dtype=dt, requires_grad=True)
    sel = torch.tensor(idx, dtype=torch.long)
    wt = torch.softmax(torch.gather(L, 1, sel), dim=1)
    y = torch.zeros(cfg.T, cfg.H, dtype=dt)
    for j in range(cfg.k):
        for e in range(cfg.e_local):
            m = (sel[:, j] == cfg.e_begin + e).nonzero().flatten()
            if m.numel() == 0:
                continue
            xe = x.index_select(0, m)
            a = torch.nn.functional.silu(xe @ Wg[e]) * (xe @ Wu[e])
            y = y.index_add(0, m, wt[m, j:j + 1] * (a @ Wd[e]))
    dy = torch.tensor(inp["dy"], dtype=dt)
    (y * dy).sum().backward()
    assert _rel(y.detach().numpy(), Y) < 1e-13
    assert _rel(x.grad.numpy(), g["dx"]) < 1e-13
    assert _rel(Wg.grad.numpy(), g["dw_gate"]) < 1e-13
    assert _rel(Wd.grad.numpy(), g["dw_down"]) < 1e-13
    dL = om.router_backward(inp["logits"], idx, w, g["d_topk_w"], 1)
    assert _rel(L.grad.numpy(), dL) < 1e-13


def test_samples_match_full_layer():
    cfg = wl.CONFIGS["tiny_bf16"].replace(e_begin=1, e_local=6)
    inp, idx, w, Y, saved, g = _run(cfg)
    toks = np.array([0, 5, 17, 63])
    s = om.token_sample(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, toks)
    assert _rel(s["y"], Y[toks]) < 1e-14 and _rel(s["dx"], g["dx"][toks]) < 1e-14
    assert _rel(s["d_topk_w"], g["d_topk_w"][toks]) < 1e-14
    es = om.expert_sample(inp, cfg.k, saved["index"], w, [0, 3, 5])
    for e, (dwg, dwu, dwd) in es.items():
        assert _rel(dwg, g["dw_gate"][e]) < 1e-14 and _rel(dwd, g["dw_down"][e]) < 1e-14
