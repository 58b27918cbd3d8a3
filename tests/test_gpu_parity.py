"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Integer outputs (top-k ids, counts, offsets, row order) must match bit for bit; float
outputs within a relative Frobenius error of 1e-2 (bf16 runs) or 1e-5 (fp32 runs).
Small layers are compared element by element in full; the full-size workloads on
sampled tokens and experts, which the oracle evaluates one by one."""
import numpy as np
import pytest

import workloads as wl
from oracle import moe as om

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import BF16_TOL, W_TOL, inputs, oracle_full, rel, run_layer, tol  # noqa: E402

SMALL = {
    "tiny_f32": wl.CONFIGS["tiny_f32"],
    "tiny_bf16": wl.CONFIGS["tiny_bf16"],
    "tiny_bf16_share": wl.CONFIGS["tiny_bf16"].replace(e_begin=3, e_local=4),
    "tiny_f32_renorm0": wl.CONFIGS["tiny_f32"].replace(renorm=0, e_begin=1, e_local=6),
    # several 128-row tiles per expert with ragged tails, and N tails of 64 columns
    "ragged_bf16": wl.MoeConfig("ragged_bf16", 700, 192, 192, 6, 2, 0, 6, 5),
    "ragged_bf16_share": wl.MoeConfig("ragged_bf16_share", 700, 192, 320, 10, 3, 4, 5, 6),
    "ragged_f32": wl.MoeConfig("ragged_f32", 300, 96, 80, 6, 2, 0, 6, 7, dtype="f32"),
    # Zipf-skewed loads with 8 empty experts; the weight gradients' 768 and 384 output
    # tiles take several rounds of the persistent grid in cost order
    "skew_bf16": wl.MoeConfig("skew_bf16", 1024, 512, 384, 64, 4, 0, 64, 10, routing="zipf"),
    # about 320 rows per expert (T k / E = 320), every bf16 row-tiled GEMM on 320-row tiles
    # (row_tile = 320; one round of the grid makes the library's own choice 256): tiles that
    # reach the second wave row, experts past 320 rows with a short second tile, 64-column
    # N tails
    "tall_bf16": wl.MoeConfig("tall_bf16", 1280, 320, 192, 8, 2, 0, 8, 11, row_tile=320),
    "tall_bf16_share": wl.MoeConfig("tall_bf16_share", 1280, 320, 192, 8, 2, 2, 5, 12, row_tile=320),
}


def _check_ints(cfg, out, ref):
    assert np.array_equal(out["topk_idx"], ref["topk_idx"])
    ix = ref["index"]
    assert np.array_equal(out["counts"], ix["counts"])
    assert np.array_equal(out["offsets"], ix["offsets"])
    assert np.array_equal(out["row_src"], ix["row_src"])
    assert np.array_equal(out["row_of"], ix["row_of"])


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("fuse", [True, False], ids=["fused_gather", "xp"])
def test_small_layer_parity(name, fuse):
    cfg = SMALL[name]
    print(f"[parity] {name} fuse={fuse}", flush=True)
    inp = inputs(cfg)
    out = run_layer(cfg, inp, fuse_gather=fuse)
    ref = oracle_full(cfg, inp)
    _check_ints(cfg, out, ref)
    assert rel(out["topk_w"], ref["topk_w"]) < W_TOL
    t = tol(cfg)
    for key in ("y", "dx", "dw_gate", "dw_up", "dw_down", "d_topk_w", "d_logits"):
        err = rel(out[key], ref[key])
        assert err < t, (key, err)
    if not fuse:
        assert np.array_equal(out["xp"], inp["x"][ix_tok(ref, cfg)])


RECOMPUTE = [n for n, c in SMALL.items() if c.dtype == "bf16"]


@pytest.mark.parametrize("name", RECOMPUTE)
def test_small_layer_parity_recompute(name):
    """Activation checkpointing (the pages time their layers with full activation
    checkpointing: the forward keeps nothing and the backward recomputes G|U and A)
    against the oracle, every output element by element."""
    cfg = SMALL[name]
    print(f"[parity-recompute] {name}", flush=True)
    inp = inputs(cfg)
    out = run_layer(cfg, inp, recompute=1)
    ref = oracle_full(cfg, inp)
    _check_ints(cfg, out, ref)
    assert rel(out["topk_w"], ref["topk_w"]) < W_TOL
    for key in ("y", "dx", "dw_gate", "dw_up", "dw_down", "d_topk_w", "d_logits"):
        err = rel(out[key], ref[key])
        assert err < BF16_TOL, (key, err)


def ix_tok(ref, cfg):
    return ref["index"]["row_src"] // cfg.k


FULL = ["qwen3_30b", "skew_zipf", "qwen3_235b_ep8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity_sampled(name):
    cfg = wl.CONFIGS[name]
    print(f"[parity-full] {name}", flush=True)
    inp = inputs(cfg)
    out = run_layer(cfg, inp)
    idx, w = om.route_topk(inp["logits"], cfg.k, cfg.renorm)
    assert np.array_equal(out["topk_idx"], idx)
    assert rel(out["topk_w"], w) < W_TOL
    ix = om.build_index(idx, cfg.e_begin, cfg.e_local)
    ref = {"topk_idx": idx, "index": ix}
    _check_ints(cfg, out, ref)
    assert int(ix["counts"].sum()) == int(out["offsets"][-1])
    rng = np.random.default_rng(123)
    toks = np.sort(rng.choice(cfg.T, size=96, replace=False))
    s = om.token_sample(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, toks)
    for key in ("y", "dx", "d_topk_w"):
        err = rel(out[key][toks], s[key])
        assert err < BF16_TOL, (key, err)
    # the router backward on the GPU's own d_topk_w (the kernel alone, fp32) and on the
    # oracle's d_topk_w (the whole chain)
    dl = om.router_backward(inp["logits"][toks], idx[toks], w[toks], out["d_topk_w"][toks], cfg.renorm)
    assert rel(out["d_logits"][toks], dl) < 1e-5
    dl_chain = om.router_backward(inp["logits"][toks], idx[toks], w[toks], s["d_topk_w"], cfg.renorm)
    err = rel(out["d_logits"][toks], dl_chain)
    assert err < BF16_TOL, ("d_logits", err)
    counts = ix["counts"]
    experts = sorted({int(np.argmax(counts)), int(np.argmin(counts)), int(rng.integers(cfg.e_local))})
    es = om.expert_sample(inp, cfg.k, ix, w, experts)
    for e, (dwg, dwu, dwd) in es.items():
        for key, refv in (("dw_gate", dwg), ("dw_up", dwu), ("dw_down", dwd)):
            if counts[e] == 0:
                assert not out[key][e].any(), (key, e)
            else:
                err = rel(out[key][e], refv)
                assert err < BF16_TOL, (key, e, int(counts[e]), err)


def test_round_trip_gather_combine_is_exact():
    """Dispatch-gather then an unweighted combine of the gathered rows gives
    bf16(n_t * x[t]) bit for bit (n_t = local slots of token t)."""
    from combine_top_router_amd.layer import MoeLayer
    import combine_top_router_amd.lib as L
    cfg = wl.CONFIGS["qwen3_30b"].replace(e_begin=40, e_local=50)
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    layer = MoeLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local, L.MOE_BF16, fuse_gather=False)
    x = torch.from_numpy(inp["x"]).cuda().to(torch.bfloat16)
    layer.route(torch.from_numpy(inp["logits"]).cuda())
    layer.dispatch(x)
    L.moe_combine(layer.shape, layer.xp.data_ptr(), layer.row_of.data_ptr(), layer.y.data_ptr(),
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    R = int(layer.offsets[-1].item())
    row_of = layer.row_of.cpu().numpy().reshape(cfg.T, cfg.k)
    n = (row_of >= 0).sum(axis=1).astype(np.float32)
    expect = wl.bf16_round(n[:, None] * inp["x"])
    assert np.array_equal(layer.y.float().cpu().numpy(), expect)
    xp = layer.xp[:R].float().cpu().numpy()
    src = layer.row_src[:R].cpu().numpy()
    assert np.array_equal(xp, inp["x"][src // cfg.k])


def test_power_of_two_weight_scaling_is_exact():
    cfg = SMALL["ragged_bf16"]
    inp = inputs(cfg)
    a = run_layer(cfg, inp)
    b = run_layer(cfg, inp, scale_up=2.0)
    assert np.array_equal(b["y"], 2 * a["y"])
    assert np.array_equal(b["dw_gate"], 2 * a["dw_gate"])


def test_deterministic_across_runs():
    cfg = SMALL["ragged_bf16_share"]
    inp = inputs(cfg)
    a = run_layer(cfg, inp)
    b = run_layer(cfg, inp)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


ROW_TILE = {
    "tall_bf16_share": SMALL["tall_bf16_share"],
    "ragged_bf16": SMALL["ragged_bf16"],
    # fp8_bwd: only the gate/up and down GEMMs are bf16 row-tiled ones
    "tall_fp8bwd": wl.MoeConfig("tall_fp8bwd", 1280, 256, 256, 8, 2, 0, 8, 21, bwd="mxfp8"),
}


@pytest.mark.parametrize("name", list(ROW_TILE))
def test_row_tile_height_does_not_change_results(name):
    # the 256- and 320-row builds run each output's K loop in the same order, so every
    # output agrees bit for bit whichever height the bf16 row-tiled GEMMs take
    cfg = ROW_TILE[name]
    inp = inputs(cfg)
    print(f"[row_tile] {name}", flush=True)
    a = run_layer(cfg.replace(row_tile=256), inp)
    b = run_layer(cfg.replace(row_tile=320), inp)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_empty_expert_and_no_tokens():
    cfg = wl.CONFIGS["tiny_bf16"]
    inp = dict(inputs(cfg))
    inp["logits"] = inp["logits"].copy()
    inp["logits"][:, 5] = -1e4
    out = run_layer(cfg, inp)
    assert out["counts"][5] == 0
    assert not out["dw_gate"][5].any() and not out["dw_up"][5].any() and not out["dw_down"][5].any()
    ref = oracle_full(cfg, inp)
    for key in ("y", "dx", "dw_gate", "dw_down", "d_logits"):
        assert rel(out[key], ref[key]) < BF16_TOL, key
    cfg0 = cfg.replace(T=0)
    inp0 = {k_: (v[:0] if k_ in ("logits", "x", "dy") else v) for k_, v in inp.items()}
    out0 = run_layer(cfg0, inp0)
    assert out0["y"].shape == (0, cfg.H)
    assert not out0["dw_gate"].any() and not out0["dw_down"].any()
    assert not out0["counts"].any() and not out0["offsets"].any()


# Degenerate and boundary shapes of the method: a single expert choice (k = 1), every
# expert chosen (k = E, where renorm = 1 equals the full softmax), one expert in all,
# one local expert, the largest k, the full-softmax weights in bf16, the smallest H and I
# the bf16 path takes (64) and an I that leaves a 64-column tail in every 256-wide tile.
EDGE = {
    "k1": wl.MoeConfig("k1", 300, 128, 64, 4, 1, 0, 4, 21),
    "k_eq_E": wl.MoeConfig("k_eq_E", 200, 192, 128, 4, 4, 0, 4, 22),
    "one_expert": wl.MoeConfig("one_expert", 150, 64, 64, 1, 1, 0, 1, 23),
    "one_local": wl.MoeConfig("one_local", 256, 128, 192, 16, 4, 7, 1, 24),
    "k16": wl.MoeConfig("k16", 64, 128, 64, 32, 16, 0, 32, 25),
    "renorm0_bf16": wl.MoeConfig("renorm0_bf16", 256, 128, 128, 8, 3, 2, 5, 26, renorm=0),
    "tail_cols": wl.MoeConfig("tail_cols", 333, 320, 320, 6, 2, 0, 6, 27),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_shapes(name):
    cfg = EDGE[name]
    print(f"[parity-edge] {name}", flush=True)
    inp = inputs(cfg)
    out = run_layer(cfg, inp)
    ref = oracle_full(cfg, inp)
    _check_ints(cfg, out, ref)
    assert int(out["counts"].sum()) == int(out["offsets"][-1])
    assert rel(out["topk_w"], ref["topk_w"]) < W_TOL
    t = tol(cfg)
    for key in ("y", "dx", "dw_gate", "dw_up", "dw_down", "d_topk_w", "d_logits"):
        err = rel(out[key], ref[key])
        assert err < t, (key, err)
    if cfg.k == cfg.E:
        # every token reaches every expert: the counts are T, the weights sum to one
        assert np.all(out["counts"] == cfg.T)
        assert np.allclose(out["topk_w"].sum(axis=1), 1.0, atol=1e-5)


def _random_configs(n, seed=2024):
    """Seeded random small layers across the shape space the bf16 path accepts: H and I
    multiples of 64, any E up to 40 with k <= min(E, 16), a random local expert range,
    both weight modes; sized so the oracle finishes each in a few seconds."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(E, 16) + 1))
        el = int(rng.integers(1, E + 1))
        eb = int(rng.integers(0, E - el + 1))
        H = 64 * int(rng.integers(1, 7))
        I = 64 * int(rng.integers(1, 7))
        T = int(rng.integers(1, 400))
        out.append(wl.MoeConfig(f"rand{i}", T, H, I, E, k, eb, el, 100 + i, renorm=int(rng.integers(0, 2))))
    return out


RANDOM = {c.name: c for c in _random_configs(10)}


@pytest.mark.parametrize("name", list(RANDOM))
def test_random_shapes(name):
    cfg = RANDOM[name]
    print(f"[parity-random] {cfg}", flush=True)
    inp = inputs(cfg)
    out = run_layer(cfg, inp)
    ref = oracle_full(cfg, inp)
    _check_ints(cfg, out, ref)
    assert rel(out["topk_w"], ref["topk_w"]) < W_TOL
    for key in ("y", "dx", "dw_gate", "dw_up", "dw_down", "d_topk_w", "d_logits"):
        err = rel(out[key], ref[key])
        assert err < BF16_TOL, (key, err)


def test_repeated_ids_stay_within_r_cap():
    """A token's k ids must be distinct; if they repeat a local expert while e_local < k,
    the dispatch keeps the first R_cap rows of the expert-major order and gives the later
    slots no row.  Every token here picks experts [0, 0, 1, 1] of the local pair, so
    expert 0 alone fills R_cap = 2T rows: counts [2T, 0], offsets stop at R_cap, expert 1's
    slots get row_of = -1, and nothing is written past R_cap (guard entries untouched)."""
    import combine_top_router_amd.lib as L
    T, H, E, k = 64, 128, 8, 4
    s = L.MoeShape(T, H, 64, E, k, 0, 2, L.MOE_BF16, 0, 1, 0, 0)
    R_cap, G = T * 2, 256
    dev = "cuda"
    topk = torch.tensor([[0, 0, 1, 1]] * T, dtype=torch.int32, device=dev)
    x = torch.randn(T, H, device=dev).to(torch.bfloat16)
    counts = torch.full((2,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((3,), -7, dtype=torch.int32, device=dev)
    row_src = torch.full((R_cap + G,), -7, dtype=torch.int32, device=dev)
    row_of = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    xp = torch.full((R_cap + 8, H), 5.0, dtype=torch.bfloat16, device=dev)
    _, scratch_b = L.moe_workspace_bytes(s)
    scratch = torch.empty(max(scratch_b, 256), dtype=torch.uint8, device=dev)
    L.moe_dispatch(s, topk.data_ptr(), x.data_ptr(), counts.data_ptr(), offsets.data_ptr(), row_src.data_ptr(),
                   row_of.data_ptr(), xp.data_ptr(), scratch.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    slots = np.arange(T * k).reshape(T, k)
    assert counts.cpu().tolist() == [R_cap, 0]
    assert offsets.cpu().tolist() == [0, R_cap, R_cap]
    assert np.array_equal(row_src[:R_cap].cpu().numpy(), slots[:, :2].reshape(-1))
    assert np.all(row_src[R_cap:].cpu().numpy() == -7)
    ro = row_of.cpu().numpy().reshape(T, k)
    assert np.array_equal(ro[:, :2].reshape(-1), np.arange(R_cap)) and np.all(ro[:, 2:] == -1)
    assert torch.equal(xp[:R_cap], x.repeat_interleave(2, dim=0))
    assert torch.all(xp[R_cap:] == 5.0)
