"""Parity of the router GEMM (moe_router_fwd / moe_router_bwd) with the oracle.

Forward: logits within 1e-5 (relative Frobenius) of the fp64 x W_r (bf16 inputs are
exact, the GPU sums in fp32); the routing is an integer decision taken in fp32, so
topk_idx must equal the oracle's routing applied to the GPU's own fp32 logits, bit for
bit, and the weights match within 2e-6.  Backward: dx (= dx_in + d_logits W_r^T) and
dW_r within 1e-2 of the fp64 results (d_logits enters the bf16 MFMAs rounded to bf16), with dx_in absent,
given, and the same buffer as dx.  Small ragged shapes, the tiny layer, routers over 512 and
1024 experts and the full Qwen3-30B-A3B router (T=4096, H=2048, E=128)."""
import numpy as np
import pytest

import workloads as wl
from oracle import moe as om

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import BF16_TOL, W_TOL, rel, to_dev  # noqa: E402

CASES = {
    "tiny": wl.CONFIGS["tiny_bf16"],
    "ragged": wl.MoeConfig("ragged_router", 700, 192, 64, 40, 3, 0, 40, 21),
    "one_token": wl.MoeConfig("one_token_router", 1, 64, 64, 16, 4, 0, 16, 22),
    # wide routers: E past the 16-lane routing kernel's 256 and at the ABI's 1024
    "wide_512": wl.MoeConfig("wide_router", 100, 128, 64, 512, 8, 0, 512, 23),
    "wide_1024_k16": wl.MoeConfig("wide_router_k16", 50, 64, 64, 1024, 16, 0, 1024, 24, renorm=0),
    "qwen3_30b": wl.CONFIGS["qwen3_30b"],
}


def _shape(cfg):
    import combine_top_router_amd.lib as L
    return L.MoeShape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local, L.MOE_BF16, 0, cfg.renorm, 0, 0)


@pytest.mark.parametrize("name", list(CASES))
def test_router_parity(name):
    import combine_top_router_amd.lib as L
    cfg = CASES[name]
    print(f"[router] {name}", flush=True)
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    w_r = wl.make_router_weight(cfg)
    s = _shape(cfg)
    _, scratch_b = L.moe_workspace_bytes(s)
    dev = "cuda"
    x, w = to_dev(inp["x"], torch.bfloat16), to_dev(w_r, torch.bfloat16)
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    scratch = torch.empty(scratch_b, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    L.moe_router_fwd(s, x.data_ptr(), w.data_ptr(), logits.data_ptr(), idx.data_ptr(), tw.data_ptr(),
                     scratch.data_ptr(), stream)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert rel(lg, om.router_logits(inp["x"], w_r)) < 1e-5
    ridx, rw = om.route_topk(lg, k, cfg.renorm)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert rel(tw.cpu().numpy(), rw) < W_TOL

    rng = np.random.default_rng(cfg.seed + 100)
    dl = rng.standard_normal((T, E)).astype(np.float32)
    dx_in = wl.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    dx_r, dw_ref = om.router_gemm_backward(inp["x"], w_r, dl)
    dlt = torch.from_numpy(dl).to(dev)
    dw = torch.empty(H, E, dtype=torch.bfloat16, device=dev)
    for mode in ("none", "given", "inplace"):
        dx = to_dev(dx_in, torch.bfloat16) if mode == "inplace" else torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        din = to_dev(dx_in, torch.bfloat16) if mode == "given" else (dx if mode == "inplace" else None)
        L.moe_router_bwd(s, x.data_ptr(), w.data_ptr(), dlt.data_ptr(), 0 if din is None else din.data_ptr(),
                         dx.data_ptr(), dw.data_ptr(), scratch.data_ptr(), stream)
        torch.cuda.synchronize()
        want = dx_r if mode == "none" else dx_in + dx_r
        err_dx, err_dw = rel(dx.float().cpu().numpy(), want), rel(dw.float().cpu().numpy(), dw_ref)
        print(f"  {mode}: dx {err_dx:.3e}  dW_r {err_dw:.3e}", flush=True)
        assert err_dx < BF16_TOL and err_dw < BF16_TOL, (mode, err_dx, err_dw)


@pytest.mark.parametrize("name", ["ragged", "wide_512", "qwen3_30b"])
def test_router_end_to_end_from_fp64_logits(name):
    """The whole forward chain against the oracle's: the GPU's top-k ids and weights from
    its own router GEMM against the oracle's routing of the fp64 logits x W_r.  The fp32
    sums carry rounding errors of at most 2^-24 of each partial sum; their total stays
    within b = sqrt(H) 2^-24 sum_h |x_h w_he| (a random walk of H such errors; the test
    checks that the GPU's logits do), so a token whose k-th and (k+1)-th fp64 logits lie
    closer than 2b may legitimately pick either: such tokens are skipped and counted
    (there must be few)."""
    import combine_top_router_amd.lib as L
    cfg = CASES[name]
    print(f"[router-e2e] {name}", flush=True)
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    w_r = wl.make_router_weight(cfg)
    s = _shape(cfg)
    _, scratch_b = L.moe_workspace_bytes(s)
    T, E, k = cfg.T, cfg.E, cfg.k
    x, w = to_dev(inp["x"], torch.bfloat16), to_dev(w_r, torch.bfloat16)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    scratch = torch.empty(scratch_b, dtype=torch.uint8, device="cuda")
    L.moe_router_fwd(s, x.data_ptr(), w.data_ptr(), logits.data_ptr(), idx.data_ptr(), tw.data_ptr(),
                     scratch.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    L64 = om.router_logits(inp["x"], w_r)
    ridx, rw = om.route_topk(L64, k, cfg.renorm)
    bound = np.sqrt(cfg.H) * 2.0 ** -24 * (np.abs(inp["x"].astype(np.float64)) @ np.abs(w_r.astype(np.float64)))
    assert np.all(np.abs(logits.cpu().numpy() - L64) <= bound)
    srt = np.sort(L64, axis=1)[:, ::-1]
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    ok = gap > 2.0 * bound.max(axis=1)
    skipped = int((~ok).sum())
    print(f"  tokens {T}, skipped near ties {skipped}", flush=True)
    assert skipped <= max(2, T // 100)
    gi, gw = idx.cpu().numpy()[ok], tw.cpu().numpy()[ok]
    ri, rwk = ridx[ok], rw[ok]
    # the selected set; within it two slots may swap places where their logits lie within
    # the fp32 error of each other, so weights are compared expert by expert
    og, orf = np.argsort(gi, axis=1), np.argsort(ri, axis=1)
    assert np.array_equal(np.take_along_axis(gi, og, 1), np.take_along_axis(ri, orf, 1))
    assert rel(np.take_along_axis(gw, og, 1), np.take_along_axis(rwk, orf, 1)) < 1e-5


def test_router_no_tokens():
    import combine_top_router_amd.lib as L
    cfg = wl.CONFIGS["tiny_bf16"].replace(T=0)
    s = _shape(cfg)
    _, scratch_b = L.moe_workspace_bytes(s)
    w = to_dev(wl.make_router_weight(cfg), torch.bfloat16)
    scratch = torch.empty(max(scratch_b, 256), dtype=torch.uint8, device="cuda")
    dw = torch.full((cfg.H, cfg.E), 7.0, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    L.moe_router_fwd(s, 0, w.data_ptr(), 0, 0, 0, scratch.data_ptr(), stream)
    L.moe_router_bwd(s, 0, w.data_ptr(), 0, 0, 0, dw.data_ptr(), scratch.data_ptr(), stream)
    torch.cuda.synchronize()
    assert not dw.float().abs().sum().item()


def test_router_graph_replays_match_eager():
    """moe_router_fwd + moe_router_bwd captured as one HIP graph: every replay, with eager
    work and a host wait between replays, reproduces the eager outputs bit for bit."""
    import combine_top_router_amd.lib as L
    cfg = CASES["ragged"]
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    s = _shape(cfg)
    _, scratch_b = L.moe_workspace_bytes(s)
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    x, w = to_dev(inp["x"], torch.bfloat16), to_dev(wl.make_router_weight(cfg), torch.bfloat16)
    dl = torch.from_numpy(np.random.default_rng(5).standard_normal((T, E)).astype(np.float32)).cuda()
    outs = {"logits": torch.empty(T, E, dtype=torch.float32, device="cuda"),
            "idx": torch.empty(T, k, dtype=torch.int32, device="cuda"),
            "w": torch.empty(T, k, dtype=torch.float32, device="cuda"),
            "dx": torch.empty(T, H, dtype=torch.bfloat16, device="cuda"),
            "dw": torch.empty(H, E, dtype=torch.bfloat16, device="cuda")}
    scratch = torch.empty(scratch_b, dtype=torch.uint8, device="cuda")

    def run():
        st = torch.cuda.current_stream().cuda_stream
        L.moe_router_fwd(s, x.data_ptr(), w.data_ptr(), outs["logits"].data_ptr(), outs["idx"].data_ptr(),
                         outs["w"].data_ptr(), scratch.data_ptr(), st)
        L.moe_router_bwd(s, x.data_ptr(), w.data_ptr(), dl.data_ptr(), 0, outs["dx"].data_ptr(),
                         outs["dw"].data_ptr(), scratch.data_ptr(), st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        for t in outs.values():
            t.fill_(3)
        junk.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), (rep, n)

