"""The layer's forward + backward captured as one HIP graph and replayed.

Every call of the path launches kernels only (no allocation, copy or host wait), so the
whole step can be captured.  Each replay, with unrelated eager work and a host
synchronisation between replays, must reproduce the eager outputs bit for bit (the
kernels are deterministic)."""
import numpy as np
import pytest

import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import inputs, to_dev  # noqa: E402

CASES = {
    "tiny_bf16": wl.CONFIGS["tiny_bf16"],
    "ragged_bf16_share": wl.MoeConfig("ragged_bf16_share", 700, 192, 320, 10, 3, 4, 5, 6),
    "ragged_mx": wl.MoeConfig("ragged_mx", 700, 256, 192, 6, 2, 0, 6, 8, bwd="mxfp8"),
    "ragged_mxfp8": wl.MoeConfig("ragged_mxfp8", 700, 256, 256, 6, 2, 0, 6, 8, bwd="mxfp8", fwd="mxfp8"),
    "tiny_f32": wl.CONFIGS["tiny_f32"],
    # activation checkpointing: the backward's recompute of G|U and A is captured too
    "ragged_bf16_share_recompute": wl.MoeConfig("ragged_bf16_share", 700, 192, 320, 10, 3, 4, 5, 6),
    "ragged_mxfp8_recompute": wl.MoeConfig("ragged_mxfp8", 700, 256, 256, 6, 2, 0, 6, 8, bwd="mxfp8", fwd="mxfp8"),
    # Zipf-skewed loads: the weight gradients take their tiles from a device counter that the
    # tile table zeroes, so every replay must start the greedy schedule afresh
    "skew_bf16_dynamic": wl.MoeConfig("skew_bf16", 1024, 512, 384, 64, 4, 0, 64, 10, routing="zipf"),
    "skew_mx_dynamic": wl.MoeConfig("skew_mx", 1024, 512, 384, 64, 4, 0, 64, 10, routing="zipf", bwd="mxfp8"),
}


def _schedules_dynamically(counts):
    """Whether the tile table picks the greedy weight-gradient schedule for these expert
    loads: an expert costing over twice the mean, or one of the 8 contiguous expert ranges
    over 2 % above their mean (cost = max(ceil(rows / 64), 3) + 2 K steps per tile)."""
    El = len(counts)
    cost = [max((int(c) + 63) // 64, 3) + 2 for c in counts]
    tot = sum(cost)
    xsum = [0] * 8
    for e, c in enumerate(cost):
        xsum[e * 8 // El] += c
    return max(cost) * El > 2 * tot or max(xsum) * 8 * 50 > tot * 51


def _outputs(layer, y, g):
    out = {"y": y.clone(), "topk_idx": layer.topk_idx.clone(), "row_src": layer.row_src.clone()}
    for k, v in g.items():
        out[k] = v.clone()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    from combine_top_router_amd.layer import MoeLayer
    import combine_top_router_amd.lib as L
    cfg = CASES[name]
    print(f"[graph] {name}", flush=True)
    inp = inputs(cfg)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    layer = MoeLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local,
                     L.MOE_F32 if cfg.dtype == "f32" else L.MOE_BF16,
                     L.MOE_BWD_MXFP8 if cfg.bwd == "mxfp8" else L.MOE_BWD_SAME, cfg.renorm,
                     fwd=L.MOE_FWD_MXFP8 if cfg.fwd == "mxfp8" else L.MOE_FWD_SAME,
                     recompute=int(name.endswith("_recompute")))
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"])).cuda()
    x, wg, wu, wd, dy = (to_dev(inp[k], dt) for k in ("x", "w_gate", "w_up", "w_down", "dy"))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y = layer.forward(logits, x, wg, wu, wd)
        g = layer.backward(dy)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = _outputs(layer, y, g)
    if name.endswith("_dynamic"):
        assert _schedules_dynamically(layer.counts.cpu().numpy()), "the case must exercise the greedy schedule"

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(logits, x, wg, wu, wd)
        layer.backward(dy)
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        # clobber every output, then replay
        for t in (layer.y, layer.dx, layer.dw_gate, layer.dw_up, layer.dw_down, layer.d_topk_w, layer.d_logits):
            t.fill_(7)
        junk.add_(1.0)                 # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(layer, layer.y, {"dx": layer.dx, "dw_gate": layer.dw_gate, "dw_up": layer.dw_up,
                                        "dw_down": layer.dw_down, "d_topk_w": layer.d_topk_w,
                                        "d_logits": layer.d_logits})
        for k, v in ref.items():
            assert torch.equal(got[k], v), (name, rep, k)
    del graph, layer
    torch.cuda.empty_cache()
