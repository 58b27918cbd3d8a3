"""Opt-in per-kernel timing: records every kernel of an eager step, none under capture,
and leaves the results unchanged."""
import numpy as np
import pytest

import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import inputs, to_dev  # noqa: E402


def _layer_and_inputs(cfg):
    from combine_top_router_amd.layer import MoeLayer
    import combine_top_router_amd.lib as L
    inp = inputs(cfg)
    layer = MoeLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local, L.MOE_BF16, L.MOE_BWD_SAME,
                     cfg.renorm)
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"])).cuda()
    args = [logits] + [to_dev(inp[k], torch.bfloat16) for k in ("x", "w_gate", "w_up", "w_down")]
    return layer, args, to_dev(inp["dy"], torch.bfloat16)


def test_timing_records_each_kernel_and_not_under_capture():
    import combine_top_router_amd.lib as L
    cfg = wl.MoeConfig("timing", 700, 192, 320, 10, 3, 0, 10, 6)
    print("[timing] eager step, then capture", flush=True)
    layer, args, dy = _layer_and_inputs(cfg)
    y0 = layer.forward(*args).clone()
    dx0 = layer.backward(dy)["dx"].clone()
    torch.cuda.synchronize()

    L.moe_timing_enable(True)
    try:
        y = layer.forward(*args)
        dx = layer.backward(dy)["dx"]
        recs = L.moe_timing_read()
        names = [n for n, _ in recs]
        for n in ("route_topk", "fwd_gateup", "fwd_down", "combine", "bwd_dA", "bwd_dWd", "bwd_dX",
                  "bwd_dWgu", "unpermute_dx", "route_bwd"):
            assert n in names, (n, names)
        assert all(ms > 0 and np.isfinite(ms) for _, ms in recs), recs
        assert torch.equal(y, y0) and torch.equal(dx, dx0)
        assert L.moe_timing_read() == []

        # launches on a capturing stream are captured plainly and leave no record
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer.forward(*args)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        L.moe_timing_read()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            yg = layer.forward(*args)
        assert L.moe_timing_read() == []
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(yg, y0)
    finally:
        L.moe_timing_enable(False)
