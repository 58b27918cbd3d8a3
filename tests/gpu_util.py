"""Helpers of the GPU parity tests: run the HIP path through the C ABI on seeded inputs
and compare with the oracle."""
import functools

import numpy as np
import torch

import workloads as wl
from oracle import moe as om

BF16_TOL = 1e-2      # relative Frobenius bound for bf16 outputs and gradients
F32_TOL = 1e-5       # relative Frobenius bound for fp32 runs
W_TOL = 2e-6         # fp32 softmax weights against fp64


def rel(a, b):
    a = np.asarray(a, dtype=np.float64); b = np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


def tol(cfg):
    return F32_TOL if cfg.dtype == "f32" else BF16_TOL


@functools.lru_cache(maxsize=2)
def inputs(cfg):
    return wl.make_inputs(cfg)


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def run_layer(cfg, inp, fuse_gather=True, scale_up=1.0, recompute=0):
    """Forward + backward on the GPU; returns host copies of every output."""
    from combine_top_router_amd.layer import MoeLayer
    import combine_top_router_amd.lib as L
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    layer = MoeLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local,
                     L.MOE_F32 if cfg.dtype == "f32" else L.MOE_BF16,
                     L.MOE_BWD_MXFP8 if cfg.bwd == "mxfp8" else L.MOE_BWD_SAME, cfg.renorm,
                     fuse_gather=fuse_gather, fwd=L.MOE_FWD_MXFP8 if cfg.fwd == "mxfp8" else L.MOE_FWD_SAME,
                     recompute=recompute, row_tile=cfg.row_tile)
    assert (layer.saved is None) == bool(recompute)
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"])).cuda()
    x = to_dev(inp["x"], dt)
    wg = to_dev(inp["w_gate"], dt)
    wu = to_dev(inp["w_up"] * scale_up, dt)
    wd = to_dev(inp["w_down"], dt)
    dy = to_dev(inp["dy"], dt)
    y = layer.forward(logits, x, wg, wu, wd)
    g = layer.backward(dy)
    torch.cuda.synchronize()
    out = {"topk_idx": host(layer.topk_idx), "topk_w": host(layer.topk_w), "counts": host(layer.counts),
           "offsets": host(layer.offsets), "y": host(y)}
    R = int(out["offsets"][-1])
    out["row_src"] = host(layer.row_src)[:R]
    out["row_of"] = host(layer.row_of)[: cfg.T * cfg.k]
    for k_, v in g.items():
        out[k_] = host(v)
    if layer.xp is not None:
        out["xp"] = host(layer.xp)[:R]
    del layer, x, wg, wu, wd, dy, logits
    torch.cuda.empty_cache()
    return out


def oracle_full(cfg, inp):
    idx, w = om.route_topk(inp["logits"], cfg.k, cfg.renorm)
    Y, saved = om.layer_forward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w)
    g = om.layer_backward(inp, cfg.k, cfg.e_begin, cfg.e_local, idx, w, saved)
    g["d_logits"] = om.router_backward(inp["logits"], idx, w, g["d_topk_w"], cfg.renorm)
    g["y"] = Y
    g["topk_idx"], g["topk_w"] = idx, w
    g["index"] = saved["index"]
    return g
