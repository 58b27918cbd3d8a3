"""moe_dispatch_noscratch (the dispatch for callers that cannot allocate: its scratch is a
static device buffer) against moe_dispatch with a caller-owned scratch, bit for bit, on
two calls in a row, the second with a smaller input (the static buffer keeps the first
call's histograms, which the second must not see)."""
import numpy as np
import pytest

import workloads as wl
from oracle import moe as om

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dispatch(cfg, noscratch):
    import combine_top_router_amd.lib as L
    s = L.MoeShape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local, L.MOE_BF16, 0, 1, 0, 0)
    inp = wl.make_inputs(cfg, with_weights=False, with_dy=False)
    idx, _ = om.route_topk(inp["logits"], cfg.k)
    dev = "cuda"
    R_cap = cfg.T * min(cfg.k, cfg.e_local)
    topk = torch.from_numpy(idx).to(dev)
    x = torch.from_numpy(inp["x"]).to(dev).to(torch.bfloat16)
    out = {"counts": torch.full((cfg.e_local,), -7, dtype=torch.int32, device=dev),
           "offsets": torch.full((cfg.e_local + 1,), -7, dtype=torch.int32, device=dev),
           "row_src": torch.full((R_cap,), -7, dtype=torch.int32, device=dev),
           "row_of": torch.full((cfg.T * cfg.k,), -7, dtype=torch.int32, device=dev),
           "xp": torch.zeros((R_cap, cfg.H), dtype=torch.bfloat16, device=dev)}
    st = torch.cuda.current_stream().cuda_stream
    p = {n: t.data_ptr() for n, t in out.items()}
    if noscratch:
        L.moe_dispatch_noscratch(s, topk.data_ptr(), x.data_ptr(), p["counts"], p["offsets"], p["row_src"],
                                 p["row_of"], p["xp"], st)
    else:
        _, scratch_b = L.moe_workspace_bytes(s)
        scratch = torch.empty(max(scratch_b, 256), dtype=torch.uint8, device=dev)
        L.moe_dispatch(s, topk.data_ptr(), x.data_ptr(), p["counts"], p["offsets"], p["row_src"], p["row_of"],
                       p["xp"], scratch.data_ptr(), st)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


CASES = [
    # the Qwen3-30B-A3B routing (128 experts, top-8, 4096 tokens), then a smaller local share
    wl.CONFIGS["qwen3_30b"].replace(H=256),
    wl.MoeConfig("noscratch_small", 300, 128, 64, 16, 4, 3, 9, 77),
]


def test_dispatch_noscratch_matches_dispatch_twice():
    for cfg in CASES:
        print(f"[noscratch] {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k} local=[{cfg.e_begin}, +{cfg.e_local})",
              flush=True)
        a = _dispatch(cfg, noscratch=True)
        b = _dispatch(cfg, noscratch=False)
        R = int(b["offsets"][-1])
        for n in ("counts", "offsets", "row_of"):
            assert torch.equal(a[n], b[n]), n
        assert torch.equal(a["row_src"][:R], b["row_src"][:R])
        assert torch.equal(a["xp"][:R], b["xp"][:R])
