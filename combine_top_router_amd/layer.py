"""Device buffers of one MoE layer pass, allocated with PyTorch, and the call order of
the C ABI.  Every step runs in libmoe; torch only provides memory and the stream."""
from __future__ import annotations

import torch

from . import lib as L

_DT = {L.MOE_BF16: torch.bfloat16, L.MOE_F32: torch.float32}


def _p(t):
    return 0 if t is None else t.data_ptr()


def stream_handle(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class MoeLayer:
    """One GPU's share of a dropless MoE layer: experts [e_begin, e_begin + e_local) of E.

    ``forward`` runs route -> dispatch -> expert MLP -> combine and ``backward`` runs the
    expert backward and the router backward.  ``recompute=1`` keeps nothing between the two
    (activation checkpointing: the backward recomputes the gate/up GEMM).  With ``fuse_gather`` the token rows are
    read from x through row_src inside the GEMMs instead of a gathered copy xp.
    """

    def __init__(self, T, H, I, E, k, e_begin=0, e_local=None, dtype=L.MOE_BF16, bwd=L.MOE_BWD_SAME,
                 renorm=1, device="cuda", fuse_gather=True, fwd=L.MOE_FWD_SAME, recompute=0, row_tile=0):
        e_local = E if e_local is None else e_local
        self.shape = L.MoeShape(T, H, I, E, k, e_begin, e_local, dtype, bwd, renorm, fwd, recompute, row_tile)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = _DT[dtype]
        saved_b, scratch_b = L.moe_workspace_bytes(self.shape)
        self.R_cap = T * min(k, e_local)
        dev, i32, f32 = self.device, torch.int32, torch.float32
        self.topk_idx = torch.empty(T, k, dtype=i32, device=dev)
        self.topk_w = torch.empty(T, k, dtype=f32, device=dev)
        self.counts = torch.empty(e_local, dtype=i32, device=dev)
        self.offsets = torch.empty(e_local + 1, dtype=i32, device=dev)
        self.row_src = torch.empty(max(self.R_cap, 1), dtype=i32, device=dev)
        self.row_of = torch.empty(max(T * k, 1), dtype=i32, device=dev)
        self.xp = None if fuse_gather else torch.empty(self.R_cap, H, dtype=self.dtype, device=dev)
        self.yp = torch.empty(max(self.R_cap, 1), H, dtype=self.dtype, device=dev)
        self.y = torch.empty(T, H, dtype=self.dtype, device=dev)
        # with recompute nothing is kept between forward and backward: no saved buffer at all
        self.saved = None if recompute else torch.empty(max(saved_b, 256), dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(max(scratch_b, 256), dtype=torch.uint8, device=dev)
        self.dx = torch.empty(T, H, dtype=self.dtype, device=dev)
        self.dw_gate = torch.empty(e_local, H, I, dtype=self.dtype, device=dev)
        self.dw_up = torch.empty(e_local, H, I, dtype=self.dtype, device=dev)
        self.dw_down = torch.empty(e_local, I, H, dtype=self.dtype, device=dev)
        self.d_topk_w = torch.empty(T, k, dtype=f32, device=dev)
        self.d_logits = torch.empty(T, E, dtype=f32, device=dev)
        self.inputs = None

    def _check(self, t, shape, dtype, name):
        if t.device != self.device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {self.device}, got "
                             f"{t.dtype} {tuple(t.shape)} on {t.device}")

    def route(self, logits, stream=None):
        s = self.shape
        self._check(logits, (s.T, s.E), torch.float32, "logits")
        L.moe_route_topk(s, _p(logits), _p(self.topk_idx), _p(self.topk_w), stream_handle(stream))

    def dispatch(self, x, stream=None):
        L.moe_dispatch(self.shape, _p(self.topk_idx), _p(x), _p(self.counts), _p(self.offsets), _p(self.row_src),
                       _p(self.row_of), _p(self.xp), _p(self.scratch), stream_handle(stream))

    def experts(self, x, w_gate, w_up, w_down, stream=None):
        L.moe_fwd(self.shape, _p(x), _p(self.xp), _p(self.offsets), _p(self.row_src), _p(self.topk_w), _p(w_gate),
                  _p(w_up), _p(w_down), _p(self.yp), _p(self.saved), _p(self.scratch), stream_handle(stream))

    def combine(self, stream=None):
        L.moe_combine(self.shape, _p(self.yp), _p(self.row_of), _p(self.y), stream_handle(stream))

    def forward(self, logits, x, w_gate, w_up, w_down, stream=None):
        s = self.shape
        self._check(x, (s.T, s.H), self.dtype, "x")
        self._check(w_gate, (s.e_local, s.H, s.I), self.dtype, "w_gate")
        self._check(w_up, (s.e_local, s.H, s.I), self.dtype, "w_up")
        self._check(w_down, (s.e_local, s.I, s.H), self.dtype, "w_down")
        self.inputs = (logits, x, w_gate, w_up, w_down)
        self.route(logits, stream)
        self.dispatch(x, stream)
        self.experts(x, w_gate, w_up, w_down, stream)
        self.combine(stream)
        return self.y

    def backward(self, dy, stream=None):
        s = self.shape
        self._check(dy, (s.T, s.H), self.dtype, "dy")
        logits, x, w_gate, w_up, w_down = self.inputs
        h = stream_handle(stream)
        L.moe_bwd(s, _p(dy), _p(x), _p(self.xp), _p(self.offsets), _p(self.row_src), _p(self.row_of),
                  _p(self.topk_w), _p(w_gate), _p(w_up), _p(w_down), _p(self.saved), _p(self.dx),
                  _p(self.dw_gate), _p(self.dw_up), _p(self.dw_down), _p(self.d_topk_w), _p(self.scratch), h)
        L.moe_route_topk_bwd(s, _p(logits), _p(self.topk_idx), _p(self.topk_w), _p(self.d_topk_w),
                             _p(self.d_logits), h)
        return {"dx": self.dx, "dw_gate": self.dw_gate, "dw_up": self.dw_up, "dw_down": self.dw_down,
                "d_topk_w": self.d_topk_w, "d_logits": self.d_logits}
