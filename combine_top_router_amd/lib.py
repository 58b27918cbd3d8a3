"""ctypes binding of libmoe.so: the C ABI of include/moe.h, same names, argument
marshalling only.  Pointers are passed as Python ints (device addresses), streams as
ints (a hipStream_t, 0 = the null stream).  A failing call raises MoeError."""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE", "MOE_EHIP",
    "MOE_F32", "MOE_BF16", "MOE_BWD_SAME", "MOE_BWD_MXFP8", "MOE_FWD_SAME", "MOE_FWD_MXFP8",
    "MoeShape", "MoeError", "load", "lib_path", "EXPORTS",
    "moe_abi_version", "moe_last_error", "moe_workspace_bytes", "moe_route_topk",
    "moe_dispatch", "moe_dispatch_noscratch", "moe_fwd", "moe_combine", "moe_bwd", "moe_route_topk_bwd",
    "moe_mx_quantize", "moe_mx_quantize_cols", "moe_timing_enable", "moe_timing_read",
    "moe_router_fwd", "moe_router_bwd",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_BWD_SAME, MOE_BWD_MXFP8 = 0, 1
MOE_FWD_SAME, MOE_FWD_MXFP8 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "I", "E", "k", "e_begin", "e_local", "dtype", "bwd", "renorm", "fwd", "recompute",
                 "row_tile")]

    def __repr__(self):
        return "MoeShape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class MoeError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} failed with status {code}: {msg}")
        self.code = code


_P = ctypes.c_void_p
_S = ctypes.POINTER(MoeShape)
_SIG = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (ctypes.c_int, [_S, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route_topk": (ctypes.c_int, [_S, _P, _P, _P, _P]),
    "moe_dispatch": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_noscratch": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_fwd": (ctypes.c_int, [_S] + [_P] * 12),
    "moe_combine": (ctypes.c_int, [_S, _P, _P, _P, _P]),
    "moe_bwd": (ctypes.c_int, [_S] + [_P] * 18),
    "moe_route_topk_bwd": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
    "moe_mx_quantize": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "moe_mx_quantize_cols": (ctypes.c_int, [_P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P, _P, _P, _P,
                                            _P, _P]),
    "moe_router_fwd": (ctypes.c_int, [_S] + [_P] * 7),
    "moe_router_bwd": (ctypes.c_int, [_S] + [_P] * 8),
    "moe_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "moe_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]),
}
EXPORTS = tuple(_SIG)

_lib = None


def load():
    """Load libmoe.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m combine_top_router_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIG.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int, func: str):
    if rc != MOE_OK:
        raise MoeError(rc, func, moe_last_error())


def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_workspace_bytes(shape: MoeShape):
    saved = ctypes.c_size_t(0)
    scratch = ctypes.c_size_t(0)
    _check(load().moe_workspace_bytes(ctypes.byref(shape), ctypes.byref(saved), ctypes.byref(scratch)),
           "moe_workspace_bytes")
    return saved.value, scratch.value


def moe_route_topk(shape, logits, topk_idx, topk_w, stream=0):
    _check(load().moe_route_topk(ctypes.byref(shape), logits, topk_idx, topk_w, stream), "moe_route_topk")


def moe_dispatch(shape, topk_idx, x, counts, offsets, row_src, row_of, xp, scratch, stream=0):
    _check(load().moe_dispatch(ctypes.byref(shape), topk_idx, x, counts, offsets, row_src, row_of, xp,
                               scratch, stream), "moe_dispatch")


def moe_dispatch_noscratch(shape, topk_idx, x, counts, offsets, row_src, row_of, xp, stream=0):
    _check(load().moe_dispatch_noscratch(ctypes.byref(shape), topk_idx, x, counts, offsets, row_src, row_of, xp,
                                         stream), "moe_dispatch_noscratch")


def moe_fwd(shape, x, xp, offsets, row_src, topk_w, w_gate, w_up, w_down, yp, saved, scratch, stream=0):
    _check(load().moe_fwd(ctypes.byref(shape), x, xp, offsets, row_src, topk_w, w_gate, w_up, w_down, yp,
                          saved, scratch, stream), "moe_fwd")


def moe_combine(shape, yp, row_of, y, stream=0):
    _check(load().moe_combine(ctypes.byref(shape), yp, row_of, y, stream), "moe_combine")


def moe_bwd(shape, dy, x, xp, offsets, row_src, row_of, topk_w, w_gate, w_up, w_down, saved, dx,
            dw_gate, dw_up, dw_down, d_topk_w, scratch, stream=0):
    _check(load().moe_bwd(ctypes.byref(shape), dy, x, xp, offsets, row_src, row_of, topk_w, w_gate, w_up,
                          w_down, saved, dx, dw_gate, dw_up, dw_down, d_topk_w, scratch, stream), "moe_bwd")


def moe_route_topk_bwd(shape, logits, topk_idx, topk_w, d_topk_w, d_logits, stream=0):
    _check(load().moe_route_topk_bwd(ctypes.byref(shape), logits, topk_idx, topk_w, d_topk_w, d_logits, stream),
           "moe_route_topk_bwd")


def moe_mx_quantize(x, rows, K, codes, scales, stream=0):
    _check(load().moe_mx_quantize(x, rows, K, codes, scales, stream), "moe_mx_quantize")


def moe_mx_quantize_cols(x, N, offsets, groups, Rp, poff, codes, scales, row_codes=0, row_scales=0, stream=0):
    _check(load().moe_mx_quantize_cols(x, N, offsets, groups, Rp, poff, codes, scales, row_codes, row_scales,
                                       stream), "moe_mx_quantize_cols")


def moe_router_fwd(shape, x, w_r, logits, topk_idx, topk_w, scratch, stream=0):
    _check(load().moe_router_fwd(ctypes.byref(shape), x, w_r, logits, topk_idx, topk_w, scratch, stream),
           "moe_router_fwd")


def moe_router_bwd(shape, x, w_r, d_logits, dx_in, dx, dw_r, scratch, stream=0):
    _check(load().moe_router_bwd(ctypes.byref(shape), x, w_r, d_logits, dx_in, dx, dw_r, scratch, stream),
           "moe_router_bwd")


def moe_timing_enable(on: bool = True):
    _check(load().moe_timing_enable(1 if on else 0), "moe_timing_enable")


def moe_timing_read(capacity: int = 256):
    """[(kernel name, milliseconds)] of the kernels launched since the last read."""
    names = (ctypes.c_char_p * capacity)()
    ms = (ctypes.c_float * capacity)()
    n = ctypes.c_int(0)
    _check(load().moe_timing_read(capacity, names, ms, ctypes.byref(n)), "moe_timing_read")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n.value, capacity))]
