"""MI355X-native dropless MoE layer: top-k routing, dispatch, grouped SwiGLU expert MLP
and combine, forward and backward, as hand-written HIP kernels for gfx950 behind the
C ABI of include/moe.h (libmoe.so).

libmoe.so is loaded on first use; every entry point raises ImportError if it has not
been built (``python -m combine_top_router_amd.build``).  There is no fallback path."""
from . import lib
from .lib import *  # noqa: F401,F403

__all__ = list(lib.__all__) + ["MoeLayer"]


def __getattr__(name):
    if name == "MoeLayer":
        from .layer import MoeLayer
        return MoeLayer
    raise AttributeError(name)
