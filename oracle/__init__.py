"""CPU oracle for the dropless MoE layer (test infrastructure).

A plain, slow, obviously correct fp64 implementation of what the layer computes:
top-k softmax routing, the stable expert-major permutation, the per-expert SwiGLU
MLP, the weighted combine, the full backward, the router backward, and the MXFP8
quantize-dequantize used by the MXFP8 backward.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library: it never imports
``combine_top_router_amd`` and the library never imports it.  Inputs come from
``workloads`` (random numbers only).

Method source: the Prime Mega MoE write-ups (Polish, Thai and Spanish pages; the
fused chain "EP dispatch, two expert linear layers, SwiGLU, combine") and NVIDIA's
DeepSeek-V3 MoE article (dropless MoE, grouped GEMM, group-aware MXFP8
quantization, dispatch/combine).  The pages give no formulas; every formula here is
the plainest reading and is listed with its reading in the module docstrings.
"""
from . import moe, mx  # noqa: F401
