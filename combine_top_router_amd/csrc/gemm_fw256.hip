// Every GEMM of the layer on the fused stream of the GEMM engine with 256-row tiles
// (eight waves that each load one eighth of every operand step and compute a 128 x 64
// sub-tile): the bf16 row-tiled GEMMs of 256 rows, the weight gradients and all MXFP8
// GEMMs, and the host-side launch order of the forward and backward passes.  The
// kernels are those of gemm.hip.
#define MOE_GEMM_FW 256
#include "gemm.hip"
