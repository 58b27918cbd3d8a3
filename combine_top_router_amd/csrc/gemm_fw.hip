// The bf16 row-tiled GEMMs (gate/up, down, dA, dX) on the fused stream of the GEMM
// engine: 256 x 256 tiles, eight waves that each load one eighth of every operand step
// and compute a 128 x 64 sub-tile.  The kernels are those of gemm.hip, compiled with
// the engine's fused-stream constants.
#define MOE_GEMM_FW 1
#include "gemm.hip"
