// The bf16 row-tiled GEMMs (gate/up, down, dA', dX') on the fused stream of the GEMM
// engine with 320-row tiles: eight waves that each load one eighth of every operand step
// and compute a 160 x 64 sub-tile.  The kernels are those of gemm.hip; the layer puts a
// GEMM on this build when its expected tile rounds favour the taller tile.
#define MOE_GEMM_FW 320
#include "gemm.hip"
