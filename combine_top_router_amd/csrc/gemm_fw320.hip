// The bf16 gate/up, down and dX GEMMs on the fused stream of the GEMM engine with
// 320-row tiles: eight waves that each load one eighth of every operand step and compute
// a 160 x 64 sub-tile.  The kernels are those of gemm.hip, compiled with the engine's
// fused-stream constants; the layer takes this build when the experts' expected row
// counts pad least to multiples of 320.
#define MOE_GEMM_FW 320
#include "gemm.hip"
