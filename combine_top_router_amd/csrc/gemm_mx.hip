// The MXFP8 grouped GEMMs (forward and backward launchers of gemm.hip) compiled with
// one load wave per SIMD: 8 compute + 4 load waves, 168 registers per wave, where the fp8
// kernels' compute side fits without spilling (at 16 waves and 128 registers it spills
// 16-64 bytes per lane).  gemm.hip itself builds the bf16 kernels with two load waves per
// SIMD.
#define MOE_GEMM_MX_TU 1
#include "gemm.hip"
