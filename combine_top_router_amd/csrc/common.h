// Internal helpers shared by the HIP kernels and the host entry points of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bits

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define MOE_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair (lo in bits 0..15), round to nearest even, with
// gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// x / k for 0 <= x < 2^31 and 1 <= k <= 16, given inv_k = 1.0 / k: (x + 1/2) / k lies at
// least 1 / (2k) from an integer, far more than the double product's rounding error
// (below 2^-20 here), so truncating it gives the exact quotient in three instructions.
__device__ __forceinline__ int div_k(int x, double inv_k) { return (int)(((double)x + 0.5) * inv_k); }

template <typename T> struct elem;
template <> struct elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
template <> struct elem<bf16_t> {
  __device__ static float load(const bf16_t* p) { return bf2f(*p); }
  __device__ static void store(bf16_t* p, float v) { *p = f2bf(v); }
};

// logistic function with the hardware reciprocal (v_rcp_f32, 1 ulp): exp(-g) = inf gives 0
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

// MX scale exponent of a 32-element block with absolute maximum amax (E4M3 elements,
// e8m0 scale 2^X): the smallest X with amax <= 448 * 2^X, clamped to [-127, 127]; 0 for
// an all-zero block.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float m = frexpf(amax, &e);    // amax = m * 2^e, m in [0.5, 1)
  // amax in [2^(e-1), 2^e): X = e - 9, plus one if amax > 1.75 * 2^(e-1) = 448 * 2^(e-9)
  int X = e - 9 + (m > 0.875f ? 1 : 0);
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// E4M3 codes of x0..x3 * 2^-X packed little-endian (|x * 2^-X| <= 448 by the scale
// rule).  The scaling by a power of two is exact; gfx950's v_cvt_pk_fp8_f32 converts to
// the OCP E4M3 format rounding to nearest, ties to even (the default mode), with the
// sign of the input, also for results that round to zero.
__device__ __forceinline__ uint32_t e4m3_pack4(float x0, float x1, float x2, float x3, int X) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x0, -X), ldexpf(x1, -X), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x2, -X), ldexpf(x3, -X), lo, true);
}

// Host-side: the launch configuration constants shared by the host code and kernels.
constexpr int kGemmBMMx = 256;  // rows of one row-group tile of the MXFP8 row-tiled GEMMs
constexpr int kZeroBytes = 512;  // zeroed scratch area read in place of rows past a group's end
// (token, slot) pairs per histogram chunk of the dispatch index: at least 1024, a
// multiple of 256, and few enough chunks (<= 256 and <= 32768 / El) that every
// workgroup can read the whole chunk-by-expert histogram
inline int index_chunk(int64_t TK, int El) {
  int64_t nmax = 32768 / El;
  if (nmax > 256) nmax = 256;
  if (nmax < 1) nmax = 1;
  int64_t c = (TK + nmax - 1) / nmax;
  c = (c + 255) / 256 * 256;
  return (int)(c < 1024 ? 1024 : c);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// moe_dispatch_noscratch: the size of its static chunk-histogram buffer (int32 entries),
// and the device address of the current GPU's copy
constexpr int kStaticHistInts = 32768;
hipError_t static_hist_scratch(int32_t** out);

// Opt-in per-kernel timing of the calling host thread (moe_timing_enable): a pair of
// HIP events handed to hipExtLaunchKernel, which stamps them with the dispatch's own
// start and end; with timing off (and always under graph capture) the plain launch.
bool ktimer_pair(const char* name, hipStream_t st, hipEvent_t* start, hipEvent_t* stop);
#define MOE_LAUNCH(name, kernel, grid, block, shmem, st, ...)                               \
  do {                                                                                      \
    hipEvent_t moe_e0_, moe_e1_;                                                            \
    if (::moe::ktimer_pair(name, st, &moe_e0_, &moe_e1_))                                   \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, moe_e0_, moe_e1_, 0, __VA_ARGS__); \
    else                                                                                    \
      hipLaunchKernelGGL(kernel, grid, block, shmem, st, __VA_ARGS__);                      \
  } while (0)

// ---- launch wrappers (defined in the .hip files) ----
hipError_t launch_route_topk(const moe_shape& s, const float* logits, int32_t* idx, float* w,
                             hipStream_t st);
hipError_t launch_route_bwd(const moe_shape& s, const float* logits, const int32_t* idx,
                            const float* w, const float* dw, float* dlogits, hipStream_t st);
hipError_t launch_index(const moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                        int32_t* row_src, int32_t* row_of, int32_t* chunk_hist, hipStream_t st);
hipError_t launch_tile_table(const moe_shape& s, const int32_t* offsets, int bm, int32_t* tiles,
                             int32_t* zeros, int32_t* order, hipStream_t st, int bm2 = 0,
                             int32_t* tiles2 = nullptr);
hipError_t launch_gather(const moe_shape& s, const void* x, const int32_t* offsets,
                         const int32_t* row_src, void* xp, hipStream_t st);
// bf16 with part != null: also d_topk_w from the partial row-dots (the dX combine)
hipError_t launch_combine(const moe_shape& s, const void* rows, const int32_t* row_of, void* out,
                          hipStream_t st, const char* name = "combine", const float* part = nullptr,
                          int nparts = 0, float* d_topk_w = nullptr);
// router GEMM (router_gemm.hip): wt = W_r^T scratch [E, H]; part = fp32 partial dW_r
// [router_dw_slices(T, H, E), H, E]
int router_dw_slices(int T, int H, int E);
hipError_t launch_router_fwd(const moe_shape& s, const bf16_t* x, const bf16_t* w, bf16_t* wt, float* logits,
                             hipStream_t st);
hipError_t launch_router_bwd(const moe_shape& s, const bf16_t* x, const bf16_t* w, const float* dl,
                             const bf16_t* dx_in, bf16_t* dx, bf16_t* dw, float* part, hipStream_t st);
hipError_t launch_dtopk(const moe_shape& s, const float* dw_part, int nparts, const int32_t* row_of,
                        float* d_topk_w, hipStream_t st);

// bf16 MFMA grouped GEMMs
struct FwdArgs {
  int T, H, I, k, El;
  const bf16_t* x;        // [T, H]
  const bf16_t* xp;       // [R_cap, H] or null (gather through row_src)
  const int32_t* offsets; // [El + 1]
  const int32_t* row_src; // [R_cap]
  const float* topk_w;    // [T, k]
  const bf16_t* wg;       // [El, H, I]
  const bf16_t* wu;
  const bf16_t* wd;       // [El, I, H]
  const int32_t* tiles;   // row-group tile table
  int max_tiles;
  bf16_t* gu;             // [R_cap, 2I]  (g | u), or null: not kept
  bf16_t* a;              // [R_cap, I]
  bf16_t* yp;             // [R_cap, H]
  // fp8_bwd: the row-wise MXFP8 codes of the weights for the backward, written by the
  // GEMM that streams them (null: not written).  Gate/up: [W_gate | W_up] along I,
  // [El*H, 2I] codes and [El*H, 2I/32] scales; down: W_down along H, [El*I, H] and
  // [El*I, H/32].  Only experts with rows get codes.
  uint8_t* q_wrows;
  uint8_t* s_wrows;
};
// The bf16 forward GEMMs on the fused stream, one build per tile height (a.tiles holds
// tiles of that height): 256 rows (gemm_fw256.hip) or 320 rows (gemm_fw320.hip).
namespace fw256 {
hipError_t launch_fwd_gateup_bf16(const FwdArgs& a, hipStream_t st);  // K1
hipError_t launch_fwd_down_bf16(const FwdArgs& a, hipStream_t st);    // K2
}  // namespace fw256
namespace fw320 {
hipError_t launch_fwd_gateup_bf16(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_down_bf16(const FwdArgs& a, hipStream_t st);
}  // namespace fw320
// compute units the GEMMs' persistent grids are sized for
int gemm_cus();

struct BwdArgs {
  int T, H, I, k, El;
  const bf16_t* dy;       // [T, H]
  const bf16_t* x;
  const bf16_t* xp;       // or null
  const int32_t* offsets;
  const int32_t* row_src;
  const float* topk_w;
  const bf16_t* wg;
  const bf16_t* wu;
  const bf16_t* wd;
  const bf16_t* gu;       // saved
  const bf16_t* a;        // saved
  const int32_t* tiles;   // 256-row tiles (kGemmBMMx: the MXFP8 B1 and B3; bf16 ones of 256 rows)
  const int32_t* tiles320;// 320-row tiles (bf16 B1 or B3 of 320 rows), same entry bound
  int max_tiles;
  int bm_da, bm_dx;       // tile heights of the bf16 B1 and B3: 256 or 320
  bf16_t* dgu;            // scratch [R_cap, 2I]
  bf16_t* dxp;            // scratch [R_cap, H]
  float* dw_part;         // scratch [R_cap, nparts]
  bf16_t* aw;             // scratch [R_cap, I]: w * A
  const bf16_t* zeros;    // scratch: kZeroBytes of zeros
  int32_t* order;         // scratch [El + 3]: the weight-gradient GEMMs' expert order, its dynamic
                          // flag and their two item counters (written by k_tile_table)
  bf16_t* dwg;            // [El, H, I]
  bf16_t* dwu;
  bf16_t* dwd;            // [El, I, H]
};
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st);
// B1 alone and B3 alone on the fused stream, each build on the table of its height; the
// weight gradients on the 256-row build
namespace fw256 {
hipError_t launch_bwd_da_bf16(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dx_bf16(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dwd_bf16(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dwgu_bf16(const BwdArgs& a, hipStream_t st);
}  // namespace fw256
namespace fw320 {
hipError_t launch_bwd_da_bf16(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dx_bf16(const BwdArgs& a, hipStream_t st);
}  // namespace fw320
// column parts of the B1 row-dot partials per row (dw_part is [R_cap, nparts])
int bwd_bf16_nparts(int I);

// MXFP8 backward: E4M3 values with one e8m0 scale per 32 along each GEMM's contraction
// axis.  Row-wise buffers are [rows, K] codes + [rows, K/32] scales; column-wise ones
// are stored transposed, [N, Rp] codes + [N, Rp/32] scales, over a padded row space in
// which every expert's rows start at poff[e], a multiple of kMxRowPad.
constexpr int kMxRowPad = 128;
struct MxArgs {
  uint8_t* q_dy; uint8_t* s_dy;      // row-wise dY' (gathered dY rows)   [R_cap, H]
  uint8_t* q_wd; uint8_t* s_wd;      // row-wise W_down along H           [El*I, H]
  uint8_t* q_dgu; uint8_t* s_dgu;    // row-wise dG|dU along I            [R_cap, 2I]
  uint8_t* q_wg; uint8_t* s_wg;      // row-wise [W_gate | W_up] along I  [El*H, 2I]
  uint8_t* qt_a; uint8_t* st_a;      // column-wise A, transposed         [I, Rp]
  uint8_t* qt_dy; uint8_t* st_dy;    // column-wise w * dY', transposed   [H, Rp]
  uint8_t* qt_x; uint8_t* st_x;      // column-wise Xp, transposed        [H, Rp]
  uint8_t* qt_dgu; uint8_t* st_dgu;  // column-wise dG|dU, transposed     [2I, Rp]
  int32_t* poff;                     // [El + 1] padded row offsets
  int Rp;                            // padded row capacity (multiple of kMxRowPad)
  int64_t R_cap;                     // row capacity of the row-wise activation buffers
  bool w_ready;                      // q_wd / q_wg hold the weights' codes (written by the forward)
};
inline int64_t mx_rp_cap(int64_t R_cap, int El) { return ceil_div(R_cap + (int64_t)(kMxRowPad - 1) * El, kMxRowPad) * kMxRowPad; }

// row-wise quantization of rows of K codes (K % 32 == 0).  rows >= 0 and no gather: a
// fixed count; otherwise the count is offsets[El] (device-resident) and rows_bound an
// upper bound.  With row_src, row r reads source row row_src[r] / k; with src2, the
// last K / 2 columns of row r come from src2 (two matrices side by side).
hipError_t launch_mx_rows(const bf16_t* src, const bf16_t* src2, int ld, const int32_t* row_src, int k,
                          const int32_t* offsets, int El, int64_t rows, int64_t rows_bound, int K, uint8_t* q,
                          uint8_t* s, const char* name, hipStream_t st);
// column-wise, group-aware quantization into the padded transposed layout; optional row
// gather (row_src / k) and per-row scaling by topk_w[row_src[r]]; with qr, also the
// row-wise quantization of the same (gathered, unscaled) rows into qr [rows, ldr], sr
// [rows, ldr / 32] (ldr <= 0: ldr = N)
hipError_t launch_mx_cols(const bf16_t* src, int ld, const int32_t* row_src, int k, const float* topk_w,
                          const int32_t* offsets, const int32_t* poff, int El, int N, int Rp, uint8_t* qt,
                          uint8_t* stt, const char* name, hipStream_t st, uint8_t* qr = nullptr,
                          uint8_t* sr = nullptr, int ldr = 0);
hipError_t launch_poff(const int32_t* offsets, int El, int32_t* poff, hipStream_t st);
hipError_t launch_bwd_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st);
// out[e] = e * step for e = 0..n (the group offsets of n equal weight matrices)
hipError_t launch_mx_iota(int32_t* out, int n, int step, hipStream_t st);

// MXFP8 forward operands (scratch).  The weights are quantised column-wise into the
// transposed layout of launch_mx_cols with one group per expert: column n of expert e's
// matrix at codes[n * Rp + e * K .. + K - 1] (K = H for W_gate / W_up, I for W_down,
// both multiples of 128, so the groups need no padding and Rp = El * K).
struct MxFwdArgs {
  uint8_t* q_x; uint8_t* s_x;        // row-wise Xp along H               [R_cap, H]
  uint8_t* q_a; uint8_t* s_a;        // row-wise A along I                [R_cap, I]
  uint8_t* qt_wgu; uint8_t* st_wgu;  // column-wise [W_gate | W_up] along H, transposed [2I, El*H]
  uint8_t* qt_wd; uint8_t* st_wd;    // column-wise W_down along I, transposed          [H, El*I]
  int32_t* goff_h;                   // [El + 1]: e * H
  int32_t* goff_i;                   // [El + 1]: e * I
  int64_t R_cap;
  // optional (an MXFP8 backward follows): the same passes also write the backward's
  // row-wise weight codes, W_down along H [El*I, H] and [W_gate | W_up] along I [El*H, 2I]
  uint8_t* q_wd_rows; uint8_t* s_wd_rows;
  uint8_t* q_wgu_rows; uint8_t* s_wgu_rows;
};
// k1_only: the gate/up GEMM and what it needs (the backward's recompute)
hipError_t launch_fwd_mx(const FwdArgs& a, const MxFwdArgs& m, hipStream_t st, bool k1_only = false);
// the MXFP8 row-tiled GEMMs on the 256-row fused stream (a.tiles: kGemmBMMx-row tiles)
namespace fw256 {
hipError_t launch_fwd_gateup_mx(const FwdArgs& a, const MxFwdArgs& m, hipStream_t st);
hipError_t launch_fwd_down_mx(const FwdArgs& a, const MxFwdArgs& m, hipStream_t st);
hipError_t launch_bwd_da_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st);
hipError_t launch_bwd_dx_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st);
hipError_t launch_bwd_dwd_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st);
hipError_t launch_bwd_dwgu_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st);
}  // namespace fw256

// fp32 (SIMT) grouped GEMMs: the same chain in fp32 arithmetic
struct FwdArgsF32 {
  int T, H, I, k, El;
  const float* x; const float* xp; const int32_t* offsets; const int32_t* row_src;
  const float* topk_w; const float* wg; const float* wu; const float* wd;
  const int32_t* tiles; int max_tiles;
  float* gu; float* a; float* yp;
};
hipError_t launch_fwd_f32(const FwdArgsF32& a, hipStream_t st);
struct BwdArgsF32 {
  int T, H, I, k, El;
  const float* dy; const float* x; const float* xp; const int32_t* offsets; const int32_t* row_src;
  const float* topk_w; const float* wg; const float* wu; const float* wd;
  const float* gu; const float* a; const int32_t* tiles; int max_tiles;
  float* dgu; float* dxp; float* dw_part;
  float* dwg; float* dwu; float* dwd;
};
hipError_t launch_bwd_f32(const BwdArgsF32& a, hipStream_t st);

}  // namespace moe
