// fp32 grouped GEMMs of the expert MLP (one thread per output element).
//
// The same chain as the bf16 MFMA kernels -- gate/up + SwiGLU, down * routing weight,
// dA' with the SwiGLU backward, dX, dW_down, dW_gate/dW_up -- in fp32 arithmetic with
// fp32 storage.  Meant for fp32 runs of small layers; the hot path is bf16.
#include "common.h"

namespace moe {

namespace {

// expert of row r: the last e with offsets[e] <= r (empty experts are skipped)
__device__ __forceinline__ int expert_of(const int32_t* offsets, int El, int r) {
  int lo = 0, hi = El - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void k_f32_gateup(FwdArgsF32 a) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int i = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= a.offsets[a.El] || i >= a.I) return;
  const int e = expert_of(a.offsets, a.El, r);
  const float* xr = a.xp ? a.xp + (size_t)r * a.H : a.x + (size_t)(a.row_src[r] / a.k) * a.H;
  const float* wg = a.wg + (size_t)e * a.H * a.I + i;
  const float* wu = a.wu + (size_t)e * a.H * a.I + i;
  float g = 0.f, u = 0.f;
  for (int h = 0; h < a.H; ++h) {
    g = fmaf(xr[h], wg[(size_t)h * a.I], g);
    u = fmaf(xr[h], wu[(size_t)h * a.I], u);
  }
  a.gu[(size_t)r * 2 * a.I + i] = g;
  a.gu[(size_t)r * 2 * a.I + a.I + i] = u;
  a.a[(size_t)r * a.I + i] = silu_f(g) * u;
}

__global__ __launch_bounds__(256) void k_f32_down(FwdArgsF32 a) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= a.offsets[a.El] || h >= a.H) return;
  const int e = expert_of(a.offsets, a.El, r);
  const float* ar = a.a + (size_t)r * a.I;
  const float* wd = a.wd + (size_t)e * a.I * a.H + h;
  float acc = 0.f;
  for (int i = 0; i < a.I; ++i) acc = fmaf(ar[i], wd[(size_t)i * a.H], acc);
  a.yp[(size_t)r * a.H + h] = a.topk_w[a.row_src[r]] * acc;
}

__global__ __launch_bounds__(256) void k_f32_bwd_da(BwdArgsF32 a) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int i = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= a.offsets[a.El] || i >= a.I) return;
  const int e = expert_of(a.offsets, a.El, r);
  const int src = a.row_src[r];
  const float* dyr = a.dy + (size_t)(src / a.k) * a.H;
  const float* wd = a.wd + ((size_t)e * a.I + i) * a.H;
  float dap = 0.f;
  for (int h = 0; h < a.H; ++h) dap = fmaf(dyr[h], wd[h], dap);
  const size_t I2 = 2 * (size_t)a.I;
  const float g = a.gu[r * I2 + i], u = a.gu[r * I2 + a.I + i];
  const float w = a.topk_w[src];
  a.dw_part[(size_t)r * a.I + i] = dap * a.a[(size_t)r * a.I + i];
  const float da = w * dap;
  const float sg = sigmoid_f(g);
  a.dgu[r * I2 + a.I + i] = da * g * sg;
  a.dgu[r * I2 + i] = da * u * sg * (1.f + g * (1.f - sg));
}

__global__ __launch_bounds__(256) void k_f32_bwd_dx(BwdArgsF32 a) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= a.offsets[a.El] || h >= a.H) return;
  const int e = expert_of(a.offsets, a.El, r);
  const float* dg = a.dgu + (size_t)r * 2 * a.I;
  const float* du = dg + a.I;
  const float* wg = a.wg + ((size_t)e * a.H + h) * a.I;
  const float* wu = a.wu + ((size_t)e * a.H + h) * a.I;
  float acc = 0.f;
  for (int i = 0; i < a.I; ++i) acc = fmaf(dg[i], wg[i], fmaf(du[i], wu[i], acc));
  a.dxp[(size_t)r * a.H + h] = acc;
}

// which = 0: dWd[e][m=i][n=h] = sum_r A[r][i] w_r dY'[r][h];
// which = 1: dWg/dWu[e][m=h][n] = sum_r Xp[r][h] dGU[r][n], n < 2I.
__global__ __launch_bounds__(256) void k_f32_wgrad(BwdArgsF32 a, int which, int M, int N) {
  const int e = blockIdx.z;
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int r0 = a.offsets[e], r1 = a.offsets[e + 1];
  float acc = 0.f;
  for (int r = r0; r < r1; ++r) {
    const int src = a.row_src[r];
    if (which == 0) {
      acc = fmaf(a.a[(size_t)r * a.I + m] * a.topk_w[src], a.dy[(size_t)(src / a.k) * a.H + n], acc);
    } else {
      const float xv = a.xp ? a.xp[(size_t)r * a.H + m] : a.x[(size_t)(src / a.k) * a.H + m];
      acc = fmaf(xv, a.dgu[(size_t)r * 2 * a.I + n], acc);
    }
  }
  if (which == 0) a.dwd[((size_t)e * a.I + m) * a.H + n] = acc;
  else if (n < a.I) a.dwg[((size_t)e * a.H + m) * a.I + n] = acc;
  else a.dwu[((size_t)e * a.H + m) * a.I + (n - a.I)] = acc;
  (void)M;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgsF32& a, hipStream_t st) {
  const int64_t R_cap = (int64_t)a.T * (a.k < a.El ? a.k : a.El);
  if (R_cap == 0) return hipSuccess;
  const unsigned gx = (unsigned)ceil_div(R_cap, 4);
  MOE_LAUNCH("f32_gateup", k_f32_gateup, dim3(gx, (unsigned)ceil_div(a.I, 64)), dim3(256), 0, st, a);
  MOE_LAUNCH("f32_down", k_f32_down, dim3(gx, (unsigned)ceil_div(a.H, 64)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdArgsF32& a, hipStream_t st) {
  const int64_t R_cap = (int64_t)a.T * (a.k < a.El ? a.k : a.El);
  if (R_cap > 0) {
    const unsigned gx = (unsigned)ceil_div(R_cap, 4);
    MOE_LAUNCH("f32_bwd_dA", k_f32_bwd_da, dim3(gx, (unsigned)ceil_div(a.I, 64)), dim3(256), 0, st, a);
    MOE_LAUNCH("f32_bwd_dX", k_f32_bwd_dx, dim3(gx, (unsigned)ceil_div(a.H, 64)), dim3(256), 0, st, a);
  }
  MOE_LAUNCH("f32_bwd_dWd", k_f32_wgrad, dim3((unsigned)ceil_div(a.H, 256), a.I, a.El), dim3(256), 0, st, a, 0, a.I, a.H);
  MOE_LAUNCH("f32_bwd_dWgu", k_f32_wgrad, dim3((unsigned)ceil_div(2 * a.I, 256), a.H, a.El), dim3(256), 0, st, a, 1, a.H,
                     2 * a.I);
  return hipGetLastError();
}

}  // namespace moe
