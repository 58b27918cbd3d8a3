// Router GEMM and its backward, bf16 MFMA for gfx950.
//
// NVIDIA's DeepSeek-V3 MoE article ("Optimization 2"): fused router kernels assign each
// token to its experts before dispatch.  The router here is one linear map without
// bias over every expert, logits [T, E] = x [T, H] W_r [H, E], accumulated in fp32 and
// kept in fp32 (the routing selects on them); its backward adds d_logits W_r^T to dX
// and gives dW_r = x^T d_logits.  The work is small (2 T H E flops, x read once), so the
// kernels aim at reading x once from HBM with enough waves in flight, not at a deep
// LDS pipeline:
//   logits : each workgroup a 32-row x 64-expert tile, 16 waves = 2 column blocks x 8
//            slices of H, slices summed through LDS; A and B fragments straight from
//            global memory (x rows and a transposed copy of W_r, both K-contiguous).
//   dx     : each workgroup a 128-token x 256-column tile (so W_r is read T / 128 times
//            and d_logits H / 256 times), each wave 32 x 128 of it over K = E, its
//            d_logits fragments (rounded to bf16 as they are loaded) read once for four
//            32-column blocks; W_r rows are already K-contiguous; adds dx_in in fp32.
//   dW_r   : 64 x 64 tiles over a slice of the tokens, x and d_logits staged transposed
//            in LDS (token-contiguous) for 16-byte fragment reads; the slices' fp32
//            partial sums reduced in a fixed order by a second kernel (deterministic).
//
// v_mfma_f32_32x32x16_bf16 operand layout: lane l supplies row (or column) l % 32 and
// the 8 contraction indices 8 (l / 32) .. 8 (l / 32) + 7 of each 16-step; result
// element j of lane l is row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
#include "common.h"

namespace moe {

namespace {

typedef __bf16 rbf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ rbf16x8 load8(const bf16_t* p) { return *reinterpret_cast<const rbf16x8*>(p); }
__device__ __forceinline__ rbf16x8 zero8() {
  rbf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (__bf16)0.f;
  return z;
}
// 8 fp32 values -> bf16 (round to nearest even)
__device__ __forceinline__ rbf16x8 cvt8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  rbf16x8 o;
  o[0] = (__bf16)a[0]; o[1] = (__bf16)a[1]; o[2] = (__bf16)a[2]; o[3] = (__bf16)a[3];
  o[4] = (__bf16)b[0]; o[5] = (__bf16)b[1]; o[6] = (__bf16)b[2]; o[7] = (__bf16)b[3];
  return o;
}
__device__ __forceinline__ int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

// W_r [H, E] -> W_rT [E, H] through a 32 x 32 LDS tile
__global__ __launch_bounds__(256) void k_router_wt(const bf16_t* __restrict__ w, int H, int E,
                                                   bf16_t* __restrict__ wt) {
  __shared__ bf16_t tile[32][33];
  const int h0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 8 rows per pass
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = h0 + ty + 8 * i, e = e0 + tx;
    tile[ty + 8 * i][tx] = (h < H && e < E) ? w[(size_t)h * E + e] : (bf16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + ty + 8 * i, h = h0 + tx;
    if (e < E && h < H) wt[(size_t)e * H + h] = tile[tx][ty + 8 * i];
  }
}

constexpr int LG_KSPLIT = 8;   // slices of H per logits tile
constexpr int LG_COLS = 64;    // experts per logits tile

// logits [T, E] = x [T, H] W_r [H, E]; H % 64 == 0 (a slice of H is a multiple of 8 and
// the loop steps 16 with the last half step masked)
__global__ __launch_bounds__(1024) void k_router_logits(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wt,
                                                       int T, int H, int E, float* __restrict__ logits) {
  __shared__ f32x16 red[LG_KSPLIT - 1][2][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cb = wv & 1, ks = wv >> 1;
  const int r0 = blockIdx.x * 32, c0 = blockIdx.y * LG_COLS + cb * 32;
  const int row = min(r0 + (lane & 31), T - 1), col = min(c0 + (lane & 31), E - 1);
  const int kl = H / LG_KSPLIT;
  const bf16_t* pa = x + (size_t)row * H + ks * kl + (lane >> 5) * 8;
  const bf16_t* pb = wt + (size_t)col * H + ks * kl + (lane >> 5) * 8;
  f32x16 acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  const bool k16 = kl % 16 == 0;               // uniform: no masked half step
#pragma unroll 8
  for (int k = 0; k < kl; k += 16) {
    const bool in = k16 || k + (lane >> 5) * 8 < kl;   // kl % 8 == 0: a lane's 8 indices all in or all out
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(in ? load8(pa + k) : zero8(), in ? load8(pb + k) : zero8(), acc, 0,
                                                   0, 0);
  }
  if (ks > 0) red[ks - 1][cb][lane] = acc;
  __syncthreads();
  if (ks == 0) {
#pragma unroll 1
    for (int s = 0; s < LG_KSPLIT - 1; ++s) {
      const f32x16 o = red[s][cb][lane];
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] += o[j];
    }
    const int c = c0 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + acc_row(j, lane);
      if (r < T && c < E) logits[(size_t)r * E + c] = acc[j];
    }
  }
}

constexpr int DX_BLOCKS = 4;                  // 32-column blocks of dX per wave
constexpr int DX_ROWS = 128;                  // tokens per workgroup: 4 row blocks of waves
constexpr int DX_COLS = 2 * 32 * DX_BLOCKS;   // columns per workgroup: 2 column halves of waves

// dx [T, H] = dx_in + d_logits [T, E] W_r^T; E % 8 == 0 (E16: E % 16 == 0, no masked
// half step).  Wave wv: rows 32 (wv % 4), columns 128 (wv / 4) of the workgroup's tile.
template <bool E16>
__global__ __launch_bounds__(512) void k_router_dx(const float* __restrict__ dl, const bf16_t* __restrict__ w, int T,
                                                   int H, int E, const bf16_t* dx_in, bf16_t* dx) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r0 = blockIdx.x * DX_ROWS + (wv & 3) * 32, c0 = blockIdx.y * DX_COLS + (wv >> 2) * 32 * DX_BLOCKS;
  if (c0 >= H || r0 >= T) return;
  const int row = min(r0 + (lane & 31), T - 1);
  const float* pa = dl + (size_t)row * E + (lane >> 5) * 8;
  const bf16_t* pb[DX_BLOCKS];
#pragma unroll
  for (int b = 0; b < DX_BLOCKS; ++b) pb[b] = w + (size_t)min(c0 + 32 * b + (lane & 31), H - 1) * E + (lane >> 5) * 8;
  f32x16 acc[DX_BLOCKS];
#pragma unroll
  for (int b = 0; b < DX_BLOCKS; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[b][j] = 0.f;
#pragma unroll 2
  for (int k = 0; k < E; k += 16) {
    // E % 8 == 0: a lane's 8 indices are all in or all out
    const bool in = E16 || k + (lane >> 5) * 8 < E;
    const rbf16x8 a = in ? cvt8(pa + k) : zero8();
#pragma unroll
    for (int b = 0; b < DX_BLOCKS; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, in ? load8(pb[b] + k) : zero8(), acc[b], 0, 0, 0);
  }
  // dx_in may be dx itself: every dx_in value of the lane is loaded before the first store,
  // so the loads are issued together instead of one after each store
  if (dx_in) {
    bf16_t din[DX_BLOCKS][16];
#pragma unroll
    for (int b = 0; b < DX_BLOCKS; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = min(r0 + acc_row(j, lane), T - 1), c = min(c0 + 32 * b + (lane & 31), H - 1);
        din[b][j] = dx_in[(size_t)r * H + c];
      }
#pragma unroll
    for (int b = 0; b < DX_BLOCKS; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[b][j] += bf2f(din[b][j]);
  }
#pragma unroll
  for (int b = 0; b < DX_BLOCKS; ++b) {
    const int c = c0 + 32 * b + (lane & 31);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + acc_row(j, lane);
      if (r < T && c < H) dx[(size_t)r * H + c] = f2bf(acc[b][j]);
    }
  }
}

constexpr int DW_TILE = 64;   // h and e per tile
constexpr int DW_CHUNK = 32;  // tokens staged per step
constexpr int DW_LD = 40;     // LDS row stride (elements): 16-byte aligned rows

// partial dW_r [H, E] of token slice blockIdx.z: sum over its tokens of x[t, h] dl[t, e]
__global__ __launch_bounds__(256) void k_router_dw(const bf16_t* __restrict__ x, const float* __restrict__ dl, int T,
                                                   int H, int E, int tslice, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) bf16_t xs[DW_TILE][DW_LD];  // [h][t]
  __shared__ __attribute__((aligned(16))) bf16_t ds[DW_TILE][DW_LD];  // [e][t]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h0 = blockIdx.x * DW_TILE, e0 = blockIdx.y * DW_TILE;
  const int t_begin = blockIdx.z * tslice, t_end = min(T, t_begin + tslice);
  const int bh = (wv & 1) * 32, be = (wv >> 1) * 32;   // the wave's 32 x 32 block
  f32x16 acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  // staging map: thread -> token tid / 8 of the chunk, 8 consecutive columns (tid % 8) * 8
  const int st_t = tid >> 3, st_c = (tid & 7) * 8;
  for (int t0 = t_begin; t0 < t_end; t0 += DW_CHUNK) {
    const int t = t0 + st_t;
    float xv[8], dv[8];
    if (t < t_end && h0 + st_c < H) {
      const i32x4 u = *reinterpret_cast<const i32x4*>(x + (size_t)t * H + h0 + st_c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[2 * q] = __uint_as_float((uint32_t)u[q] << 16);
        xv[2 * q + 1] = __uint_as_float((uint32_t)u[q] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) xv[q] = 0.f;
    }
    if (t < t_end && e0 + st_c < E) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(dl + (size_t)t * E + e0 + st_c);
      const f32x4 b = *reinterpret_cast<const f32x4*>(dl + (size_t)t * E + e0 + st_c + 4);
      dv[0] = a[0]; dv[1] = a[1]; dv[2] = a[2]; dv[3] = a[3]; dv[4] = b[0]; dv[5] = b[1]; dv[6] = b[2]; dv[7] = b[3];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) dv[q] = 0.f;
    }
    __syncthreads();   // the previous chunk's fragments have been read
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      xs[st_c + q][st_t] = f2bf(xv[q]);
      ds[st_c + q][st_t] = f2bf(dv[q]);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < DW_CHUNK / 16; ++kk) {
      const int kt = kk * 16 + (lane >> 5) * 8;
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load8(&xs[bh + (lane & 31)][kt]), load8(&ds[be + (lane & 31)][kt]),
                                                     acc, 0, 0, 0);
    }
  }
  const int e = e0 + be + (lane & 31);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int h = h0 + bh + acc_row(j, lane);
    if (h < H && e < E) part[((size_t)blockIdx.z * H + h) * E + e] = acc[j];
  }
}

// dW_r = the slices' partial sums, added in slice order, rounded once to bf16
__global__ __launch_bounds__(256) void k_router_dw_sum(const float* __restrict__ part, int slices, int64_t n,
                                                       bf16_t* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < slices; ++z) s += part[(size_t)z * n + i];
  dw[i] = f2bf(s);
}

}  // namespace

int router_dw_slices(int T, int H, int E) {
  const int64_t tiles = ceil_div(H, DW_TILE) * ceil_div(E, DW_TILE);
  int64_t s = ceil_div(1024, tiles);
  const int64_t smax = ceil_div(T, DW_CHUNK);
  if (s > smax) s = smax;
  return (int)(s < 1 ? 1 : s);
}

hipError_t launch_router_fwd(const moe_shape& s, const bf16_t* x, const bf16_t* w, bf16_t* wt, float* logits,
                             hipStream_t st) {
  MOE_LAUNCH("router_wt", k_router_wt, dim3((unsigned)ceil_div(s.H, 32), (unsigned)ceil_div(s.E, 32)), dim3(256), 0,
             st, w, s.H, s.E, wt);
  if (s.T == 0) return hipGetLastError();
  MOE_LAUNCH("router_logits", k_router_logits, dim3((unsigned)ceil_div(s.T, 32), (unsigned)ceil_div(s.E, LG_COLS)),
             dim3(1024), 0, st, x, wt, s.T, s.H, s.E, logits);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const moe_shape& s, const bf16_t* x, const bf16_t* w, const float* dl,
                             const bf16_t* dx_in, bf16_t* dx, bf16_t* dw, float* part, hipStream_t st) {
  const int64_t n = (int64_t)s.H * s.E;
  {
    const dim3 grid((unsigned)ceil_div(s.T, DX_ROWS), (unsigned)ceil_div(s.H, DX_COLS));
    if (s.T > 0 && s.E % 16 == 0)
      MOE_LAUNCH("router_dx", k_router_dx<true>, grid, dim3(512), 0, st, dl, w, s.T, s.H, s.E, dx_in, dx);
    else if (s.T > 0)
      MOE_LAUNCH("router_dx", k_router_dx<false>, grid, dim3(512), 0, st, dl, w, s.T, s.H, s.E, dx_in, dx);
  }
  const int slices = router_dw_slices(s.T, s.H, s.E);
  const int tslice = (int)(ceil_div(ceil_div(s.T, slices), DW_CHUNK) * DW_CHUNK);
  MOE_LAUNCH("router_dw", k_router_dw,
             dim3((unsigned)ceil_div(s.H, DW_TILE), (unsigned)ceil_div(s.E, DW_TILE), (unsigned)slices), dim3(256), 0,
             st, x, dl, s.T, s.H, s.E, tslice, part);
  MOE_LAUNCH("router_dw_sum", k_router_dw_sum, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, part, slices, n,
             dw);
  return hipGetLastError();
}

}  // namespace moe
