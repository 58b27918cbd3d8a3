// MXFP8 quantizers: E4M3 (OCP "FN": bias 7, max 448, no infinities) elements with one
// e8m0 scale (2^(code - 127)) per block of 32 along a GEMM's contraction axis.
//
// The fp8 backward mode of the Prime Mega MoE pages (bf16 forward, FP8 backward) with
// the group-aware MXFP8 quantisation of NVIDIA's DeepSeek-V3 MoE article: column-wise
// blocks of 32 token rows start at each expert's first row and never cross experts.
//
// Scale rule: X = the smallest integer with amax <= 448 * 2^X (so x / 2^X never
// saturates), clamped to [-127, 127], X = 0 for an all-zero block.  Elements: x / 2^X
// rounded to the nearest E4M3 value, ties to even, sign bit from x.  The scale is exact
// exponent arithmetic and the element conversion is correctly rounded, so identical
// inputs give identical codes on any correct implementation.
#include "common.h"

namespace moe {

namespace {

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Row-wise: one wave per row, in passes of 512 columns per 64 lanes: lane l takes the
// 8-element groups l + 64 i (8 consecutive columns each), so the 4 lanes 4j .. 4j + 3 of
// a pass hold one 32-element block.  A lane issues the loads of up to RG passes (RG x 16
// bytes) before it quantises any of them.  rows_fixed < 0 (or a gather) means the row
// count is offsets[El]; with src2, columns >= K / 2 of row r come from src2 (two
// [rows, K / 2] matrices side by side).
constexpr int RG = 8;
__global__ __launch_bounds__(256) void k_mx_rows(const bf16_t* __restrict__ src, const bf16_t* __restrict__ src2,
                                                 int ld, const int32_t* __restrict__ row_src, int k,
                                                 const int32_t* __restrict__ offsets, int El, int64_t rows_fixed,
                                                 int K, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t rows = (row_src || rows_fixed < 0) ? (int64_t)offsets[El] : rows_fixed;
  const int lane = threadIdx.x & 63;
  const int half = K / 2;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += (int64_t)gridDim.x * 4) {
    const int64_t sr = row_src ? (int64_t)(row_src[r] / k) : r;
    const bf16_t* const p1 = src + sr * ld;
    const bf16_t* const p2 = src2 ? src2 + sr * ld - half : nullptr;
    uint8_t* const qr = q + r * K;
    uint8_t* const sq = s + r * (K / 32);
    for (int c0 = 0; c0 < K; c0 += 512 * RG) {
      i32x4 u[RG];
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int c = c0 + 512 * i + 8 * lane;
        u[i] = i32x4{0, 0, 0, 0};
        if (c < K) u[i] = *reinterpret_cast<const i32x4*>((p2 && c >= half ? p2 : p1) + c);
      }
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int c = c0 + 512 * i + 8 * lane;
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[2 * j] = bf_lo((uint32_t)u[i][j]); v[2 * j + 1] = bf_hi((uint32_t)u[i][j]); }
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
        am = fmaxf(am, __shfl_xor(am, 2, 64));
        if (c < K) {   // K is a multiple of 32: a block lies wholly inside or outside the row
          const int X = mx_scale_exp(am);
          const uint32_t w0 = e4m3_pack4(v[0], v[1], v[2], v[3], X);
          const uint32_t w1 = e4m3_pack4(v[4], v[5], v[6], v[7], X);
          *reinterpret_cast<uint2*>(qr + c) = make_uint2(w0, w1);
          if ((lane & 3) == 0) sq[c >> 5] = (uint8_t)(X + 127);
        }
      }
    }
  }
}

// Column-wise, transposed: one workgroup per (padded 128-row chunk, 128 columns); a chunk
// lies inside one expert's padded segment (segments are multiples of 128 rows).  The
// chunk's row sources and weights are read once into LDS and its rows staged as bf16
// (32 KB, so several workgroups share a CU); thread t takes the 32-row block t / 128 of
// column t % 128 into registers (applying the optional row weight in fp32), quantizes
// it, the codes then overwrite the staged tile, and the workgroup writes each column's
// 128 codes as one 128-byte line and its four scales as one word.  With qr given, the same staged tile also yields
// the row-wise quantisation of the unweighted values (codes at qr[r * ldr + n] for the
// dispatched row r, scales at sr[r * (ldr / 32) + n / 32]): thread t takes the 32
// columns (t % 4) of staged row t / 4, so a matrix that both layouts need is read once.
constexpr int COL_ROWS = 128, COL_COLS = 128;
constexpr int COL_THREADS = 4 * COL_COLS;   // one per (column, 32-row block)
static_assert(COL_ROWS == kMxRowPad, "a column chunk spans one padding unit");
__global__ __launch_bounds__(COL_THREADS, 8) void k_mx_cols(const bf16_t* __restrict__ src, int ld,
                                                 const int32_t* __restrict__ row_src, int k,
                                                 const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ poff, int El, int N, int Rp,
                                                 uint8_t* __restrict__ qt, uint8_t* __restrict__ stt,
                                                 uint8_t* __restrict__ qr, uint8_t* __restrict__ sr, int ldr) {
  // the codes [COL_COLS][COL_ROWS / 4 + 4] (u32) take the staged tile's place once it is
  // read, so the workgroup holds 33 KB of LDS and four fit on a CU
  __shared__ __attribute__((aligned(16))) uint16_t tile[COL_ROWS][COL_COLS];
  uint32_t (*const codes)[COL_ROWS / 4 + 4] = reinterpret_cast<uint32_t (*)[COL_ROWS / 4 + 4]>(&tile[0][0]);
  static_assert(COL_COLS * (COL_ROWS / 4 + 4) * 4 <= COL_ROWS * COL_COLS * 2, "the codes fit over the tile");
  __shared__ uint32_t scales[COL_COLS];
  __shared__ int srow[COL_ROWS];
  __shared__ float wrow[COL_ROWS];
  const int pr0 = blockIdx.x * COL_ROWS;     // padded row of the chunk
  if (pr0 >= poff[El]) return;
  int lo = 0, hi = El - 1;                   // expert: last e with poff[e] <= pr0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= pr0) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int r0 = offsets[e] + (pr0 - poff[e]);
  const int nrow = min(COL_ROWS, offsets[e + 1] - r0);   // may be <= 0 in an expert's padding
  const int n0 = blockIdx.y * COL_COLS;
  const int tid = threadIdx.x;
  if (tid < COL_ROWS) {
    int sr = 0;
    float w = 1.f;
    if (tid < nrow) {
      const int r = r0 + tid;
      const int s = row_src ? row_src[r] : 0;
      sr = row_src ? s / k : r;
      if (topk_w) w = topk_w[s];
    }
    srow[tid] = sr;
    wrow[tid] = w;
  }
  __syncthreads();
  // stage: 128 rows x 64 columns of bf16, one 16-byte load per (row, 8 columns)
  {
    constexpr int IT = COL_ROWS * (COL_COLS / 8) / COL_THREADS;
    i32x4 u[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + COL_THREADS * it;
      const int rr = i / (COL_COLS / 8), cc = (i % (COL_COLS / 8)) * 8;
      u[it] = i32x4{0, 0, 0, 0};
      if (rr < nrow && n0 + cc < N) u[it] = *reinterpret_cast<const i32x4*>(src + (size_t)srow[rr] * ld + n0 + cc);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + COL_THREADS * it;
      const int rr = i / (COL_COLS / 8), cc = (i % (COL_COLS / 8)) * 8;
      *reinterpret_cast<i32x4*>(&tile[rr][cc]) = u[it];
    }
  }
  __syncthreads();
  if (qr) {
    const int rr = tid / (COL_COLS / 32), h = tid % (COL_COLS / 32);   // staged row, 32-column block
    const int n = n0 + 32 * h;
    if (rr < nrow && n < N) {
      const i32x4* t4 = reinterpret_cast<const i32x4*>(&tile[rr][32 * h]);
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x4 u = t4[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * q + 2 * j] = bf_lo((uint32_t)u[j]);
          v[8 * q + 2 * j + 1] = bf_hi((uint32_t)u[j]);
        }
      }
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(v[j]));
      const int X = mx_scale_exp(am);
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = e4m3_pack4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], X);
      const size_t r = (size_t)(r0 + rr);
      uint4* dst = reinterpret_cast<uint4*>(qr + r * ldr + n);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      sr[r * (ldr / 32) + n / 32] = (uint8_t)(X + 127);
    }
  }
  const int c = tid % COL_COLS, b = tid / COL_COLS;   // column, 32-row block
  uint32_t q[8];
  {
    float v[32];
    float am = 0.f;
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) {
      const int r = b * 32 + rr;
      v[rr] = __uint_as_float((uint32_t)tile[r][c] << 16);
      if (topk_w) v[rr] *= wrow[r];
      am = fmaxf(am, fabsf(v[rr]));
    }
    const int X = mx_scale_exp(am);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = e4m3_pack4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], X);
    reinterpret_cast<uint8_t*>(scales)[c * 4 + b] = (uint8_t)(X + 127);
  }
  __syncthreads();   // every read of the staged tile is done: the codes take its place
#pragma unroll
  for (int j = 0; j < 8; ++j) codes[c][b * 8 + j] = q[j];
  __syncthreads();
  // write-out: COL_COLS columns x 128 codes, eight lanes per 128-byte line
#pragma unroll
  for (int it = 0; it < COL_COLS * 8 / COL_THREADS; ++it) {
    const int i = tid + COL_THREADS * it;
    const int c = i / 8, part = i % 8;
    const int n = n0 + c;
    if (n < N)
      *reinterpret_cast<uint4*>(qt + (size_t)n * Rp + pr0 + part * 16) =
          *reinterpret_cast<const uint4*>(&codes[c][part * 4]);
  }
  if (tid < COL_COLS && n0 + tid < N)
    *reinterpret_cast<uint32_t*>(stt + (size_t)(n0 + tid) * (Rp / 32) + pr0 / 32) = scales[tid];
}

// padded offsets: every expert's rows rounded up to kMxRowPad
__global__ __launch_bounds__(1024) void k_poff(const int32_t* __restrict__ offsets, int El, int32_t* __restrict__ poff) {
  __shared__ int32_t buf[1024];
  const int e = threadIdx.x;
  const int n = e < El ? (offsets[e + 1] - offsets[e] + kMxRowPad - 1) / kMxRowPad * kMxRowPad : 0;
  buf[e] = n;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? buf[e - off] : 0;
    __syncthreads();
    buf[e] += v;
    __syncthreads();
  }
  if (e < El) poff[e + 1] = buf[e];
  if (e == 0) poff[0] = 0;
}

__global__ __launch_bounds__(256) void k_iota(int32_t* __restrict__ out, int n, int step) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e <= n) out[e] = e * step;
}

}  // namespace

hipError_t launch_mx_iota(int32_t* out, int n, int step, hipStream_t st) {
  MOE_LAUNCH("mx_goff", k_iota, dim3((unsigned)ceil_div(n + 1, 256)), dim3(256), 0, st, out, n, step);
  return hipGetLastError();
}

hipError_t launch_mx_rows(const bf16_t* src, const bf16_t* src2, int ld, const int32_t* row_src, int k,
                          const int32_t* offsets, int El, int64_t rows, int64_t rows_bound, int K, uint8_t* q,
                          uint8_t* s, const char* name, hipStream_t st) {
  if (rows_bound <= 0) return hipSuccess;
  const int64_t blocks = ceil_div(rows_bound, 4);   // four rows (waves) per workgroup
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  MOE_LAUNCH(name, k_mx_rows, dim3(grid), dim3(256), 0, st, src, src2, ld, row_src, k, offsets, El, rows, K, q, s);
  return hipGetLastError();
}

hipError_t launch_mx_cols(const bf16_t* src, int ld, const int32_t* row_src, int k, const float* topk_w,
                          const int32_t* offsets, const int32_t* poff, int El, int N, int Rp, uint8_t* qt,
                          uint8_t* stt, const char* name, hipStream_t st, uint8_t* qr, uint8_t* sr, int ldr) {
  if (Rp <= 0) return hipSuccess;
  MOE_LAUNCH(name, k_mx_cols, dim3((unsigned)(Rp / COL_ROWS), (unsigned)ceil_div(N, COL_COLS)), dim3(COL_THREADS), 0, st,
             src, ld, row_src, k, topk_w, offsets, poff, El, N, Rp, qt, stt, qr, sr, ldr > 0 ? ldr : N);
  return hipGetLastError();
}

hipError_t launch_poff(const int32_t* offsets, int El, int32_t* poff, hipStream_t st) {
  MOE_LAUNCH("mx_poff", k_poff, dim3(1), dim3(1024), 0, st, offsets, El, poff);
  return hipGetLastError();
}

}  // namespace moe
