// bf16 MFMA grouped GEMMs of the expert MLP, forward and backward, for gfx950.
//
// Grouped GEMM over each expert's real row count in one launch, shapes read on the
// device (NVIDIA DeepSeek-V3 MoE article, "Optimization 1"); the two expert linear
// layers with SwiGLU between them and the routing-weight scaling fused into the
// GEMMs (Prime Mega MoE pages: one call fusing the linears, SwiGLU and combine, with
// scratch buffers instead of intermediate tensors).
//
// Engine: 256-thread workgroups (4 wave64), 128x128 output tile, K step 64, four
// v_mfma_f32_32x32x16_bf16 accumulators per wave (64x64 per wave).  Operand tiles go
// global -> registers -> LDS with a two-stage LDS ring (one barrier per K step).
// An operand whose contraction axis is contiguous in memory ("K-major") is stored
// [rows][64] and read with 16-byte LDS reads; an operand contiguous along M or N
// ("MN-major": row-major weights as the B of x*W, and both operands of the weight
// gradients, which contract over token rows) is stored [64][128] and read with the
// gfx950 transposing LDS read ds_read_b64_tr_b16, so no operand is transposed in
// memory.  Both layouts are XOR-swizzled by 16-byte chunk against LDS bank conflicts.
//
// Kernels:
//   K1 fwd_gateup : G = Xp Wg, U = Xp Wu (dual B tile), epilogue saves G|U and A = silu(G) U
//   K2 fwd_down   : Yp = w * (A Wd)
//   B1 bwd_dA     : dA' = dY' Wd^T; epilogue: rowdot(dA', A) partials, SwiGLU backward -> dG|dU
//   B3 bwd_dX     : dXp = dG Wg^T + dU Wu^T (K = 2I)
//   B2 bwd_dWd    : dWd[e] = A_e^T (w dY')_e over the expert's rows
//   B4 bwd_dWgu   : [dWg | dWu][e] = Xp_e^T [dG | dU]_e over the expert's rows
#include "common.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int TILE_ELEMS = 128 * 64;  // both LDS layouts hold 8192 bf16

// ---- LDS layouts ----
// K-major [128][64]: 8 chunks of 16 B per row; chunk c of row r lives at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int kmaj_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }
// MN-major [64][128]: 16 chunks per k-row; chunk c of k-row r lives at c ^ ((r & 3) << 2).
__device__ __forceinline__ int mnmaj_off(int r, int c) { return r * 128 + ((c ^ ((r & 3) << 2)) << 3); }

// MFMA 32x32x16 operand fragment: lane l gets 8 consecutive k of row/col (l & 31),
// k = 8 * (l >> 5) .. +7 inside the 16-wide k sub-step kk.
__device__ __forceinline__ bf16x8 frag_kmaj(const bf16_t* s, int base, int kk, int lane) {
  const int r = base + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(s + kmaj_off(r, c));
}

// Same fragment from an MN-major tile with two transposing reads: in each 16-lane group
// g, lane 4j + q points at k-row j of its 4-row slab and columns 4q..4q+3 of the
// group's 16 columns; the hardware hands lane i of the group column i of the 4 rows.
__device__ __forceinline__ bf16x8 frag_mnmaj(const bf16_t* s, int base, int kk, int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  const int col = base + 16 * (g & 1) + 4 * q;
  s16x4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = kk * 16 + 8 * (g >> 1) + 4 * h + j;
    const int off = r * 128 + (((col >> 3) ^ ((r & 3) << 2)) << 3) + (col & 7);
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(s + off));
  }
  bf16x8 out;
  __builtin_memcpy(&out, v, 16);
  return out;
}

__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  // workgroups are dispatched round-robin over the 8 XCDs; make consecutive virtual
  // ids run on one XCD so that tiles sharing operands share its L2
  return (bid & 7) * (nwg >> 3) + (bid >> 3);
}

__device__ __forceinline__ i32x4 scale_bf16x8(i32x4 v, float w) {
  i32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t u = (uint32_t)v[q];
    float lo = __uint_as_float(u << 16) * w, hi = __uint_as_float(u & 0xffff0000u) * w;
    o[q] = (int)((uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16));
  }
  return o;
}

// Register staging of one 128x64 operand tile: 4 chunks of 16 B per thread.
struct Stage {
  i32x4 a[4], b[4];
};

__device__ __forceinline__ void store_kmaj(bf16_t* s, const i32x4* v, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i, c = tid & 7;
    *reinterpret_cast<i32x4*>(s + kmaj_off(r, c)) = v[i];
  }
}
__device__ __forceinline__ void store_mnmaj(bf16_t* s, const i32x4* v, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i, c = tid & 15;
    *reinterpret_cast<i32x4*>(s + mnmaj_off(r, c)) = v[i];
  }
}

// The main loop: acc[mi][ni] (32x32 blocks) of this wave's 64x64 sub-tile.
// P supplies load(kt, Stage&), the operand layouts and the wave's N-block columns.
// Global loads run two K steps ahead of the MFMAs (two register stages), the LDS ring
// has two stages, and there is one barrier per K step.
template <class P>
__device__ __forceinline__ void store_stage(bf16_t* buf, const Stage& st, int tid) {
  if (P::A_KMAJ) store_kmaj(buf, st.a, tid); else store_mnmaj(buf, st.a, tid);
  if (P::B_KMAJ) store_kmaj(buf + TILE_ELEMS, st.b, tid); else store_mnmaj(buf + TILE_ELEMS, st.b, tid);
}

template <class P>
__device__ __forceinline__ void mma_stage(const bf16_t* buf, f32x16 (&acc)[2][2], int lane, int wm, int wn) {
  const bf16_t* As = buf;
  const bf16_t* Bs = buf + TILE_ELEMS;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8 af[2], bf[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      af[mi] = P::A_KMAJ ? frag_kmaj(As, wm * 64 + mi * 32, kk, lane) : frag_mnmaj(As, wm * 64 + mi * 32, kk, lane);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      bf[ni] = P::B_KMAJ ? frag_kmaj(Bs, P::ncol(wn, ni), kk, lane) : frag_mnmaj(Bs, P::ncol(wn, ni), kk, lane);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
  }
}

template <class P>
__device__ __forceinline__ void mainloop(P& p, int nk, bf16_t* lds, f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
  if (nk <= 0) return;
  Stage s0, s1;
  p.load(0, s0);
  store_stage<P>(lds, s0, tid);
  if (nk > 1) p.load(1, s0);
  __syncthreads();
  // K steps in pairs so that the two register stages keep fixed registers
  for (int kt = 0; kt < nk; kt += 2) {
    // step kt: s0 holds step kt + 1, s1 receives step kt + 2
    if (kt + 2 < nk) p.load(kt + 2, s1);
    mma_stage<P>(lds, acc, lane, wm, wn);
    if (kt + 1 < nk) store_stage<P>(lds + 2 * TILE_ELEMS, s0, tid);
    __syncthreads();
    if (kt + 1 >= nk) break;
    // step kt + 1: s1 holds step kt + 2, s0 receives step kt + 3
    if (kt + 3 < nk) p.load(kt + 3, s0);
    mma_stage<P>(lds + 2 * TILE_ELEMS, acc, lane, wm, wn);
    if (kt + 2 < nk) store_stage<P>(lds, s1, tid);
    __syncthreads();
  }
}

// ---- epilogue staging ----
// After the main loop the LDS ring is free.  Each wave writes one 32-row half (mi) of
// its 64x64 fp32 accumulator to its own [32][EP_LD] region, so that lanes can then read
// 8 consecutive columns of one row and issue 16-byte global loads and stores.
constexpr int EP_LD = 72;  // row stride in floats: rows r and r + 4 fall on disjoint banks

__device__ __forceinline__ void stage_acc(float* wsm, const f32x16 (&acc)[2][2], int mi, int lane) {
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      wsm[r * EP_LD + ni * 32 + (lane & 31)] = acc[mi][ni][i];
    }
}

__device__ __forceinline__ void read8(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}

__device__ __forceinline__ i32x4 pack8(const float (&v)[8]) {
  i32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (int)((uint32_t)f2bf(v[2 * q]) | ((uint32_t)f2bf(v[2 * q + 1]) << 16));
  return o;
}

__device__ __forceinline__ void unpack8(i32x4 u, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(((uint32_t)u[q]) << 16);
    v[2 * q + 1] = __uint_as_float(((uint32_t)u[q]) & 0xffff0000u);
  }
}

// Generic epilogue walk for the "wn * 64 + ni * 32" column mapping: calls
// f(row_in_tile, col_in_tile, v[8]) for every 8-column chunk of this wave's sub-tile.
template <class F>
__device__ __forceinline__ void epilogue_rows(bf16_t* lds, const f32x16 (&acc)[2][2], F&& f) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
  float* wsm = reinterpret_cast<float*>(lds) + wv * 32 * EP_LD;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    __syncthreads();
    stage_acc(wsm, acc, mi, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = (lane >> 3) + 8 * j, cc = (lane & 7) * 8;
      float v[8];
      read8(wsm + rr * EP_LD + cc, v);
      f(wm * 64 + mi * 32 + rr, wn * 64 + cc, v);
    }
  }
}

// Row (within the 128-row tile) and column (within the 128-col tile) held by element
// i of accumulator block (mi, ni) of this lane.
__device__ __forceinline__ int acc_row(int wm, int mi, int i, int lane) {
  return wm * 64 + mi * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
}

// Common setup of the row-group GEMMs: virtual tile v -> expert, first row, valid rows
// and column tile, in the expert-major order of the tile table (see k_tile_table).
struct RowTile {
  int e, rs, cnt, nt;
};
__device__ __forceinline__ bool row_tile(const int32_t* tiles, const int32_t* offsets, int v, int NT, RowTile& t) {
  const int q = v / NT;
  if (q >= tiles[0]) return false;
  const i32x4 ent = *reinterpret_cast<const i32x4*>(tiles + 4 + 4 * q);
  t.e = ent[0];
  const int local = v - ent[1] * NT;
  const int mt = local % ent[2];
  t.nt = local / ent[2];
  t.rs = offsets[t.e] + mt * BM;
  t.cnt = min(BM, offsets[t.e + 1] - t.rs);
  return true;
}

// ---------------- K1: gate/up + SwiGLU ----------------
struct PGateUp {
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  // gate columns 0..63 and up columns 64..127 of the B tile; wave wn takes the same
  // 32 intermediate columns of both so G and U of one element share a lane
  __device__ static int ncol(int wn, int ni) { return ni * 64 + wn * 32; }
  const bf16_t* arow[4];
  const bf16_t* wg;
  const bf16_t* wu;
  int I, n0;
  __device__ void load(int kt, Stage& s) const {
    const int tid = threadIdx.x;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.a[i] = *reinterpret_cast<const i32x4*>(arow[i] + k0 + (tid & 7) * 8);
    const int c = tid & 15;
    const bf16_t* w = c < 8 ? wg : wu;
    const int col = n0 + (c & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      s.b[i] = *reinterpret_cast<const i32x4*>(w + (size_t)(k0 + r) * I + col);
    }
  }
};

__global__ __launch_bounds__(NT, 2) void k_fwd_gateup(FwdArgs a, int nvirt, int nwg) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * TILE_ELEMS];
  const int v = xcd_remap(blockIdx.x, nwg);
  if (v >= nvirt) return;
  RowTile t;
  if (!row_tile(a.tiles, a.offsets, v, a.I / 64, t)) return;
  const int tid = threadIdx.x, nt = t.nt;
  PGateUp p;
  for (int i = 0; i < 4; ++i) {
    const int r = t.rs + min((tid >> 3) + 32 * i, t.cnt - 1);
    p.arow[i] = a.xp ? a.xp + (size_t)r * a.H : a.x + (size_t)(a.row_src[r] / a.k) * a.H;
  }
  p.wg = a.wg + (size_t)t.e * a.H * a.I;
  p.wu = a.wu + (size_t)t.e * a.H * a.I;
  p.I = a.I;
  p.n0 = nt * 64;
  f32x16 acc[2][2];
  mainloop(p, a.H / BK, lds, acc);
  // epilogue: lane takes 8 intermediate columns of one row, G from block ni = 0 and U
  // from ni = 1 (same columns), and writes 16-byte chunks of G, U and A
  const int lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
  float* wsm = reinterpret_cast<float*>(lds) + wv * 32 * EP_LD;
  const size_t I2 = 2 * (size_t)a.I;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    __syncthreads();
    stage_acc(wsm, acc, mi, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rr = (lane >> 2) + 16 * j, cc = (lane & 3) * 8;
      const int rt = wm * 64 + mi * 32 + rr;
      float g[8], u[8], av[8];
      read8(wsm + rr * EP_LD + cc, g);
      read8(wsm + rr * EP_LD + 32 + cc, u);
      if (rt < t.cnt) {
        const size_t r = (size_t)(t.rs + rt);
        const int col = p.n0 + wn * 32 + cc;
#pragma unroll
        for (int q = 0; q < 8; ++q) av[q] = silu_f(g[q]) * u[q];
        *reinterpret_cast<i32x4*>(a.gu + r * I2 + col) = pack8(g);
        *reinterpret_cast<i32x4*>(a.gu + r * I2 + a.I + col) = pack8(u);
        *reinterpret_cast<i32x4*>(a.a + r * a.I + col) = pack8(av);
      }
    }
  }
}

// ---------------- K2: down projection * routing weight ----------------
struct PDown {
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  __device__ static int ncol(int wn, int ni) { return wn * 64 + ni * 32; }
  const bf16_t* arow[4];
  const bf16_t* wd;
  int H, n0;
  __device__ void load(int kt, Stage& s) const {
    const int tid = threadIdx.x;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.a[i] = *reinterpret_cast<const i32x4*>(arow[i] + k0 + (tid & 7) * 8);
    int col = n0 + (tid & 15) * 8;
    if (col >= H) col = n0;  // tail columns: any valid address, results are discarded
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      s.b[i] = *reinterpret_cast<const i32x4*>(wd + (size_t)(k0 + r) * H + col);
    }
  }
};

__global__ __launch_bounds__(NT, 2) void k_fwd_down(FwdArgs a, int nvirt, int nwg) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * TILE_ELEMS];
  const int v = xcd_remap(blockIdx.x, nwg);
  if (v >= nvirt) return;
  RowTile t;
  if (!row_tile(a.tiles, a.offsets, v, (int)ceil_div(a.H, BN), t)) return;
  const int tid = threadIdx.x, nt = t.nt;
  PDown p;
  for (int i = 0; i < 4; ++i) {
    const int r = t.rs + min((tid >> 3) + 32 * i, t.cnt - 1);
    p.arow[i] = a.a + (size_t)r * a.I;
  }
  p.wd = a.wd + (size_t)t.e * a.I * a.H;
  p.H = a.H;
  p.n0 = nt * BN;
  f32x16 acc[2][2];
  mainloop(p, a.I / BK, lds, acc);
  epilogue_rows(lds, acc, [&](int rt, int ct, const float (&v)[8]) {
    const int col = p.n0 + ct;
    if (rt < t.cnt && col < a.H) {
      const size_t r = (size_t)(t.rs + rt);
      const float w = a.topk_w[a.row_src[r]];
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = w * v[q];
      *reinterpret_cast<i32x4*>(a.yp + r * a.H + col) = pack8(o);
    }
  });
}

// ---------------- B1: dA' = dY' Wd^T, SwiGLU backward ----------------
struct PBwdDA {
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  __device__ static int ncol(int wn, int ni) { return wn * 64 + ni * 32; }
  const bf16_t* arow[4];
  const bf16_t* brow[4];
  __device__ void load(int kt, Stage& s) const {
    const int tid = threadIdx.x;
    const int k0 = kt * BK + (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.a[i] = *reinterpret_cast<const i32x4*>(arow[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s.b[i] = *reinterpret_cast<const i32x4*>(brow[i] + k0);
  }
};

__global__ __launch_bounds__(NT, 2) void k_bwd_da(BwdArgs a, int nvirt, int nwg, int nparts) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * TILE_ELEMS];
  const int v = xcd_remap(blockIdx.x, nwg);
  if (v >= nvirt) return;
  RowTile t;
  if (!row_tile(a.tiles, a.offsets, v, (int)ceil_div(a.I, BN), t)) return;
  const int tid = threadIdx.x, nt = t.nt;
  const int n0 = nt * BN;
  PBwdDA p;
  const bf16_t* wd = a.wd + (size_t)t.e * a.I * a.H;
  for (int i = 0; i < 4; ++i) {
    const int r = t.rs + min((tid >> 3) + 32 * i, t.cnt - 1);
    p.arow[i] = a.dy + (size_t)(a.row_src[r] / a.k) * a.H;
    const int n = min(n0 + (tid >> 3) + 32 * i, a.I - 1);
    p.brow[i] = wd + (size_t)n * a.H;
  }
  f32x16 acc[2][2];
  mainloop(p, a.H / BK, lds, acc);
  // epilogue: SwiGLU backward on 8 columns per lane; the rowdot of dA' and A over this
  // wave's 64 columns is reduced across the 8 lanes that share the row
  const int lane = tid & 63, wn = (tid >> 6) >> 1;
  const size_t I2 = 2 * (size_t)a.I;
  epilogue_rows(lds, acc, [&](int rt, int ct, const float (&dap)[8]) {
    const int col = n0 + ct;
    const bool ok = rt < t.cnt && col < a.I;
    float part = 0.f;
    size_t r = 0;
    if (ok) {
      r = (size_t)(t.rs + rt);
      const float w = a.topk_w[a.row_src[r]];
      float g[8], u[8], av[8], dg[8], du[8];
      unpack8(*reinterpret_cast<const i32x4*>(a.gu + r * I2 + col), g);
      unpack8(*reinterpret_cast<const i32x4*>(a.gu + r * I2 + a.I + col), u);
      unpack8(*reinterpret_cast<const i32x4*>(a.a + r * a.I + col), av);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        part += dap[q] * av[q];
        const float da = w * dap[q];
        const float sg = sigmoid_f(g[q]);
        du[q] = da * g[q] * sg;
        dg[q] = da * u[q] * sg * (1.f + g[q] * (1.f - sg));
      }
      *reinterpret_cast<i32x4*>(a.dgu + r * I2 + col) = pack8(dg);
      *reinterpret_cast<i32x4*>(a.dgu + r * I2 + a.I + col) = pack8(du);
    }
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    if (rt < t.cnt && (lane & 7) == 0) a.dw_part[(size_t)(t.rs + rt) * nparts + nt * 2 + wn] = part;
  });
}

// ---------------- B3: dXp = dG Wg^T + dU Wu^T ----------------
struct PBwdDX {
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  __device__ static int ncol(int wn, int ni) { return wn * 64 + ni * 32; }
  const bf16_t* arow[4];
  const bf16_t* grow[4];
  const bf16_t* urow[4];
  int I;
  __device__ void load(int kt, Stage& s) const {
    const int tid = threadIdx.x;
    const int k0 = kt * BK;
    const int kc = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.a[i] = *reinterpret_cast<const i32x4*>(arow[i] + k0 + kc);
    if (k0 < I) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s.b[i] = *reinterpret_cast<const i32x4*>(grow[i] + k0 + kc);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s.b[i] = *reinterpret_cast<const i32x4*>(urow[i] + (k0 - I) + kc);
    }
  }
};

__global__ __launch_bounds__(NT, 2) void k_bwd_dx(BwdArgs a, int nvirt, int nwg) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * TILE_ELEMS];
  const int v = xcd_remap(blockIdx.x, nwg);
  if (v >= nvirt) return;
  RowTile t;
  if (!row_tile(a.tiles, a.offsets, v, (int)ceil_div(a.H, BN), t)) return;
  const int tid = threadIdx.x, nt = t.nt;
  const int n0 = nt * BN;
  PBwdDX p;
  p.I = a.I;
  const size_t woff = (size_t)t.e * a.H * a.I;
  for (int i = 0; i < 4; ++i) {
    const int r = t.rs + min((tid >> 3) + 32 * i, t.cnt - 1);
    p.arow[i] = a.dgu + (size_t)r * 2 * a.I;
    const int n = min(n0 + (tid >> 3) + 32 * i, a.H - 1);
    p.grow[i] = a.wg + woff + (size_t)n * a.I;
    p.urow[i] = a.wu + woff + (size_t)n * a.I;
  }
  f32x16 acc[2][2];
  mainloop(p, 2 * a.I / BK, lds, acc);
  epilogue_rows(lds, acc, [&](int rt, int ct, const float (&v)[8]) {
    const int col = n0 + ct;
    if (rt < t.cnt && col < a.H)
      *reinterpret_cast<i32x4*>(a.dxp + (size_t)(t.rs + rt) * a.H + col) = pack8(v);
  });
}

// ---------------- weight gradients: contraction over an expert's rows ----------------
// Both operands are MN-major tiles of 64 token rows; rows past the expert's end are
// loaded as zeros.
struct PWgrad {
  static constexpr bool A_KMAJ = false, B_KMAJ = false;
  __device__ static int ncol(int wn, int ni) { return wn * 64 + ni * 32; }
  // A: rows of an [R, lda] (or gathered [T, lda]) matrix, columns m0.. ; B likewise
  const bf16_t* abase; int lda; bool agather;
  const bf16_t* bbase; int ldb; bool bgather;
  const int32_t* row_src; const float* topk_w; int k;
  bool bscale;   // multiply B rows by the routing weight
  int rs, cnt, m0, n0, M, N;
  __device__ void load(int kt, Stage& s) const {
    const int tid = threadIdx.x;
    const int c = tid & 15;
    int ca = m0 + c * 8; if (ca >= M) ca = m0;
    int cb = n0 + c * 8; if (cb >= N) cb = n0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = kt * BK + (tid >> 4) + 16 * i;
      if (kr < cnt) {
        const int r = rs + kr;
        const int src = row_src[r];
        const size_t ra = agather ? (size_t)(src / k) : (size_t)r;
        const size_t rb = bgather ? (size_t)(src / k) : (size_t)r;
        s.a[i] = *reinterpret_cast<const i32x4*>(abase + ra * lda + ca);
        i32x4 bv = *reinterpret_cast<const i32x4*>(bbase + rb * ldb + cb);
        s.b[i] = bscale ? scale_bf16x8(bv, topk_w[src]) : bv;
      } else {
        s.a[i] = i32x4{0, 0, 0, 0};
        s.b[i] = i32x4{0, 0, 0, 0};
      }
    }
  }
};

// B2 (WHICH = 0): dWd[e] [I, H] = A_e^T (w dY')_e.   B4 (WHICH = 1): [dWg | dWu][e] [H, 2I] = Xp_e^T [dG | dU]_e.
template <int WHICH>
__global__ __launch_bounds__(NT, 2) void k_bwd_wgrad(BwdArgs a, int tm, int tn, int nvirt, int nwg) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * TILE_ELEMS];
  const int v = xcd_remap(blockIdx.x, nwg);
  if (v >= nvirt) return;
  const int e = v / (tm * tn);
  const int rem = v - e * tm * tn;
  const int mt = rem / tn, nt = rem - mt * tn;
  PWgrad p;
  p.rs = a.offsets[e];
  p.cnt = a.offsets[e + 1] - p.rs;
  p.m0 = mt * BM;
  p.n0 = nt * BN;
  p.row_src = a.row_src; p.topk_w = a.topk_w; p.k = a.k;
  if (WHICH == 0) {
    p.abase = a.a; p.lda = a.I; p.agather = false;
    p.bbase = a.dy; p.ldb = a.H; p.bgather = true; p.bscale = true;
    p.M = a.I; p.N = a.H;
  } else {
    if (a.xp) { p.abase = a.xp; p.agather = false; } else { p.abase = a.x; p.agather = true; }
    p.lda = a.H;
    p.bbase = a.dgu; p.ldb = 2 * a.I; p.bgather = false; p.bscale = false;
    p.M = a.H; p.N = 2 * a.I;
  }
  f32x16 acc[2][2];
  mainloop(p, (p.cnt + BK - 1) / BK, lds, acc);
  epilogue_rows(lds, acc, [&](int rt, int ct, const float (&vv)[8]) {
    const int m = p.m0 + rt, n = p.n0 + ct;
    if (m >= p.M || n >= p.N) return;
    const i32x4 o = pack8(vv);
    if (WHICH == 0) {
      *reinterpret_cast<i32x4*>(a.dwd + ((size_t)e * a.I + m) * a.H + n) = o;
    } else if (n < a.I) {
      *reinterpret_cast<i32x4*>(a.dwg + ((size_t)e * a.H + m) * a.I + n) = o;
    } else {
      *reinterpret_cast<i32x4*>(a.dwu + ((size_t)e * a.H + m) * a.I + (n - a.I)) = o;
    }
  });
}

inline int round8(int n) { return (n + 7) & ~7; }

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  {
    const int nvirt = a.max_tiles * (a.I / 64), nwg = round8(nvirt);
    MOE_LAUNCH("fwd_gateup", k_fwd_gateup, dim3(nwg), dim3(NT), 0, st, a, nvirt, nwg);
  }
  {
    const int nvirt = a.max_tiles * (int)ceil_div(a.H, BN), nwg = round8(nvirt);
    MOE_LAUNCH("fwd_down", k_fwd_down, dim3(nwg), dim3(NT), 0, st, a, nvirt, nwg);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  const int nparts = 2 * (int)ceil_div(a.I, BN);
  if (a.max_tiles > 0) {
    const int nvirt = a.max_tiles * (int)ceil_div(a.I, BN), nwg = round8(nvirt);
    MOE_LAUNCH("bwd_dA", k_bwd_da, dim3(nwg), dim3(NT), 0, st, a, nvirt, nwg, nparts);
  }
  {
    const int tm = (int)ceil_div(a.I, BM), tn = (int)ceil_div(a.H, BN);
    const int nvirt = a.El * tm * tn, nwg = round8(nvirt);
    MOE_LAUNCH("bwd_dWd", k_bwd_wgrad<0>, dim3(nwg), dim3(NT), 0, st, a, tm, tn, nvirt, nwg);
  }
  if (a.max_tiles > 0) {
    const int nvirt = a.max_tiles * (int)ceil_div(a.H, BN), nwg = round8(nvirt);
    MOE_LAUNCH("bwd_dX", k_bwd_dx, dim3(nwg), dim3(NT), 0, st, a, nvirt, nwg);
  }
  {
    const int tm = (int)ceil_div(a.H, BM), tn = (int)ceil_div(2 * a.I, BN);
    const int nvirt = a.El * tm * tn, nwg = round8(nvirt);
    MOE_LAUNCH("bwd_dWgu", k_bwd_wgrad<1>, dim3(nwg), dim3(NT), 0, st, a, tm, tn, nvirt, nwg);
  }
  return hipGetLastError();
}

int bwd_bf16_nparts(int I) { return 2 * (int)ceil_div(I, BN); }

}  // namespace moe
