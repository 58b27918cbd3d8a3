// bf16 MFMA grouped GEMMs of the expert MLP, forward and backward, for gfx950.
//
// Grouped GEMM over each expert's real row count in one launch, shapes read on the
// device (NVIDIA DeepSeek-V3 MoE article, "Optimization 1"); the two expert linear
// layers with SwiGLU between them and the routing-weight scaling fused into the
// GEMMs (Prime Mega MoE pages: one call fusing the linears, SwiGLU and combine, with
// scratch buffers instead of intermediate tensors).
//
// Engine: persistent 512-thread workgroups (8 wave64, one workgroup per CU), 128x256
// output tile, K step 64, each wave a 64x64 sub-tile as four v_mfma_f32_32x32x16_bf16
// accumulators.  Operand tiles move global -> LDS with the gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4) into a three-stage LDS ring, issued two K steps ahead, one
// barrier per K step.  An operand whose contraction axis is contiguous in memory
// ("K-major") is stored [rows][64] and read with 16-byte LDS reads; an operand
// contiguous along M or N ("MN-major": row-major weights as the B of x*W, and both
// operands of the weight gradients, which contract over token rows) is stored
// [64][width] and read with the transposing LDS read ds_read_b64_tr_b16, so no operand
// is transposed in memory.  Both layouts are XOR-swizzled by 16-byte chunk against LDS
// bank conflicts; the swizzle is applied by choosing which global chunk each lane of a
// direct-to-LDS load fetches.
//
// Kernels:
//   K1 fwd_gateup : G = Xp Wg, U = Xp Wu (dual B tile), epilogue saves G|U and A = silu(G) U
//   K2 fwd_down   : Yp = w * (A Wd)
//   B1 bwd_dA     : dA' = dY' Wd^T; epilogue: rowdot(dA', A) partials, SwiGLU backward -> dG|dU,
//                   and w * A for B2
//   B3 bwd_dX     : dXp = dG Wg^T + dU Wu^T (K = 2I)
//   B2 bwd_dWd    : dWd[e] = (w A)_e^T dY'_e over the expert's rows
//   B4 bwd_dWgu   : [dWg | dWu][e] = Xp_e^T [dG | dU]_e over the expert's rows
#include "common.h"

namespace moe {

namespace {

#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8
#endif
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
constexpr int BM = 128, BN = 256, BK = MOE_GEMM_BK;
constexpr int NSTAGE = BK == 64 ? 3 : 6;  // LDS ring stages (48 KB or 24 KB each)
constexpr int DEPTH = NSTAGE - 1;         // K steps in flight ahead of the MFMAs
constexpr int NW = MOE_GEMM_WAVES;   // waves per workgroup: 2 along M x NW/2 along N
constexpr int NTHR = 64 * NW;
constexpr int WN = NW / 2;           // waves along N
constexpr int NI = 8 / WN;           // 32-column accumulator blocks per wave
constexpr int WCOLS = 32 * NI;       // columns per wave
constexpr int A_ELEMS = BM * BK;                  // 8192 bf16
constexpr int B_ELEMS = BN * BK;                  // 16384 bf16
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;    // 48 KB per stage
constexpr int A_LOADS = A_ELEMS * 2 / 16 / NTHR;  // 16-byte loads per thread per stage
constexpr int B_LOADS = B_ELEMS * 2 / 16 / NTHR;
constexpr int LOADS = A_LOADS + B_LOADS;
constexpr int LDS_ELEMS = NSTAGE * STAGE_ELEMS;   // 144 KB
constexpr int IDS_SLOT = 64;                      // ints per index slot (one per lane)
constexpr int IDS_INTS = NW * 2 * IDS_SLOT;       // per wave, two K steps of gathered row indices

// ---- LDS layouts (16-byte chunk granularity) ----
// K-major [rows][BK]: CPR_K chunks per row, RPW rows per 256-byte bank window; chunk c
// of row r lives at c ^ ((r / RPW) % CPR_K), so the 16 rows a 16-byte LDS read touches
// at once fall on distinct banks.
constexpr int CPR_K = BK / 8, RPW = 128 / BK;
__device__ __forceinline__ int kmaj_chunk(int r, int c) { return c ^ ((r / RPW) & (CPR_K - 1)); }
// MN-major [BK][W]: chunk c of k-row r lives at c ^ ((r & 3) << 2).
__device__ __forceinline__ int mnmaj_chunk(int r, int c) { return c ^ ((r & 3) << 2); }

// Slot s of a tile (16 bytes at element offset 8 s) -> (row, logical chunk).
__device__ __forceinline__ void kmaj_slot(int s, int& r, int& c) {
  r = s / CPR_K;
  c = kmaj_chunk(r, s % CPR_K);
}
template <int W>
__device__ __forceinline__ void mnmaj_slot(int s, int& r, int& c) {
  constexpr int CPR = W / 8;
  r = s / CPR;
  c = mnmaj_chunk(r, s % CPR);
}

// Slot written by load q of this thread: each wave instruction fills 64 consecutive
// slots (1 KB), lane l the l-th.
__device__ __forceinline__ int load_slot(int q, int wv, int lane) { return (q * NW + wv) * 64 + lane; }

// Direct-to-LDS loads, written as inline assembly: the wave's 64 lanes each fetch 16
// (or 4) bytes from their own global address into consecutive LDS slots starting at
// the wave-uniform base held in M0.  The compiler does not see these as LDS writes, so
// it adds no waits of its own; the main loop orders them with explicit vmcnt waits.
// M0 is restored after each load.
__device__ __forceinline__ void dma16(const void* g, bf16_t* lds_wave_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((MOE_LDS void*)lds_wave_base));
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(g), "s"(m) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, void* lds_wave_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((MOE_LDS void*)lds_wave_base));
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(g), "s"(m) : "memory");
}

// MFMA 32x32x16 operand fragment: lane l gets 8 consecutive k of row/col (l & 31),
// k = 8 * (l >> 5) .. +7 inside the 16-wide k sub-step kk.
__device__ __forceinline__ bf16x8 frag_kmaj(const bf16_t* s, int base, int kk, int lane) {
  const int r = base + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(s + r * BK + (kmaj_chunk(r, c) << 3));
}

// Same fragment from an MN-major tile of width W with two transposing reads: in each
// 16-lane group g, lane 4j + q points at k-row j of its 4-row slab and columns
// 4q..4q+3 of the group's 16 columns; the hardware hands lane i of the group column i
// of the 4 rows.
template <int W>
__device__ __forceinline__ bf16x8 frag_mnmaj(const bf16_t* s, int base, int kk, int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  const int col = base + 16 * (g & 1) + 4 * q;
  s16x4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = kk * 16 + 8 * (g >> 1) + 4 * h + j;
    const int off = r * W + (mnmaj_chunk(r, col >> 3) << 3) + (col & 7);
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(s + off));
  }
  bf16x8 out;
  __builtin_memcpy(&out, v, 16);
  return out;
}

template <class P>
__device__ __forceinline__ void mma_stage(const bf16_t* st, f32x16 (&acc)[2][NI], int lane, int wm, int wn) {
  const bf16_t* As = st;
  const bf16_t* Bs = st + A_ELEMS;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 af[2], bf[NI];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      af[mi] = P::A_KMAJ ? frag_kmaj(As, wm * 64 + mi * 32, kk, lane) : frag_mnmaj<BM>(As, wm * 64 + mi * 32, kk, lane);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      bf[ni] = P::B_KMAJ ? frag_kmaj(Bs, P::ncol(wn, ni), kk, lane) : frag_mnmaj<BN>(Bs, P::ncol(wn, ni), kk, lane);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
  }
}

// The main loop over nk K steps.  P::issue(kt, stage) issues this thread's P::NVMEM
// direct-to-LDS loads of K step kt and no other vector memory instruction.  Loads run
// two steps ahead (the step index is clamped, so the count in flight is fixed); before
// reading a stage each thread waits for its own loads of that stage, and the barrier
// then makes every thread's loads visible and frees the stage the next loads
// overwrite.  `active` is false for waves whose 64 rows all lie past the tile's valid
// rows: they skip the MFMAs.
template <class P>
__device__ __forceinline__ void mainloop(P& p, int nk, bf16_t* lds, f32x16 (&acc)[2][NI], bool active) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
  if (nk <= 0) return;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) p.issue(min(d, nk - 1), lds + d * STAGE_ELEMS);
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // wait for this thread's loads of step kt (the DEPTH - 1 later steps may still
    // fly) and its LDS reads of step kt - 1, then a plain barrier (__syncthreads()
    // would also wait for every load in flight)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"((DEPTH - 1) * P::NVMEM) : "memory");
    const int nxt = cur == 0 ? NSTAGE - 1 : cur - 1;  // (kt + DEPTH) % NSTAGE: the stage read in step kt - 1
    p.issue(min(kt + DEPTH, nk - 1), lds + nxt * STAGE_ELEMS);
    if (active) mma_stage<P>(lds + cur * STAGE_ELEMS, acc, lane, wm, wn);
    cur = cur == NSTAGE - 1 ? 0 : cur + 1;
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // the trailing duplicate loads
}

// ---- epilogue staging ----
// After the main loop the LDS ring is free.  Each wave writes one 32-row half (mi) of
// its 64 x WCOLS fp32 accumulator to its own [32][EP_LD] region, so that lanes can then
// read 8 consecutive columns of one row and issue 16-byte global loads and stores.
constexpr int EP_LD = WCOLS + 8;  // row stride in floats: rows r and r + 4 fall on disjoint banks
static_assert(NW * 32 * EP_LD * 4 <= LDS_ELEMS * 2, "epilogue staging must fit in the LDS ring");

__device__ __forceinline__ void stage_acc(float* wsm, const f32x16 (&acc)[2][NI], int mi, int lane) {
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
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

// Epilogue walk for the "wn * WCOLS + ni * 32" column mapping: calls
// f(row_in_tile, col_in_tile, v[8]) for every 8-column chunk of this wave's sub-tile;
// the EP_LPR lanes sharing a row are consecutive.
constexpr int EP_LPR = WCOLS / 8;      // lanes per row
constexpr int EP_RPP = 64 / EP_LPR;    // rows per pass
template <class F>
__device__ __forceinline__ void epilogue_rows(bf16_t* lds, const f32x16 (&acc)[2][NI], F&& f) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
  float* wsm = reinterpret_cast<float*>(lds) + wv * 32 * EP_LD;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    stage_acc(wsm, acc, mi, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32 / EP_RPP; ++j) {
      const int rr = lane / EP_LPR + EP_RPP * j, cc = (lane % EP_LPR) * 8;
      float v[8];
      read8(wsm + rr * EP_LD + cc, v);
      f(wm * 64 + mi * 32 + rr, wn * WCOLS + cc, v);
    }
    __syncthreads();
  }
}

// ---- persistent scheduling ----
// Workgroup b runs on XCD b % 8.  The V work items are split into 8 contiguous
// ranges, one per XCD, and the XCD's workgroups walk their range in order, so work
// items sharing operands run together on one XCD and share its L2.
struct Sched {
  int v, hi, step;
  __device__ explicit Sched(int V) {
    const int x = blockIdx.x & 7;
    const int lo = (int)(((int64_t)V * x) >> 3);
    hi = (int)(((int64_t)V * (x + 1)) >> 3);
    v = lo + (int)(blockIdx.x >> 3);
    step = (int)(gridDim.x >> 3);
  }
  __device__ bool more() const { return v < hi; }
  __device__ void next() { v += step; }
};

// Row-group tile: virtual item v -> expert, first row, valid rows and column tile, in
// the expert-major order of the tile table (k_tile_table).
struct RowTile {
  int e, rs, cnt, nt;
};
__device__ __forceinline__ void row_tile(const int32_t* tiles, const int32_t* offsets, int v, int NT, RowTile& t) {
  const int q = v / NT;
  const i32x4 ent = *reinterpret_cast<const i32x4*>(tiles + 4 + 4 * q);
  t.e = ent[0];
  const int local = v - ent[1] * NT;
  const int mt = local % ent[2];
  t.nt = local / ent[2];
  t.rs = offsets[t.e] + mt * BM;
  t.cnt = min(BM, offsets[t.e + 1] - t.rs);
}

// K-major operand with fixed rows: per load q, the row pointer (already offset by the
// lane's chunk) of the slot it fills; step kt adds kt * 64 elements.
template <int NL>
struct KRows {
  const bf16_t* p[NL];
  __device__ void issue(int kt, bf16_t* tile, int wv) const {
#pragma unroll
    for (int q = 0; q < NL; ++q) dma16(p[q] + kt * BK, tile + (q * NW + wv) * 64 * 8);
  }
};

// ---------------- K1: gate/up + SwiGLU ----------------
struct PGateUp {
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  static constexpr int NVMEM = LOADS;
  // gate columns 0..127 and up columns 128..255 of the B tile; wave wn takes the same
  // WCOLS / 2 intermediate columns of both (blocks ni < NI / 2 gate, the rest up), so
  // G and U of one element share a lane
  __device__ static int ncol(int wn, int ni) {
    return (ni < NI / 2 ? 0 : 128) + wn * (WCOLS / 2) + (ni % (NI / 2)) * 32;
  }
  KRows<A_LOADS> a;
  const bf16_t* b[B_LOADS];  // weight row k = 0 of the slot's column
  size_t bstep;              // elements per K step of the weights (64 rows)
  int wv;
  __device__ void issue(int kt, bf16_t* st) const {
    a.issue(kt, st, wv);
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) dma16(b[q] + kt * bstep, st + A_ELEMS + (q * NW + wv) * 64 * 8);
  }
};

__device__ __forceinline__ const bf16_t* a_row_ptr(const bf16_t* x, const bf16_t* xp, const int32_t* row_src,
                                                   int k, int ld, int r) {
  return xp ? xp + (size_t)r * ld : x + (size_t)(row_src[r] / k) * ld;
}

__global__ __launch_bounds__(NTHR, 1) void k_fwd_gateup(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  const int NT = (int)ceil_div(a.I, 128);
  Sched sc(a.tiles[0] * NT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
  for (; sc.more(); sc.next()) {
    RowTile t;
    row_tile(a.tiles, a.offsets, sc.v, NT, t);
    const int n0 = t.nt * 128;
    PGateUp p;
    p.wv = wv;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      p.a.p[q] = a_row_ptr(a.x, a.xp, a.row_src, a.k, a.H, t.rs + min(r, t.cnt - 1)) + c * 8;
    }
    const bf16_t* wg = a.wg + (size_t)t.e * a.H * a.I;
    const bf16_t* wu = a.wu + (size_t)t.e * a.H * a.I;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      int r, c;
      mnmaj_slot<BN>(load_slot(q, wv, lane), r, c);
      int col = n0 + (c & 15) * 8;  // intermediate column; chunks 16..31 are W_up's
      if (col >= a.I) col = n0;      // tail columns: any valid address, results are discarded
      p.b[q] = (c < 16 ? wg : wu) + col + (size_t)r * a.I;
    }
    p.bstep = (size_t)BK * a.I;
    f32x16 acc[2][NI];
    mainloop(p, a.H / BK, lds, acc, wm * 64 < t.cnt);
    // epilogue: lane takes 8 intermediate columns of one row, G from the gate blocks and
    // U from the up blocks (same columns), and writes 16-byte chunks of G, U and A
    constexpr int LPR = WCOLS / 16, RPP = 64 / LPR;
    float* wsm = reinterpret_cast<float*>(lds) + wv * 32 * EP_LD;
    const size_t I2 = 2 * (size_t)a.I;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      stage_acc(wsm, acc, mi, lane);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 32 / RPP; ++j) {
        const int rr = lane / LPR + RPP * j, cc = (lane % LPR) * 8;
        const int rt = wm * 64 + mi * 32 + rr;
        float g[8], u[8], av[8];
        read8(wsm + rr * EP_LD + cc, g);
        read8(wsm + rr * EP_LD + WCOLS / 2 + cc, u);
        const int col = n0 + wn * (WCOLS / 2) + cc;
        if (rt < t.cnt && col < a.I) {
          const size_t r = (size_t)(t.rs + rt);
#pragma unroll
          for (int q = 0; q < 8; ++q) av[q] = silu_f(g[q]) * u[q];
          *reinterpret_cast<i32x4*>(a.gu + r * I2 + col) = pack8(g);
          *reinterpret_cast<i32x4*>(a.gu + r * I2 + a.I + col) = pack8(u);
          *reinterpret_cast<i32x4*>(a.a + r * a.I + col) = pack8(av);
        }
      }
      __syncthreads();
    }
  }
}

// ---------------- K2: down projection * routing weight ----------------
struct PMnB {
  // K-major A rows, MN-major B (row-major weights [K, N])
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  static constexpr int NVMEM = LOADS;
  __device__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  KRows<A_LOADS> a;
  const bf16_t* b[B_LOADS];
  size_t bstep;
  int wv;
  __device__ void issue(int kt, bf16_t* st) const {
    a.issue(kt, st, wv);
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) dma16(b[q] + kt * bstep, st + A_ELEMS + (q * NW + wv) * 64 * 8);
  }
};

__global__ __launch_bounds__(NTHR, 1) void k_fwd_down(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  const int NT = (int)ceil_div(a.H, BN);
  Sched sc(a.tiles[0] * NT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1;
  for (; sc.more(); sc.next()) {
    RowTile t;
    row_tile(a.tiles, a.offsets, sc.v, NT, t);
    const int n0 = t.nt * BN;
    PMnB p;
    p.wv = wv;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      p.a.p[q] = a.a + (size_t)(t.rs + min(r, t.cnt - 1)) * a.I + c * 8;
    }
    const bf16_t* wd = a.wd + (size_t)t.e * a.I * a.H;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      int r, c;
      mnmaj_slot<BN>(load_slot(q, wv, lane), r, c);
      int col = n0 + c * 8;
      if (col >= a.H) col = n0;  // tail columns: any valid address, results are discarded
      p.b[q] = wd + (size_t)r * a.H + col;
    }
    p.bstep = (size_t)BK * a.H;
    f32x16 acc[2][NI];
    mainloop(p, a.I / BK, lds, acc, wm * 64 < t.cnt);
    epilogue_rows(lds, acc, [&](int rt, int ct, const float (&v)[8]) {
      const int col = n0 + ct;
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
}

// ---------------- B1 / B3: both operands K-major ----------------
struct PKK {
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  static constexpr int NVMEM = LOADS;
  __device__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  KRows<A_LOADS> a;
  const bf16_t* b[B_LOADS];   // B rows for K steps [0, ksplit)
  const bf16_t* b2[B_LOADS];  // B3: W_up rows for K steps [ksplit, nk)
  int ksplit;                 // B3: I / 64; B1: larger than any step count
  int wv;
  __device__ void issue(int kt, bf16_t* st) const {
    a.issue(kt, st, wv);
    const bool second = kt >= ksplit;
    const int k0 = (second ? kt - ksplit : kt) * BK;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q)
      dma16((second ? b2[q] : b[q]) + k0, st + A_ELEMS + (q * NW + wv) * 64 * 8);
  }
};

// B1: dA' = dY' Wd^T.  Epilogue: SwiGLU backward on 8 columns per lane, w * A for B2, and
// the rowdot of dA' and A over this wave's 64 columns, reduced across the 8 lanes of a row.
__global__ __launch_bounds__(NTHR, 1) void k_bwd_da(BwdArgs a, int nparts) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  const int NT = (int)ceil_div(a.I, BN);
  Sched sc(a.tiles[0] * NT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
  for (; sc.more(); sc.next()) {
    RowTile t;
    row_tile(a.tiles, a.offsets, sc.v, NT, t);
    const int n0 = t.nt * BN;
    PKK p;
    p.wv = wv;
    p.ksplit = 1 << 30;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      p.a.p[q] = a.dy + (size_t)(a.row_src[t.rs + min(r, t.cnt - 1)] / a.k) * a.H + c * 8;
    }
    const bf16_t* wd = a.wd + (size_t)t.e * a.I * a.H;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      p.b[q] = wd + (size_t)min(n0 + r, a.I - 1) * a.H + c * 8;
      p.b2[q] = p.b[q];
    }
    f32x16 acc[2][NI];
    mainloop(p, a.H / BK, lds, acc, wm * 64 < t.cnt);
    const size_t I2 = 2 * (size_t)a.I;
    epilogue_rows(lds, acc, [&](int rt, int ct, const float (&dap)[8]) {
      const int col = n0 + ct;
      const bool ok = rt < t.cnt && col < a.I;
      float part = 0.f;
      if (ok) {
        const size_t r = (size_t)(t.rs + rt);
        const float w = a.topk_w[a.row_src[r]];
        float g[8], u[8], av[8], dg[8], du[8], aw[8];
        unpack8(*reinterpret_cast<const i32x4*>(a.gu + r * I2 + col), g);
        unpack8(*reinterpret_cast<const i32x4*>(a.gu + r * I2 + a.I + col), u);
        unpack8(*reinterpret_cast<const i32x4*>(a.a + r * a.I + col), av);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          part += dap[q] * av[q];
          aw[q] = w * av[q];
          const float da = w * dap[q];
          const float sg = sigmoid_f(g[q]);
          du[q] = da * g[q] * sg;
          dg[q] = da * u[q] * sg * (1.f + g[q] * (1.f - sg));
        }
        *reinterpret_cast<i32x4*>(a.dgu + r * I2 + col) = pack8(dg);
        *reinterpret_cast<i32x4*>(a.dgu + r * I2 + a.I + col) = pack8(du);
        *reinterpret_cast<i32x4*>(a.aw + r * a.I + col) = pack8(aw);
      }
#pragma unroll
      for (int off = 1; off < EP_LPR; off <<= 1) part += __shfl_xor(part, off, 64);
      if (rt < t.cnt && lane % EP_LPR == 0) a.dw_part[(size_t)(t.rs + rt) * nparts + t.nt * WN + wn] = part;
    });
  }
}

// B3: dXp = dG Wg^T + dU Wu^T, K = 2I: the first I/64 steps read W_gate rows, the rest W_up.
__global__ __launch_bounds__(NTHR, 1) void k_bwd_dx(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  const int NT = (int)ceil_div(a.H, BN);
  Sched sc(a.tiles[0] * NT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1;
  for (; sc.more(); sc.next()) {
    RowTile t;
    row_tile(a.tiles, a.offsets, sc.v, NT, t);
    const int n0 = t.nt * BN;
    PKK p;
    p.wv = wv;
    p.ksplit = a.I / BK;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      p.a.p[q] = a.dgu + (size_t)(t.rs + min(r, t.cnt - 1)) * 2 * a.I + c * 8;
    }
    const size_t woff = (size_t)t.e * a.H * a.I;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      const size_t n = (size_t)min(n0 + r, a.H - 1);
      p.b[q] = a.wg + woff + n * a.I + c * 8;
      p.b2[q] = a.wu + woff + n * a.I + c * 8;
    }
    f32x16 acc[2][NI];
    mainloop(p, 2 * a.I / BK, lds, acc, wm * 64 < t.cnt);
    epilogue_rows(lds, acc, [&](int rt, int ct, const float (&v)[8]) {
      const int col = n0 + ct;
      if (rt < t.cnt && col < a.H)
        *reinterpret_cast<i32x4*>(a.dxp + (size_t)(t.rs + rt) * a.H + col) = pack8(v);
    });
  }
}

// ---------------- weight gradients: contraction over an expert's rows ----------------
// Both operands are MN-major tiles of 64 token rows; rows past the expert's end are
// loaded from a zeroed scratch area.  For a gathered operand (rows of x or dy picked
// by row_src) each wave also copies the 64 row_src entries of a K step into its own
// LDS slot one step ahead, with one more direct-to-LDS load, so the vector memory
// queue holds only direct-to-LDS loads and the counts stay exact.  Within issue(kt)
// the index load of step kt + 1 goes first, and issue(kt + 1) waits for it with
// vmcnt(LOADS): only the six operand loads of step kt may still be in flight.
template <bool AG, bool BG>
struct PWgrad {
  static constexpr bool A_KMAJ = false, B_KMAJ = false;
  static constexpr bool GATHER = AG || BG;
  static constexpr int NVMEM = LOADS + (GATHER ? 1 : 0);
  static constexpr int AR = 4, BR = 2;  // token rows per wave instruction of A and B
  __device__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  const bf16_t* abase; int lda;
  const bf16_t* bbase; int ldb;
  const int32_t* row_src; const bf16_t* zeros; int k;
  int rs, cnt, wv, lane;
  int32_t* ids;                    // this wave's two LDS slots of BK row indices
  int acol[A_LOADS], bcol[B_LOADS];  // element column of the lane's chunk
  __device__ void fetch_ids(int kt) const {  // row_src of step kt -> slot kt & 1
    dma4(row_src + rs + min(kt * BK + lane, cnt - 1), ids + (kt & 1) * IDS_SLOT);
  }
  __device__ void issue(int kt, bf16_t* st) const {
    const int32_t* my = ids + (kt & 1) * IDS_SLOT;
    if (GATHER) {
      if (kt == 0) {
        fetch_ids(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LOADS) : "memory");
      }
    }
    const bf16_t* ap[A_LOADS];
    const bf16_t* bp[B_LOADS];
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      const int kr = (q * NW + wv) * AR + (lane >> 4);
      int row = rs + kt * BK + kr;
      if (AG) row = my[kr] / k;
      ap[q] = kt * BK + kr < cnt ? abase + (size_t)row * lda + acol[q] : zeros;
    }
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      const int kr = (q * NW + wv) * BR + (lane >> 5);
      int row = rs + kt * BK + kr;
      if (BG) row = my[kr] / k;
      bp[q] = kt * BK + kr < cnt ? bbase + (size_t)row * ldb + bcol[q] : zeros;
    }
    if (GATHER) fetch_ids(kt + 1);
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) dma16(ap[q], st + (q * NW + wv) * 64 * 8);
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) dma16(bp[q], st + A_ELEMS + (q * NW + wv) * 64 * 8);
  }
};

template <int WHICH, bool AG, bool BG>
__device__ __forceinline__ void wgrad_tile(const BwdArgs& a, bf16_t* lds, int32_t* ids, int e, int m0, int n0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int M = WHICH == 0 ? a.I : a.H, N = WHICH == 0 ? a.H : 2 * a.I;
  PWgrad<AG, BG> p;
  p.rs = a.offsets[e];
  p.cnt = a.offsets[e + 1] - p.rs;
  p.row_src = a.row_src; p.zeros = a.zeros; p.k = a.k;
  p.wv = wv;
  p.lane = lane;
  p.ids = ids + wv * 2 * IDS_SLOT;
  if (WHICH == 0) {
    p.abase = a.aw; p.lda = a.I;
    p.bbase = a.dy; p.ldb = a.H;
  } else {
    p.abase = AG ? a.x : a.xp; p.lda = a.H;
    p.bbase = a.dgu; p.ldb = 2 * a.I;
  }
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q) {
    int r, c;
    mnmaj_slot<BM>(load_slot(q, wv, lane), r, c);
    const int col = m0 + c * 8;
    p.acol[q] = col < M ? col : m0;
  }
#pragma unroll
  for (int q = 0; q < B_LOADS; ++q) {
    int r, c;
    mnmaj_slot<BN>(load_slot(q, wv, lane), r, c);
    const int col = n0 + c * 8;
    p.bcol[q] = col < N ? col : n0;
  }
  f32x16 acc[2][NI];
  mainloop(p, (p.cnt + BK - 1) / BK, lds, acc, true);
  epilogue_rows(lds, acc, [&](int rt, int ct, const float (&vv)[8]) {
    const int m = m0 + rt, n = n0 + ct;
    if (m >= M || n >= N) return;
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

// B2 (WHICH = 0): dWd[e] [I, H] = (w A)_e^T dY'_e.   B4 (WHICH = 1): [dWg | dWu][e] [H, 2I] = Xp_e^T [dG | dU]_e.
// B2 (WHICH = 0): dWd[e] [I, H] = (w A)_e^T dY'_e.   B4 (WHICH = 1): [dWg | dWu][e] [H, 2I] = Xp_e^T [dG | dU]_e.
template <int WHICH>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_wgrad(BwdArgs a, int tm, int tn) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) int32_t ids[IDS_INTS];
  for (Sched sc(a.El * tm * tn); sc.more(); sc.next()) {
    const int e = sc.v / (tm * tn);
    const int rem = sc.v - e * tm * tn;
    const int mt = rem / tn, nt = rem - mt * tn;
    if (WHICH == 0) wgrad_tile<0, false, true>(a, lds, ids, e, mt * BM, nt * BN);
    else if (a.xp) wgrad_tile<1, false, false>(a, lds, ids, e, mt * BM, nt * BN);
    else wgrad_tile<1, true, false>(a, lds, ids, e, mt * BM, nt * BN);
  }
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// persistent grid: at most one workgroup per CU, a multiple of 8 (one share per XCD)
inline int grid_for(int64_t work) {
  int g = num_cus();
  if (work < g) g = (int)work;
  g = (g + 7) & ~7;
  return g < 8 ? 8 : g;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MOE_LAUNCH("fwd_gateup", k_fwd_gateup, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.I, 128))), dim3(NTHR), 0, st,
             a);
  MOE_LAUNCH("fwd_down", k_fwd_down, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.H, BN))), dim3(NTHR), 0, st, a);
  return hipGetLastError();
}

int bwd_bf16_nparts(int I) { return WN * (int)ceil_div(I, BN); }

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  const int nparts = bwd_bf16_nparts(a.I);
  if (a.max_tiles > 0)
    MOE_LAUNCH("bwd_dA", k_bwd_da, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.I, BN))), dim3(NTHR), 0, st, a,
               nparts);
  {
    const int tm = (int)ceil_div(a.I, BM), tn = (int)ceil_div(a.H, BN);
    MOE_LAUNCH("bwd_dWd", k_bwd_wgrad<0>, dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st, a, tm, tn);
  }
  if (a.max_tiles > 0)
    MOE_LAUNCH("bwd_dX", k_bwd_dx, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.H, BN))), dim3(NTHR), 0, st, a);
  {
    const int tm = (int)ceil_div(a.H, BM), tn = (int)ceil_div(2 * a.I, BN);
    MOE_LAUNCH("bwd_dWgu", k_bwd_wgrad<1>, dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st, a, tm, tn);
  }
  return hipGetLastError();
}

}  // namespace moe
