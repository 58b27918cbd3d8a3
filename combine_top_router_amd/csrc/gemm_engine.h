// Shared GEMM engine of the bf16 and MXFP8 grouped GEMMs (internal header).
//
// Persistent 512-thread workgroups (8 wave64, one workgroup per CU), 128x256 output
// tile, each wave a 64x64 sub-tile as 32x32 MFMA accumulator blocks.  Operand tiles
// move global -> LDS with the gfx950 direct-to-LDS loads (global_load_lds_dwordx4)
// into an LDS ring, issued DEPTH K steps ahead, one barrier per K step.  An operand
// whose contraction axis is contiguous in memory ("K-major") is stored [rows][BK] and
// read with 16-byte LDS reads; an operand contiguous along M or N ("MN-major") is
// stored [BK][width] and read with the transposing LDS read ds_read_b64_tr_b16.  Both
// layouts are XOR-swizzled by 16-byte chunk against LDS bank conflicts; the swizzle is
// applied by choosing which global chunk each lane of a direct-to-LDS load fetches.
#pragma once

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

// bf16 policies: the MFMAs of one stage
template <class Derived>
struct Bf16Mma {
  __device__ void compute(const bf16_t* st, int, f32x16 (&acc)[2][NI], int lane, int wm, int wn) const {
    mma_stage<Derived>(st, acc, lane, wm, wn);
  }
};

// The main loop over nk K steps.  P::issue(kt, stage, slot) issues this thread's P::NVMEM
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
  for (int d = 0; d < DEPTH; ++d) p.issue(min(d, nk - 1), lds + d * STAGE_ELEMS, d);
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // wait for this thread's loads of step kt (the DEPTH - 1 later steps may still
    // fly) and its LDS reads of step kt - 1, then a plain barrier (__syncthreads()
    // would also wait for every load in flight)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"((DEPTH - 1) * P::NVMEM) : "memory");
    const int nxt = cur == 0 ? NSTAGE - 1 : cur - 1;  // (kt + DEPTH) % NSTAGE: the stage read in step kt - 1
    p.issue(min(kt + DEPTH, nk - 1), lds + nxt * STAGE_ELEMS, nxt);
    if (active) p.compute(lds + cur * STAGE_ELEMS, cur, acc, lane, wm, wn);
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
}  // namespace moe
