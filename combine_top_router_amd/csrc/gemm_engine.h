// Shared GEMM engine of the bf16 and MXFP8 grouped GEMMs (internal header).
//
// Persistent workgroups (one per CU) of eight waves.  BM x 256 output tile (BM = 256 or
// 320 rows, one build each), each wave a (BM / 2) x 64 sub-tile as 32x32 MFMA
// accumulator blocks.  Operand tiles move global -> LDS with the gfx950 direct-to-LDS
// loads (global_load_lds_dwordx4) into a two-stage ring, one barrier per K step: every
// wave issues one eighth of the next step's loads, then computes the current one (the
// fused stream).  An operand whose contraction axis is contiguous in memory ("K-major")
// is stored [rows][BK] and read with 16-byte LDS reads; an operand contiguous along M or
// N ("MN-major") is stored [BK][width] and read with the transposing LDS read
// ds_read_b64_tr_b16.  Both layouts are XOR-swizzled by 16-byte chunk against LDS bank
// conflicts; the swizzle is applied by choosing which global chunk each lane of a load
// fetches.
//
// A workgroup's tiles form one stream of K steps: the loads of the next tile's first
// step are issued while the current tile's last step computes, and the current tile's
// epilogue runs in the ring stage that its last step freed while those loads are in
// flight.  Tile descriptors and gathered row indices are read with scalar loads.
#pragma once

#include "common.h"

namespace moe {
namespace {

// The tile height is the translation unit's MOE_GEMM_FW (256 in gemm_fw256.hip, 320 in
// gemm_fw320.hip): 256 or 320 rows of 256 columns, 64 or 72 KB stages.  Eight waves per CU
// leave each 256 registers, room for up to 160 accumulators.
#if MOE_GEMM_FW != 256 && MOE_GEMM_FW != 320
#error "gemm.hip is compiled through gemm_fw256.hip or gemm_fw320.hip"
#endif
constexpr int BM = MOE_GEMM_FW, BN = 256, BK = 64;
constexpr int NSTAGE = 2;            // LDS ring stages
constexpr int DEPTH = NSTAGE - 1;    // K steps in flight ahead of the MFMAs
constexpr int NW = 8;                // waves: 2 along M x 4 along N
constexpr int NP = NW;               // every wave issues its share of each step's loads
constexpr int NTHR = 64 * NW;
constexpr int WM = 2;                // waves along M
constexpr int WN = NW / WM;          // waves along N
constexpr int MI = BM / (32 * WM);   // 32-row accumulator blocks per wave
constexpr int NI = BN / (32 * WN);   // 32-column accumulator blocks per wave
constexpr int WROWS = 32 * MI;       // rows per wave
constexpr int WCOLS = 32 * NI;       // columns per wave
constexpr int A_ELEMS = BM * BK;
constexpr int B_ELEMS = BN * BK;
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
constexpr int A_INSTR = A_ELEMS * 2 / 1024;       // 1 KB wave loads per stage, of A
constexpr int B_INSTR = B_ELEMS * 2 / 1024;       // and of B
constexpr int A_LP = A_INSTR / NP;                // per wave
constexpr int B_LP = B_INSTR / NP;
constexpr int LDS_ELEMS = NSTAGE * STAGE_ELEMS;
using Acc = f32x16[MI][NI];                       // a wave's accumulators
static_assert(MI * NI * 16 <= 160, "accumulators of one wave");
static_assert(A_LP * NP == A_INSTR && B_LP * NP == B_INSTR, "wave loads divide among the waves");
constexpr int IDS_SLOT = 64;                      // ints per index slot (one per lane)
constexpr int IDS_INTS = NP * 2 * IDS_SLOT;       // per wave, two positions of gathered row indices

// ---- scalar loads ----
// A wave-uniform load through the scalar data cache (address space 4): it is counted
// by lgkmcnt, not vmcnt.  The address is made wave-uniform.
template <class T>
__device__ __forceinline__ T sload(const T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return *(const __attribute__((address_space(4))) T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

// Wave load q of load wave pw is instruction q * NP + pw of its region; instruction I
// fills slots 64 I .. 64 I + 63 (1 KB), lane l the l-th.
__device__ __forceinline__ int load_instr(int q, int pw) { return q * NP + pw; }
__device__ __forceinline__ int load_slot(int q, int pw, int lane) { return load_instr(q, pw) * 64 + lane; }

// Direct-to-LDS loads, written as inline assembly: the wave's 64 lanes each fetch 16
// (or 4) bytes from their own global address into consecutive LDS slots starting at
// the wave-uniform base held in M0.  The compiler does not see these as LDS writes, so
// it adds no waits of its own; the stream orders them with explicit vmcnt waits.
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
// LDS address of wave load q of load wave pw in the A or B region of a stage
__device__ __forceinline__ bf16_t* a_dst(bf16_t* st, int q, int pw) { return st + load_instr(q, pw) * 512; }
__device__ __forceinline__ bf16_t* b_dst(bf16_t* st, int q, int pw) { return st + A_ELEMS + load_instr(q, pw) * 512; }


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

// The rows [base, end) of a row tile of cnt rows that compute wave row wm holds, in nblk
// 32-row accumulator blocks with rows (wave-uniform): wave row wm takes rows
// wm * WROWS .. + WROWS - 1.  A wave without rows (nblk = 0) skips its MFMAs.
struct WaveRows {
  int base, end, nblk;
};
__device__ __forceinline__ WaveRows wave_rows(int cnt, int wm) {
  const int b = wm * WROWS, e = min(cnt, b + WROWS);
  return {b, e, e > b ? (e - b + 31) >> 5 : 0};
}

// The bf16 MFMAs of one stage for a job J (J::A_KMAJ, J::B_KMAJ, J::ncol) over the
// wave's MI 32-row blocks from row w.base (blocks past w.nblk compute on rows that the
// tile does not hold and their results are discarded: skipping them by branch measured
// slower).  With J::TRANS
// the two fragments enter the MFMA in swapped roles, so that each 32x32 accumulator block
// holds the transpose of its block of C (see trans_chunks).
template <class J>
__device__ __forceinline__ void mma_stage(const bf16_t* st, Acc& acc, int lane, const WaveRows& w, int wn) {
  const bf16_t* As = st;
  const bf16_t* Bs = st + A_ELEMS;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 af[MI], bf[NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      af[mi] = J::A_KMAJ ? frag_kmaj(As, w.base + mi * 32, kk, lane) : frag_mnmaj<BM>(As, w.base + mi * 32, kk, lane);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      bf[ni] = J::B_KMAJ ? frag_kmaj(Bs, J::ncol(wn, ni), kk, lane) : frag_mnmaj<BN>(Bs, J::ncol(wn, ni), kk, lane);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = J::TRANS ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[ni], af[mi], acc[mi][ni], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    // 320-row fused stream: the next sub-step's fragments are not read ahead of these
    // MFMAs (160 accumulators leave no room for them; the SIMD's other wave fills the
    // LDS wait)
    if constexpr (MI > 4) __builtin_amdgcn_sched_barrier(0);
  }
}

// A transposed accumulator block as bf16 row chunks.  The 32x32 MFMA leaves row
// 8 (r / 4) + 4 (l / 32) + r % 4 and column l % 32 of its result in register r of lane l;
// for a block accumulated with swapped operands (J::TRANS) that result is C^T, so lane l
// holds row l % 32 of C and, in registers 4q .. 4q + 3, its columns 8q + 4 (l / 32) .. + 3.
// Packed to bf16 pairs, lanes l and l + 32 trade halves with v_permlane32_swap (which
// swaps lanes 32..63 of its first operand with lanes 0..31 of its second), after which
// lane l holds two 16-byte chunks of its row: chunk s = columns 16 s + 8 (l / 32) .. + 7.
__device__ __forceinline__ void trans_chunks(const f32x16& a, i32x4 (&out)[2]) {
  uint32_t d[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    d[q][0] = pk_bf16(a[4 * q], a[4 * q + 1]);
    d[q][1] = pk_bf16(a[4 * q + 2], a[4 * q + 3]);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const auto r = __builtin_amdgcn_permlane32_swap(d[2 * s][c], d[2 * s + 1][c], false, false);
      d[2 * s][c] = r[0];
      d[2 * s + 1][c] = r[1];
    }
    out[s] = i32x4{(int)d[2 * s][0], (int)d[2 * s][1], (int)d[2 * s + 1][0], (int)d[2 * s + 1][1]};
  }
}

// One 32-row band (accumulator block row mi) of a wave's sub-tile, given as trans_chunks
// output ch[b][s] of NB 32-column blocks (lane l: row l % 32, 16-byte chunk
// 4 b + 2 s + l / 32 of the row's NCH = 4 NB chunks), passes through the wave's own LDS
// region [32][8 NCH] bf16 so that afterwards NCH consecutive lanes hold the NCH chunks of
// one row: store(row_in_band, column_in_band, chunk) is called for rows lane / NCH +
// (64 / NCH) j, and one store instruction writes whole row segments of 16 NCH bytes.
// Chunk c of row r sits at slot c ^ band_swz(r).  A write puts one chunk of 32
// consecutive rows; band_swz gives any 8 consecutive rows distinct 16-byte slots of a
// 128-byte window and any 16 distinct slots of a 256-byte window (rows of 128 bytes: the
// row parity picks the window half; of 64 bytes: r % 4 picks the quarter), which is what
// keeps 16-byte LDS writes free of bank conflicts on gfx950 (the form c ^ (r / 2), free
// for 16-byte reads, measured 16 % conflicted cycles in the weight gradients).  A read
// takes whole rows, so any swizzle keeps it conflict-free.
static_assert(WCOLS == 64, "a band row holds at most 8 chunks of 16 bytes");
constexpr int BAND_ELEMS = 32 * WCOLS;  // per wave
static_assert(NW * BAND_ELEMS <= STAGE_ELEMS, "the bands of all waves fit in one ring stage");
template <int NCH>
__device__ __forceinline__ int band_swz(int r) {
  static_assert(NCH == 4 || NCH == 8, "rows of 64 or 128 bytes");
  if constexpr (NCH == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}
template <int NB, class F>
__device__ __forceinline__ void band_store(bf16_t* wreg, const i32x4 (&ch)[NB][2], F&& store) {
  constexpr int NCH = 4 * NB, W = 8 * NCH;
  static_assert(NB == 1 || NB == 2, "one or two 32-column blocks per band row");
  const int lane = threadIdx.x & 63, r = lane & 31;
  const int swr = band_swz<NCH>(r);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = b * 4 + 2 * s + (lane >> 5);
      *reinterpret_cast<i32x4*>(wreg + r * W + ((c ^ swr) << 3)) = ch[b][s];
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  i32x4 v[NCH / 2];
  const int rr0 = lane / NCH, cc = lane % NCH;
#pragma unroll
  for (int j = 0; j < NCH / 2; ++j) {
    const int rr = rr0 + (64 / NCH) * j;
    v[j] = *reinterpret_cast<const i32x4*>(wreg + rr * W + ((cc ^ band_swz<NCH>(rr)) << 3));
  }
#pragma unroll
  for (int j = 0; j < NCH / 2; ++j) store(lane / NCH + (64 / NCH) * j, (lane % NCH) * 8, v[j]);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the region is free for the next band
}

// The row-wise MXFP8 codes of a transposed accumulator block's 32 columns of row l % 32
// (the rows' values x in fp32, in the trans_chunks layout): lanes l and l + 32 together
// hold the row's 32 values, so the block's maximum takes one v_permlane32_swap; the
// codes (E4M3 of x / 2^X, X the block's scale exponent) are rearranged as trans_chunks
// does, after which lane l holds codes of columns 16 (l / 32) .. + 15 of its row.
__device__ __forceinline__ i32x4 mx_row_codes(const f32x16& x, int& X) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am), false, false);
  am = fmaxf(am, __uint_as_float((threadIdx.x & 32) ? pr[0] : pr[1]));
  X = mx_scale_exp(am);
  uint32_t e[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) e[q] = e4m3_pack4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3], X);
  const auto s02 = __builtin_amdgcn_permlane32_swap(e[0], e[2], false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(e[1], e[3], false, false);
  return i32x4{(int)s02[0], (int)s02[1], (int)s13[0], (int)s13[1]};
}

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
}

// ---- persistent scheduling ----
// Workgroup b runs on XCD b % 8.  Two ways to hand out the V work items:
// * contiguous: the items are split into 8 contiguous ranges, one per XCD, and the
//   XCD's workgroups walk their range in order, so work items sharing operands run
//   together on one XCD and share its L2 (what a job of equal-cost items wants);
// * dynamic, for items sorted by cost, largest first: workgroup b starts with item w,
//   its XCD-major rank (b % 8) (G / 8) + b / 8, and each further item is G plus the old
//   value of a counter that the launch's G workgroups share, taken when the workgroup
//   starts its current tile: greedy longest-first, so a workgroup that finishes early
//   takes the costliest item left and every workgroup ends within about one item of
//   the others.  Wave 0 takes the item at the tile's first position and publishes it in
//   LDS; the waves read it there at the tile's next-to-last position, so a dynamic tile
//   spans at least DEPTH + 2 stream positions.
// Jobs with DYN = true choose per launch (J::dynamic(), a uniform device flag, and
// J::counter(), zero before the launch).
// Column halves (contiguous ranges of a job with NSPLIT): when the last round of an XCD's
// range is at most half full (rem items for its G / 8 workgroups, 2 rem <= G / 8), each of
// those rem tiles is handed out as two halves of BN / 2 columns, so that the round keeps
// every workgroup busy on about half a tile instead of half the workgroups on whole ones.
// A half computes its own output columns (no partial sums to combine), so results do not
// change.  The stream walks work indices u; enc(u) is the job's value: the item, or for
// NSPLIT jobs item * 4 + hs with hs = 0 (whole tile), 1 (left half) or 2 (right half).
template <bool DYN, bool NSPLIT = false>
struct Sched {
  int v;          // the workgroup's first work index; < 0: none
  int hi;         // contiguous: end of the XCD's work indices; dynamic: V
  int step;       // contiguous: stride
  int g;          // grid size
  bool dyn;
  int32_t* ctr;   // dynamic: the launch's item counter
  int lo;         // contiguous: the XCD's first item
  int whole;      // contiguous: work indices below it are whole tiles
  __device__ Sched(int V, bool dynamic, int32_t* counter) {
    const int x = blockIdx.x & 7;
    dyn = DYN && dynamic;
    ctr = counter;
    g = (int)gridDim.x;
    lo = 0;
    whole = 0;
    if (dyn) {
      const int w = x * (g >> 3) + (int)(blockIdx.x >> 3);
      hi = V;
      step = 0;
      v = w < V ? w : -1;
    } else {
      lo = (int)(((int64_t)V * x) >> 3);
      const int n = (int)(((int64_t)V * (x + 1)) >> 3) - lo;
      step = (int)(gridDim.x >> 3);
      whole = n;
      hi = n;
      if constexpr (NSPLIT) {
        const int R = n / step, rem = n - R * step;
        if (rem > 0 && 2 * rem <= step) {
          whole = R * step;
          hi = whole + 2 * rem;
        }
      }
      v = (int)(blockIdx.x >> 3);
      if (v >= hi) v = -1;
    }
  }
  // the job's value of work index u
  __device__ __forceinline__ int enc(int u) const {
    if (dyn) return u;
    if constexpr (NSPLIT) {
      if (u < whole) return (lo + u) << 2;
      const int h = u - whole;
      return ((lo + whole + (h >> 1)) << 2) | (1 + (h & 1));
    } else {
      return lo + u;
    }
  }
  // stream positions a tile of nk K steps takes
  __device__ __forceinline__ int len(int nk) const { return max(nk, dyn ? DEPTH + 2 : DEPTH + 1); }
  // contiguous: the work index after u (one of this workgroup's), or -1
  __device__ __forceinline__ int next(int u) const {
    const int n = u + step;
    return n < hi ? n : -1;
  }
  // dynamic: the next item from the shared counter, or -1 (one lane calls it)
  __device__ __forceinline__ int grab() const {
    const int n = g + atomicAdd(ctr, 1);
    return n >= g && n < hi ? n : -1;
  }
};

// ---- the tile stream ----
// A workgroup's tiles form one stream of K steps ("positions"); every tile takes
// Sched::len(nk) positions (max(nk, DEPTH + 1), or DEPTH + 2 under dynamic scheduling),
// positions past nk repeating a valid step's loads and skipping the MFMAs.
//
// A job J supplies: items(); the compute side -- Tile, tile(v, Tile&) (what the epilogue
// needs, scalar loads only), rows(const Tile&, wm) (the WaveRows of wave row wm),
// compute(stage pointer, stage index, acc, lane, WaveRows, wn) and epilogue(const Tile&,
// acc, staging); and the load side -- Ld, setup(v, Ld&, pw, lane) and Ld::GATHER,
// Ld::issue(kt, stage pointer, stage index, parity, fetch_next) and Ld::fetch(kt,
// parity) (fetch_next, when the loader calls it, fetches the row indices of the next
// position into the other index slot); a gathering loader's job also supplies
// fetch_first(v, pw, lane, parity), the row indices of item v's first step.
// The fused stream: every wave is compute wave wv and load wave wv, with one K step
// in flight.  At each position a wave waits for everything it has issued (its loads of
// the position and its index fetch for the next, and any epilogue stores), meets the
// other waves at the barrier (after which the position's stage is complete and the
// stage read one position ago is free), issues its loads of the next position into that
// free stage and runs the position's MFMAs.  After a tile's last position the waves meet
// once more and run the epilogue in the stage just read, which the next issue refills
// only after the next barrier.  Tiles may differ in K steps (Sched::len).  The next tile
// is fixed at the current tile's next-to-last position: at once for contiguous ranges;
// under dynamic scheduling wave 0 takes it at the tile's first position and publishes it
// in LDS, and the waves read it after a later barrier (a dynamic tile spans at least
// DEPTH + 2 positions).  The loads of that next-to-last position also fetch the next
// tile's first row indices for a gathering loader (J::fetch_first); the loader is set up
// for the next tile in place when its first loads are issued.
template <class J, class S>
__device__ __forceinline__ void fused_stream(const J& job, bf16_t* lds, S sc, int wv, int lane) {
  static_assert(DEPTH == 1, "the fused stream keeps one K step in flight");
  using P = typename J::Ld;
  using T = typename J::Tile;
  const int wm = (int)((unsigned)wv % WM), wn = (int)((unsigned)wv / WM);
  int32_t* slot = nullptr;   // dynamic: two LDS slots for the next item, by tile parity
  if constexpr (J::DYN) slot = job.dslot;
  auto clampk = [](int kt, int nk) { return max(0, min(kt, nk - 1)); };
  // an opaque copy of the lane index for the per-tile load setup: the per-lane load
  // offsets are recomputed per tile rather than held in registers across the stream
  auto setup = [&](int item, P& L) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    job.setup(item, L, wv, ln);
  };
  P lcur;
  T cur;
  int v = sc.v, vn = -1;   // work indices (sc.enc gives the job's value)
  setup(sc.enc(v), lcur);
  job.tile(sc.enc(v), cur);
  WaveRows wr = job.rows(cur, wm);
  if constexpr (J::NSPLIT)
    if (wn * WCOLS >= cur.ncols) wr.nblk = 0;   // a column half: this wave's columns lie outside it
  int len = sc.len(cur.nk);
  bool has_nxt = false;
  int gpar = 0;   // index slot of the next issue
  if (P::GATHER) {
    lcur.fetch(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  lcur.issue(0, lds, 0, gpar, [&] { lcur.fetch(1, gpar ^ 1); });   // len >= 2
  gpar ^= 1;
  Acc acc;
  zero_acc(acc);
  int cs = 0, grabbed = 0;
  for (int t = 0;; ++t) {
    for (int kc = 0; kc < len; ++kc) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (sc.dyn && kc == 0 && wv == 0 && lane == 0) grabbed = sc.grab();
      if (kc + 2 == len) {   // the next tile, before the issue that fetches its first indices
        vn = sc.dyn ? uni(slot[t & 1]) : sc.next(v);
        has_nxt = vn >= 0;
      }
      bf16_t* const st = lds + (cs ^ 1) * STAGE_ELEMS;   // NSTAGE = 2: the stage freed
      if (kc + 1 < len) {
        const int k1 = kc + 1;
        lcur.issue(clampk(k1, lcur.nk), st, cs ^ 1, gpar, [&] {
          if (k1 + 1 < len) {
            lcur.fetch(clampk(k1 + 1, lcur.nk), gpar ^ 1);
          } else if (has_nxt) {
            if constexpr (P::GATHER) job.fetch_first(sc.enc(vn), wv, lane, gpar ^ 1);
          } else {
            lcur.fetch(clampk(k1, lcur.nk), gpar ^ 1);
          }
        });
        gpar ^= 1;
      } else if (has_nxt) {
        setup(sc.enc(vn), lcur);
        lcur.issue(0, st, cs ^ 1, gpar, [&] { lcur.fetch(1, gpar ^ 1); });
        gpar ^= 1;
      }
      // extra work of every wave on the position's stage, ahead of its MFMAs so that its
      // stores are on their way long before the next position's wait
      if constexpr (J::SIDE)
        if (kc < cur.nk) job.side(lds + cs * STAGE_ELEMS, cur, kc, wv * 64 + lane);
      if (kc < cur.nk && wr.nblk > 0) job.compute(lds + cs * STAGE_ELEMS, cs, acc, lane, wr, wn);
      if (sc.dyn && kc == 0 && wv == 0) {   // published after the MFMAs, read after a barrier
        const int n = uni(grabbed);
        if (lane == 0) slot[t & 1] = n;
      }
      cs ^= 1;
    }
    if constexpr (J::EPI_LDS) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    bool epi = true;
    if constexpr (J::NSPLIT) epi = wn * WCOLS < cur.ncols;
    if (epi) job.epilogue(cur, acc, reinterpret_cast<float*>(lds + (cs ^ 1) * STAGE_ELEMS));
    zero_acc(acc);
    if (!has_nxt) break;
    v = vn;
    has_nxt = false;
    job.tile(sc.enc(v), cur);
    wr = job.rows(cur, wm);
    if constexpr (J::NSPLIT)
      if (wn * WCOLS >= cur.ncols) wr.nblk = 0;
    len = sc.len(cur.nk);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class J>
__device__ __forceinline__ void run_stream(const J& job, bf16_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wv = uni(tid >> 6);
  bool dyn = false;
  int32_t* ctr = nullptr;
  if constexpr (J::DYN) {
    dyn = job.dynamic();
    ctr = job.counter();
  }
  Sched<J::DYN, J::NSPLIT> sc(job.items(), dyn, ctr);
  if (sc.v < 0) return;
  fused_stream(job, lds, sc, wv, lane);
}

// ---- epilogue staging ----
// Each wave stages 16-row pieces of its WROWS x WCOLS fp32 accumulator in its own
// [16][EP_LD] region of the free ring stage, so that lanes can then read 8 consecutive
// columns of one row and issue 16-byte global loads and stores.  The regions are
// private to their waves, so no workgroup barrier is needed between quarters.
constexpr int EP_LD = WCOLS + 8;  // row stride in floats: rows r and r + 4 fall on disjoint banks
constexpr int EP_ROWS = 16;
static_assert(NW * EP_ROWS * EP_LD * 4 <= STAGE_ELEMS * 2, "epilogue staging must fit in one ring stage");

// stage rows 16 h .. 16 h + 15 of accumulator block row mi (registers 8 h .. 8 h + 7)
__device__ __forceinline__ void stage_quarter(float* wsm, const Acc& acc, int mi, int h, int lane) {
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      wsm[r * EP_LD + ni * 32 + (lane & 31)] = acc[mi][ni][8 * h + i];
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void staging_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 8 consecutive floats of staged row r: the rows lie EP_LD * 4 = 288 bytes apart (32 mod
// 256), so in one 16-byte read the lanes of rows r and r + 1 would meet on the same banks;
// odd rows read their two halves in the other order, which puts them on the other banks
__device__ __forceinline__ void read8(const float* p, int r, float (&v)[8]) {
  const int h = (r & 1) * 4;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + h);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + (4 - h));
  v[0] = h ? b[0] : a[0]; v[1] = h ? b[1] : a[1]; v[2] = h ? b[2] : a[2]; v[3] = h ? b[3] : a[3];
  v[4] = h ? a[0] : b[0]; v[5] = h ? a[1] : b[1]; v[6] = h ? a[2] : b[2]; v[7] = h ? a[3] : b[3];
}

__device__ __forceinline__ i32x4 pack8(const float (&v)[8]) {
  i32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (int)pk_bf16(v[2 * q], v[2 * q + 1]);
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
// f(row_in_tile, col_in_tile, v[8], slot) for every 8-column chunk of this wave's
// sub-tile (slot numbers the lane's rows, see ep_row); the EP_LPR lanes sharing a row
// are consecutive.
constexpr int EP_LPR = WCOLS / 8;      // lanes per row
constexpr int EP_RPP = 64 / EP_LPR;    // rows per pass
// With UNROLL the row passes of a staged piece are unrolled, so their LDS reads and
// global stores can overlap (jobs with small epilogues; the heavy ones keep them rolled
// to stay within the register budget).
template <bool UNROLL = false, class F>
__device__ __forceinline__ void epilogue_rows(float* stage, const Acc& acc, const WaveRows& w, F&& f) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wn = (int)((unsigned)wv / WM);
  float* wsm = stage + wv * EP_ROWS * EP_LD;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      stage_quarter(wsm, acc, mi, h, lane);
      if constexpr (UNROLL) {
        float v[EP_ROWS / EP_RPP][8];
#pragma unroll
        for (int j = 0; j < EP_ROWS / EP_RPP; ++j)
          read8(wsm + (lane / EP_LPR + EP_RPP * j) * EP_LD + (lane % EP_LPR) * 8, lane / EP_LPR + EP_RPP * j, v[j]);
#pragma unroll
        for (int j = 0; j < EP_ROWS / EP_RPP; ++j)
          f(w.base + mi * 32 + h * 16 + lane / EP_LPR + EP_RPP * j, wn * WCOLS + (lane % EP_LPR) * 8, v[j],
            (mi * 2 + h) * (EP_ROWS / EP_RPP) + j);
      } else {
#pragma unroll 1
        for (int j = 0; j < EP_ROWS / EP_RPP; ++j) {
          const int rr = lane / EP_LPR + EP_RPP * j, cc = (lane % EP_LPR) * 8;
          float v[8];
          read8(wsm + rr * EP_LD + cc, rr, v);
          f(w.base + mi * 32 + h * 16 + rr, wn * WCOLS + cc, v, (mi * 2 + h) * (EP_ROWS / EP_RPP) + j);
        }
      }
      staging_done();
    }
}

// Row-group tile: virtual item v -> expert, first row, valid rows and column tile, in
// the expert-major order of the tile table (k_tile_table).  Scalar loads only.
struct RowTile {
  int e, rs, cnt, nt;
  int mt, nmt;   // the tile's index among its expert's row tiles, and their number
};
__device__ __forceinline__ void row_tile(const int32_t* tiles, const int32_t* offsets, int v, int NT, RowTile& t) {
  const int q = uni(v / NT);
  const i32x4 ent = sload(reinterpret_cast<const i32x4*>(tiles + 4 + 4 * q));
  t.e = uni(ent[0]);
  const int local = uni(v - ent[1] * NT);
  const int mt = uni(local % ent[2]);
  t.nt = uni(local / ent[2]);
  const int o0 = sload(offsets + t.e), o1 = sload(offsets + t.e + 1);
  t.mt = mt;
  t.nmt = uni(ent[2]);
  t.rs = uni(o0 + mt * BM);
  t.cnt = uni(min(BM, o1 - t.rs));
}

// Row-source indices of the A rows a load wave's K-major loads cover (load q fills rows
// 8 I .. 8 I + 7 of the tile, I = q * NP + pw, lane l row 8 I + l / 8), clamped to the
// tile's valid rows, read with scalar loads and selected per lane.
__device__ __forceinline__ void gather_rows_a(const int32_t* row_src, const RowTile& t, int pw, int lane,
                                              int (&src)[A_LP]) {
  static_assert(CPR_K == 8, "a wave load covers 8 rows of 8 chunks");
  const int j = lane >> 3;
#pragma unroll
  for (int q = 0; q < A_LP; ++q) {
    const int r0 = load_instr(q, pw) * 8;
    int s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = sload(row_src + t.rs + min(r0 + i, t.cnt - 1));
    const int lo = (j & 1) ? s[1] : s[0], lo2 = (j & 1) ? s[3] : s[2];
    const int hi = (j & 1) ? s[5] : s[4], hi2 = (j & 1) ? s[7] : s[6];
    const int a = (j & 2) ? lo2 : lo, b = (j & 2) ? hi2 : hi;
    src[q] = (j & 4) ? b : a;
  }
}

// K-major operand with fixed rows: per wave load q, the row pointer (already offset by
// the lane's chunk) of the slot it fills; step kt adds kt * 64 elements.
struct KRows {
  const bf16_t* p[A_LP];
  __device__ __forceinline__ void dma(int kt, bf16_t* st, int pw) const {
#pragma unroll
    for (int q = 0; q < A_LP; ++q) dma16(p[q] + kt * BK, a_dst(st, q, pw));
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
