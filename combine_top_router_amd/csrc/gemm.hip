// bf16 and MXFP8 MFMA grouped GEMMs of the expert MLP, forward and backward, for gfx950.
//
// Grouped GEMM over each expert's real row count in one launch, shapes read on the
// device (NVIDIA DeepSeek-V3 MoE article, "Optimization 1"); the two expert linear
// layers with SwiGLU between them and the routing-weight scaling fused into the
// GEMMs (Prime Mega MoE pages: one call fusing the linears, SwiGLU and combine, with
// scratch buffers instead of intermediate tensors).
//
// Engine (gemm_engine.h): persistent workgroups (one per CU), BM x 256 output tile, K
// step 64, each of 8 waves a (BM / 2) x 64 sub-tile of v_mfma_f32_32x32x16_bf16
// accumulators.  Operand tiles move global -> LDS with the gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4) into a two-stage LDS ring, one K step ahead, one barrier per
// K step, and a workgroup's tiles form one stream of K steps, so the next tile's loads
// fly while the current tile's epilogue runs (the fused stream: every wave loads and
// computes).  This file is compiled twice, by gemm_fw256.hip (256-row tiles: every GEMM,
// and the host-side launch order of the bf16 and MXFP8 passes) and gemm_fw320.hip
// (320-row tiles: the bf16 row-tiled GEMMs).  An operand whose contraction axis is contiguous in
// memory ("K-major") is stored [rows][64] and read with 16-byte LDS reads; an operand
// contiguous along M or N ("MN-major": row-major weights as the B of x*W, and both
// operands of the weight gradients, which contract over token rows) is stored
// [64][width] and read with the transposing LDS read ds_read_b64_tr_b16, so no operand
// is transposed in memory.
//
// Kernels:
//   K1 fwd_gateup : G = Xp Wg, U = Xp Wu (dual B tile), epilogue saves G|U and A = silu(G) U
//   K2 fwd_down   : Yp = w * (A Wd)
//   B1 bwd_dA     : dA' = dY' Wd^T; epilogue: rowdot(dA', A) partials, SwiGLU backward -> dG|dU,
//                   and w * A for B2
//   B3 bwd_dX     : dXp = dG Wg^T + dU Wu^T (K = 2I)
//   B2 bwd_dWd    : dWd[e] = (w A)_e^T dY'_e over the expert's rows
//   B4 bwd_dWgu   : [dWg | dWu][e] = Xp_e^T [dG | dU]_e over the expert's rows
// Each has an MXFP8 variant on v_mfma_scale_f32_32x32x64_f8f6f4 over E4M3 codes with e8m0
// scales per 32 along K (the fp8 forward's K1 also writes A's row-wise codes).
#include <type_traits>

#include "gemm_engine.h"

namespace moe {

namespace {

// ---------------- shared pieces ----------------
// What the waves of a row-tiled kernel know about a tile.
struct RowTileInfo {
  RowTile t;
  int n0;
  int nk;
  int ncols;   // output columns from n0 (BN, or BN / 2 for a column half)
};
// Column halves (jobs with NSPLIT, see Sched): the job's value is item * 4 + hs
__device__ __forceinline__ int split_item(int v) { return v >> 2; }
__device__ __forceinline__ int split_off(int v) { return (v & 3) == 2 ? BN / 2 : 0; }
__device__ __forceinline__ int split_cols(int v) { return (v & 3) ? BN / 2 : BN; }

// Row-tiled bf16 loader state common to the fused-stream kernels: issue(kt, stage, ...)
// issues the wave's direct-to-LDS loads of K step kt; the rows are fixed per tile, so
// there are no row indices to fetch.
struct RowLd {
  static constexpr bool GATHER = false;
  int nk;
  int pw;
  __device__ __forceinline__ void fetch(int, int) const {}
};

// K-major A rows of a row tile for load wave pw: the lane's chunk of each of its A_LP
// rows, from a dense [rows, ld] buffer (dense != nullptr) or gathered through row_src.
__device__ __forceinline__ void a_rows_kmaj(KRows& a, const bf16_t* dense, const bf16_t* gsrc,
                                            const int32_t* row_src, int k, int ld, const RowTile& t, int pw,
                                            int lane) {
  int src[A_LP];
  if (!dense) gather_rows_a(row_src, t, pw, lane, src);
#pragma unroll
  for (int q = 0; q < A_LP; ++q) {
    int r, c;
    kmaj_slot(load_slot(q, pw, lane), r, c);
    a.p[q] = (dense ? dense + (size_t)(t.rs + min(r, t.cnt - 1)) * ld : gsrc + (size_t)(src[q] / k) * ld) + c * 8;
  }
}

__device__ __forceinline__ void row_tile_info(const int32_t* tiles, const int32_t* offsets, int v, int NT, int nk,
                                              int ntw, RowTileInfo& p) {
  row_tile(tiles, offsets, v, NT, p.t);
  p.n0 = p.t.nt * ntw;
  p.nk = nk;
  p.ncols = BN;
}
// a job's tile for its value v (a column half when NS and v says so)
template <bool NS>
__device__ __forceinline__ void row_tile_info_split(const int32_t* tiles, const int32_t* offsets, int v, int NT,
                                                    int nk, RowTileInfo& p) {
  row_tile_info(tiles, offsets, NS ? split_item(v) : v, NT, nk, BN, p);
  if constexpr (NS) {
    p.n0 += split_off(v);
    p.ncols = split_cols(v);
  }
}

// ---------------- MXFP8 operands (mxfp8 forward, fp8_bwd / mxfp8 backward) ----------------
// Both operands K-major E4M3 codes [rows][K] with e8m0 scales [rows][K/32].  One K step
// is 128 codes: the same 128 bytes per row as a bf16 step of 64, so the LDS ring,
// slots and swizzle are shared.  For v_mfma_scale_f32_32x32x64_f8f6f4 lane l of row
// l & 31 holds codes 16 (l >> 5) .. +15 of each of the two 32-blocks of a 64-code
// sub-step and supplies the scale of block l >> 5 of its row.  The scales of a step (4
// bytes per row) come with 512 / (64 NP) more direct-to-LDS loads per wave into a small
// ring: scale slot t < BM carries A row t, BM <= t < BM + BN B row t - BM (the slots past
// BM + BN repeat A row 0).
constexpr int MX_STEP = 128;               // codes per K step
constexpr int MX_SC_SLOT = 512 * 4;        // scale bytes per stage
constexpr int MX_SC_LP = 512 / (64 * NP);  // scale loads per wave
static_assert(B_LP % 2 == 0, "a column half is B_LP / 2 whole loads");
static_assert(MX_STEP == 2 * BK, "an fp8 step must span the bytes of a bf16 step");
// (the 320-row fused-stream build compiles no MXFP8 kernel)
static_assert(BM == 320 || (MX_SC_LP * NP * 64 == 512 && BM + BN <= 512), "scale slots");

__device__ __forceinline__ i32x8 frag_fp8(const bf16_t* tile, int r, int kk, int lane) {
  const int c0 = kk * 4 + (lane >> 5);
  const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + r * BK + (kmaj_chunk(r, c0) << 3));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + r * BK + (kmaj_chunk(r, c0 + 2) << 3));
  i32x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

// The scaled MFMAs of one stage for a job J: B rows J::ncol(wn, ni) as in mma_stage.
template <class J>
__device__ __forceinline__ void mx_compute(const bf16_t* st, const uint8_t* sc, Acc& acc, int lane,
                                           const WaveRows& w, int wn) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    i32x8 af[MI], bf[NI];
    int sa[MI], sb[NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = w.base + mi * 32 + (lane & 31);
      af[mi] = frag_fp8(st, r, kk, lane);
      sa[mi] = sc[r * 4 + kk * 2 + (lane >> 5)];
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int r = J::ncol(wn, ni) + (lane & 31);
      bf[ni] = frag_fp8(st + A_ELEMS, r, kk, lane);
      sb[ni] = sc[(BM + r) * 4 + kk * 2 + (lane >> 5)];
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = J::TRANS ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[ni], af[mi], acc[mi][ni], 0, 0, 0,
                                                                                sb[ni], 0, sa[mi])
                               : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bf[ni], acc[mi][ni], 0, 0, 0,
                                                                                sa[mi], 0, sb[ni]);
  }
}

struct LMx {
  static constexpr bool GATHER = false;
  int nk, pw;
  const uint8_t* a[A_LP];       // codes of the lane's slot at K step 0
  const uint8_t* b[B_LP];
  const uint8_t* sp[MX_SC_LP];  // scale rows of the lane's scale slots at K step 0
  uint8_t* scring;              // NSTAGE x MX_SC_SLOT bytes of LDS
  __device__ __forceinline__ void fetch(int, int) const {}
  template <class F>
  __device__ __forceinline__ void issue(int kt, bf16_t* st, int slot, int, F&&) const {
#pragma unroll
    for (int q = 0; q < A_LP; ++q) dma16(a[q] + kt * MX_STEP, a_dst(st, q, pw));
#pragma unroll
    for (int q = 0; q < B_LP; ++q) dma16(b[q] + kt * MX_STEP, b_dst(st, q, pw));
#pragma unroll
    for (int q = 0; q < MX_SC_LP; ++q)
      dma4(sp[q] + kt * (MX_STEP / 32), scring + slot * MX_SC_SLOT + load_instr(q, pw) * 256);
  }
  // operand rows: A row r (of tile) at a_base + ra(r) * lda, B row n at b_base + rb(n) * ldb;
  // both matrices' scales have row stride ld / 32 and start at s_a / s_b
  template <class RA, class RB>
  __device__ __forceinline__ void setup(const uint8_t* a_codes, const uint8_t* a_scales, int lda, RA ra,
                                        const uint8_t* b_codes, const uint8_t* b_scales, int ldb, RB rb, int k0,
                                        uint8_t* ring, int lane) {
    scring = ring;
#pragma unroll
    for (int q = 0; q < A_LP; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, pw, lane), r, c);
      a[q] = a_codes + (size_t)ra(r) * lda + k0 + c * 16;
    }
#pragma unroll
    for (int q = 0; q < B_LP; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, pw, lane), r, c);
      b[q] = b_codes + (size_t)rb(r) * ldb + k0 + c * 16;
    }
#pragma unroll
    for (int q = 0; q < MX_SC_LP; ++q) {
      const int t = load_slot(q, pw, lane);
      if (t < BM) sp[q] = a_scales + (size_t)ra(t) * (lda / 32) + k0 / 32;
      else if (t < BM + BN) sp[q] = b_scales + (size_t)rb(t - BM) * (ldb / 32) + k0 / 32;
      else sp[q] = a_scales + (size_t)ra(0) * (lda / 32) + k0 / 32;   // unused slot, any valid row
    }
  }
};

// ---------------- fp8_bwd: the weights' row-wise codes from the forward's B stages ----------------
// The bf16 forward streams every weight slice of an expert through the B stages of each
// of that expert's row tiles, MN-major [BK][BN]: k-row r of step kt is weight row
// kt * BK + r, chunk c its output columns 8c .. 8c + 7.  Row tile mt of n also writes
// the row-wise MXFP8 codes of the steps kt with kt mod n = mt for the backward (blocks
// of 32 along the output columns, the scale and rounding rule of k_mx_rows, so the
// codes are the same bytes).
// Thread t takes the chunk pairs t + NTHR i (16 columns each): the two lanes of a block
// are adjacent, so its maximum takes one lane exchange; 16 lanes read one k-row's 512
// bytes and write its 256 code bytes, 16 per lane.  put(r, c, codes, X) stores the
// codes of chunks c, c + 1 (c even; the block's scale from the lanes with c % 4 = 0).
template <class Put>
__device__ __forceinline__ void quant_bstage(const bf16_t* Bs, int tid, Put&& put) {
#pragma unroll 1
  for (int it = 0; it < BK * BN / 16 / NTHR; ++it) {
    const int g = it * NTHR + tid, r = g / (BN / 16), c = 2 * (g % (BN / 16));
    const bf16_t* const row = Bs + r * BN;
    const i32x4 u0 = *reinterpret_cast<const i32x4*>(row + (mnmaj_chunk(r, c) << 3));
    const i32x4 u1 = *reinterpret_cast<const i32x4*>(row + (mnmaj_chunk(r, c + 1) << 3));
    // the block maximum of |x| from the bf16 magnitudes (integer order is magnitude
    // order; a NaN counts as 0, as fmaxf drops it)
    uint32_t mb = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t w = (uint32_t)(q < 4 ? u0[q] : u1[q - 4]);
      const uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
      mb = max(mb, max(lo > 0x7f80u ? 0u : lo, hi > 0x7f80u ? 0u : hi));
    }
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 1, 64));
    const int X = mx_scale_exp(__uint_as_float(mb << 16));
    auto f = [&](int q, int h) {
      const uint32_t w = (uint32_t)(q < 4 ? u0[q] : u1[q - 4]);
      return __uint_as_float(h ? w & 0xffff0000u : w << 16);
    };
    uint4 cw;
    cw.x = e4m3_pack4(f(0, 0), f(0, 1), f(1, 0), f(1, 1), X);
    cw.y = e4m3_pack4(f(2, 0), f(2, 1), f(3, 0), f(3, 1), X);
    cw.z = e4m3_pack4(f(4, 0), f(4, 1), f(5, 0), f(5, 1), X);
    cw.w = e4m3_pack4(f(6, 0), f(6, 1), f(7, 0), f(7, 1), X);
    put(r, c, cw, X);
  }
}

// ---------------- K1: gate/up + SwiGLU ----------------
// B tile: gate columns 0..BN/2-1 and up columns BN/2..BN-1; compute wave wn takes the same
// WCOLS / 2 intermediate columns of both (blocks ni < NI / 2 gate, the rest up), so G
// and U of one element share a lane.
struct LGateUp : RowLd {
  KRows a;
  const bf16_t* b[B_LP];  // weight row k = 0 of the slot's column
  size_t bstep;           // elements per K step of the weights (64 rows)
  template <class F>
  __device__ __forceinline__ void issue(int kt, bf16_t* st, int, int, F&&) const {
    a.dma(kt, st, pw);
#pragma unroll
    for (int q = 0; q < B_LP; ++q) dma16(b[q] + kt * bstep, b_dst(st, q, pw));
  }
};

// MX: Xp rows (row-wise codes along H) against the transposed column-wise codes of
// [W_gate | W_up] (rows n < I gate, I + n up; expert e's K range starts at e * H).
// QW (fp8_bwd, bf16 operands): the expert's row tiles also write the row-wise codes of
// [W_gate | W_up] (quant_bstage).
template <bool MX, bool QW = false>
struct JGateUp {
  using Tile = RowTileInfo;
  using Ld = typename std::conditional<MX, LMx, LGateUp>::type;
  static constexpr bool A_KMAJ = true, B_KMAJ = MX;
  static constexpr bool DYN = false, TRANS = true, EPI_LDS = true;
  static constexpr bool NSPLIT = false;   // column halves of a last round (Sched)
  static constexpr bool SIDE = QW;
  static_assert(!(MX && QW), "the weight codes come from bf16 B stages");
  __device__ __forceinline__ static int ncol(int wn, int ni) {
    return (ni < NI / 2 ? 0 : BN / 2) + wn * (WCOLS / 2) + (ni % (NI / 2)) * 32;
  }
  FwdArgs a;
  MxFwdArgs m;
  int NT;
  uint8_t* scring;
  __device__ __forceinline__ int items() const { return sload(a.tiles) * NT; }
  __device__ __forceinline__ int nk() const { return MX ? a.H / MX_STEP : a.H / BK; }
  __device__ __forceinline__ void tile(int v, Tile& p) const {
    row_tile_info(a.tiles, a.offsets, v, NT, nk(), BN / 2, p);
  }
  __device__ __forceinline__ WaveRows rows(const Tile& p, int wm) const { return wave_rows(p.t.cnt, wm); }
  __device__ __forceinline__ void compute(const bf16_t* st, int slot, Acc& acc, int lane, const WaveRows& w,
                                          int wn) const {
    if constexpr (MX) mx_compute<JGateUp>(st, scring + slot * MX_SC_SLOT, acc, lane, w, wn);
    else mma_stage<JGateUp>(st, acc, lane, w, wn);
  }
  __device__ __forceinline__ void setup(int v, Ld& p, int pw, int lane) const {
    RowTile t;
    row_tile(a.tiles, a.offsets, v, NT, t);
    const int n0 = t.nt * (BN / 2);
    p.pw = pw;
    p.nk = nk();
    if constexpr (MX) {
      const size_t ldw = (size_t)a.El * a.H;  // codes per transposed weight column
      const size_t eoff = (size_t)t.e * a.H;
      // B tile row r: gate column n0 + r for r < BN / 2, else up column n0 + r - BN / 2;
      // tail columns read any valid column (their results are discarded)
      p.setup(m.q_x, m.s_x, a.H, [&](int r) { return t.rs + min(r, t.cnt - 1); }, m.qt_wgu + eoff,
              m.st_wgu + eoff / 32, (int)ldw,
              [&](int r) { return (r < BN / 2 ? 0 : a.I) + min(n0 + r % (BN / 2), a.I - 1); }, 0, scring, lane);
    } else {
      setup_bf16(t, n0, p, pw, lane);
    }
  }
  // B chunk c: gate (c < BN / 16) or up column p.n0 + 8 (c % (BN / 16)), row e * H + h of the codes
  __device__ __forceinline__ void side(const bf16_t* st, const Tile& p, int kt, int tid) const {
    if (kt % p.t.nmt != p.t.mt) return;   // the expert's row tiles share the steps
    const uint32_t I2 = 2u * (uint32_t)a.I;
    uint8_t* const qb = a.q_wrows + ((size_t)p.t.e * a.H + (size_t)kt * BK) * I2;
    uint8_t* const sb = a.s_wrows + ((size_t)p.t.e * a.H + (size_t)kt * BK) * (I2 / 32);
    quant_bstage(st + A_ELEMS, tid, [&](int r, int c, uint4 w, int X) {
      constexpr int HC = BN / 16;
      const int col = p.n0 + (c % HC) * 8;
      if (col < a.I) {
        const uint32_t cc = (c < HC ? 0u : (uint32_t)a.I) + (uint32_t)col;
        *reinterpret_cast<uint4*>(qb + (uint32_t)r * I2 + cc) = w;
        if ((c & 3) == 0) sb[(uint32_t)r * (I2 / 32) + cc / 32] = (uint8_t)(X + 127);
      }
    });
  }
  __device__ __forceinline__ void setup_bf16(const RowTile& t, int n0, LGateUp& p, int pw, int lane) const {
    a_rows_kmaj(p.a, a.xp, a.x, a.row_src, a.k, a.H, t, pw, lane);
    const bf16_t* wg = a.wg + (size_t)t.e * a.H * a.I;
    const bf16_t* wu = a.wu + (size_t)t.e * a.H * a.I;
#pragma unroll
    for (int q = 0; q < B_LP; ++q) {
      int r, c;
      mnmaj_slot<BN>(load_slot(q, pw, lane), r, c);
      constexpr int HC = BN / 16;    // chunks per half: HC..2 HC - 1 are W_up's
      int col = n0 + (c % HC) * 8;   // intermediate column
      if (col >= a.I) col = n0;      // tail columns: any valid address, results are discarded
      p.b[q] = (c < HC ? wg : wu) + col + (size_t)r * a.I;
    }
    p.bstep = (size_t)BK * a.I;
  }
  // The accumulators hold C^T (trans_chunks): gate block 0 and up block 1 of a band hold
  // G and U of the same elements, so A = silu(G) U is formed in registers (MX: and its
  // row-wise codes, from the fp32 values); G|U and A leave through the wave's LDS band.
  __device__ __forceinline__ void epilogue(const Tile& p, const Acc& acc, float* stage) const {
    static_assert(NI == 2, "one gate and one up block per band");
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = (int)((unsigned)wv % WM), wn = (int)((unsigned)wv / WM);
    bf16_t* const wreg = reinterpret_cast<bf16_t*>(stage) + wv * BAND_ELEMS;
    const uint32_t I2 = 2u * (uint32_t)a.I;
    // the tile's first row (uniform); lanes add 32-bit offsets.  G|U is not kept when the
    // backward recomputes it.
    const bool keep_gu = a.gu != nullptr;
    bf16_t* const gub = keep_gu ? a.gu + (size_t)p.t.rs * I2 : nullptr;
    bf16_t* const ab = a.a + (size_t)p.t.rs * a.I;
    const int colw = p.n0 + wn * (WCOLS / 2);  // the wave's first intermediate column
    const WaveRows w = wave_rows(p.t.cnt, wm);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rb = w.base + mi * 32;   // the band's first row in the tile
      f32x16 av;
#pragma unroll
      for (int i = 0; i < 16; ++i) av[i] = silu_f(acc[mi][0][i]) * acc[mi][1][i];
      if constexpr (MX) {
        // the down GEMM's row-wise codes of A: the wave's 32 columns are one MX block
        int X;
        const i32x4 codes = mx_row_codes(av, X);
        const int rt = rb + (lane & 31);
        if (rt < w.end && colw < a.I) {
          const size_t r = (size_t)(p.t.rs + rt);
          *reinterpret_cast<i32x4*>(m.q_a + r * a.I + colw + 16 * (lane >> 5)) = codes;
          if (lane < 32) m.s_a[r * (a.I / 32) + colw / 32] = (uint8_t)(X + 127);
        }
      }
      if (keep_gu) {
        // G and U (I columns apart in each G|U row) as two one-block bands
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          i32x4 ch[1][2];
          trans_chunks(acc[mi][g], ch[0]);
          band_store(wreg, ch, [&](int rr, int cb, i32x4 v) {
            const int rt = rb + rr, col = colw + cb;
            if (rt < w.end && col < a.I)
              *reinterpret_cast<i32x4*>(gub + ((uint32_t)rt * I2 + (uint32_t)col + (g ? (uint32_t)a.I : 0u))) = v;
          });
        }
      }
      i32x4 ca[1][2];
      trans_chunks(av, ca[0]);
      band_store(wreg, ca, [&](int rr, int cb, i32x4 v) {
        const int rt = rb + rr, col = colw + cb;
        if (rt < w.end && col < a.I)
          *reinterpret_cast<i32x4*>(ab + ((uint32_t)rt * (uint32_t)a.I + (uint32_t)col)) = v;
      });
    }
  }
};

template <bool MX, bool QW = false>
__global__ __launch_bounds__(NTHR, 1) void k_fwd_gateup(FwdArgs a, MxFwdArgs m) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  JGateUp<MX, QW> job{a, m, (int)ceil_div(a.I, BN / 2), scring};
  run_stream(job, lds);
}

// ---------------- K2: down projection * routing weight ----------------
// K-major A rows, MN-major B (row-major weights [K, N])
struct LMnB : RowLd {
  KRows a;
  const bf16_t* b[B_LP];
  size_t bstep;
  template <class F>
  __device__ __forceinline__ void issue(int kt, bf16_t* st, int, int, F&&) const {
    a.dma(kt, st, pw);
#pragma unroll
    for (int q = 0; q < B_LP; ++q) dma16(b[q] + kt * bstep, b_dst(st, q, pw));
  }
};

// MX: A rows (row-wise codes along I) against the transposed column-wise codes of
// W_down (row n = hidden column n; expert e's K range starts at e * I).
// QW (fp8_bwd, bf16 operands): the expert's row tiles also write the row-wise codes of
// W_down along H (quant_bstage).
template <bool MX, bool QW = false>
struct JDown {
  using Tile = RowTileInfo;
  using Ld = typename std::conditional<MX, LMx, LMnB>::type;
  static constexpr bool A_KMAJ = true, B_KMAJ = MX;
  static constexpr bool DYN = false, TRANS = true, EPI_LDS = true;
  static constexpr bool NSPLIT = false;   // column halves of a last round (Sched)
  static constexpr bool SIDE = QW;
  static_assert(!(MX && QW), "the weight codes come from bf16 B stages");
  __device__ __forceinline__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  FwdArgs a;
  MxFwdArgs m;
  int NT;
  uint8_t* scring;
  __device__ __forceinline__ int items() const { return sload(a.tiles) * NT; }
  __device__ __forceinline__ int nk() const { return MX ? a.I / MX_STEP : a.I / BK; }
  __device__ __forceinline__ void tile(int v, Tile& p) const {
    row_tile_info_split<NSPLIT>(a.tiles, a.offsets, v, NT, nk(), p);
  }
  __device__ __forceinline__ WaveRows rows(const Tile& p, int wm) const { return wave_rows(p.t.cnt, wm); }
  __device__ __forceinline__ void compute(const bf16_t* st, int slot, Acc& acc, int lane, const WaveRows& w,
                                          int wn) const {
    if constexpr (MX) mx_compute<JDown>(st, scring + slot * MX_SC_SLOT, acc, lane, w, wn);
    else mma_stage<JDown>(st, acc, lane, w, wn);
  }
  __device__ __forceinline__ void setup(int v, Ld& p, int pw, int lane) const {
    RowTile t;
    row_tile(a.tiles, a.offsets, NSPLIT ? split_item(v) : v, NT, t);
    const int n0 = t.nt * BN + (NSPLIT ? split_off(v) : 0);
    p.pw = pw;
    p.nk = nk();
    if constexpr (MX) {
      const size_t ldw = (size_t)a.El * a.I;
      const size_t eoff = (size_t)t.e * a.I;
      p.setup(m.q_a, m.s_a, a.I, [&](int r) { return t.rs + min(r, t.cnt - 1); }, m.qt_wd + eoff, m.st_wd + eoff / 32,
              (int)ldw, [&](int r) { return min(n0 + r, a.H - 1); }, 0, scring, lane);
    } else {
      setup_bf16(t, n0, p, pw, lane);
    }
  }
  // B chunk c: hidden columns p.n0 + 8c .., row e * I + i of the codes
  __device__ __forceinline__ void side(const bf16_t* st, const Tile& p, int kt, int tid) const {
    if (kt % p.t.nmt != p.t.mt) return;   // the expert's row tiles share the steps
    const uint32_t H = (uint32_t)a.H;
    uint8_t* const qb = a.q_wrows + ((size_t)p.t.e * a.I + (size_t)kt * BK) * H;
    uint8_t* const sb = a.s_wrows + ((size_t)p.t.e * a.I + (size_t)kt * BK) * (H / 32);
    quant_bstage(st + A_ELEMS, tid, [&](int r, int c, uint4 w, int X) {
      const uint32_t col = (uint32_t)(p.n0 + c * 8);
      if (col < H) {
        *reinterpret_cast<uint4*>(qb + (uint32_t)r * H + col) = w;
        if ((c & 3) == 0) sb[(uint32_t)r * (H / 32) + col / 32] = (uint8_t)(X + 127);
      }
    });
  }
  __device__ __forceinline__ void setup_bf16(const RowTile& t, int n0, LMnB& p, int pw, int lane) const {
    a_rows_kmaj(p.a, a.a, nullptr, nullptr, 1, a.I, t, pw, lane);
    const bf16_t* wd = a.wd + (size_t)t.e * a.I * a.H;
#pragma unroll
    for (int q = 0; q < B_LP; ++q) {
      int r, c;
      mnmaj_slot<BN>(load_slot(q, pw, lane), r, c);
      int col = n0 + c * 8;
      if (col >= a.H) col = n0;  // tail columns: any valid address, results are discarded
      p.b[q] = wd + (size_t)r * a.H + col;
    }
    p.bstep = (size_t)BK * a.H;
  }
  // C^T accumulators: lane l holds row l % 32 of each band, so it scales by that row's
  // routing weight alone, then the band leaves through LDS (band_store).
  __device__ __forceinline__ void epilogue(const Tile& p, const Acc& acc, float* stage) const {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = (int)((unsigned)wv % WM), wn = (int)((unsigned)wv / WM);
    bf16_t* const wreg = reinterpret_cast<bf16_t*>(stage) + wv * BAND_ELEMS;
    const WaveRows w = wave_rows(p.t.cnt, wm);
    float wr[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rt = min(w.base + mi * 32 + (lane & 31), p.t.cnt - 1);
      wr[mi] = a.topk_w[a.row_src[p.t.rs + rt]];
    }
    bf16_t* const yb = a.yp + (size_t)p.t.rs * a.H;  // the tile's first row
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rb = w.base + mi * 32;
      i32x4 ch[NI][2];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) trans_chunks(acc[mi][ni] * wr[mi], ch[ni]);
      band_store(wreg, ch, [&](int rr, int cb, i32x4 v) {
        const int rt = rb + rr, col = p.n0 + wn * WCOLS + cb;
        if (rt < w.end && col < a.H)
          *reinterpret_cast<i32x4*>(yb + ((uint32_t)rt * (uint32_t)a.H + (uint32_t)col)) = v;
      });
    }
  }
};

template <bool MX, bool QW = false>
__global__ __launch_bounds__(NTHR, 1) void k_fwd_down(FwdArgs a, MxFwdArgs m) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  JDown<MX, QW> job{a, m, (int)ceil_div(a.H, BN), scring};
  run_stream(job, lds);
}

// ---------------- B1 / B3: both operands K-major ----------------
template <bool NS>
struct LKK : RowLd {
  KRows a;
  const bf16_t* b[B_LP];   // B rows for K steps [0, ksplit)
  const bf16_t* b2[B_LP];  // B3: W_up rows for K steps [ksplit, nk)
  int ksplit;              // B3: I / 64; B1: larger than any step count
  // a column half (uniform): B load q fills tile rows 64 q .. 64 q + 63 (one eighth
  // of each to every wave), so the half's BN / 2 rows are loads q < B_LP / 2 exactly
  int half;
  template <class F>
  __device__ __forceinline__ void issue(int kt, bf16_t* st, int, int, F&&) const {
    a.dma(kt, st, pw);
    const bool second = kt >= ksplit;
    const int k0 = (second ? kt - ksplit : kt) * BK;
#pragma unroll
    for (int q = 0; q < B_LP; ++q)
      if (!NS || q < B_LP / 2 || !half) dma16((second ? b2[q] : b[q]) + k0, b_dst(st, q, pw));
  }
};

template <bool MX, bool NS>
using KKLd = typename std::conditional<MX, LMx, LKK<NS>>::type;

// B1: dA' = dY' Wd^T.  Epilogue: SwiGLU backward on 8 columns per lane, w * A for B2, and
// the rowdot of dA' and A over this wave's 64 columns, reduced across the 8 lanes of a row.
// MX: both operands from the fp8 row-wise buffers (dY' rows, W_down rows along H), and
// no w * A output (the MXFP8 dW_down quantises A and w * dY').
template <bool MX>
struct JDa {
  using Tile = RowTileInfo;
  using Ld = KKLd<MX, !MX>;
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  static constexpr bool DYN = false, TRANS = false, EPI_LDS = true;
  static constexpr bool NSPLIT = !MX;   // column halves of a last round (Sched)
  static constexpr bool SIDE = false;   // no extra per-step work
  __device__ __forceinline__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  BwdArgs a;
  MxArgs m;
  int NT, nparts;
  uint8_t* scring;
  float* wrow;  // LDS [NW][WROWS]: the routing weights of each compute wave's rows
  __device__ __forceinline__ int items() const { return sload(a.tiles) * NT; }
  __device__ __forceinline__ int nk() const { return MX ? a.H / MX_STEP : a.H / BK; }
  __device__ __forceinline__ void tile(int v, Tile& p) const {
    row_tile_info_split<NSPLIT>(a.tiles, a.offsets, v, NT, nk(), p);
  }
  __device__ __forceinline__ WaveRows rows(const Tile& p, int wm) const { return wave_rows(p.t.cnt, wm); }
  __device__ __forceinline__ void compute(const bf16_t* st, int slot, Acc& acc, int lane, const WaveRows& w,
                                          int wn) const {
    if constexpr (MX) mx_compute<JDa>(st, scring + slot * MX_SC_SLOT, acc, lane, w, wn);
    else mma_stage<JDa>(st, acc, lane, w, wn);
  }
  __device__ __forceinline__ void setup(int v, Ld& p, int pw, int lane) const {
    RowTile t;
    row_tile(a.tiles, a.offsets, NSPLIT ? split_item(v) : v, NT, t);
    const int n0 = t.nt * BN + (NSPLIT ? split_off(v) : 0);
    p.pw = pw;
    p.nk = nk();
    if constexpr (MX) {
      p.setup(m.q_dy, m.s_dy, a.H, [&](int r) { return t.rs + min(r, t.cnt - 1); }, m.q_wd, m.s_wd, a.H,
              [&](int r) { return t.e * a.I + min(n0 + r, a.I - 1); }, 0, scring, lane);
    } else {
      p.ksplit = 1 << 30;
      a_rows_kmaj(p.a, nullptr, a.dy, a.row_src, a.k, a.H, t, pw, lane);
      const bf16_t* wd = a.wd + (size_t)t.e * a.I * a.H;
      const int ncols = NSPLIT ? split_cols(v) : BN;
      p.half = uni(ncols < BN ? 1 : 0);
#pragma unroll
      for (int q = 0; q < B_LP; ++q) {
        int r, c;
        kmaj_slot(load_slot(q, pw, lane), r, c);
        p.b[q] = wd + (size_t)min(n0 + r, a.I - 1) * a.H + c * 8;
        p.b2[q] = p.b[q];
      }
    }
  }
  __device__ __forceinline__ void epilogue(const Tile& p, const Acc& acc, float* stage) const {
    const int lane = threadIdx.x & 63, wn = (int)((threadIdx.x >> 6) / WM);
    const int wm = (int)((unsigned)(threadIdx.x >> 6) % WM);
    const uint32_t I2 = 2u * (uint32_t)a.I;
    // the tile's first row (uniform); lanes add 32-bit offsets
    const bf16_t* const gub = a.gu + (size_t)p.t.rs * I2;
    const bf16_t* const ab = a.a + (size_t)p.t.rs * a.I;
    bf16_t* const dgub = a.dgu + (size_t)p.t.rs * I2;
    bf16_t* const awb = a.aw + (size_t)p.t.rs * a.I;
    // the routing weights of the wave's WROWS rows into the wave's LDS slots before the
    // staging starts (read back by row: no per-lane array indexed in the rolled row loop,
    // which would live in scratch memory)
    const int wv = threadIdx.x >> 6;
    const WaveRows w = wave_rows(p.t.cnt, wm);
#pragma unroll
    for (int i = lane; i < WROWS; i += 64)
      wrow[wv * WROWS + i] = a.topk_w[a.row_src[p.t.rs + min(w.base + i, p.t.cnt - 1)]];
    epilogue_rows(stage, acc, w, [&](int rt, int ct, const float (&dap)[8], int) {
      const int col = p.n0 + ct;
      const bool ok = rt < w.end && col < a.I;
      float part = 0.f;
      if (ok) {
        const uint32_t og = (uint32_t)rt * I2 + (uint32_t)col, oa = (uint32_t)rt * (uint32_t)a.I + (uint32_t)col;
        const float wt = wrow[wv * WROWS + (rt - w.base)];
        // two columns at a time, straight from and back to packed bf16 pairs
        __builtin_amdgcn_sched_barrier(0);
        const i32x4 gw = *reinterpret_cast<const i32x4*>(gub + og);
        const i32x4 uw = *reinterpret_cast<const i32x4*>(gub + og + a.I);
        const i32x4 aw4 = *reinterpret_cast<const i32x4*>(ab + oa);
        i32x4 dgo, duo, awo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float dg2[2], du2[2], aw2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t gb = (uint32_t)gw[q], ub = (uint32_t)uw[q], ab = (uint32_t)aw4[q];
            const float g = __uint_as_float(h ? gb & 0xffff0000u : gb << 16);
            const float u = __uint_as_float(h ? ub & 0xffff0000u : ub << 16);
            const float av = __uint_as_float(h ? ab & 0xffff0000u : ab << 16);
            const float d = dap[2 * q + h];
            part += d * av;
            aw2[h] = wt * av;
            const float da = wt * d;
            const float sg = sigmoid_f(g);
            du2[h] = da * g * sg;
            dg2[h] = da * u * sg * (1.f + g * (1.f - sg));
          }
          dgo[q] = (int)pk_bf16(dg2[0], dg2[1]);
          duo[q] = (int)pk_bf16(du2[0], du2[1]);
          awo[q] = (int)pk_bf16(aw2[0], aw2[1]);
        }
        *reinterpret_cast<i32x4*>(dgub + og) = dgo;
        *reinterpret_cast<i32x4*>(dgub + og + a.I) = duo;
        if (!MX) *reinterpret_cast<i32x4*>(awb + oa) = awo;
      }
#pragma unroll
      for (int off = 1; off < EP_LPR; off <<= 1) part += __shfl_xor(part, off, 64);
      // the wave's absolute 64-column block of the tile (a right column half starts at BN / 2)
      if (rt < w.end && lane % EP_LPR == 0)
        a.dw_part[(size_t)(p.t.rs + rt) * nparts + p.t.nt * WN + (p.n0 - p.t.nt * BN) / WCOLS + wn] = part;
    });
  }
};

template <bool MX>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_da(BwdArgs a, MxArgs m, int nparts) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  __shared__ float wrow[NW * WROWS];
  JDa<MX> job{a, m, (int)ceil_div(a.I, BN), nparts, scring, wrow};
  run_stream(job, lds);
}

// B3: dXp = dG Wg^T + dU Wu^T, K = 2I: the first I/64 steps read W_gate rows, the rest W_up.
// MX: dG|dU rows against the rows of the concatenated [W_gate | W_up] (both along 2I).
template <bool MX>
struct JDx {
  using Tile = RowTileInfo;
  using Ld = KKLd<MX, false>;
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  static constexpr bool DYN = false, TRANS = true, EPI_LDS = true;
  static constexpr bool NSPLIT = false;   // column halves of a last round (Sched)
  static constexpr bool SIDE = false;   // no extra per-step work
  __device__ __forceinline__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  BwdArgs a;
  MxArgs m;
  int NT;
  uint8_t* scring;
  __device__ __forceinline__ int items() const { return sload(a.tiles) * NT; }
  __device__ __forceinline__ int nk() const { return MX ? 2 * a.I / MX_STEP : 2 * a.I / BK; }
  __device__ __forceinline__ void tile(int v, Tile& p) const {
    row_tile_info_split<NSPLIT>(a.tiles, a.offsets, v, NT, nk(), p);
  }
  __device__ __forceinline__ WaveRows rows(const Tile& p, int wm) const { return wave_rows(p.t.cnt, wm); }
  __device__ __forceinline__ void compute(const bf16_t* st, int slot, Acc& acc, int lane, const WaveRows& w,
                                          int wn) const {
    if constexpr (MX) mx_compute<JDx>(st, scring + slot * MX_SC_SLOT, acc, lane, w, wn);
    else mma_stage<JDx>(st, acc, lane, w, wn);
  }
  __device__ __forceinline__ void setup(int v, Ld& p, int pw, int lane) const {
    RowTile t;
    row_tile(a.tiles, a.offsets, NSPLIT ? split_item(v) : v, NT, t);
    const int n0 = t.nt * BN + (NSPLIT ? split_off(v) : 0);
    p.pw = pw;
    p.nk = nk();
    if constexpr (MX) {
      p.setup(m.q_dgu, m.s_dgu, 2 * a.I, [&](int r) { return t.rs + min(r, t.cnt - 1); }, m.q_wg, m.s_wg, 2 * a.I,
              [&](int r) { return t.e * a.H + min(n0 + r, a.H - 1); }, 0, scring, lane);
    } else {
      p.ksplit = a.I / BK;
      a_rows_kmaj(p.a, a.dgu, nullptr, nullptr, 1, 2 * a.I, t, pw, lane);
      const size_t woff = (size_t)t.e * a.H * a.I;
#pragma unroll
      for (int q = 0; q < B_LP; ++q) {
        int r, c;
        kmaj_slot(load_slot(q, pw, lane), r, c);
        const size_t n = (size_t)min(n0 + r, a.H - 1);
        p.b[q] = a.wg + woff + n * a.I + c * 8;
        p.b2[q] = a.wu + woff + n * a.I + c * 8;
      }
    }
  }
  // C^T accumulators leave as bf16 row bands (trans_chunks, band_store)
  __device__ __forceinline__ void epilogue(const Tile& p, const Acc& acc, float* stage) const {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = (int)((unsigned)wv % WM), wn = (int)((unsigned)wv / WM);
    bf16_t* const wreg = reinterpret_cast<bf16_t*>(stage) + wv * BAND_ELEMS;
    bf16_t* const xb = a.dxp + (size_t)p.t.rs * a.H;  // the tile's first row
    const WaveRows w = wave_rows(p.t.cnt, wm);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rb = w.base + mi * 32;
      i32x4 ch[NI][2];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) trans_chunks(acc[mi][ni], ch[ni]);
      band_store(wreg, ch, [&](int rr, int cb, i32x4 v) {
        const int rt = rb + rr, col = p.n0 + wn * WCOLS + cb;
        if (rt < w.end && col < a.H)
          *reinterpret_cast<i32x4*>(xb + ((uint32_t)rt * (uint32_t)a.H + (uint32_t)col)) = v;
      });
    }
  }
};

template <bool MX>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_dx(BwdArgs a, MxArgs m) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  JDx<MX> job{a, m, (int)ceil_div(a.H, BN), scring};
  run_stream(job, lds);
}

// ---------------- weight gradients: contraction over an expert's rows ----------------
// Both operands are MN-major tiles of 64 token rows; rows past the expert's end are
// loaded from a zeroed scratch area.  For a gathered operand (rows of x or dy picked
// by row_src) each wave also copies the 64 row_src entries of a stream position into its
// own LDS index slot one position ahead, with one more direct-to-LDS load; the stream's
// full wait at the next position completes it before the next issue() reads the slot.
template <bool AG, bool BG>
struct LWgrad {
  static constexpr bool GATHER = AG || BG;
  static constexpr int AR = 512 / BM, BR = 512 / BN;  // token rows per wave load of A and B
  const bf16_t* abase; int lda;
  const bf16_t* bbase; int ldb;
  const int32_t* row_src; const bf16_t* zeros; double inv_k;  // 1 / top-k
  int rs, cnt, pw, lane;
  int nk;
  int32_t* ids;                  // this wave's two LDS slots of BK row indices
  int acol[A_LP], bcol[B_LP];    // element column of the lane's chunk
  // row_src of step kt of rows [rs, rs + cnt) -> index slot par of a wave's slots ids
  __device__ __forceinline__ static void fetch_rows(const int32_t* row_src, const bf16_t* zeros, int rs, int cnt,
                                                    int32_t* ids, int lane, int kt, int par) {
    const int32_t* src = cnt > 0 ? row_src + rs + min(kt * BK + lane, cnt - 1) : reinterpret_cast<const int32_t*>(zeros);
    dma4(src, ids + par * IDS_SLOT);
  }
  __device__ __forceinline__ void fetch(int kt, int par) const {  // row_src of step kt -> slot par
    if (GATHER) fetch_rows(row_src, zeros, rs, cnt, ids, lane, kt, par);
  }
  template <class F>
  __device__ __forceinline__ void issue(int kt, bf16_t* st, int, int par, F&& fetch_next) const {
    const int32_t* my = ids + par * IDS_SLOT;
    const bf16_t* ap[A_LP];
    const bf16_t* bp[B_LP];
    // all gathered indices are read (the slot holds valid entries for every row) before
    // any address is formed, so their LDS reads go out together and are waited for once
    int ia[A_LP], ib[B_LP];
#pragma unroll
    for (int q = 0; q < A_LP; ++q) ia[q] = AG ? my[load_instr(q, pw) * AR + (int)((unsigned)lane / (64 / AR))] : 0;
#pragma unroll
    for (int q = 0; q < B_LP; ++q) ib[q] = BG ? my[load_instr(q, pw) * BR + (int)((unsigned)lane / (64 / BR))] : 0;
#pragma unroll
    for (int q = 0; q < A_LP; ++q) asm volatile("" : "+v"(ia[q]));
#pragma unroll
    for (int q = 0; q < B_LP; ++q) asm volatile("" : "+v"(ib[q]));
#pragma unroll
    for (int q = 0; q < A_LP; ++q) {
      const int kr = load_instr(q, pw) * AR + (int)((unsigned)lane / (64 / AR));
      const int row = AG ? div_k(ia[q], inv_k) : rs + kt * BK + kr;
      ap[q] = kt * BK + kr < cnt ? abase + (size_t)row * lda + acol[q] : zeros;
    }
#pragma unroll
    for (int q = 0; q < B_LP; ++q) {
      const int kr = load_instr(q, pw) * BR + (int)((unsigned)lane / (64 / BR));
      const int row = BG ? div_k(ib[q], inv_k) : rs + kt * BK + kr;
      bp[q] = kt * BK + kr < cnt ? bbase + (size_t)row * ldb + bcol[q] : zeros;
    }
    if (GATHER) fetch_next();
#pragma unroll
    for (int q = 0; q < A_LP; ++q) dma16(ap[q], a_dst(st, q, pw));
#pragma unroll
    for (int q = 0; q < B_LP; ++q) dma16(bp[q], b_dst(st, q, pw));
  }
};

struct WgradTile {
  int e, m0, n0, nk;
};

// B2 (WHICH = 0): dWd[e] [I, H] = (w A)_e^T dY'_e (MX: Q(A)^T Q(w dY')).
// B4 (WHICH = 1): [dWg | dWu][e] [H, 2I] = Xp_e^T [dG | dU]_e.
template <int WHICH, bool AG, bool BG, bool MX>
struct JWgrad {
  using Tile = WgradTile;
  using Ld = typename std::conditional<MX, LMx, LWgrad<AG, BG>>::type;
  static constexpr bool A_KMAJ = false, B_KMAJ = false;
  // items: position p in a.order, then the expert's tm x tn output tiles, m-major.
  // a.order lists the experts by cost, most rows first, and a.order[El] = 1, when
  // their loads are skewed enough for dynamic (greedy longest-first) scheduling to pay;
  // else it is the identity, a.order[El] = 0, and the items go out in contiguous XCD
  // ranges.  a.order[El + 1 + WHICH] is the launch's item counter (zeroed with the order).
  // the accumulators hold C^T; the epilogue writes them as bf16 row bands (band_store)
  static constexpr bool DYN = true, TRANS = true, EPI_LDS = true;
  static constexpr bool NSPLIT = false;   // column halves of a last round (Sched)
  static constexpr bool SIDE = false;   // no extra per-step work
  __device__ __forceinline__ bool dynamic() const { return sload(a.order + a.El) != 0; }
  __device__ __forceinline__ int32_t* counter() const { return a.order + a.El + 1 + WHICH; }
  __device__ __forceinline__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  BwdArgs a;
  MxArgs m;
  int tm, tn;
  int32_t* ids;
  uint8_t* scring;
  int32_t* dslot;   // LDS: the next item under dynamic scheduling, two slots by tile parity
  __device__ __forceinline__ int items() const { return a.El * tm * tn; }
  __device__ __forceinline__ void tile(int v, Tile& p) const {
    const int pos = uni(v / (tm * tn));
    p.e = sload(a.order + pos);
    const int rem = uni(v - pos * tm * tn);
    p.m0 = uni(rem / tn) * BM;
    p.n0 = uni(rem % tn) * BN;
    if constexpr (MX) {
      p.nk = uni((sload(m.poff + p.e + 1) - sload(m.poff + p.e)) / MX_STEP);
    } else {
      const int cnt = sload(a.offsets + p.e + 1) - sload(a.offsets + p.e);
      p.nk = uni((cnt + BK - 1) / BK);
    }
  }
  __device__ __forceinline__ WaveRows rows(const Tile&, int wm) const { return {wm * WROWS, BM, MI}; }
  // fused stream, gathering loaders: the row indices of item v's first K step into index
  // slot par of load wave pw (as its loader's fetch(0, par) would)
  __device__ __forceinline__ void fetch_first(int v, int pw, int lane, int par) const {
    const int e = sload(a.order + uni(v / (tm * tn)));
    const int o0 = sload(a.offsets + e), o1 = sload(a.offsets + e + 1);
    Ld::fetch_rows(a.row_src, a.zeros, o0, uni(o1 - o0), ids + pw * 2 * IDS_SLOT, lane, 0, par);
  }
  __device__ __forceinline__ void compute(const bf16_t* st, int slot, Acc& acc, int lane, const WaveRows& w,
                                          int wn) const {
    if constexpr (MX) mx_compute<JWgrad>(st, scring + slot * MX_SC_SLOT, acc, lane, w, wn);
    else mma_stage<JWgrad>(st, acc, lane, w, wn);
  }
  __device__ __forceinline__ void setup(int v, Ld& p, int pw, int lane) const {
    const int M = WHICH == 0 ? a.I : a.H, N = WHICH == 0 ? a.H : 2 * a.I;
    Tile t;
    tile(v, t);
    const int e = t.e, m0 = t.m0, n0 = t.n0;
    p.pw = pw;
    p.nk = t.nk;
    if constexpr (MX) {
      // transposed column-wise codes: rows are the output's M / N indices, K runs over
      // the expert's padded row range [poff[e], poff[e + 1]); an expert without rows
      // reads the zero area (its steps only keep the stream's counts)
      const int k0 = sload(m.poff + e);
      auto ra = [&](int r) { return min(m0 + r, M - 1); };
      auto rb = [&](int r) { return min(n0 + r, N - 1); };
      if (t.nk == 0) {
        const uint8_t* z = reinterpret_cast<const uint8_t*>(a.zeros);
        auto r0 = [](int) { return 0; };
        p.setup(z, z, 0, r0, z, z, 0, r0, 0, scring, lane);
      } else if (WHICH == 0) {
        p.setup(m.qt_a, m.st_a, m.Rp, ra, m.qt_dy, m.st_dy, m.Rp, rb, k0, scring, lane);
      } else {
        p.setup(m.qt_x, m.st_x, m.Rp, ra, m.qt_dgu, m.st_dgu, m.Rp, rb, k0, scring, lane);
      }
    } else {
      const int o0 = sload(a.offsets + e), o1 = sload(a.offsets + e + 1);
      p.rs = o0;
      p.cnt = uni(o1 - o0);
      p.row_src = a.row_src; p.zeros = a.zeros; p.inv_k = 1.0 / a.k;
      p.lane = lane;
      p.ids = ids + pw * 2 * IDS_SLOT;
      if (WHICH == 0) {
        p.abase = a.aw; p.lda = a.I;
        p.bbase = a.dy; p.ldb = a.H;
      } else {
        p.abase = AG ? a.x : a.xp; p.lda = a.H;
        p.bbase = a.dgu; p.ldb = 2 * a.I;
      }
#pragma unroll
      for (int q = 0; q < A_LP; ++q) {
        int r, c;
        mnmaj_slot<BM>(load_slot(q, pw, lane), r, c);
        const int col = m0 + c * 8;
        p.acol[q] = col < M ? col : m0;
      }
#pragma unroll
      for (int q = 0; q < B_LP; ++q) {
        int r, c;
        mnmaj_slot<BN>(load_slot(q, pw, lane), r, c);
        const int col = n0 + c * 8;
        p.bcol[q] = col < N ? col : n0;
      }
    }
  }
  // The transposed accumulator blocks become bf16 row chunks (trans_chunks) and leave
  // through the wave's LDS band (band_store), 8 lanes to a 128-byte row segment.
  __device__ __forceinline__ void epilogue(const Tile& p, const Acc& acc, float* stage) const {
    const int M = WHICH == 0 ? a.I : a.H, N = WHICH == 0 ? a.H : 2 * a.I;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = (int)((unsigned)wv % WM), wn = (int)((unsigned)wv / WM);
    // the tile's first output row in dW_down, or in dW_gate and dW_up (uniform)
    const uint32_t ld = WHICH == 0 ? (uint32_t)a.H : (uint32_t)a.I;
    const size_t row0 = ((size_t)p.e * M + p.m0) * ld;
    bf16_t* const wreg = reinterpret_cast<bf16_t*>(stage) + wv * BAND_ELEMS;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      i32x4 ch[NI][2];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) trans_chunks(acc[mi][ni], ch[ni]);
      const int rb = wm * WROWS + mi * 32;   // the band's first row in the tile
      band_store(wreg, ch, [&](int rr, int cw, i32x4 v) {
        const int rt = rb + rr, n = p.n0 + wn * WCOLS + cw;
        if (p.m0 + rt >= M || n >= N) return;
        bf16_t* dst = WHICH == 0 ? a.dwd + row0 + n : (n < a.I ? a.dwg + row0 + n : a.dwu + row0 + (n - a.I));
        // weight gradients are not read again by this pass: streaming stores
        __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(dst + (uint32_t)rt * ld));
      });
    }
  }
};

// GX (bf16 dW_gate|dW_up only): the Xp rows gathered from x through row_src (no Xp buffer)
template <int WHICH, bool MX, bool GX = false>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_wgrad(BwdArgs a, MxArgs m, int tm, int tn) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) int32_t ids[MX ? 4 : IDS_INTS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  __shared__ int32_t dslot[2];
  if constexpr (MX) {
    JWgrad<WHICH, false, false, true> job{a, m, tm, tn, ids, scring, dslot};
    run_stream(job, lds);
  } else if constexpr (WHICH == 0) {
    JWgrad<0, false, true, false> job{a, m, tm, tn, ids, scring, dslot};
    run_stream(job, lds);
  } else {
    JWgrad<1, GX, false, false> job{a, m, tm, tn, ids, scring, dslot};
    run_stream(job, lds);
  }
}

template <bool MX>
hipError_t launch_bwd_gemms(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  const int nparts = bwd_bf16_nparts(a.I);
  if (a.max_tiles > 0)
    MOE_LAUNCH(MX ? "bwd_dA_mx" : "bwd_dA", k_bwd_da<MX>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.I, BN))),
               dim3(NTHR), 0, st, a, m, nparts);
  return hipGetLastError();
}

}  // namespace

// The bf16 row-tiled GEMMs on the fused stream, in namespace fw256 or fw320 by tile height:
// FwdArgs::tiles holds tiles of that height, BwdArgs holds both tables (tiles, tiles320).
#define MOE_FW_CAT2(a, b) a##b
#define MOE_FW_CAT(a, b) MOE_FW_CAT2(a, b)
namespace MOE_FW_CAT(fw, MOE_GEMM_FW) {
hipError_t launch_fwd_gateup_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MxFwdArgs m{};
  const dim3 grid(grid_for((int64_t)a.max_tiles * ceil_div(a.I, BN / 2)));
  if (a.q_wrows) MOE_LAUNCH("fwd_gateup", (k_fwd_gateup<false, true>), grid, dim3(NTHR), 0, st, a, m);
  else MOE_LAUNCH("fwd_gateup", k_fwd_gateup<false>, grid, dim3(NTHR), 0, st, a, m);
  return hipGetLastError();
}

hipError_t launch_fwd_down_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MxFwdArgs m{};
  const dim3 grid(grid_for((int64_t)a.max_tiles * ceil_div(a.H, BN)));
  if (a.q_wrows) MOE_LAUNCH("fwd_down", (k_fwd_down<false, true>), grid, dim3(NTHR), 0, st, a, m);
  else MOE_LAUNCH("fwd_down", k_fwd_down<false>, grid, dim3(NTHR), 0, st, a, m);
  return hipGetLastError();
}

// the backward's table of this build's tile height
static BwdArgs own_tiles(const BwdArgs& a) {
  BwdArgs b = a;
  if (MOE_GEMM_FW == 320) b.tiles = a.tiles320;
  return b;
}

hipError_t launch_bwd_da_bf16(const BwdArgs& a, hipStream_t st) {
  MxArgs m{};
  return launch_bwd_gemms<false>(own_tiles(a), m, st);
}

hipError_t launch_bwd_dx_bf16(const BwdArgs& a, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MxArgs m{};
  const BwdArgs b = own_tiles(a);
  MOE_LAUNCH("bwd_dX", k_bwd_dx<false>, dim3(grid_for((int64_t)b.max_tiles * ceil_div(b.H, BN))), dim3(NTHR), 0, st,
             b, m);
  return hipGetLastError();
}

#if MOE_GEMM_FW == 256
// The MXFP8 row-tiled GEMMs (256-row tiles only: a step's scale slots, one per A and B
// row, fill the 512 the loads carry).  a.tiles holds 256-row tiles.
hipError_t launch_fwd_gateup_mx(const FwdArgs& a, const MxFwdArgs& m, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MOE_LAUNCH("fwd_gateup_mx", k_fwd_gateup<true>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.I, BN / 2))),
             dim3(NTHR), 0, st, a, m);
  return hipGetLastError();
}

hipError_t launch_fwd_down_mx(const FwdArgs& a, const MxFwdArgs& m, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MOE_LAUNCH("fwd_down_mx", k_fwd_down<true>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.H, BN))), dim3(NTHR), 0,
             st, a, m);
  return hipGetLastError();
}

hipError_t launch_bwd_da_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  return launch_bwd_gemms<true>(a, m, st);
}

hipError_t launch_bwd_dx_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  if (a.max_tiles == 0) return hipSuccess;
  MOE_LAUNCH("bwd_dX_mx", k_bwd_dx<true>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.H, BN))), dim3(NTHR), 0,
             st, a, m);
  return hipGetLastError();
}

// The bf16 weight gradients: 256 x 256 output tiles of each expert's dW, K over its rows.
hipError_t launch_bwd_dwd_bf16(const BwdArgs& a, hipStream_t st) {
  MxArgs m{};
  const int tm = (int)ceil_div(a.I, BM), tn = (int)ceil_div(a.H, BN);
  MOE_LAUNCH("bwd_dWd", (k_bwd_wgrad<0, false>), dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st, a, m,
             tm, tn);
  return hipGetLastError();
}

hipError_t launch_bwd_dwgu_bf16(const BwdArgs& a, hipStream_t st) {
  MxArgs m{};
  const int tm = (int)ceil_div(a.H, BM), tn = (int)ceil_div(2 * a.I, BN);
  const dim3 grid(grid_for((int64_t)a.El * tm * tn));
  if (a.xp)
    MOE_LAUNCH("bwd_dWgu", (k_bwd_wgrad<1, false, false>), grid, dim3(NTHR), 0, st, a, m, tm, tn);
  else
    MOE_LAUNCH("bwd_dWgu", (k_bwd_wgrad<1, false, true>), grid, dim3(NTHR), 0, st, a, m, tm, tn);
  return hipGetLastError();
}

// the fp8 weight gradients (transposed column-wise codes over the padded row space)
hipError_t launch_bwd_dwd_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  const int tm = (int)ceil_div(a.I, BM), tn = (int)ceil_div(a.H, BN);
  MOE_LAUNCH("bwd_dWd_mx", (k_bwd_wgrad<0, true>), dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st, a,
             m, tm, tn);
  return hipGetLastError();
}

hipError_t launch_bwd_dwgu_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  const int tm = (int)ceil_div(a.H, BM), tn = (int)ceil_div(2 * a.I, BN);
  MOE_LAUNCH("bwd_dWgu_mx", (k_bwd_wgrad<1, true>), dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st,
             a, m, tm, tn);
  return hipGetLastError();
}
#endif  // MOE_GEMM_FW == 256

}  // namespace fw256 / fw320

// The host-side launch order of the passes, compiled once (in the 256-row build).
#if MOE_GEMM_FW == 256
// MXFP8 forward.  Order: quantise W_gate, W_up and W_down column-wise (one group per
// expert) and the Xp rows row-wise; K1 on fp8 operands writes G|U and A (bf16) and the
// row-wise codes of A (from its fp32 values); K2 on fp8 operands.  K1 and K2 run on the
// 256-row fused stream (gemm_fw256.hip; a.tiles holds 256-row tiles).
hipError_t launch_fwd_mx(const FwdArgs& a, const MxFwdArgs& m, hipStream_t st, bool k1_only) {
  if (a.max_tiles == 0) return hipSuccess;
  hipError_t e;
  const int El = a.El, H = a.H, I = a.I;
  const int RpH = El * H, RpI = El * I;
#define MOE_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  MOE_TRY(launch_mx_iota(m.goff_h, El, H, st));
  MOE_TRY(launch_mx_iota(m.goff_i, El, I, st));
  // with q_wgu_rows, gate and up codes sit side by side in rows of 2I codes
  const bool rows = m.q_wgu_rows != nullptr;
  MOE_TRY(launch_mx_cols(a.wg, I, nullptr, 1, nullptr, m.goff_h, m.goff_h, El, I, RpH, m.qt_wgu, m.st_wgu,
                         "mx_qt_wgate", st, m.q_wgu_rows, m.s_wgu_rows, 2 * I));
  MOE_TRY(launch_mx_cols(a.wu, I, nullptr, 1, nullptr, m.goff_h, m.goff_h, El, I, RpH, m.qt_wgu + (size_t)I * RpH,
                         m.st_wgu + (size_t)I * (RpH / 32), "mx_qt_wup", st, rows ? m.q_wgu_rows + I : nullptr,
                         rows ? m.s_wgu_rows + I / 32 : nullptr, 2 * I));
  if (!k1_only)
    MOE_TRY(launch_mx_cols(a.wd, H, nullptr, 1, nullptr, m.goff_i, m.goff_i, El, H, RpI, m.qt_wd, m.st_wd,
                           "mx_qt_wdown", st, m.q_wd_rows, m.s_wd_rows, H));
  if (a.xp)
    MOE_TRY(launch_mx_rows(a.xp, nullptr, H, nullptr, 1, a.offsets, El, -1, m.R_cap, H, m.q_x, m.s_x, "mx_q_x", st));
  else
    MOE_TRY(launch_mx_rows(a.x, nullptr, H, a.row_src, a.k, a.offsets, El, -1, m.R_cap, H, m.q_x, m.s_x, "mx_q_x",
                           st));
  MOE_TRY(fw256::launch_fwd_gateup_mx(a, m, st));
  if (!k1_only) MOE_TRY(fw256::launch_fwd_down_mx(a, m, st));
#undef MOE_TRY
  return hipSuccess;
}

int bwd_bf16_nparts(int I) { return WN * (int)ceil_div(I, BN); }
int gemm_cus() { return num_cus(); }

// B1 and B3 run on the fused stream (gemm_fw256.hip or gemm_fw320.hip, by a.bm_da and
// a.bm_dx), the weight gradients on its 256-row build.
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  hipError_t e = a.bm_da == 320 ? fw320::launch_bwd_da_bf16(a, st) : fw256::launch_bwd_da_bf16(a, st);
  if (e == hipSuccess) e = fw256::launch_bwd_dwd_bf16(a, st);
  if (e == hipSuccess) e = a.bm_dx == 320 ? fw320::launch_bwd_dx_bf16(a, st) : fw256::launch_bwd_dx_bf16(a, st);
  if (e == hipSuccess) e = fw256::launch_bwd_dwgu_bf16(a, st);
  return e;
}

// MXFP8 backward (every GEMM on the 256-row fused stream; a.tiles holds 256-row tiles).
// Order: quantise the weights row-wise (unless the forward left
// their codes in the saved buffer), and dY' row-wise together with
// w * dY' column-wise per expert; B1 (fp8) writes dG|dU (bf16); quantise dG|dU row-wise
// and column-wise in one pass, A and Xp column-wise; then B2, B3, B4 on fp8 operands.
hipError_t launch_bwd_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  hipError_t e;
  const int El = a.El, H = a.H, I = a.I;
#define MOE_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  MOE_TRY(launch_poff(a.offsets, El, m.poff, st));
  const int64_t WdRows = (int64_t)El * I, WgRows = (int64_t)El * H;
  if (!m.w_ready) {
    MOE_TRY(launch_mx_rows(a.wd, nullptr, H, nullptr, 1, a.offsets, El, WdRows, WdRows, H, m.q_wd, m.s_wd,
                           "mx_q_wdown", st));
    MOE_TRY(launch_mx_rows(a.wg, a.wu, I, nullptr, 1, a.offsets, El, WgRows, WgRows, 2 * I, m.q_wg, m.s_wg,
                           "mx_q_wgateup", st));
  }
  // dY' rows: row-wise for B1 and, from the same read, column-wise w * dY' for B2
  MOE_TRY(launch_mx_cols(a.dy, H, a.row_src, a.k, a.topk_w, a.offsets, m.poff, El, H, m.Rp, m.qt_dy, m.st_dy,
                         "mx_q_dy", st, m.q_dy, m.s_dy));
  MOE_TRY(fw256::launch_bwd_da_mx(a, m, st));
  // dG|dU: row-wise for B3 and column-wise for B4 in one pass
  MOE_TRY(launch_mx_cols(a.dgu, 2 * I, nullptr, 1, nullptr, a.offsets, m.poff, El, 2 * I, m.Rp, m.qt_dgu, m.st_dgu,
                         "mx_q_dgu", st, m.q_dgu, m.s_dgu));
  MOE_TRY(launch_mx_cols(a.a, I, nullptr, 1, nullptr, a.offsets, m.poff, El, I, m.Rp, m.qt_a, m.st_a, "mx_qt_a", st));
  if (a.xp)
    MOE_TRY(launch_mx_cols(a.xp, H, nullptr, 1, nullptr, a.offsets, m.poff, El, H, m.Rp, m.qt_x, m.st_x, "mx_qt_x",
                           st));
  else
    MOE_TRY(launch_mx_cols(a.x, H, a.row_src, a.k, nullptr, a.offsets, m.poff, El, H, m.Rp, m.qt_x, m.st_x,
                           "mx_qt_x", st));
  MOE_TRY(fw256::launch_bwd_dwd_mx(a, m, st));
  MOE_TRY(fw256::launch_bwd_dx_mx(a, m, st));
  MOE_TRY(fw256::launch_bwd_dwgu_mx(a, m, st));
#undef MOE_TRY
  return hipGetLastError();
}

#endif  // MOE_GEMM_FW == 256

}  // namespace moe
