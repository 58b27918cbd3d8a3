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
#include "gemm_engine.h"

namespace moe {

namespace {

// ---------------- K1: gate/up + SwiGLU ----------------
struct PGateUp : Bf16Mma<PGateUp> {
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
  __device__ void issue(int kt, bf16_t* st, int) const {
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
struct PMnB : Bf16Mma<PMnB> {
  // K-major A rows, MN-major B (row-major weights [K, N])
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  static constexpr int NVMEM = LOADS;
  __device__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  KRows<A_LOADS> a;
  const bf16_t* b[B_LOADS];
  size_t bstep;
  int wv;
  __device__ void issue(int kt, bf16_t* st, int) const {
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
struct PKK : Bf16Mma<PKK> {
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  static constexpr int NVMEM = LOADS;
  __device__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  KRows<A_LOADS> a;
  const bf16_t* b[B_LOADS];   // B rows for K steps [0, ksplit)
  const bf16_t* b2[B_LOADS];  // B3: W_up rows for K steps [ksplit, nk)
  int ksplit;                 // B3: I / 64; B1: larger than any step count
  int wv;
  __device__ void issue(int kt, bf16_t* st, int) const {
    a.issue(kt, st, wv);
    const bool second = kt >= ksplit;
    const int k0 = (second ? kt - ksplit : kt) * BK;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q)
      dma16((second ? b2[q] : b[q]) + k0, st + A_ELEMS + (q * NW + wv) * 64 * 8);
  }
};

// ---------------- MXFP8 operands (backward GEMMs in fp8_bwd mode) ----------------
// Both operands K-major E4M3 codes [rows][K] with e8m0 scales [rows][K/32].  One K step
// is 128 codes: the same 128 bytes per row as a bf16 step of 64, so the LDS ring,
// slots and swizzle are shared.  For v_mfma_scale_f32_32x32x64_f8f6f4 lane l of row
// l & 31 holds codes 16 (l >> 5) .. +15 of each of the two 32-blocks of a 64-code
// sub-step and supplies the scale of block l >> 5 of its row.  The scales of a step (4
// bytes per row) come with one more direct-to-LDS load per thread into a small ring:
// thread slot t < 128 carries A row t, 128 <= t < 384 B row t - 128.
constexpr int MX_STEP = 128;               // codes per K step
constexpr int MX_SC_SLOT = NW * 64 * 4;    // scale bytes per stage
static_assert(MX_STEP == 2 * BK, "an fp8 step must span the bytes of a bf16 step");

__device__ __forceinline__ i32x8 frag_fp8(const bf16_t* tile, int r, int kk, int lane) {
  const int c0 = kk * 4 + (lane >> 5);
  const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + r * BK + (kmaj_chunk(r, c0) << 3));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + r * BK + (kmaj_chunk(r, c0 + 2) << 3));
  i32x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

struct PMx {
  static constexpr int NVMEM = LOADS + 1;
  __device__ static int ncol(int wn, int ni) { return wn * WCOLS + ni * 32; }
  const uint8_t* a[A_LOADS];   // codes of the lane's slot at K step 0
  const uint8_t* b[B_LOADS];
  const uint8_t* sp;           // this thread's scale row at K step 0
  uint8_t* scring;             // NSTAGE x MX_SC_SLOT bytes of LDS
  int wv;
  __device__ void issue(int kt, bf16_t* st, int slot) const {
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) dma16(a[q] + kt * MX_STEP, st + (q * NW + wv) * 64 * 8);
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) dma16(b[q] + kt * MX_STEP, st + A_ELEMS + (q * NW + wv) * 64 * 8);
    dma4(sp + kt * (MX_STEP / 32), scring + slot * MX_SC_SLOT + wv * 256);
  }
  __device__ void compute(const bf16_t* st, int slot, f32x16 (&acc)[2][NI], int lane, int wm, int wn) const {
    const uint8_t* sc = scring + slot * MX_SC_SLOT;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x8 af[2], bf[NI];
      int sa[2], sb[NI];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = wm * 64 + mi * 32 + (lane & 31);
        af[mi] = frag_fp8(st, r, kk, lane);
        sa[mi] = sc[r * 4 + kk * 2 + (lane >> 5)];
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = ncol(wn, ni) + (lane & 31);
        bf[ni] = frag_fp8(st + A_ELEMS, r, kk, lane);
        sb[ni] = sc[(BM + r) * 4 + kk * 2 + (lane >> 5)];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bf[ni], acc[mi][ni], 0, 0, 0, sa[mi],
                                                                       0, sb[ni]);
    }
  }
  // operand rows: A row r (of tile) at a_base + ra(r) * lda, B row n at b_base + rb(n) * ldb;
  // both matrices' scales have row stride ld / 32 and start at s_a / s_b
  template <class RA, class RB>
  __device__ void setup(const uint8_t* a_codes, const uint8_t* a_scales, int lda, RA ra, const uint8_t* b_codes,
                        const uint8_t* b_scales, int ldb, RB rb, int k0, uint8_t* ring, int lane) {
    wv = threadIdx.x >> 6;
    scring = ring;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      a[q] = a_codes + (size_t)ra(r) * lda + k0 + c * 16;
    }
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      int r, c;
      kmaj_slot(load_slot(q, wv, lane), r, c);
      b[q] = b_codes + (size_t)rb(r) * ldb + k0 + c * 16;
    }
    const int t = wv * 64 + lane;
    if (t < BM) sp = a_scales + (size_t)ra(t) * (lda / 32) + k0 / 32;
    else if (t < BM + BN) sp = b_scales + (size_t)rb(t - BM) * (ldb / 32) + k0 / 32;
    else sp = a_scales + (size_t)ra(0) * (lda / 32) + k0 / 32;   // unused slot, any valid row
  }
};

// B1: dA' = dY' Wd^T.  Epilogue: SwiGLU backward on 8 columns per lane, w * A for B2, and
// the rowdot of dA' and A over this wave's 64 columns, reduced across the 8 lanes of a row.
// MX: both operands from the fp8 row-wise buffers (dY' rows, W_down rows along H), and
// no w * A output (the MXFP8 dW_down quantises A and w * dY').
template <bool MX>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_da(BwdArgs a, MxArgs m, int nparts) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  const int NT = (int)ceil_div(a.I, BN);
  Sched sc(a.tiles[0] * NT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1, wn = wv >> 1;
  for (; sc.more(); sc.next()) {
    RowTile t;
    row_tile(a.tiles, a.offsets, sc.v, NT, t);
    const int n0 = t.nt * BN;
    f32x16 acc[2][NI];
    if constexpr (MX) {
      PMx p;
      p.setup(m.q_dy, m.s_dy, a.H, [&](int r) { return t.rs + min(r, t.cnt - 1); }, m.q_wd, m.s_wd, a.H,
              [&](int r) { return t.e * a.I + min(n0 + r, a.I - 1); }, 0, scring, lane);
      mainloop(p, a.H / MX_STEP, lds, acc, wm * 64 < t.cnt);
    } else {
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
      mainloop(p, a.H / BK, lds, acc, wm * 64 < t.cnt);
    }
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
        if (!MX) *reinterpret_cast<i32x4*>(a.aw + r * a.I + col) = pack8(aw);
      }
#pragma unroll
      for (int off = 1; off < EP_LPR; off <<= 1) part += __shfl_xor(part, off, 64);
      if (rt < t.cnt && lane % EP_LPR == 0) a.dw_part[(size_t)(t.rs + rt) * nparts + t.nt * WN + wn] = part;
    });
  }
}

// B3: dXp = dG Wg^T + dU Wu^T, K = 2I: the first I/64 steps read W_gate rows, the rest W_up.
// MX: dG|dU rows against the rows of the concatenated [W_gate | W_up] (both along 2I).
template <bool MX>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_dx(BwdArgs a, MxArgs m) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  const int NT = (int)ceil_div(a.H, BN);
  Sched sc(a.tiles[0] * NT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv & 1;
  for (; sc.more(); sc.next()) {
    RowTile t;
    row_tile(a.tiles, a.offsets, sc.v, NT, t);
    const int n0 = t.nt * BN;
    f32x16 acc[2][NI];
    if constexpr (MX) {
      PMx p;
      p.setup(m.q_dgu, m.s_dgu, 2 * a.I, [&](int r) { return t.rs + min(r, t.cnt - 1); }, m.q_wg, m.s_wg, 2 * a.I,
              [&](int r) { return t.e * a.H + min(n0 + r, a.H - 1); }, 0, scring, lane);
      mainloop(p, 2 * a.I / MX_STEP, lds, acc, wm * 64 < t.cnt);
    } else {
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
      mainloop(p, 2 * a.I / BK, lds, acc, wm * 64 < t.cnt);
    }
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
struct PWgrad : Bf16Mma<PWgrad<AG, BG>> {
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
  __device__ void issue(int kt, bf16_t* st, int) const {
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

template <int WHICH, bool AG, bool BG, bool MX>
__device__ __forceinline__ void wgrad_tile(const BwdArgs& a, const MxArgs& m, bf16_t* lds, int32_t* ids,
                                           uint8_t* scring, int e, int m0, int n0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int M = WHICH == 0 ? a.I : a.H, N = WHICH == 0 ? a.H : 2 * a.I;
  f32x16 acc[2][NI];
  if constexpr (MX) {
    // transposed column-wise codes: rows are the output's M / N indices, K runs over
    // the expert's padded row range [poff[e], poff[e + 1])
    PMx p;
    const int k0 = m.poff[e];
    const int nk = (m.poff[e + 1] - k0) / MX_STEP;
    auto ra = [&](int r) { return min(m0 + r, M - 1); };
    auto rb = [&](int r) { return min(n0 + r, N - 1); };
    if (WHICH == 0) p.setup(m.qt_a, m.st_a, m.Rp, ra, m.qt_dy, m.st_dy, m.Rp, rb, k0, scring, lane);
    else p.setup(m.qt_x, m.st_x, m.Rp, ra, m.qt_dgu, m.st_dgu, m.Rp, rb, k0, scring, lane);
    mainloop(p, nk, lds, acc, true);
  } else {
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
    mainloop(p, (p.cnt + BK - 1) / BK, lds, acc, true);
  }
  epilogue_rows(lds, acc, [&](int rt, int ct, const float (&vv)[8]) {
    const int mm = m0 + rt, n = n0 + ct;
    if (mm >= M || n >= N) return;
    const i32x4 o = pack8(vv);
    if (WHICH == 0) {
      *reinterpret_cast<i32x4*>(a.dwd + ((size_t)e * a.I + mm) * a.H + n) = o;
    } else if (n < a.I) {
      *reinterpret_cast<i32x4*>(a.dwg + ((size_t)e * a.H + mm) * a.I + n) = o;
    } else {
      *reinterpret_cast<i32x4*>(a.dwu + ((size_t)e * a.H + mm) * a.I + (n - a.I)) = o;
    }
  });
}

// B2 (WHICH = 0): dWd[e] [I, H] = (w A)_e^T dY'_e (MX: Q(A)^T Q(w dY')).
// B4 (WHICH = 1): [dWg | dWu][e] [H, 2I] = Xp_e^T [dG | dU]_e.
template <int WHICH, bool MX>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_wgrad(BwdArgs a, MxArgs m, int tm, int tn) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) int32_t ids[MX ? 4 : IDS_INTS];
  __shared__ __attribute__((aligned(16))) uint8_t scring[MX ? NSTAGE * MX_SC_SLOT : 4];
  for (Sched sc(a.El * tm * tn); sc.more(); sc.next()) {
    const int e = sc.v / (tm * tn);
    const int rem = sc.v - e * tm * tn;
    const int mt = rem / tn, nt = rem - mt * tn;
    if (MX) wgrad_tile<WHICH, false, false, true>(a, m, lds, ids, scring, e, mt * BM, nt * BN);
    else if (WHICH == 0) wgrad_tile<0, false, true, false>(a, m, lds, ids, scring, e, mt * BM, nt * BN);
    else if (a.xp) wgrad_tile<1, false, false, false>(a, m, lds, ids, scring, e, mt * BM, nt * BN);
    else wgrad_tile<1, true, false, false>(a, m, lds, ids, scring, e, mt * BM, nt * BN);
  }
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

template <bool MX>
hipError_t launch_bwd_gemms(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  const int nparts = bwd_bf16_nparts(a.I);
  if (a.max_tiles > 0)
    MOE_LAUNCH(MX ? "bwd_dA_mx" : "bwd_dA", k_bwd_da<MX>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.I, BN))),
               dim3(NTHR), 0, st, a, m, nparts);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  MxArgs m{};
  hipError_t e = launch_bwd_gemms<false>(a, m, st);
  if (e != hipSuccess) return e;
  {
    const int tm = (int)ceil_div(a.I, BM), tn = (int)ceil_div(a.H, BN);
    MOE_LAUNCH("bwd_dWd", (k_bwd_wgrad<0, false>), dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st, a, m,
               tm, tn);
  }
  if (a.max_tiles > 0)
    MOE_LAUNCH("bwd_dX", k_bwd_dx<false>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(a.H, BN))), dim3(NTHR), 0, st,
               a, m);
  {
    const int tm = (int)ceil_div(a.H, BM), tn = (int)ceil_div(2 * a.I, BN);
    MOE_LAUNCH("bwd_dWgu", (k_bwd_wgrad<1, false>), dim3(grid_for((int64_t)a.El * tm * tn)), dim3(NTHR), 0, st, a, m,
               tm, tn);
  }
  return hipGetLastError();
}

// MXFP8 backward.  Order: quantise the weights and dY' row-wise; B1 (fp8) writes dG|dU
// (bf16); quantise dG|dU row-wise and, with A, w * dY' and Xp, column-wise per expert;
// then B2, B3, B4 on fp8 operands.
hipError_t launch_bwd_mx(const BwdArgs& a, const MxArgs& m, hipStream_t st) {
  hipError_t e;
  const int El = a.El, H = a.H, I = a.I;
#define MOE_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  MOE_TRY(launch_poff(a.offsets, El, m.poff, st));
  const int64_t WdRows = (int64_t)El * I, WgRows = (int64_t)El * H;
  MOE_TRY(launch_mx_rows(a.wd, nullptr, H, nullptr, 1, a.offsets, El, WdRows, WdRows, H, m.q_wd, m.s_wd,
                         "mx_q_wdown", st));
  MOE_TRY(launch_mx_rows(a.wg, a.wu, I, nullptr, 1, a.offsets, El, WgRows, WgRows, 2 * I, m.q_wg, m.s_wg,
                         "mx_q_wgateup", st));
  MOE_TRY(launch_mx_rows(a.dy, nullptr, H, a.row_src, a.k, a.offsets, El, -1, m.R_cap, H, m.q_dy, m.s_dy, "mx_q_dy",
                         st));
  MOE_TRY(launch_bwd_gemms<true>(a, m, st));
  MOE_TRY(launch_mx_rows(a.dgu, nullptr, 2 * I, nullptr, 1, a.offsets, El, -1, m.R_cap, 2 * I, m.q_dgu, m.s_dgu,
                         "mx_q_dgu", st));
  MOE_TRY(launch_mx_cols(a.a, I, nullptr, 1, nullptr, a.offsets, m.poff, El, I, m.Rp, m.qt_a, m.st_a, "mx_qt_a", st));
  MOE_TRY(launch_mx_cols(a.dy, H, a.row_src, a.k, a.topk_w, a.offsets, m.poff, El, H, m.Rp, m.qt_dy, m.st_dy,
                         "mx_qt_wdy", st));
  if (a.xp)
    MOE_TRY(launch_mx_cols(a.xp, H, nullptr, 1, nullptr, a.offsets, m.poff, El, H, m.Rp, m.qt_x, m.st_x, "mx_qt_x",
                           st));
  else
    MOE_TRY(launch_mx_cols(a.x, H, a.row_src, a.k, nullptr, a.offsets, m.poff, El, H, m.Rp, m.qt_x, m.st_x,
                           "mx_qt_x", st));
  MOE_TRY(launch_mx_cols(a.dgu, 2 * I, nullptr, 1, nullptr, a.offsets, m.poff, El, 2 * I, m.Rp, m.qt_dgu, m.st_dgu,
                         "mx_qt_dgu", st));
#undef MOE_TRY
  {
    const int tm = (int)ceil_div(I, BM), tn = (int)ceil_div(H, BN);
    MOE_LAUNCH("bwd_dWd_mx", (k_bwd_wgrad<0, true>), dim3(grid_for((int64_t)El * tm * tn)), dim3(NTHR), 0, st, a, m,
               tm, tn);
  }
  if (a.max_tiles > 0)
    MOE_LAUNCH("bwd_dX_mx", k_bwd_dx<true>, dim3(grid_for((int64_t)a.max_tiles * ceil_div(H, BN))), dim3(NTHR), 0, st,
               a, m);
  {
    const int tm = (int)ceil_div(H, BM), tn = (int)ceil_div(2 * I, BN);
    MOE_LAUNCH("bwd_dWgu_mx", (k_bwd_wgrad<1, true>), dim3(grid_for((int64_t)El * tm * tn)), dim3(NTHR), 0, st, a, m,
               tm, tn);
  }
  return hipGetLastError();
}

}  // namespace moe
