// Host entry points of libmoe: argument checks, workspace layout and launch order.
// The declarations and their contracts are in include/moe.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "common.h"

namespace moe {
}

using namespace moe;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int64_t R_cap;
  size_t es;         // element size of the data dtype
  int max_tiles;     // row-group tile bound (256-row tiles; 320-row ones are fewer)
  int nparts;        // rowdot partials per row
  int nchunks;
  // saved
  size_t off_gu, off_a, saved_bytes;
  // mxfp8 mode (MXFP8 forward and backward): the backward's row-wise weight codes, written
  // by the forward's weight passes into saved (codes, scales of W_down, [W_gate | W_up])
  bool wrows_saved;
  size_t off_wrows[4];
  // recompute: G|U and A in scratch, behind every other scratch buffer
  size_t off_rgu, off_ra;
  size_t off_router_part;
  // scratch
  size_t off_tiles, off_tiles320, off_zeros, off_order, off_dgu, off_dxp, off_part, off_aw, scratch_bytes;
  // MXFP8 backward buffers (scratch), 0 when unused
  int64_t Rp;
  size_t off_mx[17];
  // MXFP8 forward buffers (scratch, after the tile table), 0 when unused
  size_t off_mxf[10];
};

int check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_EINVAL, "shape is NULL");
  if (s->T < 0) return fail(MOE_EINVAL, "T = %d < 0", s->T);
  if (s->H <= 0 || s->I <= 0 || s->H > (1 << 20) || s->I > (1 << 20))
    return fail(MOE_EINVAL, "H = %d and I = %d must lie in 1..2^20", s->H, s->I);
  if (s->E < 1 || s->E > 1024) return fail(MOE_EINVAL, "E = %d outside 1..1024", s->E);
  if (s->k < 1 || s->k > s->E || s->k > 16) return fail(MOE_EINVAL, "k = %d outside 1..min(E, 16)", s->k);
  if (s->e_local < 1 || s->e_begin < 0 || (int64_t)s->e_begin + s->e_local > s->E)
    return fail(MOE_EINVAL, "local experts [%d, %d + %d) outside [0, E = %d)", s->e_begin, s->e_begin,
                s->e_local, s->E);
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return fail(MOE_EINVAL, "dtype = %d", s->dtype);
  if (s->bwd != MOE_BWD_SAME && s->bwd != MOE_BWD_MXFP8) return fail(MOE_EINVAL, "bwd = %d", s->bwd);
  if (s->renorm != 0 && s->renorm != 1) return fail(MOE_EINVAL, "renorm = %d", s->renorm);
  if ((int64_t)s->T * s->k > 0x7fffffffLL) return fail(MOE_EINVAL, "T * k exceeds 2^31 - 1");
  if (s->dtype == MOE_BF16 && (s->H % 64 != 0 || s->I % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "bf16 needs H and I multiples of 64 (H = %d, I = %d)", s->H, s->I);
  if (s->dtype == MOE_F32 && s->H % 4 != 0)
    return fail(MOE_EUNSUPPORTED, "fp32 needs H a multiple of 4 (H = %d)", s->H);
  if (s->bwd == MOE_BWD_MXFP8 && s->dtype != MOE_BF16)
    return fail(MOE_EUNSUPPORTED, "the MXFP8 backward needs bf16 data");
  if (s->bwd == MOE_BWD_MXFP8 && s->H % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "the MXFP8 backward needs H a multiple of 128 (H = %d)", s->H);
  if (s->bwd == MOE_BWD_MXFP8) {  // the kernels index the padded row space with int
    const int64_t R_cap = (int64_t)s->T * (s->k < s->e_local ? s->k : s->e_local);
    const int64_t Rp = mx_rp_cap(R_cap, s->e_local);
    if (Rp > 0x7fffffffLL)
      return fail(MOE_EUNSUPPORTED, "the MXFP8 backward's padded row space (%lld rows) exceeds 2^31 - 1",
                  (long long)Rp);
  }
  if (s->fwd != MOE_FWD_SAME && s->fwd != MOE_FWD_MXFP8) return fail(MOE_EINVAL, "fwd = %d", s->fwd);
  if (s->recompute != 0 && s->recompute != 1) return fail(MOE_EINVAL, "recompute = %d", s->recompute);
  if (s->recompute && s->dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "recompute needs bf16 data");
  if (s->row_tile != 0 && s->row_tile != 256 && s->row_tile != 320)
    return fail(MOE_EINVAL, "row_tile = %d (0, 256 or 320)", s->row_tile);
  if (s->fwd == MOE_FWD_MXFP8) {  // e_local * H <= 2^30 by the limits above: int column strides
    if (s->dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "the MXFP8 forward needs bf16 data");
    if (s->H % 128 != 0 || s->I % 128 != 0)
      return fail(MOE_EUNSUPPORTED, "the MXFP8 forward needs H and I multiples of 128 (H = %d, I = %d)", s->H, s->I);
  }
  return MOE_OK;
}

// Tile heights of the bf16 row-tiled GEMMs on the fused stream, 256 or 320 rows, per GEMM.
// A token picks a given expert with probability k / E, so an expert's row count c is
// Binomial(T, k / E); read as a normal law (continuity-corrected), it needs
// E[ceil(c / bm)] = sum over j >= 0 of P(c > j bm) tiles of height bm.  A GEMM with nt
// column tiles gives the persistent grid about ceil(El E[..] nt / CUs) rounds of tiles,
// each taking time in proportion to its height (MFMA work and operand bytes per K step),
// and the height with the fewer rounds x rows wins; 256 on a tie (less padding and fewer
// bytes per step).  Qwen3-30B-A3B (about 256 rows an expert): 320 for all four; the
// 235B-A22B share (about 1024): 320 for the gate/up GEMM only.
struct RowTiles {
  int k1, k2, da, dx;
};

static double tiles_per_expert(const moe_shape& s, int bm) {
  const double p = (double)s.k / s.E, m = s.T * p, sd = sqrt(s.T * p * (1.0 - p));
  double t = 0.0;
  for (int j = 0;; ++j) {
    const double x = (double)j * bm;  // P(c > x) = P(c >= x + 1)
    if (x > m + 12.0 * sd) break;
    t += sd > 0.0 ? 0.5 * erfc((x + 0.5 - m) / (sd * sqrt(2.0))) : (m > x ? 1.0 : 0.0);
  }
  return t;
}

RowTiles row_tile_heights(const moe_shape& s) {
  if (s.row_tile != 0) return {s.row_tile, s.row_tile, s.row_tile, s.row_tile};
  const double t256 = s.e_local * tiles_per_expert(s, 256), t320 = s.e_local * tiles_per_expert(s, 320);
  const int64_t cus = gemm_cus();
  auto pick = [&](int64_t nt) {
    const int64_t c256 = ceil_div(llround(t256 * nt), cus) * 256, c320 = ceil_div(llround(t320 * nt), cus) * 320;
    return c320 < c256 ? 320 : 256;
  };
  return {pick(ceil_div(s.I, 128)), pick(ceil_div(s.H, 256)), pick(ceil_div(s.I, 256)), pick(ceil_div(s.H, 256))};
}

// The 256-row and / or the 320-row tile table (one launch; zeros and order, when given,
// are written with them)
static hipError_t tile_tables(const moe_shape& s, const int32_t* offsets, bool n256, bool n320, int32_t* t256,
                              int32_t* t320, int32_t* zeros, int32_t* order, hipStream_t st) {
  if (n256 || !n320)
    return launch_tile_table(s, offsets, 256, t256, zeros, order, st, n320 ? 320 : 0, n320 ? t320 : nullptr);
  return launch_tile_table(s, offsets, 320, t320, zeros, order, st);
}

// fp8_bwd: the forward's bf16 GEMMs write the weights' row-wise codes for the backward
// when each expert's weight slices pass through at least three row tiles of both GEMMs
// (the row tiles share the quantising steps; the 235B-A22B share has about four).  With
// fewer, those tiles' extra stores cost more than the backward's own weight passes (an
// expert of one row tile would quantise every step of its stream).
static bool fwd_writes_wcodes(const moe_shape& s) {
  if (s.dtype != MOE_BF16 || s.bwd != MOE_BWD_MXFP8 || s.fwd == MOE_FWD_MXFP8 || s.recompute) return false;
  const RowTiles h = row_tile_heights(s);
  return tiles_per_expert(s, h.k1) >= 3.0 && tiles_per_expert(s, h.k2) >= 3.0;
}

void layout(const moe_shape& s, Layout& L) {
  const int El = s.e_local;
  L.R_cap = (int64_t)s.T * (s.k < El ? s.k : El);
  L.es = s.dtype == MOE_BF16 ? 2 : 4;
  L.max_tiles = (int)ceil_div(L.R_cap, 256) + El;
  L.nparts = s.dtype == MOE_BF16 ? bwd_bf16_nparts(s.I) : s.I;
  L.nchunks = (int)ceil_div((int64_t)s.T * s.k, index_chunk((int64_t)s.T * s.k, El));
  const size_t R = (size_t)L.R_cap;
  L.off_gu = 0;
  L.off_a = align_up(R * 2 * s.I * L.es);
  L.saved_bytes = s.recompute ? 0 : L.off_a + align_up(R * s.I * L.es);
  // the weights' row-wise codes for the MXFP8 backward, written by the forward (its weight
  // passes in mxfp8, its bf16 GEMMs' B stages in fp8_bwd where that pays) and kept with
  // the activations; else the backward quantises the weights itself
  L.wrows_saved = s.bwd == MOE_BWD_MXFP8 && !s.recompute && (s.fwd == MOE_FWD_MXFP8 || fwd_writes_wcodes(s));
  for (int i = 0; i < 4; ++i) L.off_wrows[i] = 0;
  if (L.wrows_saved) {
    const size_t Eh = (size_t)El * s.H, Ei = (size_t)El * s.I;
    const size_t sizes[4] = {Ei * s.H, Ei * s.H / 32, Eh * 2 * s.I, Eh * 2 * s.I / 32};
    for (int i = 0; i < 4; ++i) {
      L.off_wrows[i] = L.saved_bytes;
      L.saved_bytes += align_up(sizes[i]);
    }
  }
  const size_t dispatch_bytes = align_up((size_t)L.nchunks * El * 4);
  L.off_tiles = 0;
  L.off_tiles320 = align_up((size_t)(4 + 4 * L.max_tiles) * 4);
  L.off_zeros = L.off_tiles320 + align_up((size_t)(4 + 4 * L.max_tiles) * 4);
  L.off_order = L.off_zeros + align_up(kZeroBytes);
  L.off_dgu = L.off_order + align_up((size_t)(El + 3) * 4);
  L.off_dxp = L.off_dgu + align_up(R * 2 * s.I * L.es);
  L.off_part = L.off_dxp + align_up(R * s.H * L.es);
  L.off_aw = L.off_part + align_up(R * L.nparts * 4);
  size_t bwd_bytes = L.off_aw + (s.dtype == MOE_BF16 ? align_up(R * s.I * L.es) : 0);
  L.Rp = 0;
  for (int i = 0; i < 17; ++i) L.off_mx[i] = 0;
  if (s.bwd == MOE_BWD_MXFP8) {
    const size_t H = (size_t)s.H, I = (size_t)s.I, Eh = (size_t)El * s.H, Ei = (size_t)El * s.I;
    L.Rp = mx_rp_cap(L.R_cap, El);
    const size_t Rp = (size_t)L.Rp;
    // codes then scales of: dY' rows, W_down rows, dG|dU rows, [W_gate|W_up] rows,
    // A^T, (w dY')^T, Xp^T, (dG|dU)^T; then the padded offsets
    // (the weights' row-wise codes live in saved when the forward writes them)
    const size_t wsz = L.wrows_saved ? 0 : 1;
    const size_t sizes[17] = {R * H, R * H / 32, wsz * Ei * H, wsz * Ei * H / 32, R * 2 * I, R * 2 * I / 32,
                              wsz * Eh * 2 * I, wsz * Eh * 2 * I / 32, I * Rp, I * Rp / 32, H * Rp, H * Rp / 32,
                              H * Rp, H * Rp / 32, 2 * I * Rp, 2 * I * Rp / 32, (size_t)(El + 1) * 4};
    size_t off = bwd_bytes;
    for (int i = 0; i < 17; ++i) {
      L.off_mx[i] = off;
      off += align_up(sizes[i]);
    }
    bwd_bytes = off;
  }
  L.scratch_bytes = bwd_bytes > dispatch_bytes ? bwd_bytes : dispatch_bytes;
  for (int i = 0; i < 10; ++i) L.off_mxf[i] = 0;
  if (s.fwd == MOE_FWD_MXFP8) {
    const size_t H = (size_t)s.H, I = (size_t)s.I, Eh = (size_t)El * s.H, Ei = (size_t)El * s.I;
    // codes then scales of: Xp rows, A rows, [W_gate | W_up]^T, W_down^T; the group offsets
    const size_t sizes[10] = {R * H, R * H / 32, R * I, R * I / 32, 2 * I * Eh, 2 * I * Eh / 32, H * Ei, H * Ei / 32,
                              (size_t)(El + 1) * 4, (size_t)(El + 1) * 4};
    size_t off = L.off_dgu;  // the tile table and the zeroed area stay in front
    for (int i = 0; i < 10; ++i) {
      L.off_mxf[i] = off;
      off += align_up(sizes[i]);
    }
    if (off > L.scratch_bytes) L.scratch_bytes = off;
  }
  // the router GEMM's scratch (a separate call: overlaps everything above): W_r^T, then the
  // fp32 partial sums of dW_r
  L.off_router_part = align_up((size_t)s.E * s.H * 2);
  const size_t router_bytes = L.off_router_part +
                              align_up((size_t)router_dw_slices(s.T, s.H, s.E) * s.H * s.E * 4);
  if (router_bytes > L.scratch_bytes) L.scratch_bytes = router_bytes;
  L.off_rgu = L.off_ra = 0;
  if (s.recompute) {
    L.off_rgu = L.scratch_bytes;
    L.off_ra = L.off_rgu + align_up(R * 2 * s.I * L.es);
    L.scratch_bytes = L.off_ra + align_up(R * s.I * L.es);
  }
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off); }
template <typename T>
const T* at(const void* base, size_t off) { return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off); }

// ---- opt-in per-kernel timing of this host thread ----
struct TimingRec {
  const char* name;
  int e0, e1;
};
// The events are created once, by moe_timing_enable, so that no hot-path call creates
// one; a kernel launched when the pool is used up is not recorded.
constexpr int kTimingEvents = 4096;
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> pool;
  int used = 0;
  std::vector<TimingRec> recs;
  hipEvent_t next() { return used < (int)pool.size() ? pool[used++] : nullptr; }
};
thread_local Timing g_timing;

#define REQUIRE(p) do { if (!(p)) return fail(MOE_EINVAL, "%s: %s is NULL", __func__, #p); } while (0)
#define REQUIRE_WS(p) do { if (!(p)) return fail(MOE_EWORKSPACE, "%s: workspace %s is NULL", __func__, #p); } while (0)

}  // namespace

namespace moe {
bool ktimer_pair(const char* name, hipStream_t st, hipEvent_t* start, hipEvent_t* stop) {
  Timing& T = g_timing;
  if (!T.on || T.used + 2 > (int)T.pool.size()) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
  *start = T.next();
  *stop = T.next();
  T.recs.push_back({name, T.used - 2, T.used - 1});
  return true;
}
}  // namespace moe

extern "C" {

int moe_timing_enable(int on) {
  Timing& T = g_timing;
  T.on = false;
  T.used = 0;
  T.recs.clear();
  if (on) {
    while ((int)T.pool.size() < kTimingEvents) {
      hipEvent_t ev = nullptr;
      // timestamps only: no system-scope fence (and so no cache writeback) per event
      const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
      if (e != hipSuccess) return hip_status(e, __func__);
      T.pool.push_back(ev);
    }
    T.on = true;
  }
  return MOE_OK;
}

int moe_timing_read(int capacity, const char** names, float* ms, int* count) {
  REQUIRE(count);
  Timing& T = g_timing;
  *count = (int)T.recs.size();
  if (capacity > 0) {
    REQUIRE(names);
    REQUIRE(ms);
  }
  int rc = MOE_OK;
  if (!T.recs.empty()) {
    hipError_t e = hipEventSynchronize(T.pool[T.used - 1]);
    if (e != hipSuccess) rc = hip_status(e, __func__);
    for (int i = 0; i < (int)T.recs.size() && i < capacity && rc == MOE_OK; ++i) {
      names[i] = T.recs[i].name;
      ms[i] = 0.f;
      if (T.recs[i].e1 >= 0) hipEventElapsedTime(&ms[i], T.pool[T.recs[i].e0], T.pool[T.recs[i].e1]);
    }
  }
  T.used = 0;
  T.recs.clear();
  return rc;
}


int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_workspace_bytes(const moe_shape* shape, size_t* saved_bytes, size_t* scratch_bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE(saved_bytes);
  REQUIRE(scratch_bytes);
  Layout L;
  layout(*shape, L);
  *saved_bytes = L.saved_bytes;
  *scratch_bytes = L.scratch_bytes;
  return MOE_OK;
}

int moe_route_topk(const moe_shape* shape, const float* logits, int32_t* topk_idx, float* topk_w,
                   void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (shape->T == 0) return MOE_OK;
  REQUIRE(logits);
  REQUIRE(topk_idx);
  REQUIRE(topk_w);
  return hip_status(launch_route_topk(*shape, logits, topk_idx, topk_w, (hipStream_t)stream), __func__);
}

int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                 int32_t* offsets, int32_t* row_src, int32_t* row_of, void* xp, void* scratch,
                 void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE(counts);
  REQUIRE(offsets);
  REQUIRE_WS(scratch);
  if (shape->T > 0) {
    REQUIRE(topk_idx);
    REQUIRE(row_src);
    REQUIRE(row_of);
    if (xp) REQUIRE(x);
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_index(*shape, topk_idx, counts, offsets, row_src, row_of, (int32_t*)scratch, st);
  if (e == hipSuccess && xp && shape->T > 0) e = launch_gather(*shape, x, offsets, row_src, xp, st);
  return hip_status(e, __func__);
}

int moe_dispatch_noscratch(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* row_src, int32_t* row_of, void* xp, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE(counts);
  REQUIRE(offsets);
  if (shape->T > 0) {
    REQUIRE(topk_idx);
    REQUIRE(row_src);
    REQUIRE(row_of);
    if (xp) REQUIRE(x);
  }
  const int64_t TK = (int64_t)shape->T * shape->k;
  const int64_t nchunks = ceil_div(TK, index_chunk(TK, shape->e_local));
  if (nchunks * shape->e_local > kStaticHistInts)
    return fail(MOE_EUNSUPPORTED, "%s: the index needs %lld histogram entries, past the static buffer's %d",
                __func__, (long long)(nchunks * shape->e_local), kStaticHistInts);
  int32_t* hist = nullptr;
  hipError_t e = static_hist_scratch(&hist);
  if (e != hipSuccess) return hip_status(e, __func__);
  hipStream_t st = (hipStream_t)stream;
  e = launch_index(*shape, topk_idx, counts, offsets, row_src, row_of, hist, st);
  if (e == hipSuccess && xp && shape->T > 0) e = launch_gather(*shape, x, offsets, row_src, xp, st);
  return hip_status(e, __func__);
}

int moe_fwd(const moe_shape* shape, const void* x, const void* xp, const int32_t* offsets,
            const int32_t* row_src, const float* topk_w, const void* w_gate, const void* w_up,
            const void* w_down, void* yp, void* saved, void* scratch, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const moe_shape& s = *shape;
  REQUIRE(offsets);
  REQUIRE(w_gate);
  REQUIRE(w_up);
  REQUIRE(w_down);
  if (!s.recompute) REQUIRE_WS(saved);
  REQUIRE_WS(scratch);
  if (s.T == 0) return MOE_OK;
  REQUIRE(row_src);
  REQUIRE(topk_w);
  REQUIRE(yp);
  if (!xp) REQUIRE(x);
  Layout L;
  layout(s, L);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (s.dtype == MOE_BF16) {
    // the MXFP8 GEMMs take kGemmBMMx-row tiles, the bf16 ones 256- or 320-row tiles by GEMM
    const bool mxf = s.fwd == MOE_FWD_MXFP8;
    const RowTiles h = row_tile_heights(s);
    int32_t* tiles = at<int32_t>(scratch, L.off_tiles);
    int32_t* tiles320 = at<int32_t>(scratch, L.off_tiles320);
    e = tile_tables(s, offsets, mxf || h.k1 == 256 || h.k2 == 256, !mxf && (h.k1 == 320 || h.k2 == 320), tiles,
                    tiles320, nullptr, nullptr, st);
    if (e != hipSuccess) return hip_status(e, __func__);
    FwdArgs a{};
    a.T = s.T; a.H = s.H; a.I = s.I; a.k = s.k; a.El = s.e_local;
    a.x = (const bf16_t*)x; a.xp = (const bf16_t*)xp; a.offsets = offsets; a.row_src = row_src;
    a.topk_w = topk_w; a.wg = (const bf16_t*)w_gate; a.wu = (const bf16_t*)w_up; a.wd = (const bf16_t*)w_down;
    a.tiles = tiles; a.max_tiles = L.max_tiles;
    a.gu = at<bf16_t>(saved, L.off_gu); a.a = at<bf16_t>(saved, L.off_a); a.yp = (bf16_t*)yp;
    if (s.recompute) {  // nothing kept: the down GEMM's A in scratch, no G|U
      a.gu = nullptr;
      a.a = at<bf16_t>(scratch, L.off_ra);
    }
    if (s.fwd == MOE_FWD_MXFP8) {
      MxFwdArgs m{};
      uint8_t** bufs[8] = {&m.q_x, &m.s_x, &m.q_a, &m.s_a, &m.qt_wgu, &m.st_wgu, &m.qt_wd, &m.st_wd};
      for (int i = 0; i < 8; ++i) *bufs[i] = at<uint8_t>(scratch, L.off_mxf[i]);
      m.goff_h = at<int32_t>(scratch, L.off_mxf[8]);
      m.goff_i = at<int32_t>(scratch, L.off_mxf[9]);
      m.R_cap = L.R_cap;
      if (L.wrows_saved) {
        m.q_wd_rows = at<uint8_t>(saved, L.off_wrows[0]);
        m.s_wd_rows = at<uint8_t>(saved, L.off_wrows[1]);
        m.q_wgu_rows = at<uint8_t>(saved, L.off_wrows[2]);
        m.s_wgu_rows = at<uint8_t>(saved, L.off_wrows[3]);
      }
      e = launch_fwd_mx(a, m, st);
    } else {
      FwdArgs k1 = a, k2 = a;
      k1.tiles = h.k1 == 320 ? tiles320 : tiles;
      k2.tiles = h.k2 == 320 ? tiles320 : tiles;
      if (L.wrows_saved) {  // fp8_bwd: the GEMMs also write the weights' codes for moe_bwd
        k2.q_wrows = at<uint8_t>(saved, L.off_wrows[0]);
        k2.s_wrows = at<uint8_t>(saved, L.off_wrows[1]);
        k1.q_wrows = at<uint8_t>(saved, L.off_wrows[2]);
        k1.s_wrows = at<uint8_t>(saved, L.off_wrows[3]);
      }
      e = h.k1 == 320 ? fw320::launch_fwd_gateup_bf16(k1, st) : fw256::launch_fwd_gateup_bf16(k1, st);
      if (e == hipSuccess)
        e = h.k2 == 320 ? fw320::launch_fwd_down_bf16(k2, st) : fw256::launch_fwd_down_bf16(k2, st);
    }
  } else {
    FwdArgsF32 a{};
    a.T = s.T; a.H = s.H; a.I = s.I; a.k = s.k; a.El = s.e_local;
    a.x = (const float*)x; a.xp = (const float*)xp; a.offsets = offsets; a.row_src = row_src;
    a.topk_w = topk_w; a.wg = (const float*)w_gate; a.wu = (const float*)w_up; a.wd = (const float*)w_down;
    a.tiles = nullptr; a.max_tiles = L.max_tiles;
    a.gu = at<float>(saved, L.off_gu); a.a = at<float>(saved, L.off_a); a.yp = (float*)yp;
    e = launch_fwd_f32(a, st);
  }
  return hip_status(e, __func__);
}

int moe_combine(const moe_shape* shape, const void* yp, const int32_t* row_of, void* y, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (shape->T == 0) return MOE_OK;
  REQUIRE(yp);
  REQUIRE(row_of);
  REQUIRE(y);
  return hip_status(launch_combine(*shape, yp, row_of, y, (hipStream_t)stream), __func__);
}

int moe_bwd(const moe_shape* shape, const void* dy, const void* x, const void* xp, const int32_t* offsets,
            const int32_t* row_src, const int32_t* row_of, const float* topk_w, const void* w_gate,
            const void* w_up, const void* w_down, const void* saved, void* dx, void* dw_gate, void* dw_up,
            void* dw_down, float* d_topk_w, void* scratch, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const moe_shape& s = *shape;
  REQUIRE(offsets);
  REQUIRE(w_gate);
  REQUIRE(w_up);
  REQUIRE(w_down);
  REQUIRE(dw_gate);
  REQUIRE(dw_up);
  REQUIRE(dw_down);
  if (!s.recompute) REQUIRE_WS(saved);
  REQUIRE_WS(scratch);
  if (s.T > 0) {
    REQUIRE(dy);
    REQUIRE(row_src);
    REQUIRE(row_of);
    REQUIRE(topk_w);
    REQUIRE(dx);
    REQUIRE(d_topk_w);
    if (!xp) REQUIRE(x);
  }
  Layout L;
  layout(s, L);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (s.dtype == MOE_BF16) {
    // kGemmBMMx-row tiles for the MXFP8 row-tiled GEMMs (B1, B3 and a recomputed MXFP8
    // gate/up GEMM), 256- or 320-row tiles by GEMM for the bf16 ones: one tile-table
    // launch writes the one or two tables the call needs
    const bool mxb = s.bwd == MOE_BWD_MXFP8;
    const bool mxf = s.fwd == MOE_FWD_MXFP8;
    const RowTiles h = row_tile_heights(s);
    int hb[3] = {0, 0, 0};   // heights of the bf16 row-tiled GEMMs this call runs
    if (!mxb) { hb[0] = h.da; hb[1] = h.dx; }
    if (s.recompute && !mxf) hb[2] = h.k1;
    const bool n256 = mxb || (s.recompute && mxf) || hb[0] == 256 || hb[1] == 256 || hb[2] == 256;
    const bool n320 = hb[0] == 320 || hb[1] == 320 || hb[2] == 320;
    int32_t* tiles = at<int32_t>(scratch, L.off_tiles);
    int32_t* tiles320 = at<int32_t>(scratch, L.off_tiles320);
    int32_t* zeros = at<int32_t>(scratch, L.off_zeros);
    int32_t* order = at<int32_t>(scratch, L.off_order);
    e = tile_tables(s, offsets, n256, n320, tiles, tiles320, zeros, order, st);
    if (e != hipSuccess) return hip_status(e, __func__);
    BwdArgs a{};
    a.T = s.T; a.H = s.H; a.I = s.I; a.k = s.k; a.El = s.e_local;
    a.dy = (const bf16_t*)dy; a.x = (const bf16_t*)x; a.xp = (const bf16_t*)xp; a.offsets = offsets;
    a.row_src = row_src; a.topk_w = topk_w; a.wg = (const bf16_t*)w_gate; a.wu = (const bf16_t*)w_up;
    a.wd = (const bf16_t*)w_down; a.gu = at<bf16_t>(saved, L.off_gu); a.a = at<bf16_t>(saved, L.off_a);
    a.tiles = tiles; a.max_tiles = L.max_tiles;
    a.tiles320 = tiles320; a.bm_da = h.da; a.bm_dx = h.dx;
    a.dgu = at<bf16_t>(scratch, L.off_dgu); a.dxp = at<bf16_t>(scratch, L.off_dxp);
    a.dw_part = at<float>(scratch, L.off_part);
    a.aw = at<bf16_t>(scratch, L.off_aw); a.zeros = at<bf16_t>(scratch, L.off_zeros);
    a.order = at<int32_t>(scratch, L.off_order);
    a.dwg = (bf16_t*)dw_gate; a.dwu = (bf16_t*)dw_up; a.dwd = (bf16_t*)dw_down;
    if (s.recompute) {  // G|U and A again, by the forward's gate/up GEMM, into scratch
      bf16_t* const rgu = at<bf16_t>(scratch, L.off_rgu);
      bf16_t* const ra = at<bf16_t>(scratch, L.off_ra);
      a.gu = rgu;
      a.a = ra;
      FwdArgs f{};
      f.T = s.T; f.H = s.H; f.I = s.I; f.k = s.k; f.El = s.e_local;
      f.x = a.x; f.xp = a.xp; f.offsets = offsets; f.row_src = row_src; f.topk_w = topk_w;
      f.wg = a.wg; f.wu = a.wu; f.wd = a.wd;
      f.tiles = !mxf && h.k1 == 320 ? tiles320 : tiles;
      f.max_tiles = L.max_tiles;
      f.gu = rgu; f.a = ra; f.yp = nullptr;
      if (s.fwd == MOE_FWD_MXFP8) {
        MxFwdArgs m{};
        uint8_t** bufs[8] = {&m.q_x, &m.s_x, &m.q_a, &m.s_a, &m.qt_wgu, &m.st_wgu, &m.qt_wd, &m.st_wd};
        for (int i = 0; i < 8; ++i) *bufs[i] = at<uint8_t>(scratch, L.off_mxf[i]);
        m.goff_h = at<int32_t>(scratch, L.off_mxf[8]);
        m.goff_i = at<int32_t>(scratch, L.off_mxf[9]);
        m.R_cap = L.R_cap;
        e = launch_fwd_mx(f, m, st, true);
      } else {
        e = h.k1 == 320 ? fw320::launch_fwd_gateup_bf16(f, st) : fw256::launch_fwd_gateup_bf16(f, st);
      }
      if (e != hipSuccess) return hip_status(e, __func__);
    }
    if (s.bwd == MOE_BWD_MXFP8) {
      MxArgs m{};
      uint8_t** bufs[16] = {&m.q_dy, &m.s_dy, &m.q_wd, &m.s_wd, &m.q_dgu, &m.s_dgu, &m.q_wg, &m.s_wg,
                            &m.qt_a, &m.st_a, &m.qt_dy, &m.st_dy, &m.qt_x, &m.st_x, &m.qt_dgu, &m.st_dgu};
      for (int i = 0; i < 16; ++i) *bufs[i] = at<uint8_t>(scratch, L.off_mx[i]);
      m.poff = at<int32_t>(scratch, L.off_mx[16]);
      m.Rp = (int)L.Rp;
      m.R_cap = L.R_cap;
      m.w_ready = L.wrows_saved;
      if (L.wrows_saved) {  // written by moe_fwd's weight passes
        uint8_t* saved_w = const_cast<uint8_t*>(at<uint8_t>(saved, 0));
        m.q_wd = saved_w + L.off_wrows[0];
        m.s_wd = saved_w + L.off_wrows[1];
        m.q_wg = saved_w + L.off_wrows[2];
        m.s_wg = saved_w + L.off_wrows[3];
      }
      e = launch_bwd_mx(a, m, st);
    } else {
      e = launch_bwd_bf16(a, st);
    }
    if (e == hipSuccess && s.T > 0) e = launch_combine(s, a.dxp, row_of, dx, st, "unpermute_dx", a.dw_part, L.nparts, d_topk_w);
  } else {
    BwdArgsF32 a{};
    a.T = s.T; a.H = s.H; a.I = s.I; a.k = s.k; a.El = s.e_local;
    a.dy = (const float*)dy; a.x = (const float*)x; a.xp = (const float*)xp; a.offsets = offsets;
    a.row_src = row_src; a.topk_w = topk_w; a.wg = (const float*)w_gate; a.wu = (const float*)w_up;
    a.wd = (const float*)w_down; a.gu = at<float>(saved, L.off_gu); a.a = at<float>(saved, L.off_a);
    a.tiles = nullptr; a.max_tiles = L.max_tiles;
    a.dgu = at<float>(scratch, L.off_dgu); a.dxp = at<float>(scratch, L.off_dxp);
    a.dw_part = at<float>(scratch, L.off_part);
    a.dwg = (float*)dw_gate; a.dwu = (float*)dw_up; a.dwd = (float*)dw_down;
    e = launch_bwd_f32(a, st);
    if (e == hipSuccess && s.T > 0) e = launch_combine(s, a.dxp, row_of, dx, st, "unpermute_dx");
    if (e == hipSuccess && s.T > 0) e = launch_dtopk(s, a.dw_part, L.nparts, row_of, d_topk_w, st);
  }
  return hip_status(e, __func__);
}

int moe_router_fwd(const moe_shape* shape, const void* x, const void* w_r, float* logits, int32_t* topk_idx,
                   float* topk_w, void* scratch, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const moe_shape& s = *shape;
  if (s.dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "the router GEMM needs bf16 data");
  if (s.E % 8 != 0) return fail(MOE_EUNSUPPORTED, "the router GEMM needs E a multiple of 8 (E = %d)", s.E);
  REQUIRE(w_r);
  REQUIRE_WS(scratch);
  if (s.T > 0) {
    REQUIRE(x);
    REQUIRE(logits);
    REQUIRE(topk_idx);
    REQUIRE(topk_w);
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_router_fwd(s, (const bf16_t*)x, (const bf16_t*)w_r, at<bf16_t>(scratch, 0), logits, st);
  if (e == hipSuccess && s.T > 0) e = launch_route_topk(s, logits, topk_idx, topk_w, st);
  return hip_status(e, __func__);
}

int moe_router_bwd(const moe_shape* shape, const void* x, const void* w_r, const float* d_logits,
                   const void* dx_in, void* dx, void* dw_r, void* scratch, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const moe_shape& s = *shape;
  if (s.dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "the router GEMM needs bf16 data");
  if (s.E % 8 != 0) return fail(MOE_EUNSUPPORTED, "the router GEMM needs E a multiple of 8 (E = %d)", s.E);
  REQUIRE(w_r);
  REQUIRE(dw_r);
  REQUIRE_WS(scratch);
  if (s.T > 0) {
    REQUIRE(x);
    REQUIRE(d_logits);
    REQUIRE(dx);
  }
  Layout L;
  layout(s, L);
  return hip_status(launch_router_bwd(s, (const bf16_t*)x, (const bf16_t*)w_r, d_logits, (const bf16_t*)dx_in,
                                      (bf16_t*)dx, (bf16_t*)dw_r, at<float>(scratch, L.off_router_part),
                                      (hipStream_t)stream),
                    __func__);
}

int moe_mx_quantize(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0) return fail(MOE_EINVAL, "rows = %lld < 0", (long long)rows);
  if (K <= 0 || K % 32 != 0) return fail(MOE_EINVAL, "K = %d must be a positive multiple of 32", K);
  if (rows == 0) return MOE_OK;
  REQUIRE(x);
  REQUIRE(codes);
  REQUIRE(scales);
  return hip_status(launch_mx_rows((const bf16_t*)x, nullptr, K, nullptr, 1, nullptr, 0, rows, rows, K, codes, scales,
                                   "mx_quantize", (hipStream_t)stream),
                    __func__);
}

int moe_mx_quantize_cols(const void* x, int32_t N, const int32_t* offsets, int32_t groups, int64_t Rp,
                         int32_t* poff, uint8_t* codes, uint8_t* scales, uint8_t* row_codes,
                         uint8_t* row_scales, void* stream) {
  if (groups < 1 || groups > 1024) return fail(MOE_EINVAL, "groups = %d outside 1..1024", groups);
  if (N <= 0 || N % 8 != 0) return fail(MOE_EINVAL, "N = %d must be a positive multiple of 8", N);
  if (Rp < 0 || Rp % kMxRowPad != 0 || Rp > 0x7fffffffLL)
    return fail(MOE_EINVAL, "Rp = %lld must be a multiple of %d in [0, 2^31)", (long long)Rp, kMxRowPad);
  if ((row_codes == nullptr) != (row_scales == nullptr))
    return fail(MOE_EINVAL, "row_codes and row_scales must both be given or both be NULL");
  if (row_codes && N % 32 != 0) return fail(MOE_EINVAL, "row-wise output needs N = %d a multiple of 32", N);
  REQUIRE(offsets);
  REQUIRE(poff);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_poff(offsets, groups, poff, st);
  if (e != hipSuccess || Rp == 0) return hip_status(e, __func__);
  REQUIRE(x);
  REQUIRE(codes);
  REQUIRE(scales);
  return hip_status(launch_mx_cols((const bf16_t*)x, N, nullptr, 1, nullptr, offsets, poff, groups, N, (int)Rp, codes,
                                   scales, "mx_quantize_cols", st, row_codes, row_scales),
                    __func__);
}

int moe_route_topk_bwd(const moe_shape* shape, const float* logits, const int32_t* topk_idx,
                       const float* topk_w, const float* d_topk_w, float* d_logits, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (shape->T == 0) return MOE_OK;
  REQUIRE(topk_idx);
  REQUIRE(topk_w);
  REQUIRE(d_topk_w);
  REQUIRE(d_logits);
  if (!shape->renorm) REQUIRE(logits);
  return hip_status(
      launch_route_bwd(*shape, logits, topk_idx, topk_w, d_topk_w, d_logits, (hipStream_t)stream), __func__);
}

}  // extern "C"
