// Dispatch index build, row gather, combine / unpermute-sum and the d_topk_w gather.
//
// Dispatch permutes tokens by expert and combine returns the per-expert results to
// token order, accumulating them (NVIDIA DeepSeek-V3 MoE article, "Optimization 2",
// and its Figure 3).  Expert counts stay on the device, so that no device-to-host
// copy sits on the critical path (same article, "Optimization 1").
//
// The permutation is a stable counting sort of the (token, slot) ids by local expert:
// 1) per-chunk expert histograms; 2) in one more kernel, each chunk's workgroup sums
// the histograms of the chunks before it and of all chunks (its base position inside
// every expert group, and the counts and offsets), then ranks its slots with wavefront
// ballots (no atomic ordering), so the row order is deterministic: expert-major, then
// token-ascending.
#include <mutex>

#include "common.h"

namespace moe {

// Scratch of moe_dispatch_noscratch (for callers that cannot allocate): the chunk
// histograms of the index build, kStaticHistInts int32 at most (index_chunk keeps
// nchunks * El <= 32768 for every valid shape).  One copy per GPU, shared by every call
// on that GPU; k_hist writes every entry that k_place then reads, so nothing needs
// clearing between calls.
static __device__ __align__(256) int32_t scratch[kStaticHistInts];

// The device address of this GPU's copy of `scratch`, looked up once per device with that
// device current (the host-side name is not a device address).
hipError_t static_hist_scratch(int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<int32_t*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

namespace {

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ idx, int TK, int chunk, int e_begin,
                                              int El, int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < El; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * chunk;
  const int s1 = min(TK, s0 + chunk);
  for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
    int e = idx[s] - e_begin;
    if (e >= 0 && e < El) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += blockDim.x) chunk_hist[(size_t)blockIdx.x * El + e] = hist[e];
}

// One workgroup per chunk (at least one): expert totals and this chunk's prefix from the
// chunk histograms, an exclusive scan of the totals (workgroup 0 writes counts and
// offsets), then the chunk's slots in steps of 256; wave w of the workgroup takes
// slots [64w, 64w + 64) of a step, and the waves' per-expert counts are combined in
// order.  Rows are kept only below R_cap: a token whose ids repeat a local expert could
// otherwise give more than T * min(k, El) rows; the rows past R_cap in the expert-major
// order get no row (row_of = -1) and counts / offsets stop at R_cap.
__global__ __launch_bounds__(256) void k_place(const int32_t* __restrict__ idx, int TK, int chunk, int nchunks,
                                               int e_begin, int El, int ebits, int R_cap,
                                               const int32_t* __restrict__ chunk_hist,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ row_src, int32_t* __restrict__ row_of) {
  extern __shared__ int32_t sm[];
  int32_t* base = sm;            // [El]: next free row of expert e for this chunk
  int32_t* tot = sm + El;        // [El]: rows of expert e over all chunks
  int32_t* cnt = sm + 2 * El;    // [4][El]: per-wave counts of the current step
  __shared__ int32_t part[256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < El; e += 256) {
    base[e] = tot[e] = 0;
    cnt[e] = cnt[El + e] = cnt[2 * El + e] = cnt[3 * El + e] = 0;
  }
  __syncthreads();
  const int me = blockIdx.x;
  // eight histogram loads in flight per thread before their sums
  constexpr int HU = 8;
  const int nh = nchunks * El;
  for (int i0 = tid; i0 < nh; i0 += 256 * HU) {
    int v[HU];
#pragma unroll
    for (int u = 0; u < HU; ++u) v[u] = i0 + 256 * u < nh ? chunk_hist[i0 + 256 * u] : 0;
#pragma unroll
    for (int u = 0; u < HU; ++u) {
      if (v[u]) {
        const int i = i0 + 256 * u, c = i / El, e = i - c * El;
        atomicAdd(&tot[e], v[u]);
        if (c < me) atomicAdd(&base[e], v[u]);
      }
    }
  }
  __syncthreads();
  // exclusive scan of tot: thread t owns experts [t q, t q + q), q = ceil(El / 256)
  const int q = (El + 255) / 256;
  int mine = 0;
  for (int j = 0; j < q; ++j) {
    const int e = tid * q + j;
    if (e < El) mine += tot[e];
  }
  part[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - mine;
  for (int j = 0; j < q; ++j) {
    const int e = tid * q + j;
    if (e < El) {
      if (me == 0) {
        const int o0 = min(run, R_cap), o1 = min(run + tot[e], R_cap);
        counts[e] = o1 - o0;
        offsets[e] = o0;
      }
      base[e] += run;
      run += tot[e];
    }
  }
  if (me == 0 && tid == 255) offsets[El] = min(part[255], R_cap);
  __syncthreads();
  const int s0 = me * chunk;
  const int s1 = min(TK, s0 + chunk);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int step = s0; step < s1; step += 256) {
    const int s = step + tid;
    int e = -1;
    if (s < s1) {
      e = idx[s] - e_begin;
      if (e < 0 || e >= El) {
        row_of[s] = -1;
        e = -1;
      }
    }
    const bool valid = e >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    const int tot_w = __popcll(peers);
    if (valid && rank == 0) cnt[wv * El + e] = tot_w;
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w2 = 0; w2 < wv; ++w2) pos += cnt[w2 * El + e];
      if (pos < R_cap) row_src[pos] = s;
      row_of[s] = pos < R_cap ? pos : -1;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&base[e], tot_w);
      cnt[wv * El + e] = 0;
    }
    __syncthreads();
  }
}

// Tile table of the row-group GEMMs.  tiles[0] = number of m-tiles; m-tile i (expert
// major, then row-ascending) is entry tiles[4 + 4i .. 4i + 7] = {expert e, index of the
// expert's first m-tile, number of m-tiles of the expert, 0}.  A GEMM with NT column
// tiles enumerates its work as v = first * NT + (n-tile * tiles_of_e + m-tile in e), so
// the m-tiles sharing one weight tile are adjacent and one expert's work is contiguous.
// With order given, it also sets the work order of the weight-gradient GEMMs, whose
// output tiles cost about c = max(ceil(rows / 64), 3) + 2 K steps: if one expert costs
// over twice the mean, or the costliest of the 8 contiguous expert ranges of the XCDs
// exceeds their mean by over 2 %, order[p] = the expert with the p-th most rows (ties:
// lower index first) and order[El] = 1 (dynamic, greedy longest-first scheduling); else
// order[e] = e and order[El] = 0 (contiguous ranges, which keep each expert's tiles on
// one XCD's L2).  order[El + 1] and order[El + 2], the item counters of the dW_down and
// dW_gate|dW_up launches, are zeroed.
// With tiles2 given, the same table for m-tiles of bm2 rows goes to tiles2.
__global__ __launch_bounds__(1024) void k_tile_table(const int32_t* __restrict__ offsets, int El, int bm,
                                                     int32_t* __restrict__ tiles, int bm2,
                                                     int32_t* __restrict__ tiles2, int32_t* __restrict__ zeros,
                                                     int32_t* __restrict__ order) {
  __shared__ int32_t buf[16];  // wave totals of the scan
  __shared__ int32_t rows[1024];
  __shared__ int32_t xsum[8], cmax, dyn;
  const int e = threadIdx.x;
  if (zeros && e < kZeroBytes / 4) zeros[e] = 0;
  if (e < 8) xsum[e] = 0;
  if (e == 0) cmax = 0;
  int n = 0, c = 0;
  if (e < El) {
    c = offsets[e + 1] - offsets[e];
    n = (c + bm - 1) / bm;
  }
  rows[e] = c;
  __syncthreads();
  if (order) {
    if (e < El) {
      const int cost = max((c + 63) / 64, 3) + 2;
      atomicAdd(&xsum[(int)(((int64_t)e * 8) / El)], cost);
      atomicMax(&cmax, cost);
    }
    __syncthreads();
    if (e == 0) {
      int64_t tot = 0, xm = 0;
      for (int x = 0; x < 8; ++x) {
        tot += xsum[x];
        xm = max(xm, (int64_t)xsum[x]);
      }
      dyn = (int64_t)cmax * El > 2 * tot || xm * 8 * 50 > tot * 51;
      order[El] = dyn;
      order[El + 1] = 0;   // the item counters of the two weight-gradient launches
      order[El + 2] = 0;
    }
    __syncthreads();
    if (e < El) {
      int rank = e;
      if (dyn) {
        rank = 0;
        for (int j = 0; j < El; ++j) {
          const int cj = rows[j];
          rank += cj > c || (cj == c && j < e);
        }
      }
      order[rank] = e;
    }
  }
  // inclusive scan of the tile counts: within each wave by shuffles, then over the
  // sixteen wave totals
  const int lane = e & 63, wv = e >> 6;
  for (int t = 0; t < (tiles2 ? 2 : 1); ++t) {
    int32_t* const out = t ? tiles2 : tiles;
    const int b = t ? bm2 : bm;
    n = e < El ? (c + b - 1) / b : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    __syncthreads();   // the previous table's reads of buf are done
    if (lane == 63) buf[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += buf[w];
    incl += before;
    const int start = incl - n;
    for (int j = 0; j < n; ++j) {
      i32x4 ent = {e, start, n, 0};
      *reinterpret_cast<i32x4*>(out + 4 + 4 * (start + j)) = ent;
    }
    if (e == 1023) out[0] = incl;
  }
}

// xp[r] = x[row_src[r] / k]: one wave per row, 16-byte vectors.
template <typename T>
__global__ __launch_bounds__(256) void k_gather(const T* __restrict__ x, int H, int k,
                                                const int32_t* __restrict__ offsets, int El,
                                                const int32_t* __restrict__ row_src, int R_cap,
                                                T* __restrict__ xp) {
  const int R = offsets[El];
  const int lane = threadIdx.x & 63;
  const int nvec = H * (int)sizeof(T) / 16;
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < R; r += gridDim.x * 4) {
    const int t = row_src[r] / k;
    const i32x4* src = reinterpret_cast<const i32x4*>(x + (size_t)t * H);
    i32x4* dst = reinterpret_cast<i32x4*>(xp + (size_t)r * H);
    for (int c = lane; c < nvec; c += 64) dst[c] = src[c];
  }
}

// out[t] = sum_j rows[row_of[t*k + j]] in fp32, one rounding; 0 with no local slot.
template <typename T>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ rows, int T_, int H, int k,
                                                 const int32_t* __restrict__ row_of,
                                                 T* __restrict__ out);

// bf16 rows, KM >= k row slots per token.  With part (the backward's dX combine), also
// d_topk_w of the token's slots: each the sum, in part order, of its row's nparts partial
// row-dots (0 for a slot without a local row).  A lane sums CP 16-byte columns per pass,
// all of their row loads issued before the sums that need them (CP = 4 and plain loads
// for the forward combine: 30.1 -> 26.9 us at the 30B layer; CP = 2 and non-temporal
// loads for the dX unpermute, which also reads the partials: 30.7 us against 31.8 with
// CP = 4).
template <int KM, int CP, bool NT>
__global__ __launch_bounds__(256) void k_combine_bf16(const bf16_t* __restrict__ rows, int T_, int H, int k,
                                                     const int32_t* __restrict__ row_of, bf16_t* __restrict__ out,
                                                     const float* __restrict__ part, int nparts,
                                                     float* __restrict__ d_topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int my_r = lane < k ? row_of[(size_t)t * k + lane] : -1;
  if (part && lane < k) {
    float acc = 0.f;
    if (my_r >= 0)
      for (int p = 0; p < nparts; ++p) acc += part[(size_t)my_r * nparts + p];
    d_topk_w[(size_t)t * k + lane] = acc;
  }
  int rr[KM];  // the token's rows, broadcast while every lane is active (k <= KM)
#pragma unroll
  for (int j = 0; j < KM; ++j) rr[j] = __shfl(my_r, j, 64);
  const int nvec = H / 8;
  for (int c0 = lane; c0 < nvec; c0 += 64 * CP) {
    i32x4 v[CP][KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int r = rr[j];
      if (j >= k || r < 0) continue;
      const i32x4* p = reinterpret_cast<const i32x4*>(rows + (size_t)r * H) + c0;
#pragma unroll
      for (int h = 0; h < CP; ++h)
        if (c0 + 64 * h < nvec) v[h][j] = NT ? __builtin_nontemporal_load(p + 64 * h) : p[64 * h];
    }
#pragma unroll
    for (int h = 0; h < CP; ++h) {
      if (c0 + 64 * h >= nvec) break;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j >= k || rr[j] < 0) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += __uint_as_float(((uint32_t)v[h][j][q]) << 16);
          acc[2 * q + 1] += __uint_as_float(((uint32_t)v[h][j][q]) & 0xffff0000u);
        }
      }
      i32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = (int)pk_bf16(acc[2 * q], acc[2 * q + 1]);
      reinterpret_cast<i32x4*>(out + (size_t)t * H)[c0 + 64 * h] = o;
    }
  }
}

template <>
__global__ __launch_bounds__(256) void k_combine<float>(const float* __restrict__ rows, int T_, int H, int k,
                                                        const int32_t* __restrict__ row_of,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int my_r = lane < k ? row_of[(size_t)t * k + lane] : -1;
  int rr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) rr[j] = __shfl(my_r, j, 64);
  const int nvec = H / 4;
  for (int c = lane; c < nvec; c += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = rr[j];
      if (j >= k || r < 0) continue;
      acc += reinterpret_cast<const f32x4*>(rows + (size_t)r * H)[c];
    }
    reinterpret_cast<f32x4*>(out + (size_t)t * H)[c] = acc;
  }
}

// d_topk_w[s] = sum of the row's partial rowdots, or 0 for a non-local slot.
__global__ __launch_bounds__(256) void k_dtopk(const float* __restrict__ part, int nparts,
                                               const int32_t* __restrict__ row_of, int TK,
                                               float* __restrict__ d_topk_w) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= TK) return;
  const int r = row_of[s];
  float acc = 0.f;
  if (r >= 0)
    for (int p = 0; p < nparts; ++p) acc += part[(size_t)r * nparts + p];
  d_topk_w[s] = acc;
}

}  // namespace

hipError_t launch_index(const moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                        int32_t* row_src, int32_t* row_of, int32_t* chunk_hist, hipStream_t st) {
  const int TK = s.T * s.k;
  const int El = s.e_local;
  const int chunk = index_chunk(TK, El);
  const int nchunks = (int)ceil_div(TK, chunk);
  if (nchunks > 0)
    MOE_LAUNCH("index_hist", k_hist, dim3(nchunks), dim3(256), El * sizeof(int32_t), st, idx, TK, chunk, s.e_begin,
               El, chunk_hist);
  int ebits = 0;
  while ((1 << ebits) < El) ++ebits;
  const int R_cap = s.T * (s.k < El ? s.k : El);
  MOE_LAUNCH("index_place", k_place, dim3(nchunks > 0 ? nchunks : 1), dim3(256), 6 * El * sizeof(int32_t), st, idx,
             TK, chunk, nchunks, s.e_begin, El, ebits, R_cap, chunk_hist, counts, offsets, row_src, row_of);
  return hipGetLastError();
}

hipError_t launch_tile_table(const moe_shape& s, const int32_t* offsets, int bm, int32_t* tiles,
                             int32_t* zeros, int32_t* order, hipStream_t st, int bm2, int32_t* tiles2) {
  MOE_LAUNCH("tile_table", k_tile_table, dim3(1), dim3(1024), 0, st, offsets, s.e_local, bm, tiles, bm2, tiles2,
             zeros, order);
  return hipGetLastError();
}

hipError_t launch_gather(const moe_shape& s, const void* x, const int32_t* offsets,
                         const int32_t* row_src, void* xp, hipStream_t st) {
  const int64_t R_cap = (int64_t)s.T * (s.k < s.e_local ? s.k : s.e_local);
  if (R_cap == 0) return hipSuccess;
  const int grid = (int)(ceil_div(R_cap, 4) < 8192 ? ceil_div(R_cap, 4) : 8192);
  if (s.dtype == MOE_BF16)
    MOE_LAUNCH("gather", k_gather<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)x, s.H, s.k, offsets,
                       s.e_local, row_src, (int)R_cap, (bf16_t*)xp);
  else
    MOE_LAUNCH("gather", k_gather<float>, dim3(grid), dim3(256), 0, st, (const float*)x, s.H, s.k, offsets,
                       s.e_local, row_src, (int)R_cap, (float*)xp);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_shape& s, const void* rows, const int32_t* row_of, void* out,
                          hipStream_t st, const char* name, const float* part, int nparts, float* d_topk_w) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(s.T, 4));
  if (s.dtype == MOE_BF16) {
    if (s.k <= 8 && !part) {
      MOE_LAUNCH(name, (k_combine_bf16<8, 4, false>), grid, dim3(256), 0, st, (const bf16_t*)rows, s.T, s.H, s.k,
                 row_of, (bf16_t*)out, part, nparts, d_topk_w);
    } else if (s.k <= 8) {
      MOE_LAUNCH(name, (k_combine_bf16<8, 2, true>), grid, dim3(256), 0, st, (const bf16_t*)rows, s.T, s.H, s.k,
                 row_of, (bf16_t*)out, part, nparts, d_topk_w);
    } else {
      MOE_LAUNCH(name, (k_combine_bf16<16, 2, true>), grid, dim3(256), 0, st, (const bf16_t*)rows, s.T, s.H, s.k,
                 row_of, (bf16_t*)out, part, nparts, d_topk_w);
    }
  } else {
    MOE_LAUNCH(name, k_combine<float>, grid, dim3(256), 0, st, (const float*)rows, s.T, s.H, s.k, row_of,
               (float*)out);
  }
  return hipGetLastError();
}

hipError_t launch_dtopk(const moe_shape& s, const float* dw_part, int nparts, const int32_t* row_of,
                        float* d_topk_w, hipStream_t st) {
  const int TK = s.T * s.k;
  if (TK == 0) return hipSuccess;
  MOE_LAUNCH("dtopk", k_dtopk, dim3((unsigned)ceil_div(TK, 256)), dim3(256), 0, st, dw_part, nparts, row_of, TK,
                     d_topk_w);
  return hipGetLastError();
}

}  // namespace moe
