/*
 * moe.h -- C ABI of the dropless MoE layer hot path for AMD Instinct MI355X (gfx950).
 *
 * The layer: top-k softmax routing over E experts, a stable permutation of the
 * (token, slot) pairs into ragged per-expert row groups, a grouped gate/up GEMM with
 * SwiGLU, a grouped down GEMM scaled by the routing weight, and the weighted combine
 * back to token order; plus the whole backward.  Sources: the Prime Mega MoE pages
 * (the aisight.pl article, opening section: DeepSeek's fused Mega MoE kernel runs the
 * expert-parallel dispatch, both expert linear layers with SwiGLU between them, and the
 * combine as one chain, and Prime Intellect added its backward; precision modes bf16 and
 * fp8_bwd) and NVIDIA's DeepSeek-V3 MoE article (dropless MoE; "Optimization 1": grouped GEMM
 * over each expert's real token count with device-resident shapes; "Optimization 2":
 * dispatch permutes tokens by expert, combine restores token order and accumulates
 * the per-expert outputs; group-aware MXFP8 quantisation).
 *
 * One GPU holds the local experts [e_begin, e_begin + e_local) of E.  Slots routed to
 * other experts are not local: they get no row and contribute nothing here.
 *
 * Conventions shared by every call
 *  - Pointers are device pointers unless stated.  Every call is asynchronous on
 *    `stream` (a hipStream_t; NULL = the null stream).  No call allocates memory,
 *    synchronises, copies device->host or prints.  Expert token counts never leave
 *    the device: kernels read them from `offsets`.
 *  - Arguments are checked on the host before any launch.  A call returns MOE_OK or a
 *    negative moe_status and then nothing was launched; moe_last_error() returns a
 *    thread-local message for the last failing call on this thread.
 *  - Layouts are row-major.  x, dy, y, dx: [T, H].  w_gate, w_up: [e_local, H, I];
 *    w_down: [e_local, I, H] (the local slice).  logits, d_logits: [T, E] fp32.
 *    topk_idx [T, k] int32, topk_w and d_topk_w [T, k] fp32.
 *  - Element type of x, weights, dy, y, dx, dW, xp, yp: fp32 when shape.dtype is
 *    MOE_F32, bf16 (raw 16-bit) when MOE_BF16.
 *  - Rows: R = sum of local counts <= R_cap = T * min(k, e_local).  Row order is
 *    expert-major, token-ascending.  Row buffers are sized for R_cap; rows >= R are
 *    left unspecified.
 *  - The caller owns every buffer, including `saved` and `scratch` whose sizes come
 *    from moe_workspace_bytes().  The library keeps no state between calls apart
 *    from the opt-in timing records of moe_timing_enable, the error string of
 *    moe_last_error, each device's CU count, and the device buffer of
 *    moe_dispatch_noscratch; calls with distinct buffers may run concurrently on
 *    different streams.
 *  - Outputs are overwritten, never accumulated.  dW slices of experts with no rows
 *    are written as zeros; tokens with no local slot get y = 0 and dx = 0.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* a size, range or enum value is invalid, or a required pointer is NULL */
  MOE_EUNSUPPORTED = -2, /* a valid but unsupported combination: H or I not a multiple of 64 in
                            bf16 (H of 4 in fp32), MXFP8 with fp32 data or H, I not multiples of
                            128, an MXFP8 padded row space past 2^31 - 1 rows */
  MOE_EWORKSPACE = -3,   /* a required workspace pointer (saved / scratch) is NULL */
  MOE_EHIP = -4          /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_BWD_SAME = 0, MOE_BWD_MXFP8 = 1 } moe_bwd_prec;
typedef enum { MOE_FWD_SAME = 0, MOE_FWD_MXFP8 = 1 } moe_fwd_prec;

typedef struct {
  int32_t T;        /* tokens, >= 0 */
  int32_t H;        /* hidden size, 1..2^20; MOE_BF16 supports multiples of 64, MOE_F32 of 4 */
  int32_t I;        /* expert intermediate size, 1..2^20; MOE_BF16 supports multiples of 64 */
  int32_t E;        /* routed experts, 1..1024 */
  int32_t k;        /* experts per token, 1..min(E, 16) */
  int32_t e_begin;  /* first local expert */
  int32_t e_local;  /* local experts, >= 1, e_begin + e_local <= E */
  int32_t dtype;    /* moe_dtype */
  int32_t bwd;      /* moe_bwd_prec: MOE_BWD_MXFP8 needs MOE_BF16 */
  int32_t renorm;   /* 1: weights = softmax over the k selected logits; 0: softmax over all E */
  int32_t fwd;      /* moe_fwd_prec: MOE_FWD_MXFP8 needs MOE_BF16 (added in ABI version 2) */
  int32_t recompute;/* 1: activation checkpointing, see moe_bwd; needs MOE_BF16 (ABI version 2) */
  int32_t row_tile; /* rows per tile of the bf16 row-tiled GEMMs (gate/up, down, dA', dX'):
                       0 lets the library choose per GEMM from the shape; 256 or 320 puts all
                       four on that height.  Results do not depend on it: a row's sums run in
                       the same order at either height (ABI version 3) */
} moe_shape;
/* The pages' precision modes map onto (fwd, bwd): bf16 = (SAME, SAME) with MOE_BF16,
 * fp8_bwd = (SAME, MXFP8), mxfp8 = (MXFP8, MXFP8). */

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Message of the last failing call on this thread (host memory, owned by the library). */
const char* moe_last_error(void);

/* Byte sizes of the two caller-owned workspaces for `shape`:
 *  saved   -- written by moe_fwd, read by moe_bwd (the saved G, U and A rows; in
 *             mxfp8 mode also the backward's row-wise MXFP8 codes of the weights,
 *             which the forward's weight passes produce; in fp8_bwd mode the same
 *             codes written by the forward's bf16 GEMMs from the weight tiles they
 *             stream, when the expected rows per expert fill at least three row
 *             tiles of each; else the backward quantises the weights itself);
 *  scratch -- temporary space of moe_dispatch, moe_fwd, moe_bwd, moe_router_fwd and
 *             moe_router_bwd; its contents do not need to survive between calls.
 * Both pointers must be non-NULL.  Returns MOE_EINVAL for an invalid shape.  With
 * shape.recompute = 1 saved_bytes is 0: nothing is kept between the two calls. */
int moe_workspace_bytes(const moe_shape* shape, size_t* saved_bytes, size_t* scratch_bytes);

/* Top-k routing (NVIDIA article: a learned router activates the top-K experts;
 * Prime Mega MoE pages: 128 experts, top-8).  For each token the k largest fp32
 * logits are selected (ties to the lower expert id), ordered by logit descending, and
 * weighted by a softmax over the selected logits (renorm = 1) or by the full softmax
 * over all E logits (renorm = 0).  Writes topk_idx [T, k] and topk_w [T, k]. */
int moe_route_topk(const moe_shape* shape, const float* logits, int32_t* topk_idx,
                   float* topk_w, void* stream);

/* Dispatch (NVIDIA article, "Optimization 2": tokens are permuted by expert).
 * Builds counts [e_local], offsets [e_local + 1] (exclusive prefix of counts), the
 * stable expert-major / token-ascending row order row_src [R_cap] (row -> t*k + j) and
 * its inverse row_of [T*k] (slot -> row, or -1 if the slot's expert is not local,
 * including ids outside [0, E)).  If xp is non-NULL, also gathers xp[r] = x[row_src[r]/k]
 * ([R_cap, H]); with xp == NULL the gather is left to moe_fwd / moe_bwd, which then
 * read x through row_src.  x may be NULL when xp is NULL.  Needs scratch.
 * The k ids of a token must be distinct (moe_route_topk's always are).  If they are not
 * and e_local < k, R could exceed R_cap: the kernel then keeps the first R_cap rows of
 * the expert-major order, gives the later slots no row (row_of = -1, so they contribute
 * nothing and get d_topk_w = 0) and stops counts and offsets at R_cap, so that no write
 * leaves the R_cap-sized buffers of this or any later call. */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                 int32_t* counts, int32_t* offsets, int32_t* row_src, int32_t* row_of,
                 void* xp, void* scratch, void* stream);

/* moe_dispatch without a scratch argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results as moe_dispatch (same arguments apart from scratch), with
 * the index build's chunk histograms in a static device buffer of 32768 int32 (128 KiB)
 * that the library holds on every GPU it runs on until the process ends.  That buffer
 * holds the histograms of every valid shape (their count is at most 32768 by
 * construction); a shape needing more would return MOE_EUNSUPPORTED.  The call allocates
 * nothing (no hipMalloc, no allocating library routine); its first call on a device looks
 * up that device's copy of the buffer.  All calls on one GPU share the buffer: calls that
 * overlap in time on one GPU (e.g. on two streams) race and must not be issued. */
int moe_dispatch_noscratch(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                           int32_t* counts, int32_t* offsets, int32_t* row_src, int32_t* row_of,
                           void* xp, void* stream);

/* Expert MLP forward (Prime Mega MoE pages: two expert linear layers with SwiGLU
 * between them; NVIDIA article Figure 3: two grouped GEMMs over the variable-length
 * expert groups).  For each local row r of expert e and token t = row_src[r] / k:
 *   g = x[t] W_gate[e], u = x[t] W_up[e], a = silu(g) * u,
 *   yp[r] = topk_w[t, j] * (a W_down[e])          ([R_cap, H])
 * g, u and a are kept in `saved` for moe_bwd.  xp may be NULL (rows read from x
 * through row_src) or the buffer filled by moe_dispatch.  Needs saved and scratch.
 * shape.fwd == MOE_FWD_MXFP8 (the pages' mxfp8 mode) runs both GEMMs on MXFP8 operands
 * quantised in the call, blocks of 32 along each GEMM's contraction axis, with the
 * scale and rounding rule of moe_mx_quantize: the rows of x along H and each column of
 * W_gate[e], W_up[e] in blocks of 32 consecutive h; then the rows of a along I
 * (quantised from its fp32 value, before the rounding of the saved bf16 a) and each
 * column of W_down[e] in blocks of 32 consecutive i.  g, u and a are still the
 * bf16-rounded GEMM results, and the routing weight still applies after the down GEMM.
 * Needs H and I multiples of 128 (MOE_EUNSUPPORTED otherwise). */
int moe_fwd(const moe_shape* shape, const void* x, const void* xp, const int32_t* offsets,
            const int32_t* row_src, const float* topk_w, const void* w_gate, const void* w_up,
            const void* w_down, void* yp, void* saved, void* scratch, void* stream);

/* Combine (NVIDIA article, "Optimization 2": results return to token order and the
 * per-expert outputs are accumulated): y[t] = sum over the token's local slots j of
 * yp[row_of[t*k + j]], summed in fp32 and rounded once; 0 for a token with none. */
int moe_combine(const moe_shape* shape, const void* yp, const int32_t* row_of, void* y,
                void* stream);

/* Backward of moe_fwd + moe_combine for upstream gradient dy [T, H] (Prime Mega MoE
 * pages: the backward of the fused chain; fp8_bwd runs it in FP8).  Writes
 *   dx [T, H], dw_gate / dw_up [e_local, H, I], dw_down [e_local, I, H],
 *   d_topk_w [T, k] (0 for non-local slots).
 * shape.bwd == MOE_BWD_MXFP8 runs the four backward GEMMs on MXFP8 operands (E4M3
 * values with one e8m0 scale per 32 along each GEMM's contraction axis, column-wise
 * blocks of 32 rows never crossing an expert group).  `saved` must hold what moe_fwd
 * wrote for the same inputs.  Needs scratch.
 * shape.recompute = 1 (activation checkpointing; Prime Mega MoE pages: the layers are
 * timed with full activation checkpointing, a full layer being two forwards and one
 * backward): moe_fwd keeps g, u, a only in scratch and moe_bwd recomputes them from the
 * same inputs with the same gate/up GEMM (in the forward's precision) before the backward
 * GEMMs, so `saved` may be NULL in both calls and every output is bit-identical to
 * recompute = 0.  With the MXFP8 backward it then quantises its weights itself. */
int moe_bwd(const moe_shape* shape, const void* dy, const void* x, const void* xp,
            const int32_t* offsets, const int32_t* row_src, const int32_t* row_of,
            const float* topk_w, const void* w_gate, const void* w_up, const void* w_down,
            const void* saved, void* dx, void* dw_gate, void* dw_up, void* dw_down,
            float* d_topk_w, void* scratch, void* stream);

/* Router backward through the routing weights (NVIDIA article, "What makes MoE training
 * hard": a learned router scores the experts and the top-K are kept, so the loss reaches
 * the router through the softmax weights of the kept experts; Prime Mega MoE pages: the
 * backward of the fused chain).  Writes d_logits [T, E] fp32.  renorm = 1:
 * d_logits[t, S_j] = w_j (d_w_j - sum_i w_i d_w_i) and 0 for unselected experts;
 * renorm = 0 (needs logits): d_logits[t, e] = p_e (g_e - sum_j p_{S_j} d_w_j) with
 * p = softmax(logits[t]) and g_e = d_w of the slot selecting e, else 0.  The top-k
 * selection itself is piecewise constant and contributes no gradient.  logits is read
 * only for renorm = 0 (the full softmax) and may be NULL for renorm = 1. */
int moe_route_topk_bwd(const moe_shape* shape, const float* logits, const int32_t* topk_idx,
                       const float* topk_w, const float* d_topk_w, float* d_logits,
                       void* stream);

/* Router GEMM with the routing (NVIDIA article, "Optimization 2": fused router kernels
 * assign each token to its experts before dispatch).  The router is one linear map
 * without bias over all E experts (not only the local ones):
 *   logits [T, E] fp32 = x [T, H] w_r [H, E]   (bf16 x and w_r, fp32 accumulation),
 * then the top-k softmax routing of moe_route_topk on these logits (topk_idx, topk_w).
 * Needs MOE_BF16, E a multiple of 8 (MOE_EUNSUPPORTED otherwise) and scratch. */
int moe_router_fwd(const moe_shape* shape, const void* x, const void* w_r, float* logits, int32_t* topk_idx,
                   float* topk_w, void* scratch, void* stream);

/* Backward of the router GEMM for the upstream d_logits [T, E] fp32 (what
 * moe_route_topk_bwd writes): dx [T, H] = dx_in + d_logits w_r^T and dw_r [H, E] =
 * x^T d_logits, both bf16.  dx_in may be NULL (taken as 0) or equal to dx (e.g. the dx
 * that moe_bwd wrote, so that dx becomes the whole input gradient: x feeds both the
 * router and the experts).  d_logits enters the bf16 MFMAs rounded to bf16 and the sums
 * run in fp32; dw_r sums deterministic token slices in a fixed order.  Needs MOE_BF16,
 * E a multiple of 8 and scratch. */
int moe_router_bwd(const moe_shape* shape, const void* x, const void* w_r, const float* d_logits,
                   const void* dx_in, void* dx, void* dw_r, void* scratch, void* stream);

/* MXFP8 quantisation of the backward (NVIDIA article: group-aware MXFP8 quantisation
 * for the MXFP8 grouped GEMMs; Prime Mega MoE pages: fp8_bwd mode), exposed for tests
 * and for callers that keep quantised weights: quantises `rows` rows of K bf16 values
 * (K a multiple of 32, row-major [rows, K]) in blocks of 32 along each row into E4M3
 * (OCP "FN") codes [rows, K] and e8m0 scale codes [rows, K / 32].  Scale: the smallest
 * X with amax <= 448 * 2^X, clamped to [-127, 127], X = 0 for an all-zero block, stored
 * as X + 127; codes: x / 2^X rounded to the nearest E4M3 value, ties to even, sign bit
 * from x.  moe_bwd with MOE_BWD_MXFP8 applies the same rule to every operand it
 * quantises. */
int moe_mx_quantize(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales, void* stream);

/* Group-aware column-wise MXFP8 quantisation (NVIDIA article: the weight-gradient GEMMs
 * contract over token rows, so their operands are quantised in blocks of 32 rows of one
 * column, and a block never crosses from one expert's rows into the next's), exposed for
 * tests and callers.  x: device bf16 [offsets[groups], N] row-major, N a multiple of 8;
 * offsets: device int32 [groups + 1], non-decreasing from 0, 1 <= groups <= 1024.
 * Group g's rows are placed at padded row poff[g] of a row space in which every group
 * starts at a multiple of 128: poff (device int32 [groups + 1], written) = the exclusive
 * prefix sum of the group sizes rounded up to 128.  Outputs are transposed: codes
 * [N, Rp] E4M3 and scales [N, Rp / 32] e8m0 (same scale and rounding rule as
 * moe_mx_quantize), column n's 32-row block j at codes[n][32 j .. 32 j + 31] and
 * scales[n][j]; rows of a group's padding quantise as zeros (codes 0, scale 127).  Rp
 * (a multiple of 128) bounds the padded row space: rows at or past Rp are not written,
 * so Rp >= offsets[groups] + 127 * groups rounded up to 128 always suffices; rows from
 * poff[groups] to Rp are left as they were.  With row_codes and row_scales both given
 * (N then a multiple of 32), the same pass also writes the row-wise quantisation of the
 * rows of x, as moe_mx_quantize would: row_codes [offsets[groups], N], row_scales
 * [offsets[groups], N / 32] (the backward reads dY' and dG|dU once for both layouts).
 * Errors: MOE_EINVAL for bad sizes or NULL pointers. */
int moe_mx_quantize_cols(const void* x, int32_t N, const int32_t* offsets, int32_t groups, int64_t Rp,
                         int32_t* poff, uint8_t* codes, uint8_t* scales, uint8_t* row_codes,
                         uint8_t* row_scales, void* stream);

/* Opt-in kernel timing for profilers and benchmarks (no effect on results).
 * moe_timing_enable(1) makes every kernel that this host thread launches through the
 * calls above carry two HIP events that the dispatch itself stamps at its start and end
 * (hipExtLaunchKernel; events without a system-scope fence); launches on a stream under
 * graph capture are not recorded.  (0) stops it.  Either call discards pending
 * records.  moe_timing_read() waits for the last recorded event, writes up to
 * `capacity` kernel names (static strings owned by the library) and elapsed
 * milliseconds in launch order, sets *count to the number of kernels recorded since the
 * last read or enable, and discards the records.  The events (a pool of 4096 per host
 * thread) are created by moe_timing_enable(1), so the calls above never create one; they
 * are reused and live until the process ends.  Kernels launched after the pool is used
 * up (without a read in between) are not recorded. */
int moe_timing_enable(int on);
int moe_timing_read(int capacity, const char** names, float* ms, int* count);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
