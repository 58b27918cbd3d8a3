// Top-k softmax routing and its backward, one 64-lane wavefront per token (16 lanes per
// token for the selection when E <= 256).
//
// Selection follows the top-K router of NVIDIA's DeepSeek-V3 MoE article ("What makes
// MoE training hard": a learned router activates the top-K experts) at the Prime Mega
// MoE pages' setting (128 experts, top-8).  The k largest fp32 logits win, ties going
// to the lower expert id, slots ordered by logit descending.  Weights: softmax over the
// selected logits (renorm = 1) or the full softmax evaluated at the selected experts.
#include "common.h"

namespace moe {

namespace {

struct Cand {
  float v;
  int id;
};

__device__ __forceinline__ bool better(float av, int aid, float bv, int bid) {
  return av > bv || (av == bv && aid < bid);
}

__device__ __forceinline__ Cand wave_argmax(Cand c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(c.v, off, 64);
    int oid = __shfl_xor(c.id, off, 64);
    if (better(ov, oid, c.v, c.id)) { c.v = ov; c.id = oid; }
  }
  return c;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

constexpr int kPadId = 0x7fffffff;

// VPL = logits held per lane (E <= 64 * VPL).
template <int VPL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T, int E,
                                                    int k, int renorm, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
  bool taken[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
    taken[i] = e >= E;
  }
  float my_v = 0.f, top_v = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    Cand c{-__builtin_inff(), kPadId};
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      if (!taken[i] && better(v[i], e, c.v, c.id)) { c.v = v[i]; c.id = e; }
    }
    c = wave_argmax(c);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i == c.id) taken[i] = true;
    if (j == 0) top_v = c.v;
    if (lane == j) { my_v = c.v; my_id = c.id; }
  }
  // the top-1 logit is the row maximum, so every exponent below is <= 0
  float z = lane < k ? expf(my_v - top_v) : 0.f;
  float den;
  if (renorm) {
    den = wave_sum(z);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - top_v);
    den = wave_sum(s);
  }
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = z / den;
  }
}

// The same selection and weights with 16 lanes per token (four tokens per wavefront),
// for E <= 256: VPL = E / 16 logits per lane, group reductions over 16 lanes.
__device__ __forceinline__ Cand group16_argmax(Cand c) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    float ov = __shfl_xor(c.v, off, 16);
    int oid = __shfl_xor(c.id, off, 16);
    if (better(ov, oid, c.v, c.id)) { c.v = ov; c.id = oid; }
  }
  return c;
}

__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 16);
  return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void k_route_topk16(const float* __restrict__ logits, int T, int E,
                                                      int k, int renorm, int32_t* __restrict__ idx,
                                                      float* __restrict__ w) {
  const int sub = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= T) return;   // a whole 16-lane group leaves together
  const float* row = logits + (size_t)t * E;
  float v[VPL];
  bool taken[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = sub + 16 * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
    taken[i] = e >= E;
  }
  float my_v = 0.f, top_v = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    Cand c{-__builtin_inff(), kPadId};
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = sub + 16 * i;
      if (!taken[i] && better(v[i], e, c.v, c.id)) { c.v = v[i]; c.id = e; }
    }
    c = group16_argmax(c);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (sub + 16 * i == c.id) taken[i] = true;
    if (j == 0) top_v = c.v;
    if (sub == j) { my_v = c.v; my_id = c.id; }
  }
  const float z = sub < k ? expf(my_v - top_v) : 0.f;
  float den;
  if (renorm) {
    den = group16_sum(z);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (sub + 16 * i < E) s += expf(v[i] - top_v);
    den = group16_sum(s);
  }
  if (sub < k) {
    idx[(size_t)t * k + sub] = my_id;
    w[(size_t)t * k + sub] = z / den;
  }
}

// d_logits through the softmax weights (the selection has no gradient).
template <int VPL>
__global__ __launch_bounds__(256) void k_route_bwd(const float* __restrict__ logits,
                                                   const int32_t* __restrict__ idx,
                                                   const float* __restrict__ w,
                                                   const float* __restrict__ dw, int T, int E,
                                                   int k, int renorm,
                                                   float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_id = -1;
  float my_w = 0.f, my_dw = 0.f;
  if (lane < k) {
    my_id = idx[(size_t)t * k + lane];
    my_w = w[(size_t)t * k + lane];
    my_dw = dw[(size_t)t * k + lane];
  }
  const float s = wave_sum(my_w * my_dw);  // sum_j w_j d_w_j
  float* out = dlogits + (size_t)t * E;
  if (renorm) {
    const float gsel = my_w * (my_dw - s);
    float o[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) o[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      int id = __shfl(my_id, j, 64);
      float gj = __shfl(gsel, j, 64);
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i == id) o[i] = gj;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) out[lane + 64 * i] = o[i];
  } else {
    const float* row = logits + (size_t)t * E;
    float v[VPL], g[VPL];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      v[i] = lane + 64 * i < E ? row[lane + 64 * i] : -__builtin_inff();
      mx = fmaxf(mx, v[i]);
      g[i] = 0.f;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float ssum = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      v[i] = lane + 64 * i < E ? expf(v[i] - mx) : 0.f;
      ssum += v[i];
    }
    ssum = wave_sum(ssum);
    for (int j = 0; j < k; ++j) {
      int id = __shfl(my_id, j, 64);
      float dj = __shfl(my_dw, j, 64);
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i == id) g[i] = dj;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) out[lane + 64 * i] = v[i] / ssum * (g[i] - s);
  }
}

}  // namespace

#define MOE_VPL_DISPATCH(E, CALL) \
  do {                            \
    if ((E) <= 64) { CALL(1); }   \
    else if ((E) <= 128) { CALL(2); } \
    else if ((E) <= 256) { CALL(4); } \
    else if ((E) <= 512) { CALL(8); } \
    else { CALL(16); }            \
  } while (0)

hipError_t launch_route_topk(const moe_shape& s, const float* logits, int32_t* idx, float* w,
                             hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (s.E <= 256) {
    dim3 grid((unsigned)ceil_div(s.T, 16)), block(256);
#define CALL16(V) \
  MOE_LAUNCH("route_topk", k_route_topk16<V>, grid, block, 0, st, logits, s.T, s.E, s.k, s.renorm, idx, w)
    if (s.E <= 16) CALL16(1);
    else if (s.E <= 32) CALL16(2);
    else if (s.E <= 64) CALL16(4);
    else if (s.E <= 128) CALL16(8);
    else CALL16(16);
#undef CALL16
    return hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(s.T, 4)), block(256);
#define CALL(V) MOE_LAUNCH("route_topk", k_route_topk<V>, grid, block, 0, st, logits, s.T, s.E, s.k, s.renorm, idx, w)
  MOE_VPL_DISPATCH(s.E, CALL);
#undef CALL
  return hipGetLastError();
}

hipError_t launch_route_bwd(const moe_shape& s, const float* logits, const int32_t* idx,
                            const float* w, const float* dw, float* dlogits, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(s.T, 4)), block(256);
#define CALL(V) MOE_LAUNCH("route_bwd", k_route_bwd<V>, grid, block, 0, st, logits, idx, w, dw, s.T, s.E, s.k, s.renorm, dlogits)
  MOE_VPL_DISPATCH(s.E, CALL);
#undef CALL
  return hipGetLastError();
}

}  // namespace moe
