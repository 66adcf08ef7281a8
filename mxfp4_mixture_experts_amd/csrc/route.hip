// Router top-k and renormalise: one 64-lane wavefront per token.
//
// The pages time this step as the native router's select/normalize kernel ("MTP1 Post-Portfolio
// Eager-Cycle Profile", Post-Portfolio Device Attribution table) and note that it replaced a
// generic radix select/sort costing about 2.6x more. Here the E logits of a token are spread over
// the wave's lanes (up to 8 per lane) and each of the k rounds is one register-level arg-max per
// lane plus a 6-step butterfly across the wave, with no sort and no LDS. Selection compares the fp32
// logits themselves, so the chosen ids are exact; ties go to the lower expert index.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// (v, e) ranks before (bv, be): larger value first, lower index on equal values. e < 0 = no candidate.
__device__ __forceinline__ bool ranks_before(float v, int e, float bv, int be) {
  return e >= 0 && (be < 0 || v > bv || (v == bv && e < be));
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int score_fn, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  float v[EPL];
  uint32_t avail = 0;  // bit i: expert lane + 64*i is still selectable
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
      avail |= 1u << i;
    } else {
      v[i] = 0.0f;
    }
  }

  float my_v = 0.0f;  // lane j < k keeps the value and id of rank j
  int my_e = -1;
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((avail >> i) & 1u)
        if (ranks_before(v[i], lane + 64 * i, bv, be)) {
          bv = v[i];
          be = lane + 64 * i;
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) top = bv;
  }

  const bool mine = lane < k;
  float w;
  if (score_fn == 0) {
    // softmax: exp(l - max) / sum; the maximum over all experts is the rank-0 logit
    const float s = mine ? expf(my_v - top) : 0.0f;
    float denom;
    if (renorm) {
      denom = wave_sum(s);
    } else {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) part += expf(v[i] - top);
      denom = wave_sum(part);
    }
    w = s / denom;
  } else {
    const float s = mine ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
    w = renorm ? s / wave_sum(s) : s;
  }
  if (mine) {
    ids[(size_t)t * k + lane] = my_e;
    weights[(size_t)t * k + lane] = w;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int score_fn, int renorm,
                             int32_t* ids, float* weights, hipStream_t stream) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, score_fn, renorm, ids, weights);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, score_fn, renorm, ids, weights);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, score_fn, renorm, ids, weights);
  else
    route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, score_fn, renorm, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
