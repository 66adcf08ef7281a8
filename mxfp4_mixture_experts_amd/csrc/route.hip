// Router top-k and renormalise: one 64-lane wavefront per token.
//
// The pages time this step as the native router's select/normalize kernel ("MTP1 Post-Portfolio
// Eager-Cycle Profile", Post-Portfolio Device Attribution table) and note that it replaced a
// generic radix select/sort costing about 2.6x more. Here the E logits of a token are spread over
// the wave's lanes (up to 8 per lane). Each logit becomes a 64-bit key that orders like the float
// (larger first) and then like the expert index (lower first); each of the k rounds is a per-lane
// maximum plus a 6-step DPP maximum across the wave, with no sort, no LDS and no shuffles through the
// LDS crossbar. Selection compares the fp32 logits exactly, so the chosen ids are exact.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Total-order key: float order in the high word (-0 canonicalised to +0, so equal floats tie),
// then the lower expert index wins through the inverted index in the low word.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ int key_expert(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)key);
}

// max with a DPP-moved copy; lanes outside row_mask see their own key
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max(uint64_t k) {
  const int hi = (int)(uint32_t)(k >> 32), lo = (int)(uint32_t)k;
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > k ? o : k;
}

// Maximum key over the wave, returned uniformly (the reduction ends in lane 63).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = dpp_max<0xB1, 0xF>(k);   // quad_perm [1,0,3,2]
  k = dpp_max<0x4E, 0xF>(k);   // quad_perm [2,3,0,1]
  k = dpp_max<0x141, 0xF>(k);  // row_half_mirror
  k = dpp_max<0x140, 0xF>(k);  // row_mirror
  k = dpp_max<0x142, 0xA>(k);  // row_bcast15
  k = dpp_max<0x143, 0xC>(k);  // row_bcast31
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 63);
  return ((uint64_t)hi << 32) | lo;
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
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
    key[i] = e < E ? route_key(v[i], e) : 0ull;  // 0 ranks below every real key
  }

  float my_v = 0.0f;  // lane j < k keeps the logit and id of rank j
  int my_e = -1;
  float top = 0.0f, sel_sum = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t win = wave_max_key(best);
    const int e = key_expert(win);
    const float val = key_value(win);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] == win) key[i] = 0ull;  // taken
    if (lane == j) {
      my_v = val;
      my_e = e;
    }
    if (j == 0) top = val;
    // the winner's logit is uniform, so every lane accumulates the selected scores itself
    sel_sum += score_fn == 0 ? expf(val - top) : 1.0f / (1.0f + expf(-val));
  }

  const bool mine = lane < k;
  float w;
  if (score_fn == 0) {
    // softmax: exp(l - max) / sum; the maximum over all experts is the rank-0 logit
    const float s = expf(my_v - top);
    float denom = sel_sum;
    if (!renorm) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) part += expf(v[i] - top);
      denom = wave_sum(part);
    }
    w = s / denom;
  } else {
    const float s = 1.0f / (1.0f + expf(-my_v));
    w = renorm ? s / sel_sum : s;
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
