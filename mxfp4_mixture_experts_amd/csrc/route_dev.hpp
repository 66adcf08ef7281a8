// Device code of the router top-k (one 64-lane wavefront per token), shared by the router kernel
// and the fused router + grouping kernel.
//
// The pages time this step as the native router's select/normalize kernel ("MTP1 Post-Portfolio
// Eager-Cycle Profile", Post-Portfolio Device Attribution table) and note that it replaced a
// generic radix select/sort costing about 2.6x more. Here the E logits of a token are spread over
// the wave's lanes (up to 8 per lane) as 32-bit keys that order like the floats; each of the k
// rounds is a per-lane maximum, a 6-step DPP maximum across the wave and a few ballots for the
// lowest expert index among equal maxima, with no sort and no LDS. Selection compares the fp32
// logits exactly, so the chosen ids are exact; the selected scores are summed once at the end.
#pragma once

#include "common.hpp"

namespace moe {
namespace route_dev {

// Order key of a logit: unsigned comparison of keys is float comparison of the logits (-0 is
// canonicalised to +0, so equal floats have equal keys). 0 ranks below every real key.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __builtin_bit_cast(float, u);
}

// max with a DPP-moved copy; lanes outside row_mask see their own key
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t k) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)k, (int)k, CTRL, ROW_MASK, 0xF, false);
  return o > k ? o : k;
}

// Maximum key over the wave, returned uniformly (the reduction ends in lane 63).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  k = dpp_max_u32<0xB1, 0xF>(k);   // quad_perm [1,0,3,2]
  k = dpp_max_u32<0x4E, 0xF>(k);   // quad_perm [2,3,0,1]
  k = dpp_max_u32<0x141, 0xF>(k);  // row_half_mirror
  k = dpp_max_u32<0x140, 0xF>(k);  // row_mirror
  k = dpp_max_u32<0x142, 0xA>(k);  // row_bcast15
  k = dpp_max_u32<0x143, 0xC>(k);  // row_bcast31
  return (uint32_t)__builtin_amdgcn_readlane((int)k, 63);
}

// Route token t (one wave) from its logits, held as v[i] = logit of expert lane + 64 i (0 past E):
// ids[t*k + j] and weights[t*k + j] for j < k; the ids also go to ids_copy[t*k + j] when it is not
// null (the fused kernel's LDS copy). Each of the k rounds takes the wave maximum of the keys, then
// the lowest expert index holding it (expert e lives in lane e % 64, slot e / 64, so the first slot
// with a match and its lowest lane give the lowest index).
template <int EPL>
__device__ __forceinline__ void route_values(const float (&v)[EPL], int t, int E, int k, int score_fn,
                                             int renorm, int32_t* __restrict__ ids,
                                             float* __restrict__ weights, int32_t* ids_copy) {
  const int lane = threadIdx.x & 63;
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i < E ? order_key(v[i]) : 0u;

  float my_v = 0.0f;  // lane j < k keeps the logit and id of rank j
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    const uint32_t win = wave_max_u32(best);
    int wi = EPL, wl = 0;
#pragma unroll
    for (int i = EPL - 1; i >= 0; --i) {  // keep the lowest slot with a match
      const uint64_t m = __ballot(key[i] == win);
      if (m) {
        wi = i;
        wl = __ffsll((unsigned long long)m) - 1;
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i == wi && lane == wl) key[i] = 0u;  // taken
    if (lane == j) {
      my_v = key_to_float(win);
      my_e = wl + 64 * wi;
    }
  }

  // the maximum over all experts is the rank-0 logit, held by lane 0
  const float top = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, my_v)));
  const bool mine = lane < k;
  float w;
  if (score_fn == 0) {
    // softmax: exp(l - max) / sum
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
    if (ids_copy) ids_copy[t * k + lane] = my_e;
  }
}

// Route token t (one wave) from row t of logits f32[T, E] (see route_values).
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int score_fn, int renorm, int32_t* __restrict__ ids,
                                            float* __restrict__ weights, int32_t* ids_copy) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
  }
  route_values<EPL>(v, t, E, k, score_fn, renorm, ids, weights, ids_copy);
}

}  // namespace route_dev
}  // namespace moe
