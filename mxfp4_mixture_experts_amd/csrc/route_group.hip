// Router top-k fused with the token grouping, for small batches (decode): one workgroup routes every
// token (a wave per token), keeps the chosen ids in LDS and, after one barrier, groups them (at most
// 64 pairs: the first wave alone, one pair per lane). The two
// steps then cost one launch and no round trip of the ids through memory; the outputs are the same
// as those of the two separate kernels (same device code, see route_dev.hpp and group_dev.hpp).
#include "common.hpp"
#include "group_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

// one token per wave: above 16 tokens (the workgroup's 16 waves) a wave would route several tokens
// one after the other, and the separate router kernel (a wave per token over many workgroups) plus
// the grouping kernel are faster (T = 64: 8 us against 18 us)
constexpr int kFusedMaxTokens = group_dev::kMaxWaves;
constexpr int kFusedMaxPairs = 1024;

template <int EPL>
__global__ __launch_bounds__(1024) void route_group_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score_fn, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ group_dev::Shared sh;
  __shared__ int32_t ids_lds[kFusedMaxPairs];
  const int nw = blockDim.x >> 6;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = w; t < T; t += nw)
    route_dev::route_token<EPL>(logits, t, E, k, score_fn, renorm, ids, weights, ids_lds);
  __syncthreads();
  if (T * k <= 64) {  // one pair per lane of the first wave; the other waves are done
    if (w == 0)
      group_dev::group_pairs_one_wave(static_cast<const int32_t*>(ids_lds), T * k, E, counts, offsets,
                                      sorted_pair, pair_pos, active, n_active, sh);
    return;
  }
  group_dev::group_pairs<1>(static_cast<const int32_t*>(ids_lds), T * k, E, counts, offsets, sorted_pair,
                         pair_pos, active, n_active, sh);
}

}  // namespace

bool route_group_fusable(int T, int k) { return T <= kFusedMaxTokens && T * k <= kFusedMaxPairs; }

hipError_t launch_route_group(const float* logits, int T, int E, int k, int score_fn, int renorm,
                              int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                              int32_t* n_active, hipStream_t stream) {
  const int chunks = (T * k + 63) / 64;
  int waves = T > chunks ? T : chunks;
  waves = waves < 1 ? 1 : (waves > group_dev::kMaxWaves ? group_dev::kMaxWaves : waves);
  const dim3 grid(1), block(64 * waves);
#define MOE_RG(EPL)                                                                               \
  route_group_kernel<EPL><<<grid, block, 0, stream>>>(logits, T, E, k, score_fn, renorm, ids, weights, \
                                                      counts, offsets, sorted_pair, pair_pos, active,  \
                                                      n_active)
  if (E <= 64)
    MOE_RG(1);
  else if (E <= 128)
    MOE_RG(2);
  else if (E <= 256)
    MOE_RG(4);
  else
    MOE_RG(8);
#undef MOE_RG
  return hipGetLastError();
}

}  // namespace moe
