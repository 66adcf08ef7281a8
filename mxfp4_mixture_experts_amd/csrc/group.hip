// Token-to-expert grouping kernel (the algorithm is in group_dev.hpp).
#include "common.hpp"
#include "group_dev.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(1024) void group_tokens_kernel(const int32_t* __restrict__ ids, int P,
                                                            int E, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pair,
                                                            int32_t* __restrict__ pair_pos,
                                                            int32_t* __restrict__ active,
                                                            int32_t* __restrict__ n_active) {
  __shared__ group_dev::Shared sh;
  group_dev::group_pairs<8>(ids, P, E, counts, offsets, sorted_pair, pair_pos, active, n_active, sh);
}

}  // namespace

hipError_t launch_group_tokens(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                               int32_t* n_active, hipStream_t stream) {
  const int chunks = (P + 63) / 64;
  int waves = chunks < 1 ? 1 : (chunks > group_dev::kMaxWaves ? group_dev::kMaxWaves : chunks);
  group_tokens_kernel<<<1, waves * 64, 0, stream>>>(ids, P, E, counts, offsets, sorted_pair, pair_pos,
                                                    active, n_active);
  return hipGetLastError();
}

}  // namespace moe
