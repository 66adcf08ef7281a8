// Token-to-expert grouping kernel (the algorithm is in group_dev.hpp).
#include "common.hpp"
#include "group_dev.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Above this many 64-pair chunks the grouping runs over several workgroups (group_pairs_multi): on
// MI355X one workgroup took 4.2 us for 512 pairs, 6.8 us for 2048 and 15.8 us for 8192, the
// workgroups 6.2 us for 8192 and 9.3 us for 32768. At most kGroupMaxWgs workgroups, since each one
// reads all P ids.
constexpr int kGroupOneWgChunks = 16;
constexpr int kGroupMaxWgs = 64;

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

__global__ __launch_bounds__(1024) void group_tokens_multi_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                  int cpw, int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_pair,
                                                                  int32_t* __restrict__ pair_pos,
                                                                  int32_t* __restrict__ active,
                                                                  int32_t* __restrict__ n_active) {
  __shared__ group_dev::SharedMulti sh;
  group_dev::group_pairs_multi<8>(ids, P, E, cpw, counts, offsets, sorted_pair, pair_pos, active, n_active, sh);
}

}  // namespace

hipError_t launch_group_tokens(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                               int32_t* n_active, hipStream_t stream) {
  const int chunks = (P + 63) / 64;
  if (chunks > kGroupOneWgChunks) {
    // whole workgroups of 16 waves, a wave's share growing past one chunk only beyond 64 workgroups
    const int per_wave = (chunks + group_dev::kMaxWaves * kGroupMaxWgs - 1) / (group_dev::kMaxWaves * kGroupMaxWgs);
    const int cpw = group_dev::kMaxWaves * per_wave;
    const int grid = (chunks + cpw - 1) / cpw;
    group_tokens_multi_kernel<<<grid, group_dev::kMaxWaves * 64, 0, stream>>>(ids, P, E, cpw, counts, offsets,
                                                                               sorted_pair, pair_pos, active,
                                                                               n_active);
    return hipGetLastError();
  }
  int waves = chunks < 1 ? 1 : (chunks > group_dev::kMaxWaves ? group_dev::kMaxWaves : chunks);
  group_tokens_kernel<<<1, waves * 64, 0, stream>>>(ids, P, E, counts, offsets, sorted_pair, pair_pos,
                                                    active, n_active);
  return hipGetLastError();
}

}  // namespace moe
