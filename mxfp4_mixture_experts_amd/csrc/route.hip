// Router top-k and renormalise: one 64-lane wavefront per token (see route_dev.hpp).
#include "common.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int score_fn, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_dev::route_token<EPL>(logits, t, E, k, score_fn, renorm, ids, weights, nullptr);
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
