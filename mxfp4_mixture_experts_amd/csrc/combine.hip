// Weighted combine: out[t] = bf16( sum_{j=0..k-1} topk_w[t, j] * y[pair_pos[t*k + j]] ), summed in
// fixed j order in fp32, rounded once to bfloat16 (nearest-even). Deterministic: no atomics. The
// pages do not time this step separately (it is not among the named rows of the Post-Portfolio Device
// Attribution table of "MTP1 Post-Portfolio Eager-Cycle Profile"); it completes the routed layer.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// K = k at compile time: the k row indices and weights are loaded first, then all k rows of y, so a
// thread waits for two round trips rather than two per term; the sum still runs in j order.
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ pair_pos, int H,
                                                      int tiles_per_token, uint16_t* __restrict__ out) {
  const int t = blockIdx.x / tiles_per_token;
  const int n = ((blockIdx.x % tiles_per_token) * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float w[K];
  int row[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    w[j] = topk_w[(size_t)t * K + j];
    row[j] = pair_pos[(size_t)t * K + j];
  }
  float4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = *reinterpret_cast<const float4*>(y + (size_t)row[j] * H + n);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    acc.x = fmaf(w[j], v[j].x, acc.x);
    acc.y = fmaf(w[j], v[j].y, acc.y);
    acc.z = fmaf(w[j], v[j].z, acc.z);
    acc.w = fmaf(w[j], v[j].w, acc.w);
  }
  uint2 o;
  o.x = pack_bf16x2(acc.x, acc.y);
  o.y = pack_bf16x2(acc.z, acc.w);
  *reinterpret_cast<uint2*>(out + (size_t)t * H + n) = o;
}

}  // namespace

int combine_grid(int T, int H) { return ((H / 4 + 255) / 256) * T; }

hipError_t launch_combine(const float* y, const float* topk_w, const int32_t* pair_pos, int T, int H,
                          int k, uint16_t* out, int* grid_out, hipStream_t stream) {
  const int tiles = (H / 4 + 255) / 256;
  if (grid_out) *grid_out = tiles * T;
  const dim3 grid(tiles * T), block(256);
  switch (k) {
#define MOE_CB(K) \
  case K:         \
    combine_kernel<K><<<grid, block, 0, stream>>>(y, topk_w, pair_pos, H, tiles, out); \
    break;
    MOE_CB(1) MOE_CB(2) MOE_CB(3) MOE_CB(4) MOE_CB(5) MOE_CB(6) MOE_CB(7) MOE_CB(8)
    MOE_CB(9) MOE_CB(10) MOE_CB(11) MOE_CB(12) MOE_CB(13) MOE_CB(14) MOE_CB(15) MOE_CB(16)
#undef MOE_CB
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
