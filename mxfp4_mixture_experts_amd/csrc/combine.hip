// Weighted combine: out[t] = bf16( sum_{j=0..k-1} topk_w[t, j] * y[pair_pos[t*k + j]] ), summed in
// fixed j order in fp32, rounded once to bfloat16 (nearest-even). Deterministic: no atomics. The
// pages do not time this step separately (it is not among the named rows of the Post-Portfolio Device
// Attribution table of "MTP1 Post-Portfolio Eager-Cycle Profile"); it completes the routed layer.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ pair_pos, int H,
                                                      int k, int tiles_per_token,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x / tiles_per_token;
  const int n = ((blockIdx.x % tiles_per_token) * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float w = topk_w[(size_t)t * k + j];
    const int row = pair_pos[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)row * H + n);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
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
  combine_kernel<<<dim3(tiles * T), dim3(256), 0, stream>>>(y, topk_w, pair_pos, H, k, tiles, out);
  return hipGetLastError();
}

}  // namespace moe
