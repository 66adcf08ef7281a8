// Router GEMM and top-k: logits = x . W_router^T (bf16 operands, fp32 accumulation), then the
// router's select/normalize on those logits.
//
// The pages time the router only as its select/normalize kernel ("Native router select/normalize"
// row of the Post-Portfolio Device Attribution table, "MTP1 Post-Portfolio Eager-Cycle Profile") and
// leave the projection before it undefined; here it is a dense bf16 matrix W_router[E, H].
//   - The projection runs on the matrix cores (v_mfma_f32_16x16x32_bf16). A workgroup owns 64 tokens
//     x 64 experts and one slice of K; each of its four waves computes 16 tokens x 64 experts and
//     loads its operands straight into the MFMA lane layout (lane: row / expert j16, K elements
//     8g .. 8g+7 of a 32-wide step), with no LDS: the tile is small and the weight rows are streamed
//     once per token tile.
//   - At decode there are only one or two 64 x 64 tiles per expert group, so K is split into up to 16
//     slices to spread the weight stream over the GPU; each slice writes its partial logits to the
//     workspace.
//   - One wave per token then sums its partial logits in slice order (deterministic, no atomics),
//     optionally writes the logits, and runs the same selection code as the router kernel.
#include "common.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

constexpr int kRouterTile = 64;      // tokens and experts per workgroup tile
constexpr int kRouterMaxSplits = 16;  // K slices at most
constexpr int kRouterTargetBlocks = 256;

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// part[split][t][e] = sum over K-steps [split * steps_per_split, ...) of x[t][.] . w[e][.]
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int T, int H,
                                                          int E, int tiles_t, int splits,
                                                          int steps_per_split, float* __restrict__ part) {
  const int b = blockIdx.x;
  const int split = b % splits;
  const int tile = b / splits;
  const int tt = tile % tiles_t, te = tile / tiles_t;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int t0 = tt * kRouterTile + wave * 16;
  if (t0 >= T) return;  // no token of this wave
  const int e0 = te * kRouterTile;
  const int steps = H >> 5;
  const int s0 = split * steps_per_split;
  const int s1 = min(s0 + steps_per_split, steps);

  // operand rows; rows past T or E repeat the last one (their results are not stored)
  const uint16_t* xa = x + (size_t)min(t0 + j16, T - 1) * H + g * 8;
  const uint16_t* wb[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) wb[cb] = w + (size_t)min(e0 + cb * 16 + j16, E - 1) * H + g * 8;

  f32x4_t acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int st = s0; st < s1; ++st) {
    const bf16x8_t a = ld_bf16x8(xa + st * 32);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ld_bf16x8(wb[cb] + st * 32), acc[cb], 0, 0, 0);
  }

  // lane holds tokens t0 + 4g + i and expert e0 + 16 cb + j16
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int e = e0 + cb * 16 + j16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t < T && e < E) part[((size_t)split * T + t) * E + e] = acc[cb][i];
    }
  }
}

// One wave per token: the logits as the in-order sum of the slices' partials, then the selection.
template <int EPL>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ part, int splits,
                                                            int T, int E, int k, int score_fn, int renorm,
                                                            float* __restrict__ logits,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ weights) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const size_t slice = (size_t)T * E;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float s = 0.0f;
    if (e < E) {
      const float* p = part + (size_t)t * E + e;
      s = p[0];
#pragma unroll 4
      for (int sp = 1; sp < splits; ++sp) s += p[sp * slice];
      if (logits) logits[(size_t)t * E + e] = s;
    }
    v[i] = s;
  }
  route_dev::route_values<EPL>(v, t, E, k, score_fn, renorm, ids, weights, nullptr);
}

}  // namespace

RouterPlan plan_router(int T, int H, int E) {
  RouterPlan rp;
  rp.tiles_t = (T + kRouterTile - 1) / kRouterTile;
  const int tiles = rp.tiles_t * ((E + kRouterTile - 1) / kRouterTile);
  const int steps = H / 32;
  int splits = (kRouterTargetBlocks + tiles - 1) / (tiles > 0 ? tiles : 1);
  splits = max(1, min(splits, min(kRouterMaxSplits, steps)));
  rp.steps_per_split = (steps + splits - 1) / splits;
  rp.splits = (steps + rp.steps_per_split - 1) / rp.steps_per_split;  // no empty slice
  rp.blocks = tiles * rp.splits;
  return rp;
}

size_t router_workspace_bytes(int T, int H, int E) {
  const RouterPlan rp = plan_router(T, H, E);
  return (size_t)rp.splits * T * E * sizeof(float);
}

hipError_t launch_router_gemm_topk(const uint16_t* x, const uint16_t* w, int T, int H, int E, int k,
                                   int score_fn, int renorm, float* part, float* logits, int32_t* ids,
                                   float* weights, hipStream_t stream) {
  const RouterPlan rp = plan_router(T, H, E);
  router_gemm_kernel<<<rp.blocks, 256, 0, stream>>>(x, w, T, H, E, rp.tiles_t, rp.splits, rp.steps_per_split,
                                                    part);
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_RS(EPL)                                                                                    \
  router_select_kernel<EPL><<<grid, block, 0, stream>>>(part, rp.splits, T, E, k, score_fn, renorm, logits, \
                                                        ids, weights)
  if (E <= 64)
    MOE_RS(1);
  else if (E <= 128)
    MOE_RS(2);
  else if (E <= 256)
    MOE_RS(4);
  else
    MOE_RS(8);
#undef MOE_RS
  return hipGetLastError();
}

}  // namespace moe
