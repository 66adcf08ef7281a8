// Router GEMM and top-k: logits = x . W_router^T (bf16 operands, fp32 accumulation), then the
// router's select/normalize on those logits.
//
// The pages time the router only as its select/normalize kernel ("Native router select/normalize"
// row of the Post-Portfolio Device Attribution table, "MTP1 Post-Portfolio Eager-Cycle Profile") and
// leave the projection before it undefined; here it is a dense bf16 matrix W_router[E, H].
//   - The projection runs on the matrix cores (v_mfma_f32_16x16x32_bf16). Up to 32 tokens, a workgroup
//     owns 16 NB tokens (NB = 1 or 2 16-token blocks) x 64 experts and one slice of K; each of its four
//     waves computes 16 experts for the NB blocks and loads its operands straight into the MFMA lane
//     layout (lane: token / expert j16, K elements 8g .. 8g+7 of a 32-wide step), with no LDS: the
//     activations are a few rows and each wave streams its own expert rows. Above 32 tokens a
//     workgroup owns 64 tokens x 64 experts and stages both operands through LDS in whole lines.
//   - There are few tiles (4 at decode with 256 experts, 64 at T = 1024), so K is split into
//     up to 16 slices to give the GPU about 512 workgroups; each slice writes its partial logits
//     to the workspace.
//   - One wave per token then loads all its partial logits at once, sums them in slice order
//     (deterministic, no atomics), optionally writes the logits, and runs the same selection code as
//     the router kernel.
#include <type_traits>

#include "common.hpp"
#include "group_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

constexpr int kRouterTile = 64;      // experts per workgroup tile (16 per wave)
constexpr int kRouterMaxSplits = 16;  // K slices at most
constexpr int kRouterTargetBlocks = 512;  // about two workgroups per CU; more slices add partial-sum traffic
constexpr int kRouterFusedMaxPairs = 32 * kRouterMaxTopk;  // T <= 32 tokens in the one-launch router
constexpr int kRouterFusedThreads = 512;  // eight waves: four for the tile, all eight select

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// part[split][t][e] = sum over K-steps [split * steps_per_split, ...) of x[t][.] . w[e][.]. Wave w of
// the workgroup owns experts e0 + 16 w .. +16 and NB 16-token blocks of the tile (T <= 32 only; NB = 1
// at decode, where all four waves still stream their own expert rows). The operands of U steps are
// loaded before any of their MFMAs, so a wave has U * (NB + 1) loads in flight; steps past the slice
// re-read its last step and multiply by a zeroed weight operand, which leaves the accumulator
// unchanged (for finite activations). DEV_STORE: the partials are stored past the L2 (device scope),
// for a workgroup on another XCD to read within the same launch.
template <int NB, int U, bool DEV_STORE>
__device__ __forceinline__ void router_tile(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T,
                                            int H, int E, int tiles_t, int splits, int steps_per_split,
                                            float* __restrict__ part) {
  const int b = blockIdx.x;
  const int split = b % splits;
  const int tile = b / splits;
  const int tt = tile % tiles_t, te = tile / tiles_t;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int t0 = tt * (16 * NB);
  const int eb = te * kRouterTile + wave * 16;  // the wave's 16 experts
  if (eb >= E) return;
  const int steps = H >> 5;
  const int s0 = split * steps_per_split;
  const int s1 = min(s0 + steps_per_split, steps);

  // operand rows; rows past T or E repeat the last one (their results are not stored)
  const uint16_t* xa[NB];
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) xa[tb] = x + (size_t)min(t0 + tb * 16 + j16, T - 1) * H + g * 8;
  const uint16_t* wb = w + (size_t)min(eb + j16, E - 1) * H + g * 8;

  f32x4_t acc[NB];
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int st = s0; st < s1; st += U) {
    uint4 bw[U];
    bf16x8_t ax[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(st + u, s1 - 1) * 32;
      bw[u] = *reinterpret_cast<const uint4*>(wb + s);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) ax[u][tb] = ld_bf16x8(xa[tb] + s);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t keep = st + u < s1 ? 0xffffffffu : 0u;
      const uint4 m{bw[u].x & keep, bw[u].y & keep, bw[u].z & keep, bw[u].w & keep};
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, m);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[u][tb], bop, acc[tb], 0, 0, 0);
    }
  }

  // lane holds tokens t0 + 16 tb + 4g + i and expert eb + j16
  const int e = eb + j16;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + tb * 16 + 4 * g + i;
      if (t < T && e < E) {
        float* dst = part + ((size_t)split * T + t) * E + e;
        if constexpr (DEV_STORE)
          __hip_atomic_store(dst, acc[tb][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = acc[tb][i];
      }
    }
}

template <int NB, int U>
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int T, int H,
                                                          int E, int tiles_t, int splits,
                                                          int steps_per_split, float* __restrict__ part) {
  router_tile<NB, U, false>(x, w, T, H, E, tiles_t, splits, steps_per_split, part);
}

// T > 32: a workgroup owns 64 tokens x 64 experts and stages both operands through LDS, so every
// global load reads whole 128-byte lines and each operand element is fetched once per workgroup
// (loaded straight into the lane layout, 16 lanes read 64 bytes of each of 16 rows and the four
// waves would each re-read the tile's activations). A chunk is kChunkSteps K steps (64 bytes of every
// row per step); thread tid loads 16 bytes at column tid % kRowThreads of rows tid / kRowThreads +
// kRowsPerPass i of both operands, the next chunk's loads are in flight while the waves multiply the
// current one, and wave (wr, wc)
// computes tokens 32 wr .. +32 x experts 32 wc .. +32 (four MFMAs per step). Steps past the slice
// re-read its last step and are stored as zeros, so they add nothing.
constexpr int kChunkSteps = 4;
constexpr int kLdsRowBytes = kChunkSteps * 64 + 16;  // padded: rows 4 banks apart
constexpr int kRowThreads = kChunkSteps * 4;         // threads loading one row's chunk, 16 bytes each
constexpr int kRowsPerPass = 256 / kRowThreads;
constexpr int kStageRows = kRouterTile / kRowsPerPass;  // rows of each operand per thread

__global__ __launch_bounds__(256) void router_gemm_lds_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w, int T, int H,
                                                              int E, int tiles_t, int splits,
                                                              int steps_per_split, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kRouterTile * kLdsRowBytes];  // x rows, then w rows
  const int b = blockIdx.x;
  const int split = b % splits;
  const int tile = b / splits;
  const int tt = tile % tiles_t, te = tile / tiles_t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = tt * kRouterTile, e0 = te * kRouterTile;
  const int steps = H >> 5;
  const int s0 = split * steps_per_split;
  const int s1 = min(s0 + steps_per_split, steps);
  const int nchunks = (s1 - s0 + kChunkSteps - 1) / kChunkSteps;

  // staging: rows past T or E repeat the last one (their results are not stored)
  const int c16 = tid % kRowThreads, r0 = tid / kRowThreads, cstep = c16 >> 2;
  const uint16_t* xs[kStageRows];
  const uint16_t* wsrc[kStageRows];
#pragma unroll
  for (int i = 0; i < kStageRows; ++i) {
    xs[i] = x + (size_t)min(t0 + r0 + kRowsPerPass * i, T - 1) * H + (c16 & 3) * 8;
    wsrc[i] = w + (size_t)min(e0 + r0 + kRowsPerPass * i, E - 1) * H + (c16 & 3) * 8;
  }
  uint4 rx[kStageRows], rw[kStageRows];
  uint32_t keep = 0;
  auto load = [&](int st) {  // the chunk whose first step is st
    const int s = st + cstep;
    keep = s < s1 ? 0xffffffffu : 0u;
    const int off = min(s, s1 - 1) * 32;
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
      rx[i] = *reinterpret_cast<const uint4*>(xs[i] + off);
      rw[i] = *reinterpret_cast<const uint4*>(wsrc[i] + off);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
      const uint4 vx{rx[i].x & keep, rx[i].y & keep, rx[i].z & keep, rx[i].w & keep};
      const uint4 vw{rw[i].x & keep, rw[i].y & keep, rw[i].z & keep, rw[i].w & keep};
      *reinterpret_cast<uint4*>(lds + (r0 + kRowsPerPass * i) * kLdsRowBytes + c16 * 16) = vx;
      *reinterpret_cast<uint4*>(lds + (kRouterTile + r0 + kRowsPerPass * i) * kLdsRowBytes + c16 * 16) = vw;
    }
  };

  const int wr = wave >> 1, wc = wave & 1;
  const int j16 = lane & 15, g = lane >> 4;
  const uint8_t* la = lds + (wr * 32 + j16) * kLdsRowBytes + g * 16;
  const uint8_t* lb = lds + (kRouterTile + wc * 32 + j16) * kLdsRowBytes + g * 16;
  f32x4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(s0);
  for (int ch = 0; ch < nchunks; ++ch) {
    store();
    __syncthreads();
    if (ch + 1 < nchunks) load(s0 + (ch + 1) * kChunkSteps);
#pragma unroll
    for (int u = 0; u < kChunkSteps; ++u) {
      bf16x8_t av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = *reinterpret_cast<const bf16x8_t*>(la + a * 16 * kLdsRowBytes + u * 64);
#pragma unroll
      for (int c = 0; c < 2; ++c) bv[c] = *reinterpret_cast<const bf16x8_t*>(lb + c * 16 * kLdsRowBytes + u * 64);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], bv[c], acc[a][c], 0, 0, 0);
    }
    __syncthreads();
  }

  // lane holds tokens t0 + 32 wr + 16 a + 4g + i and expert e0 + 32 wc + 16 c + j16
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int e = e0 + wc * 32 + c * 16 + j16;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wr * 32 + a * 16 + 4 * g + i;
        if (t < T && e < E) part[((size_t)split * T + t) * E + e] = acc[a][c][i];
      }
  }
}

// One wave, token t: the logits as the in-order sum of the slices' partials, then the selection.
// DEV_LOAD: the partials are read past the L2 (device scope; written in the same launch).
template <int EPL, bool DEV_LOAD>
__device__ __forceinline__ void select_token(const float* __restrict__ part, int splits, int t, int T, int E,
                                             int k, int score_fn, int renorm, float* __restrict__ logits,
                                             int32_t* __restrict__ ids, float* __restrict__ weights,
                                             int32_t* ids_copy) {
  const int lane = threadIdx.x & 63;
  const size_t slice = (size_t)T * E;
  // every partial in flight at once (slices past the last re-read it: loads under a branch would be
  // waited for one by one), then summed in slice order; absent slices are skipped, not added as
  // zeros, so the sum's bits do not depend on the bound
  float pv[EPL][kRouterMaxSplits];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    const float* p = part + (size_t)t * E + e;
#pragma unroll
    for (int sp = 0; sp < kRouterMaxSplits; ++sp) {
      const float* q = p + min(sp, splits - 1) * slice;
      if constexpr (DEV_LOAD)
        pv[i][sp] = __hip_atomic_load(const_cast<float*>(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        pv[i][sp] = *q;
    }
  }
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float s = pv[i][0];
#pragma unroll
    for (int sp = 1; sp < kRouterMaxSplits; ++sp) s = sp < splits ? s + pv[i][sp] : s;
    if (e >= E) s = 0.0f;
    else if (logits) logits[(size_t)t * E + e] = s;
    v[i] = s;
  }
  route_dev::route_values<EPL>(v, t, E, k, score_fn, renorm, ids, weights, ids_copy);
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
  select_token<EPL, false>(part, splits, t, T, E, k, score_fn, renorm, logits, ids, weights, nullptr);
}

// The projection and the selection in one launch (T <= 32): every workgroup computes its tile and
// slice as router_gemm_kernel does, storing the partials past the L2, then adds one to a device-scope
// counter; the workgroup that finds the count complete is the last, and runs the selection of every
// token (a wave per token, the same code and order as router_select_kernel, so the results are
// bitwise those of the two launches), then, with GROUP, the token grouping of the chosen ids (the
// grouping kernel's device code), and resets the counter for the next call. The counter must be zero
// before the first call.
template <int NB, int U, int EPL, bool GROUP>
__global__ __launch_bounds__(kRouterFusedThreads) void router_fused_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                           int T, int H, int E, int tiles_t, int splits,
                                                           int steps_per_split, float* __restrict__ part,
                                                           unsigned int* __restrict__ counter, int k, int score_fn,
                                                           int renorm, float* __restrict__ logits,
                                                           int32_t* __restrict__ ids, float* __restrict__ weights,
                                                           RouterGroupOut grp) {
  __shared__ int last;
  __shared__ int32_t ids_lds[GROUP ? kRouterFusedMaxPairs : 1];
  __shared__ std::conditional_t<GROUP, group_dev::Shared, char> gsh;  // LDS of the grouping, if any
  // four waves compute the tile; the other four only join the selection in the last workgroup
  if (threadIdx.x < 256) router_tile<NB, U, true>(x, w, T, H, E, tiles_t, splits, steps_per_split, part);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partials are stored
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = wave; t < T; t += kRouterFusedThreads / 64)
    select_token<EPL, true>(part, splits, t, T, E, k, score_fn, renorm, logits, ids, weights,
                            GROUP ? ids_lds : nullptr);
  if constexpr (GROUP) {
    __syncthreads();
    const int P = T * k;
    if (P <= 64) {
      if (wave == 0)
        group_dev::group_pairs_one_wave(static_cast<const int32_t*>(ids_lds), P, E, grp.counts, grp.offsets,
                                        grp.sorted_pair, grp.pair_pos, grp.active, grp.n_active, gsh);
    } else {
      group_dev::group_pairs<1>(static_cast<const int32_t*>(ids_lds), P, E, grp.counts, grp.offsets,
                                grp.sorted_pair, grp.pair_pos, grp.active, grp.n_active, gsh);
    }
  }
}

}  // namespace

RouterPlan plan_router(int T, int H, int E) {
  RouterPlan rp;
  rp.nb = T <= 16 ? 1 : (T <= 32 ? 2 : 4);  // 4: the LDS-staged kernel
  rp.tiles_t = (T + 16 * rp.nb - 1) / (16 * rp.nb);
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
  return kRouterHeaderBytes + (size_t)rp.splits * T * E * sizeof(float);
}

bool router_fusable(int T) { return T <= 32; }

namespace {

template <bool GROUP>
hipError_t launch_router_fused(const RouterPlan& rp, const uint16_t* x, const uint16_t* w, int T, int H, int E,
                               int k, int score_fn, int renorm, void* workspace, float* logits, int32_t* ids,
                               float* weights, const RouterGroupOut& grp, hipStream_t stream) {
  unsigned int* counter = static_cast<unsigned int*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kRouterHeaderBytes);
#define MOE_RF(NB, EPL)                                                                                   \
  router_fused_kernel<NB, 8, EPL, GROUP><<<rp.blocks, kRouterFusedThreads, 0, stream>>>(x, w, T, H, E, rp.tiles_t, rp.splits, \
                                                                        rp.steps_per_split, part, counter, k,   \
                                                                        score_fn, renorm, logits, ids, weights, grp)
#define MOE_RF_E(NB)  \
  if (E <= 64)        \
    MOE_RF(NB, 1);    \
  else if (E <= 128)  \
    MOE_RF(NB, 2);    \
  else if (E <= 256)  \
    MOE_RF(NB, 4);    \
  else                \
    MOE_RF(NB, 8);
  if (rp.nb == 1) {
    MOE_RF_E(1)
  } else {
    MOE_RF_E(2)
  }
#undef MOE_RF_E
#undef MOE_RF
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_gemm_topk(const uint16_t* x, const uint16_t* w, int T, int H, int E, int k,
                                   int score_fn, int renorm, void* workspace, float* logits, int32_t* ids,
                                   float* weights, bool split_launch, hipStream_t stream) {
  const RouterPlan rp = plan_router(T, H, E);
  if (router_fusable(T) && !split_launch)
    return launch_router_fused<false>(rp, x, w, T, H, E, k, score_fn, renorm, workspace, logits, ids, weights,
                                      RouterGroupOut{}, stream);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kRouterHeaderBytes);
#define MOE_RGEMM(NB, U)                                                                                 \
  router_gemm_kernel<NB, U><<<rp.blocks, 256, 0, stream>>>(x, w, T, H, E, rp.tiles_t, rp.splits,         \
                                                           rp.steps_per_split, part)
  if (rp.nb == 1)
    MOE_RGEMM(1, 8);
  else if (rp.nb == 2)
    MOE_RGEMM(2, 8);
  else
    router_gemm_lds_kernel<<<rp.blocks, 256, 0, stream>>>(x, w, T, H, E, rp.tiles_t, rp.splits,
                                                          rp.steps_per_split, part);
#undef MOE_RGEMM
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

hipError_t launch_router_group(const uint16_t* x, const uint16_t* w, int T, int H, int E, int k, int score_fn,
                               int renorm, void* workspace, float* logits, int32_t* ids, float* weights,
                               const RouterGroupOut& grp, hipStream_t stream) {
  if (router_fusable(T))
    return launch_router_fused<true>(plan_router(T, H, E), x, w, T, H, E, k, score_fn, renorm, workspace, logits,
                                     ids, weights, grp, stream);
  const hipError_t e = launch_router_gemm_topk(x, w, T, H, E, k, score_fn, renorm, workspace, logits, ids,
                                               weights, true, stream);
  if (e != hipSuccess) return e;
  return launch_group_tokens(ids, T * k, E, grp.counts, grp.offsets, grp.sorted_pair, grp.pair_pos, grp.active,
                             grp.n_active, stream);
}

}  // namespace moe
