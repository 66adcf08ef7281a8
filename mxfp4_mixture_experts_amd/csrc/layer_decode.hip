// The whole routed MoE layer for decode (T <= 16 tokens) in one launch: router top-k, grouping,
// gate_up + SwiGLU, down and the weighted combine.
//
// The separate kernels of the layer lose latency at their edges: each launch waits for the one before
// it, starts with a chain of dependent loads (counts -> list -> weights) and ends with a tail in which
// some compute units idle ("Chunk 8.0", summary: persistent kernels as a lever at low concurrency;
// vllm.cpp PR #52: launch cost per kernel; "MTP1 Post-Portfolio Eager-Cycle Profile", Decision: a
// larger producer/reduction/consumer boundary). Inside one kernel on MI355X a dependency between
// workgroups is not free either: the eight XCDs' L2 caches are not coherent with each other, so data
// one workgroup hands to another must be written back from the producer's L2 (an agent-scope
// release, buffer_wbl2, which walks the XCD's L2: ~0.5 us each, serialised per XCD) and dropped from
// the consumer's (an agent-scope acquire, buffer_inv), or written and read past the L2 (device-scope
// accesses, measured at only ~150 GB/s device-wide). This kernel is therefore laid out to need one
// exchange and one barrier:
//   1. every workgroup routes all T tokens and groups their pairs itself, in LDS (the same device
//      code as the separate router and grouping kernels, so ids and weights are bitwise the same);
//   2. the K dimension of the down projection (= the rows of gate/up, I) of every active expert is
//      cut into 32-element MX blocks; the N = n_active * I/32 (expert, block) units are split into
//      R = min(G, N) contiguous ranges, none empty, one per workgroup. A workgroup computes the gate/up
//      rows of its blocks for all of the expert's tokens (h stays in its LDS, in fp32), then the down
//      projection restricted to those K blocks, for all H outputs: a partial y per (range, expert,
//      token), stored to the workspace. No workgroup waits for another until here;
//   3. one agent-scope release per workgroup, then a grid barrier (a device-scope counter that only
//      grows: G per call), then one acquire per workgroup;
//   4. each workgroup combines a slice of the T x H outputs: a wave per four outputs sums, over the
//      token's k pairs and each pair's ranges, routing weight times partial, spread over its lanes
//      and added in a fixed tree, then one rounding to bfloat16. Every sum runs in a fixed order:
//      results are deterministic.
// Consecutive ranges run on one XCD (workgroup b runs on XCD b % 8, and holds range (b % 8) R/8 + b/8),
// so adjacent K blocks of one expert, which share the cache lines of the down rows and their scales,
// share that XCD's L2.
// The precision differs from the multi-launch path only in where h is rounded: h stays fp32 until the
// down projection turns each 32-value block into scaled fp16 (the streaming down kernel's format, built
// here from the fp32 h rather than from its bf16 hi/lo pair), and y is summed over K ranges in fp32.
#include <atomic>

#include "common.hpp"
#include "group_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"
#include "stream_dev.hpp"

namespace moe {

namespace {

using namespace stream_dev;

constexpr int kLMaxSubs = 34;  // sub-ranges (one per expert touched) of one workgroup's range (<= 32 K blocks + 1)
constexpr int kLRing = 2;      // items in flight per wave
constexpr int kDnSlots = 4;    // down rows per lane group and item
constexpr int kCombineBatch = 4;   // partial rows per lane whose loads the combine keeps in flight

struct LayerLds {
  group_dev::Shared g;
  int32_t ids[kLayerMaxPairs];
  float wts[kLayerMaxPairs];
  int32_t counts[kLayerMaxExperts];
  int32_t offsets[kLayerMaxExperts + 1];
  int32_t sorted_pair[kLayerMaxPairs];
  int32_t pair_pos[kLayerMaxPairs];
  int32_t active[kLayerMaxExperts];
  int32_t slot_of[kLayerMaxExperts];
  int32_t range_base[kLayerMaxRanges + 1];  // first partial-y row of each range
  uint32_t rbeg[kLayerMaxRanges + 1];       // first unit of each range (rbeg[R] = N)
  int32_t rrow0[kLayerMaxRanges];           // range_base[s] - offsets[first expert of range s]
  int32_t pe_slo[kLayerMaxPairs];           // per pair: first range of its expert
  int32_t pe_cnt[kLayerMaxPairs];           // ... number of ranges of its expert
  int32_t pe_pre[kLayerMaxPairs];           // ... ranges of the token's earlier pairs
  int32_t pe_row[kLayerMaxPairs];           // ... offsets[expert] + its row within the expert
  int32_t n_active;
  int32_t counter;
  int32_t n_sub;
  int32_t lpr_d;  // down: lanes per row, a power of two >= the widest sub-range (in K blocks)
  int32_t sub_a[kLMaxSubs];     // active slot of the sub-range's expert
  int32_t sub_k0[kLMaxSubs];    // first K block (of 32) within the expert
  int32_t sub_nb[kLMaxSubs];    // K blocks
  int32_t sub_h[kLMaxSubs];     // first float of its h in the dynamic LDS
  int32_t sub_y[kLMaxSubs];     // its first partial-y row
  int32_t sub_gu[kLMaxSubs + 1];  // prefix of gate_up items
  int32_t sub_dn[kLMaxSubs + 1];  // prefix of down items
};

struct LayerArgs {
  const float* logits;
  const uint16_t* x;
  const uint8_t* w13_q;
  const uint8_t* w13_s;
  const uint8_t* w2_q;
  const uint8_t* w2_s;
  int T, H, I, E, k, score_fn, renorm;
  float clamp;
  int lpr;                     // gate_up lanes per row (choose_row_split(H))
  int32_t* ids_out;            // nullable
  float* w_out;                // nullable
  float* y_part;               // [rows, H] partial down outputs
  unsigned long long* arrive;  // grid barrier counter (zero before the first call, G added per call)
  unsigned int* status;        // incremented when a barrier wait gives up
  uint16_t* out;
};

// Range of workgroup b among R <= G ranges, or -1: consecutive ranges on one XCD (workgroup b runs on
// XCD b % 8), R/8 of them on each, so every XCD streams an equal share.
__device__ __forceinline__ int range_of_block(int b, int G, int R) {
  if (G & 7) return b < R ? b : -1;
  const int x = b & 7, i = b >> 3;
  const int s = x * R / 8 + i;
  return s < (x + 1) * R / 8 ? s : -1;
}

// Unit ranges: range s holds units [floor(s N / G), floor((s + 1) N / G)). N <= 512 * 512 and
// G <= 1024 keep every product below 2^32.
__device__ __forceinline__ uint32_t range_begin(uint32_t s, uint32_t N, uint32_t G) { return s * N / G; }

// The range holding unit u: the largest s with floor(s N / G) <= u.
__device__ __forceinline__ uint32_t range_of_unit(uint32_t u, uint32_t N, uint32_t G) {
  return ((u + 1) * G - 1) / N;
}

// Sum over the 64 lanes in a fixed order (DPP tree), the total in lane 63.
__device__ __forceinline__ float wave_sum_fixed(float v) { return segment_sum(v, 64); }

// One 32-value fp32 block of h, in place in LDS, turned into 16 packed fp16 pairs scaled by a power
// of two that puts the block's largest magnitude in [2^14, 2^15) (the streaming down kernel's
// activation format), followed by the inverse scale: 17 dwords at the start of the block.
__device__ __forceinline__ void h_block_to_f16(float* blk) {
  float v[32];
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = blk[i];
    mx = max(mx, __builtin_bit_cast(uint32_t, v[i]) & 0x7F800000u);
  }
  const int eb = (int)(mx >> 23);
  const int f = min(max(268 - eb, 1), 253);  // scale 2^(f - 127)
  const float sc = __builtin_bit_cast(float, (uint32_t)f << 23);
  uint32_t* o = reinterpret_cast<uint32_t*>(blk);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    o[i] = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)(v[2 * i] * sc), (_Float16)(v[2 * i + 1] * sc)});
  blk[16] = __builtin_bit_cast(float, (uint32_t)(254 - f) << 23);
}

template <int BPL, int MT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void layer_decode_kernel(LayerArgs a) {
  __shared__ LayerLds L;
  extern __shared__ __attribute__((aligned(16))) float h_lds[];
  const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k;
  const int P = T * k;
  const int G = gridDim.x;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);

  // ---- 1. route + group, in LDS (every workgroup) -------------------------------------------------
  for (int t = w; t < T; t += NW)
    route_dev::route_token<8>(a.logits, t, E, k, a.score_fn, a.renorm, L.ids, L.wts, nullptr);
  __syncthreads();
  if (P <= 64) {
    if (w == 0)
      group_dev::group_pairs_one_wave(static_cast<const int32_t*>(L.ids), P, E, L.counts, L.offsets, L.sorted_pair,
                                      L.pair_pos, L.active, &L.n_active, L.g);
  } else {
    group_dev::group_pairs<1>(static_cast<const int32_t*>(L.ids), P, E, L.counts, L.offsets, L.sorted_pair,
                              L.pair_pos, L.active, &L.n_active, L.g);
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) L.slot_of[e] = -1;
  if (threadIdx.x == 0) L.counter = 0;
  __syncthreads();
  const int n_active = L.n_active;
  for (int i = threadIdx.x; i < n_active; i += blockDim.x) L.slot_of[L.active[i]] = i;
  if (blockIdx.x == 0) {
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
      if (a.ids_out) a.ids_out[p] = L.ids[p];
      if (a.w_out) a.w_out[p] = L.wts[p];
    }
  }

  // R = min(G, N) ranges over the N = n_active * nb units (expert slot, K block): none empty
  const uint32_t nb = (uint32_t)I >> 5;
  const uint32_t N = (uint32_t)n_active * nb;
  const int R = (int)min((uint32_t)G, N);
  for (int r = threadIdx.x; r <= R; r += blockDim.x) L.rbeg[r] = range_begin((uint32_t)r, N, (uint32_t)R);
  __syncthreads();
  // rows of partial y per range: the tokens of every expert it touches; exclusive scan by wave 0
  if (w == 0) {
    int carry = 0;
    for (int s0 = 0; s0 < R; s0 += 64) {
      const int s = s0 + lane;
      int rows = 0, first_off = 0;
      if (s < R) {
        const uint32_t u0 = L.rbeg[s], u1 = L.rbeg[s + 1];
        const int e0 = L.active[u0 / nb], e1 = L.active[(u1 - 1) / nb];
        first_off = L.offsets[e0];
        rows = L.offsets[e1] + L.counts[e1] - first_off;
      }
      const int incl = wave_inclusive_scan(rows, lane);
      if (s < R) {
        L.range_base[s] = carry + incl - rows;
        L.rrow0[s] = carry + incl - rows - first_off;
      }
      carry += wave_last(incl);
    }
    if (lane == 0) L.range_base[R] = carry;
  }
  // per pair: its expert's ranges (contiguous) and its row within the expert
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = L.ids[p];
    const uint32_t u = (uint32_t)L.slot_of[e] * nb;
    const int slo = (int)range_of_unit(u, N, (uint32_t)R);
    L.pe_slo[p] = slo;
    L.pe_cnt[p] = (int)range_of_unit(u + nb - 1, N, (uint32_t)R) - slo + 1;
    L.pe_row[p] = L.pair_pos[p];  // offsets[e] + (its row within expert e)
  }
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int t0 = p - p % k;
    int pre = 0;
    for (int q = t0; q < p; ++q) pre += L.pe_cnt[q];
    L.pe_pre[p] = pre;
  }
  // this workgroup's sub-ranges (thread 0)
  const int my_s = range_of_block(blockIdx.x, G, R);
  const uint32_t my_u0 = my_s >= 0 ? L.rbeg[my_s] : 0, my_u1 = my_s >= 0 ? L.rbeg[my_s + 1] : 0;
  const int rpw = 64 / a.lpr;
  const int gu_tile = (BPL >= 2 ? 1 : 2) * rpw;  // gate rows per item (one wave's share)
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0, hoff = 0, gu = 0, maxnb = 1;
    const int a0 = my_u1 > my_u0 ? (int)(my_u0 / nb) : 0;
    const int base_row0 = my_s >= 0 ? L.range_base[my_s] - L.offsets[L.active[a0]] : 0;
    for (uint32_t u = my_u0; u < my_u1 && n < kLMaxSubs;) {
      const uint32_t as = u / nb;
      const uint32_t u_end = min(my_u1, (as + 1) * nb);
      const int e = L.active[as];
      L.sub_a[n] = (int)as;
      L.sub_k0[n] = (int)(u - as * nb);
      L.sub_nb[n] = (int)(u_end - u);
      L.sub_h[n] = hoff;
      L.sub_y[n] = base_row0 + L.offsets[e];
      L.sub_gu[n] = gu;
      hoff += L.counts[e] * 32 * L.sub_nb[n];
      gu += (32 * L.sub_nb[n] + gu_tile - 1) / gu_tile;
      maxnb = max(maxnb, L.sub_nb[n]);
      ++n;
      u = u_end;
    }
    L.sub_gu[n] = gu;
    // down: lpr_d lanes per row (a power of two >= the widest sub-range), kDnSlots rows per lane group
    int lpr_d = 1;
    while (lpr_d < maxnb) lpr_d <<= 1;
    const int dn_tile = kDnSlots * (64 / lpr_d);
    int dn = 0;
    for (int j = 0; j < n; ++j) {
      L.sub_dn[j] = dn;
      dn += (H + dn_tile - 1) / dn_tile;
    }
    L.sub_dn[n] = dn;
    L.n_sub = n;
    L.lpr_d = lpr_d;
  }
  __syncthreads();
  const int n_sub = L.n_sub;
  const int lpr_d = L.lpr_d;

  // ---- 2a. gate_up of the range's rows, h to LDS (fp32) --------------------------------------------
  if (n_sub > 0) {
    const int lpr = a.lpr, lg = ilog2(lpr);
    const int q = lane & (lpr - 1), sub = lane >> lg;
    constexpr int S = BPL >= 2 ? 1 : 2;
    const int NB = H >> 5;
    const uint32_t qrow = (uint32_t)(H >> 1), srow = (uint32_t)NB;
    const size_t qexp = (size_t)2 * I * qrow, sexp = (size_t)2 * I * srow;
    const uint32_t up_q = (uint32_t)I * qrow, up_s = (uint32_t)I * srow;
    const bool k_exact = (NB % lpr) == 0;
    const int n_items = L.sub_gu[n_sub];

    uint4 wv[kLRing][S][2][BPL];
    uint32_t sc[kLRing][S][2][BPL];
    int ring_item[kLRing];

    auto sub_of = [&](int it) {
      int j = 0;
      while (j + 1 < n_sub && L.sub_gu[j + 1] <= it) ++j;
      return uniform(j);
    };
    auto take = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(&L.counter, 1);
      return uniform(__shfl(v, 0, 64));
    };
    auto prefetch = [&](int d) {
      ring_item[d] = take();
      const int it = min(ring_item[d], n_items - 1);
      const int j = sub_of(it);
      const int tile = it - L.sub_gu[j];
      const int e = uniform(L.active[L.sub_a[j]]);
      const uint8_t* qb = a.w13_q + (size_t)e * qexp;
      const uint8_t* sb = a.w13_s + (size_t)e * sexp;
      const int r0 = 32 * L.sub_k0[j], r1 = r0 + 32 * L.sub_nb[j];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint32_t rr = (uint32_t)min(r0 + tile * gu_tile + s * rpw + sub, r1 - 1);
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
          const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
          const uint32_t oq = rr * qrow + kb * 16, os = rr * srow + kb;
          wv[d][s][0][b] = ld16(qb, oq);
          sc[d][s][0][b] = ld8(sb, os);
          wv[d][s][1][b] = ld16(qb, oq + up_q);
          sc[d][s][1][b] = ld8(sb, os + up_s);
        }
      }
    };

    int cur_j = -1, cur_M = 0, cur_row0 = 0, cur_m0 = -1;
    uint4 xb[MT][BPL][4];
    auto consume = [&](int d) {
      const int it = ring_item[d];
      const int j = sub_of(it);
      const int tile = it - L.sub_gu[j];
      if (j != cur_j) {
        cur_j = j;
        const int e = uniform(L.active[L.sub_a[j]]);
        cur_M = uniform(L.counts[e]);
        cur_row0 = uniform(L.offsets[e]);
        cur_m0 = -1;
      }
      const int r0 = 32 * L.sub_k0[j], r1 = r0 + 32 * L.sub_nb[j];
      const int ncols = 32 * L.sub_nb[j];
      float* hj = h_lds + L.sub_h[j];
      const int n0 = r0 + tile * gu_tile;
      for (int m0 = 0; m0 < cur_M; m0 += MT) {
        const int mc = min(MT, cur_M - m0);
        if (m0 != cur_m0) {
          cur_m0 = m0;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int t = uniform(L.sorted_pair[cur_row0 + m0 + min(m, mc - 1)]) / k;
            const uint8_t* xbase = reinterpret_cast<const uint8_t*>(a.x + (size_t)t * H);
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
              const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
#pragma unroll
              for (int i = 0; i < 4; ++i) xb[m][b][i] = ld16(xbase, kb * 64 + i * 16);
            }
          }
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int b = 0; b < BPL; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i) opaque(xb[m][b][i]);
        }
        float acc[S][2][MT];
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int gu = 0; gu < 2; ++gu)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[s][gu][m] = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int n = n0 + s * rpw + sub;
#pragma unroll
          for (int gu = 0; gu < 2; ++gu) {
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
              float scale = e8m0_to_float(sc[d][s][gu][b]);
              if (!(k_exact && n < r1) && !(n < r1 && q + lpr * b < NB)) scale = 0.0f;
              if (MT == 1 || mc == MT) {
                uint4 xs[MT][4];
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                  for (int i = 0; i < 4; ++i) xs[m][i] = xb[m][b][i];
                dot_block_bf16<MT>(wv[d][s][gu][b], scale, xs, acc[s][gu]);
              } else {
                uint4 xs[1][4];
                float a1[1] = {acc[s][gu][0]};
#pragma unroll
                for (int i = 0; i < 4; ++i) xs[0][i] = xb[0][b][i];
                dot_block_bf16<1>(wv[d][s][gu][b], scale, xs, a1);
                acc[s][gu][0] = a1[0];
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int n = n0 + s * rpw + sub;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m >= mc) break;
            float g = segment_sum(acc[s][0][m], lpr);
            float u = segment_sum(acc[s][1][m], lpr);
            if (q == lpr - 1 && n < r1) {
              if (a.clamp > 0.0f) {
                g = clampf(g, a.clamp);
                u = clampf(u, a.clamp);
              }
              hj[(m0 + m) * ncols + (n - r0)] = silu_mul(g, u);
            }
          }
        }
      }
    };

#pragma unroll
    for (int d = 0; d < kLRing; ++d) prefetch(d);
    // the ring walk leaves by a jump (with a flag tested again at the top, the compiler's wait before
    // consuming an entry also covered the other entry's loads, draining the ring at every item)
    for (;;) {
#pragma unroll
      for (int d = 0; d < kLRing; ++d) {
        if (ring_item[d] >= n_items) goto gate_up_drained;
        consume(d);
        prefetch(d);
      }
    }
  gate_up_drained:;
  }
  __syncthreads();

  // ---- 2b. h blocks to scaled fp16, in place ---------------------------------------------------
  if (n_sub > 0) {
    for (int j = 0; j < n_sub; ++j) {
      const int M = L.counts[L.active[L.sub_a[j]]];
      const int nbj = L.sub_nb[j];
      for (int i = threadIdx.x; i < M * nbj; i += blockDim.x) h_block_to_f16(h_lds + L.sub_h[j] + 32 * i);
    }
    if (threadIdx.x == 0) L.counter = 0;
  }
  __syncthreads();

  // ---- 2c. down over the range's K blocks: partial y rows to the workspace --------------------------
  if (n_sub > 0) {
    const int lg = ilog2(lpr_d);
    const int q = lane & (lpr_d - 1), sub = lane >> lg;
    const int rpw_d = 64 >> lg;
    const int dn_tile = kDnSlots * rpw_d;
    const uint32_t qrow = (uint32_t)(I >> 1), srow = (uint32_t)nb;
    const size_t qexp = (size_t)H * qrow, sexp = (size_t)H * srow;
    const int n_items = L.sub_dn[n_sub];

    uint4 wv[kLRing][kDnSlots];
    uint32_t sc[kLRing][kDnSlots];
    int ring_item[kLRing];
    auto sub_of = [&](int it) {
      int j = 0;
      while (j + 1 < n_sub && L.sub_dn[j + 1] <= it) ++j;
      return uniform(j);
    };
    auto take = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(&L.counter, 1);
      return uniform(__shfl(v, 0, 64));
    };
    auto prefetch = [&](int d) {
      ring_item[d] = take();
      const int it = min(ring_item[d], n_items - 1);
      const int j = sub_of(it);
      const int tile = it - L.sub_dn[j];
      const int e = uniform(L.active[L.sub_a[j]]);
      const uint8_t* qb = a.w2_q + (size_t)e * qexp;
      const uint8_t* sb = a.w2_s + (size_t)e * sexp;
      const uint32_t kb = (uint32_t)(L.sub_k0[j] + min(q, L.sub_nb[j] - 1));
#pragma unroll
      for (int s = 0; s < kDnSlots; ++s) {
        const uint32_t rr = (uint32_t)min(tile * dn_tile + s * rpw_d + sub, H - 1);
        wv[d][s] = ld16(qb, rr * qrow + kb * 16);
        sc[d][s] = ld8(sb, rr * srow + kb);
      }
    };
    auto consume = [&](int d) {
      const int it = ring_item[d];
      const int j = sub_of(it);
      const int tile = it - L.sub_dn[j];
      const int M = uniform(L.counts[L.active[L.sub_a[j]]]);
      const int nbj = L.sub_nb[j];
      const bool qv = q < nbj;
      const float* hj = h_lds + L.sub_h[j] + 32 * min(q, nbj - 1);  // this lane's block, token 0
      const int yrow = L.sub_y[j];
      const int n0 = tile * dn_tile;
      for (int m0 = 0; m0 < M; m0 += MT) {
        const int mc = min(MT, M - m0);
        uint32_t hh[MT][16];
        float hinv[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float* hb = hj + (size_t)(m0 + min(m, mc - 1)) * 32 * nbj;
          const uint4* h4 = reinterpret_cast<const uint4*>(hb);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = h4[i];
            hh[m][4 * i] = v.x, hh[m][4 * i + 1] = v.y, hh[m][4 * i + 2] = v.z, hh[m][4 * i + 3] = v.w;
          }
          hinv[m] = hb[16];
        }
        float acc[kDnSlots][MT];
#pragma unroll
        for (int s = 0; s < kDnSlots; ++s)
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[s][m] = 0.0f;
#pragma unroll
        for (int s = 0; s < kDnSlots; ++s) {
          const int n = n0 + s * rpw_d + sub;
          float scale = e8m0_to_float(sc[d][s]);
          if (!(qv && n < H)) scale = 0.0f;
          float bs[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) bs[m] = scale * hinv[m];
          if (MT == 1 || mc == MT) {
            dot_block_f16s<MT>(wv[d][s], bs, hh, acc[s]);
          } else {
            uint32_t hs[1][16];
            float b1[1] = {bs[0]}, a1[1] = {acc[s][0]};
#pragma unroll
            for (int i = 0; i < 16; ++i) hs[0][i] = hh[0][i];
            dot_block_f16s<1>(wv[d][s], b1, hs, a1);
            acc[s][0] = a1[0];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < kDnSlots; ++s) {
          const int n = n0 + s * rpw_d + sub;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m >= mc) break;
            const float v = segment_sum(acc[s][m], lpr_d);
            if (q == lpr_d - 1 && n < H) a.y_part[(size_t)(yrow + m0 + m) * H + n] = v;
          }
        }
      }
    };

#pragma unroll
    for (int d = 0; d < kLRing; ++d) prefetch(d);
    // (the ring walk leaves by a jump, as above)
    for (;;) {
#pragma unroll
      for (int d = 0; d < kLRing; ++d) {
        if (ring_item[d] >= n_items) goto down_drained;
        consume(d);
        prefetch(d);
      }
    }
  down_drained:;
  }

  // ---- 3. grid barrier: this workgroup's partial rows are complete at the device level -----------
  // The partial rows went to this XCD's L2 with ordinary stores; one agent-scope release per
  // workgroup writes them back (device-scope stores of every row measured ~150 GB/s device-wide).
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are in L2
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned long long old =
        __hip_atomic_fetch_add(a.arrive, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long target = (old / (unsigned long long)G + 1ull) * (unsigned long long)G;
    int spins = 0;
    while (__hip_atomic_load(a.arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(16);  // ~0.5 us between polls: many pollers of one word slow its atomics
      if (++spins > (1 << 20)) {  // ~1 s: the grid was not resident; give up rather than hang
        atomicAdd(a.status, 1u);
        break;
      }
    }
  }
  // drop this XCD's L2 copies of earlier calls' partial rows before reading them
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();

  // ---- 4. combine a slice of the T x H outputs -----------------------------------------------------
  // One wave per quad of four consecutive outputs of one token. The quad's partial rows are the
  // entries (pair j, range s) in order; lane l takes entries l, l + 64, ..., loads them all (16 bytes
  // each, device scope) before summing, and adds topk_w[j] * row to its four accumulators in entry
  // order; the lanes' sums are then added in a fixed tree (DPP), so the result is deterministic.
  const int quads = T * (H >> 2);
  const int q0 = (int)((uint32_t)quads * blockIdx.x / (uint32_t)G);
  const int q1 = (int)((uint32_t)quads * (blockIdx.x + 1) / (uint32_t)G);
  for (int qd = q0 + w; qd < q1; qd += NW) {
    const int t = qd / (H >> 2), n = (qd - t * (H >> 2)) * 4;
    const int p0 = t * k;
    const int total = L.pe_pre[p0 + k - 1] + L.pe_cnt[p0 + k - 1];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = 0;
    for (int i0 = 0; i0 < total; i0 += 64 * kCombineBatch) {
      float4 y[kCombineBatch];
      float wy[kCombineBatch];
#pragma unroll
      for (int b = 0; b < kCombineBatch; ++b) {
        const int i = i0 + b * 64 + lane;
        wy[b] = 0.0f;
        y[b] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < total) {
          while (i >= L.pe_pre[p0 + j] + L.pe_cnt[p0 + j]) ++j;  // entries ascend: j only grows
          const int p = p0 + j;
          const int sr = L.pe_slo[p] + (i - L.pe_pre[p]);
          const int row = L.rrow0[sr] + L.pe_row[p];
          y[b] = *reinterpret_cast<const float4*>(a.y_part + (size_t)row * H + n);
          wy[b] = L.wts[p];
        }
      }
#pragma unroll
      for (int b = 0; b < kCombineBatch; ++b) {
        acc.x = fmaf(wy[b], y[b].x, acc.x), acc.y = fmaf(wy[b], y[b].y, acc.y);
        acc.z = fmaf(wy[b], y[b].z, acc.z), acc.w = fmaf(wy[b], y[b].w, acc.w);
      }
    }
    acc.x = wave_sum_fixed(acc.x), acc.y = wave_sum_fixed(acc.y);
    acc.z = wave_sum_fixed(acc.z), acc.w = wave_sum_fixed(acc.w);
    if (lane == 63) {
      uint2 o;
      o.x = pack_bf16x2(acc.x, acc.y);
      o.y = pack_bf16x2(acc.z, acc.w);
      *reinterpret_cast<uint2*>(a.out + (size_t)t * H + n) = o;
    }
  }
}

constexpr int layer_waves(int bpl, int mt) {
  return bpl == 1 ? 4 : bpl == 2 ? (mt == 1 ? 4 : 3) : bpl == 3 ? 3 : bpl <= 5 ? 2 : 1;
}

}  // namespace

size_t layer_workspace_bytes(int T, int H, int I, int E, int k, int num_cus) {
  const long P = (long)T * k;
  const long rows = (long)T * num_cus + 2 * P;
  return kLayerSyncBytes + (size_t)rows * H * sizeof(float);
}

// Largest LDS h of one workgroup: its range spans at most ceil(min(E, P) * I/32 / G) K blocks, each
// holding 32 fp32 values per token of its expert (at most T tokens each).
size_t layer_h_lds_bytes(int T, int I, int E, int k, int num_cus) {
  const long P = (long)T * k;
  const long nact = P < E ? P : E;
  const long blocks = (nact * (I / 32) + num_cus - 1) / num_cus;
  return (size_t)(blocks + 1) * 32 * T * sizeof(float);
}

bool layer_supported(int T, int H, int I, int E, int k, int num_cus) {
  if (T < 1 || T > kLayerMaxTokens || (long)T * k > kLayerMaxPairs || E > kLayerMaxExperts) return false;
  if (num_cus < 1 || num_cus > kLayerMaxRanges) return false;
  const long P = (long)T * k;
  const long nact = P < E ? P : E;
  const long blocks = (nact * (I / 32) + num_cus - 1) / num_cus;
  if (blocks > 32) return false;  // sub-range table (one per expert touched) and lanes per down row
  return layer_h_lds_bytes(T, I, E, k, num_cus) <= kLayerMaxHLds;
}

hipError_t launch_layer_decode(const float* logits, const uint16_t* x, int T, int H, int I, int E, int k,
                               int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                               const uint8_t* w2_q, const uint8_t* w2_s, float clamp, int32_t* ids_out,
                               float* w_out, uint16_t* out, void* workspace, int num_cus, hipStream_t stream) {
  LayerArgs a;
  a.logits = logits;
  a.x = x;
  a.w13_q = w13_q;
  a.w13_s = w13_s;
  a.w2_q = w2_q;
  a.w2_s = w2_s;
  a.T = T, a.H = H, a.I = I, a.E = E, a.k = k, a.score_fn = score_fn, a.renorm = renorm;
  a.clamp = clamp;
  const RowSplit rs = choose_row_split(H);
  a.lpr = rs.lpr;
  a.ids_out = ids_out;
  a.w_out = w_out;
  char* ws = static_cast<char*>(workspace);
  a.arrive = reinterpret_cast<unsigned long long*>(ws);
  a.status = reinterpret_cast<unsigned int*>(ws + 8);
  a.y_part = reinterpret_cast<float*>(ws + kLayerSyncBytes);
  a.out = out;
  const size_t lds = layer_h_lds_bytes(T, I, E, k, num_cus);
  const int mt = (T >= 2 && rs.bpl <= 2) ? 2 : 1;
#define MOE_LAYER(BPL, MT)                                                                            \
  {                                                                                                   \
    auto kern = layer_decode_kernel<BPL, MT, 4 * layer_waves(BPL, MT)>;                               \
    static std::atomic<bool> attr{false};                                                             \
    if (!attr.load()) {                                                                               \
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, \
                              (int)kLayerMaxHLds) != hipSuccess)                                      \
        return hipErrorInvalidValue;                                                                  \
      attr.store(true);                                                                               \
    }                                                                                                 \
    kern<<<num_cus, 256 * layer_waves(BPL, MT), lds, stream>>>(a);                                   \
  }
  switch (rs.bpl) {
    case 1: if (mt == 2) MOE_LAYER(1, 2) else MOE_LAYER(1, 1) break;
    case 2: if (mt == 2) MOE_LAYER(2, 2) else MOE_LAYER(2, 1) break;
    case 3: MOE_LAYER(3, 1) break;
    case 4: MOE_LAYER(4, 1) break;
    case 5: MOE_LAYER(5, 1) break;
    case 6: MOE_LAYER(6, 1) break;
    case 7: MOE_LAYER(7, 1) break;
    case 8: MOE_LAYER(8, 1) break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_LAYER
  return hipGetLastError();
}

}  // namespace moe
