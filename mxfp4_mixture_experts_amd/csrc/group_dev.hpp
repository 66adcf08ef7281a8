// Token-to-expert grouping: expert histogram, exclusive prefix scan and a stable permutation of the
// P = T*k routed pairs by expert ("Direct M=2 route remap" row of the Post-Portfolio Device
// Attribution table, "MTP1 Post-Portfolio Eager-Cycle Profile").
//
// Device code shared by the grouping kernel and the fused router + grouping kernel.
// One workgroup of up to 16 waves. Each wave owns a contiguous range of whole 64-pair chunks. Within
// a chunk, lanes holding the same expert are found with ten ballots over the id bits; the lowest
// such lane updates the wave's own per-expert counter in LDS, so nothing is atomic and the result is
// deterministic. A per-expert scan over the waves (in wave order) plus a scan over the experts gives
// each pair's row: offsets[e] + (pairs of e in earlier waves) + (earlier chunks of this wave) + (rank
// among equal lanes of its chunk). Rows within an expert therefore follow ascending p. With the ids
// in global memory (kIdGroup > 1) both passes load those of kIdGroup chunks at once, so a wave waits
// for one memory round trip per group rather than per chunk; ids in LDS are read one chunk at a time.
#pragma once

#include "common.hpp"

namespace moe {
namespace group_dev {

constexpr int kMaxWaves = 16;
constexpr int kMaxExperts = 512;

// LDS of group_pairs.
struct Shared {
  int hist[kMaxWaves * kMaxExperts];  // per-wave counters, then running rows
  int total[kMaxExperts];
  int base[kMaxExperts];
};

// Group the P pairs of `ids` (global or LDS) with the whole workgroup (every thread calls it);
// kIdGroup chunks' ids are loaded together.
template <int kIdGroup, typename IdPtr>
__device__ __forceinline__ void group_pairs(IdPtr ids, int P, int E, int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ sorted_pair,
                                            int32_t* __restrict__ pair_pos,
                                            int32_t* __restrict__ active,
                                            int32_t* __restrict__ n_active, Shared& sh) {
  int* hist = sh.hist;
  int* total = sh.total;
  int* base = sh.base;
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  for (int i = threadIdx.x; i < nw * E; i += blockDim.x) hist[i] = 0;
  __syncthreads();

  const int chunks = (P + 63) >> 6;
  const int per_wave = (chunks + nw - 1) / nw;
  const int c_begin = w * per_wave;
  const int c_end = min(chunks, c_begin + per_wave);
  int* my_hist = hist + w * E;

  // ids of chunks c0 .. c0 + kIdGroup - 1 of this wave (0 past the wave's range or past P)
  auto load_ids = [&](int c0, int (&ev)[kIdGroup]) {
#pragma unroll
    for (int j = 0; j < kIdGroup; ++j) {
      const int p = ((c0 + j) << 6) + lane;
      ev[j] = (c0 + j < c_end && p < P) ? ids[p] : 0;
    }
  };

  // 1. per-wave histogram
  for (int c0 = c_begin; c0 < c_end; c0 += kIdGroup) {
    int ev[kIdGroup];
    load_ids(c0, ev);
#pragma unroll
    for (int j = 0; j < kIdGroup; ++j) {
      const int c = c0 + j;
      if (c >= c_end) break;  // uniform
      const int p = (c << 6) + lane;
      const bool valid = p < P;
      const uint64_t peers = match_key(ev[j], valid);
      if (valid && lane == __ffsll((unsigned long long)peers) - 1) my_hist[ev[j]] += __popcll(peers);
    }
  }
  __syncthreads();

  // 2. per expert: exclusive prefix over waves, and the expert's total
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int v = 0; v < nw; ++v) {
      const int c = hist[v * E + e];
      hist[v * E + e] = run;
      run += c;
    }
    total[e] = run;
  }
  __syncthreads();

  // 3. exclusive scan over experts, counts/offsets, compacted active list (wave 0)
  if (w == 0) {
    int carry = 0, acarry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? total[e] : 0;
      const int incl = wave_inclusive_scan(c, lane);
      if (e < E) {
        base[e] = carry + incl - c;
        counts[e] = c;
        offsets[e] = carry + incl - c;
      }
      carry += wave_last(incl);
      const bool act = e < E && c > 0;
      const uint64_t am = __ballot(act);
      if (act) active[acarry + __popcll(am & lanemask_lt(lane))] = e;
      acarry += __popcll(am);
    }
    if (lane == 0) {
      offsets[E] = carry;
      *n_active = acarry;
    }
    for (int i = acarry + lane; i < E; i += 64) active[i] = -1;
  }
  __syncthreads();

  // 4. stable placement
  for (int c0 = c_begin; c0 < c_end; c0 += kIdGroup) {
    int ev[kIdGroup];
    load_ids(c0, ev);
#pragma unroll
    for (int j = 0; j < kIdGroup; ++j) {
      const int c = c0 + j;
      if (c >= c_end) break;  // uniform
      const int p = (c << 6) + lane;
      const bool valid = p < P;
      const int e = ev[j];
      const uint64_t peers = match_key(e, valid);
      if (valid) {
        const int pos = base[e] + my_hist[e] + __popcll(peers & lanemask_lt(lane));
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      }
      // every lane of this wave has read my_hist[e] above before the leader advances it
      __builtin_amdgcn_wave_barrier();
      if (valid && lane == __ffsll((unsigned long long)peers) - 1) my_hist[e] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// The same grouping for at most 64 pairs, by one wave alone (lane p holds pair p): the other waves
// of the workgroup may have exited. Each expert's count is written to LDS by the lowest lane
// holding it, one wave-wide scan over the experts gives counts, offsets and the active list (and
// turns the LDS counts into base rows), and each pair's row is its expert's base plus the number of
// lower lanes holding the same expert — the definition above, so the outputs are the same.
// (cnt: E ints of LDS, per expert its count, then its base row)
template <typename IdPtr, typename OutPtr>
__device__ __forceinline__ void group_pairs_one_wave(IdPtr ids, int P, int E, OutPtr counts, OutPtr offsets,
                                                     OutPtr sorted_pair, OutPtr pair_pos, OutPtr active,
                                                     OutPtr n_active, int* cnt) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  const bool valid = lane < P;
  const int my_e = valid ? ids[lane] : 0;
  const uint64_t peers = match_key(my_e, valid);
  const int rank = __popcll(peers & lanemask_lt(lane));
  // LDS accesses of one wave complete in order: the zeroing above lands before these counts
  if (valid && rank == 0) cnt[my_e] = __popcll(peers);

  int carry = 0, acarry = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int c = e < E ? cnt[e] : 0;
    const int incl = wave_inclusive_scan(c, lane);
    if (e < E) {
      counts[e] = c;
      offsets[e] = carry + incl - c;
      cnt[e] = carry + incl - c;
    }
    carry += wave_last(incl);
    const bool act = e < E && c > 0;
    const uint64_t am = __ballot(act);
    if (act) active[acarry + __popcll(am & lanemask_lt(lane))] = e;
    acarry += __popcll(am);
  }
  if (lane == 0) {
    offsets[E] = carry;
    *n_active = acarry;
  }
  for (int i = acarry + lane; i < E; i += 64) active[i] = -1;
  if (valid) {
    const int pos = cnt[my_e] + rank;
    sorted_pair[pos] = lane;
    pair_pos[lane] = pos;
  }
}

// The same grouping over several workgroups, for many pairs (one workgroup places 64-pair chunks at
// roughly one per wave every microsecond, so 8192 pairs took 16 us alone). Workgroup g owns the
// chunks [g * cpw, (g + 1) * cpw). No device scratch and no communication between workgroups:
// each one counts every expert over all P ids and over the ids before its own chunks with LDS
// atomics (integer counts, so the order of the additions does not matter), which gives it every
// expert's offset and the number of its pairs that precede the workgroup. Its waves then count and
// place their own chunks exactly as group_pairs does, starting from those numbers, so every pair
// gets the same row: offsets[e] + (pairs of e at lower p). Workgroup 0 writes counts, offsets and
// the active list. kIdGroup ids per thread are loaded together.
struct SharedMulti {
  int hist[kMaxWaves * kMaxExperts];  // per-wave counts of the workgroup's chunks, then running rows
  int total[kMaxExperts];             // pairs of each expert over all P
  int before[kMaxExperts];            // pairs of each expert before the workgroup's first chunk
  int base[kMaxExperts];              // offsets
};

template <int kIdGroup>
__device__ __forceinline__ void group_pairs_multi(const int32_t* __restrict__ ids, int P, int E, int cpw,
                                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ sorted_pair,
                                                  int32_t* __restrict__ pair_pos, int32_t* __restrict__ active,
                                                  int32_t* __restrict__ n_active, SharedMulti& sh) {
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x;

  for (int i = threadIdx.x; i < nw * E; i += blockDim.x) sh.hist[i] = 0;
  for (int i = threadIdx.x; i < E; i += blockDim.x) sh.total[i] = 0, sh.before[i] = 0;
  __syncthreads();

  const int chunks = (P + 63) >> 6;
  const int wg_c0 = min(chunks, g * cpw);
  const int wg_c1 = min(chunks, wg_c0 + cpw);
  const int p_first = wg_c0 << 6;  // first pair of the workgroup

  // 1. every expert's count over all P, and over the pairs before the workgroup's chunks
  for (int p0 = 0; p0 < P; p0 += kIdGroup * (int)blockDim.x) {
    int ev[kIdGroup];
#pragma unroll
    for (int j = 0; j < kIdGroup; ++j) {
      const int p = p0 + j * (int)blockDim.x + (int)threadIdx.x;
      ev[j] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < kIdGroup; ++j) {
      const int p = p0 + j * (int)blockDim.x + (int)threadIdx.x;
      if (ev[j] >= 0) {
        atomicAdd(&sh.total[ev[j]], 1);
        if (p < p_first) atomicAdd(&sh.before[ev[j]], 1);
      }
    }
  }

  // the wave's chunks: a contiguous share of the workgroup's
  const int per_wave = (wg_c1 - wg_c0 + nw - 1) / nw;
  const int c_begin = min(wg_c1, wg_c0 + w * per_wave);
  const int c_end = min(wg_c1, c_begin + per_wave);
  int* my_hist = sh.hist + w * E;

  // 2. per-wave counts of its chunks (the lowest lane of each expert adds the expert's lanes)
  for (int c = c_begin; c < c_end; ++c) {
    const int p = (c << 6) + lane;
    const bool valid = p < P;
    const int e = valid ? ids[p] : 0;
    const uint64_t peers = match_key(e, valid);
    if (valid && lane == __ffsll((unsigned long long)peers) - 1) my_hist[e] += __popcll(peers);
  }
  __syncthreads();

  // 3. per expert: rows before each wave's chunks = before + counts of the earlier waves
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = sh.before[e];
    for (int v = 0; v < nw; ++v) {
      const int c = sh.hist[v * E + e];
      sh.hist[v * E + e] = run;
      run += c;
    }
  }

  // 4. exclusive scan over experts (wave 0); workgroup 0 also writes counts, offsets, the active list
  if (w == 0) {
    const bool writer = g == 0;
    int carry = 0, acarry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? sh.total[e] : 0;
      const int incl = wave_inclusive_scan(c, lane);
      if (e < E) {
        sh.base[e] = carry + incl - c;
        if (writer) {
          counts[e] = c;
          offsets[e] = carry + incl - c;
        }
      }
      carry += wave_last(incl);
      const bool act = e < E && c > 0;
      const uint64_t am = __ballot(act);
      if (writer && act) active[acarry + __popcll(am & lanemask_lt(lane))] = e;
      acarry += __popcll(am);
    }
    if (writer) {
      if (lane == 0) {
        offsets[E] = carry;
        *n_active = acarry;
      }
      for (int i = acarry + lane; i < E; i += 64) active[i] = -1;
    }
  }
  __syncthreads();

  // 5. stable placement of the wave's chunks
  for (int c = c_begin; c < c_end; ++c) {
    const int p = (c << 6) + lane;
    const bool valid = p < P;
    const int e = valid ? ids[p] : 0;
    const uint64_t peers = match_key(e, valid);
    if (valid) {
      const int pos = sh.base[e] + my_hist[e] + __popcll(peers & lanemask_lt(lane));
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
    // every lane of this wave has read my_hist[e] above before the leader advances it
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == __ffsll((unsigned long long)peers) - 1) my_hist[e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename IdPtr>
__device__ __forceinline__ void group_pairs_one_wave(IdPtr ids, int P, int E, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_pair,
                                                     int32_t* __restrict__ pair_pos,
                                                     int32_t* __restrict__ active,
                                                     int32_t* __restrict__ n_active, Shared& sh) {
  group_pairs_one_wave<IdPtr, int32_t*>(ids, P, E, counts, offsets, sorted_pair, pair_pos, active, n_active,
                                        sh.total);
}

}  // namespace group_dev
}  // namespace moe
