// Weight-streaming MXFP4 expert GEMMs for experts with few routed rows (decode).
//
// At small per-expert M the expert GEMMs are bound by HBM bandwidth ("Chunk 8.0": the small
// per-expert GEMMs are memory-bandwidth-bound; "MTP1 Post-Portfolio Eager-Cycle Profile": the compact
// routed MXFP4 GEMM is the largest open kernel family at M=2). Each weight byte is used by at most a
// handful of rows, so these kernels are organised around streaming the expert weights once, at full
// width, with loads always in flight:
//   - each lane loads whole 32-element MX blocks: 16 bytes of E2M1 codes (one 128-bit load; a wave
//     load covers up to 1 KB of consecutive bytes of a row) plus the block's E8M0 scale byte;
//   - a row of K elements is split over `lpr` lanes (in-wave split-K), each owning fixed blocks, so
//     the lane's slice of the activations stays in registers for every row of an expert;
//   - the codes are decoded in registers with the gfx950 FP4 conversion (two codes per instruction)
//     and consumed by dot2 instructions with fp32 accumulation: bf16 dot2 against x (gate/up, codes
//     decoded with their scale; bf16 products are exact in fp32), fp16 dot2 against h (down, codes
//     decoded unscaled, the block's scale applied to the block's sum). h is kept in memory as two
//     bf16 planes, hi = bf16(h) and lo = bf16(h - hi); each lane rebuilds its 32-value h block as
//     hi + lo and turns it into fp16 with a power-of-two scale that puts the block's largest
//     magnitude in [2^14, 2^15), so no value overflows and each keeps fp16's 11-bit precision
//     (relative to the block maximum);
//   - partial sums are reduced across the row's lanes with DPP adds, deterministically;
//   - gate row i and up row I+i are handled by the same lanes, so SwiGLU (with the optional clamp) is
//     applied in registers and only h is written (gate_up fusion as in vllm.cpp PR #52; clamp-SwiGLU
//     epilogue as the routed clamp-SwiGLU row of the Post-Portfolio Device Attribution table).
// Scheduling: the work is a list of items (expert, tile of rows), each one wave's share. The grid
// is persistent with one workgroup per CU, holding as many waves as the register budget allows;
// each workgroup owns an equal contiguous range of items and its waves take them one at a time
// from a counter in LDS. Each wave keeps the loads of its next items in flight while it decodes
// the current one.
#include <atomic>

#include "common.hpp"
#include "group_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"
#include "stream_dev.hpp"

namespace moe {

RowSplit choose_row_split(int K) {
  RowSplit s;
  s.nb = K / 32;
  int lpr = 64;
  while (lpr > 1 && (s.nb % lpr) != 0) lpr >>= 1;  // largest power of two dividing nb
  if ((s.nb + lpr - 1) / lpr > 8) {
    lpr = 1;  // too many blocks per lane: smallest power of two giving at most 8, ragged tail
    while (lpr < 64 && (s.nb + lpr - 1) / lpr > 8) lpr <<= 1;
  }
  s.lpr = lpr;
  s.bpl = (s.nb + lpr - 1) / lpr;
  return s;
}

// LDS a workgroup can hold on the current device (at most kStageMaxBytes)
constexpr size_t kStageMaxBytes = 150 * 1024;
size_t stage_limit() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) {
    (void)hipGetLastError();
    return 65536;
  }
  const size_t lim = (size_t)v - 1024;  // the kernel's own LDS variables
  return lim < kStageMaxBytes ? lim : kStageMaxBytes;
}

namespace {

using namespace stream_dev;

// Row slots per item (one wave's share; gate_up slot = a gate row and its up row): with the ring of
// two items, about 8 block loads per lane in flight, so that 3-4 waves fit per SIMD.
constexpr int gateup_slots(int bpl) { return bpl >= 2 ? 1 : 2; }
constexpr int down_slots(int bpl) { return bpl >= 4 ? 1 : 4 / bpl; }
// Items in flight per wave (ring depth).
constexpr int gateup_ring(int bpl) { return 2; }
constexpr int down_ring(int bpl) { return 2; }


// Waves per SIMD each variant's registers allow without spilling (4 waves x 128 VGPRs, 3 x 168,
// 2 x 256, 1 x 512), read off the compiler's resource usage for these tile shapes; the workgroup
// (one per CU) has four times as many waves.
constexpr int gu_waves(int bpl, int mt) {
  return bpl == 1 ? 4 : bpl == 2 ? (mt == 1 ? 4 : 3) : bpl == 3 ? 3 : bpl <= 5 ? 2 : 1;
}
constexpr int dn_waves(int bpl, int mt) {
  return bpl == 1 ? 4 : bpl == 2 ? (mt == 1 ? 4 : 2) : bpl == 3 ? 4 : bpl <= 6 ? 2 : 1;
}


struct ItemRange {
  int begin, end;  // items [begin, end) of this workgroup
};


// Relative cost of one item of an expert with M rows when MT rows are decoded per pass: a fixed
// part per pass (the weight stream and the decode) plus one part per row (the dot products).
__device__ __forceinline__ int item_cost(int M, int MT) { return 3 * ((M + MT - 1) / MT) + M; }

// The workgroup's items: contiguous ranges of the (expert, tile) list holding equal shares of the
// total cost, so workgroups streaming experts with more rows get fewer items (`weighted`; without
// it, when every expert has the same row count, equal item counts). One wave computes the range
// from the active list and the counts (uniform values). A range boundary at cost
// position p is the first item whose cost interval starts at or after p; every workgroup evaluates
// it the same way, so the end of one range is the begin of the next.
__device__ __forceinline__ bool my_items(const int32_t* list, const int* count_ptr,
                                         const int32_t* counts, int list_cap, int tiles, int MT,
                                         int weighted, ItemRange& ir) {
  const int lane = threadIdx.x & 63;
  // the list's first 64 entries are loaded with its length (entries past the length are stale or
  // unwritten: clamped into the expert range, never used), so a list of at most 64 experts costs
  // two dependent round trips: length and entries, then row counts
  const int e_pre = weighted ? list[min(lane, list_cap - 1)] : 0;
  const int n = uniform(*count_ptr);
  if (n <= 0) return false;
  const int G = gridDim.x, b = blockIdx.x;
  if (!weighted) {  // every expert has the same row count: equal item counts, no count loads
    ir.begin = (int)((long)b * n * tiles / G);
    ir.end = (int)((long)(b + 1) * n * tiles / G);
    return ir.begin < ir.end;
  }
  if (n <= 64) {
    const int c = lane < n ? item_cost(counts[min(max(e_pre, 0), list_cap - 1)], MT) : 0;
    const int scan = wave_inclusive_scan(c, lane);
    const long total = (long)tiles * wave_last(scan);
    const long p0 = total * b / G, p1 = total * (b + 1) / G;
    const long incl = (long)tiles * scan, excl = incl - (long)tiles * c;
    const bool has0 = lane < n && p0 >= excl && p0 < incl;
    const bool has1 = lane < n && p1 >= excl && p1 < incl;
    const uint64_t m0 = __ballot(has0), m1 = __ballot(has1);
    const int v0 = lane * tiles + (int)((p0 - excl + c - 1) / (c > 0 ? c : 1));
    const int v1 = lane * tiles + (int)((p1 - excl + c - 1) / (c > 0 ? c : 1));
    ir.begin = m0 ? uniform(__shfl(v0, __ffsll((unsigned long long)m0) - 1, 64)) : n * tiles;
    ir.end = m1 ? uniform(__shfl(v1, __ffsll((unsigned long long)m1) - 1, 64)) : n * tiles;
    return ir.begin < ir.end;
  }
  // total cost
  long total = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int c = i < n ? item_cost(counts[list[i]], MT) : 0;
    total += (long)wave_last(wave_inclusive_scan(c, lane));
  }
  total *= tiles;
  const long p0 = total * b / G, p1 = total * (b + 1) / G;
  // walk the slots with a running prefix; find the items at cost positions p0 and p1
  int begin = n * tiles, end = n * tiles;
  long run = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const long c = i < n ? (long)item_cost(counts[list[i]], MT) : 0;
    const int scan = wave_inclusive_scan((int)c, lane);
    const long incl = run + (long)tiles * scan;  // prefix after slot i
    const long excl = incl - (long)tiles * c;     // prefix before slot i
    // item of slot i at position p: i*tiles + ceil((p - excl) / c), for excl <= p < incl
    const bool has0 = i < n && p0 >= excl && p0 < incl;
    const bool has1 = i < n && p1 >= excl && p1 < incl;
    const uint64_t m0 = __ballot(has0), m1 = __ballot(has1);
    if (m0) {
      const int src = __ffsll((unsigned long long)m0) - 1;
      const int v = i * tiles + (int)((p0 - excl + c - 1) / (c > 0 ? c : 1));
      begin = min(begin, uniform(__shfl(v, src, 64)));
    }
    if (m1) {
      const int src = __ffsll((unsigned long long)m1) - 1;
      const int v = i * tiles + (int)((p1 - excl + c - 1) / (c > 0 ? c : 1));
      end = min(end, uniform(__shfl(v, src, 64)));
    }
    run += (long)tiles * wave_last(scan);
  }
  ir.begin = begin;
  ir.end = end;
  return ir.begin < ir.end;
}

// The workgroup's range, computed by its first wave alone and passed to the others through LDS
// (every wave of the GPU loading the same few lines of the list and the counts at once would queue
// on those lines). Returns false, in every wave, for an empty range.
__device__ __forceinline__ bool my_items_wg(const int32_t* list, const int* count_ptr,
                                            const int32_t* counts, int list_cap, int tiles, int MT,
                                            int weighted, int* shared_range, ItemRange& ir) {
  if (threadIdx.x < 64) {
    ItemRange r{0, 0};
    if (!my_items(list, count_ptr, counts, list_cap, tiles, MT, weighted, r)) r = ItemRange{0, 0};
    if (threadIdx.x == 0) {
      shared_range[0] = r.begin;
      shared_range[1] = r.end;
    }
  }
  __syncthreads();
  ir.begin = shared_range[0];
  ir.end = shared_range[1];
  return ir.begin < ir.end;
}


// ---------------------------------------------------------------------------------------------
// Item pipeline shared by both kernels.
//
// One workgroup per CU; an item is one wave's share of work: S row slots of one expert. The
// workgroup owns a static range of items (see my_items) and its waves take items
// from that range one at a time through a counter in LDS, so every wave stays busy until the range
// is drained (with several workgroups per CU the oldest-first issue order starves the youngest one,
// which then finishes alone at a fraction of the bandwidth).
//
// A wave keeps the weight loads of its next D items in flight in a ring of register sets: it
// consumes ring entry d and refills it with a newly taken item, so D items' loads are outstanding
// while it decodes. Entries past the end of the range re-load the range's last item (L2 hits spread
// over the channels; no branch around the loads) and are never consumed. The activations of the
// current expert and token chunk stay in registers and are reloaded only when a wave's item
// changes expert (or an expert has more rows than one chunk holds); a reload waits for its loads at
// once, so the decode paths never wait on anything but the ring entry they consume.

struct Prefetch {
  int slot;                  // expert slot whose bases are cached
  const uint8_t* q;          // that expert's code and scale bases
  const uint8_t* s;
  int M, row0;               // that expert's row count and first sorted row
};

// Expert state of the item being consumed.
struct Current {
  int slot, M, row0, a_m0;
};

// Next item of the workgroup's range for this wave (uniform); >= ir.end once the range is drained.
__device__ __forceinline__ int take_item(int* counter, const ItemRange& ir) {
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(counter, 1);
  return ir.begin + uniform(__shfl(v, 0, 64));
}

// ---------------------------------------------------------------------------------------------
// gate_up: an item is S (gate row, up row) slot pairs.

// STX: all T rows of x and the token of each of the P sorted rows are copied to LDS at the start by
// the waves that do not compute the workgroup's range (so the copy overlaps that computation and
// waiting for it never waits for weight loads), and a wave reads its activation slices from there
// at every change of expert instead of fetching them from L2 behind its weight ring. The host
// enables it when both fit kXStageBytes + kTokStageBytes.
constexpr int kXStageBytes = 65536;
constexpr int kTokStageBytes = 4096;

// EPL > 0 (routed variant, decode): every workgroup first routes the T tokens itself (a wave per
// token, EPL logits per lane: the router top-k device code) and groups the T*k <= kRoutePairs pairs
// (one wave: the grouping device code) into LDS, and reads its work list, the experts' counts and
// offsets and the rows' tokens from there; workgroup 0 also writes the ids, weights and grouping to
// memory for the launches that follow. The routing and grouping are the separate kernels' code on
// the same inputs, so every workgroup holds the same result, bitwise that of those kernels. The
// layer then needs no routing launch and no memory round trip before the first weight load.
template <int BPL, int MT, int S, int D, int NW, int MODE, bool STX, int EPL>
__global__ __launch_bounds__(64 * NW, 1) void small_gateup_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, int k, int T,
    const int32_t* __restrict__ list, const int32_t* __restrict__ list_count, int list_cap, int H, int I,
    int tiles, int weighted, const uint8_t* __restrict__ w13_q, const uint8_t* __restrict__ w13_s,
    int lpr, float clamp, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
    float* __restrict__ g_ws, RouteOut ro) {
  constexpr bool kGate = MODE != kUpWithGate;
  constexpr bool kUp = MODE != kGateOnly;
  constexpr bool ROUTE = EPL > 0;
  static_assert(!ROUTE || STX, "the routed variant reads the rows' tokens from LDS");
  __shared__ int counter;
  __shared__ int range[2];
  extern __shared__ __attribute__((aligned(16))) uint8_t x_stage[];  // STX: x [T][H] bf16, tokens [P]
  // ROUTE: the ids, weights and grouping of the batch
  __shared__ int32_t r_ids[ROUTE ? kRoutePairs : 1], r_sorted[ROUTE ? kRoutePairs : 1],
      r_pair_pos[ROUTE ? kRoutePairs : 1];
  __shared__ float r_w[ROUTE ? kRoutePairs : 1];
  __shared__ int32_t r_cnt[ROUTE ? kRouteExperts : 1], r_counts[ROUTE ? kRouteExperts : 1],
      r_offsets[ROUTE ? kRouteExperts + 1 : 1], r_active[ROUTE ? kRouteExperts : 1], r_n_active[1];
  ItemRange ir;
  if (threadIdx.x == 0) counter = 0;
  if constexpr (ROUTE) {
    const int wv = threadIdx.x >> 6;
    const bool first = blockIdx.x == 0;
    if (wv < T)  // a wave per token (the host checks T <= NW)
      route_dev::route_token<EPL>(ro.logits, wv, ro.E, k, ro.score_fn, ro.renorm, first ? ro.ids : r_ids,
                                  first ? ro.weights : r_w, first ? r_ids : nullptr);
    __syncthreads();
    if (threadIdx.x < 64)
      group_dev::group_pairs_one_wave<const int32_t*, int32_t*>(r_ids, T * k, ro.E, r_counts, r_offsets, r_sorted,
                                                                r_pair_pos, r_active, r_n_active, r_cnt);
    __syncthreads();
    if (first) {  // the grouping, for the launches that follow
      for (int i = threadIdx.x; i < ro.E; i += blockDim.x) {
        ro.counts[i] = r_counts[i];
        ro.offsets[i] = r_offsets[i];
        ro.active[i] = r_active[i];
      }
      for (int i = threadIdx.x; i < T * k; i += blockDim.x) {
        ro.sorted_pair[i] = r_sorted[i];
        ro.pair_pos[i] = r_pair_pos[i];
      }
      if (threadIdx.x == 0) {
        ro.offsets[ro.E] = r_offsets[ro.E];
        *ro.n_active = r_n_active[0];
      }
    }
  }
  // the work list, the experts' row counts and first rows, and the rows' pairs: in LDS when routed
  const int32_t* Lst = ROUTE ? r_active : list;
  const int32_t* Lcnt = ROUTE ? r_n_active : list_count;
  const int32_t* Cnt = ROUTE ? r_counts : counts;
  const int32_t* Off = ROUTE ? r_offsets : offsets;
  const int32_t* Srt = ROUTE ? r_sorted : sorted_pair;
  if constexpr (STX) {
    if (threadIdx.x >= 64) {  // waves 1..NW-1; wave 0 computes the range meanwhile
      constexpr int kStagers = 64 * (NW - 1);
      constexpr int NXL = (kXStageBytes / 16 + kStagers - 1) / kStagers;
      const int st = threadIdx.x - 64;
      const int n16 = T * H / 8;
      const int P = T * k;
      const uint4* src = reinterpret_cast<const uint4*>(x);
      // every load is issued (indices clamped into the arrays), so they are in flight together;
      // only the stores are conditional
      uint4 v[NXL];
#pragma unroll
      for (int j = 0; j < NXL; ++j) v[j] = src[min(st + kStagers * j, n16 - 1)];
      constexpr int NTL = kTokStageBytes / 4 / kStagers + 1;
      int tok[NTL];
#pragma unroll
      for (int j = 0; j < NTL; ++j) tok[j] = Srt[min(st + kStagers * j, P - 1)];
      uint4* dst = reinterpret_cast<uint4*>(x_stage);
#pragma unroll
      for (int j = 0; j < NXL; ++j)
        if (st + kStagers * j < n16) dst[st + kStagers * j] = v[j];
      int32_t* tdst = reinterpret_cast<int32_t*>(x_stage + (size_t)T * H * 2);
#pragma unroll
      for (int j = 0; j < NTL; ++j)
        if (st + kStagers * j < P) tdst[st + kStagers * j] = tok[j] / k;
    }
  }
  // (the barrier inside makes the staged rows visible too)
  if (!my_items_wg(Lst, Lcnt, Cnt, list_cap, tiles, MT, weighted, range, ir)) return;

  const int lane = threadIdx.x & 63;
  const int lg = ilog2(lpr);
  const int q = lane & (lpr - 1);
  const int sub = lane >> lg;
  const int rpw = 64 >> lg;
  const int NB = H >> 5;
  const int tile_rows = S * rpw;
  const uint32_t qrow = (uint32_t)(H >> 1), srow = (uint32_t)NB;
  const size_t qexp = (size_t)2 * I * qrow, sexp = (size_t)2 * I * srow;
  const uint32_t up_q = (uint32_t)I * qrow, up_s = (uint32_t)I * srow;  // up rows follow the gate rows
  const bool k_exact = (NB % lpr) == 0;

  uint4 w[D][S][2][BPL];
  uint32_t sc[D][S][2][BPL];
  int ring_item[D];
  int ring_m[D], ring_r0[D];  // the entry's expert: row count and first row, read when its item is taken
  Prefetch pf{-1, w13_q, w13_s, 0, 0};

  // take an item into ring entry d and issue its loads; rows of a partial last tile are clamped
  // (their results are never stored)
  auto prefetch = [&](int d) {
    ring_item[d] = take_item(&counter, ir);
    const int it = min(ring_item[d], ir.end - 1);
    const int slot = uniform(it / tiles);
    const int tile = uniform(it - slot * tiles);
    if (slot != pf.slot) {
      pf.slot = slot;
      const int e = uniform(Lst[slot]);
      pf.q = w13_q + (size_t)e * qexp;
      pf.s = w13_s + (size_t)e * sexp;
      pf.M = uniform(Cnt[e]);
      pf.row0 = uniform(Off[e]);
    }
    ring_m[d] = pf.M;
    ring_r0[d] = pf.row0;
    const int n0 = tile * tile_rows;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t rr = (uint32_t)min(n0 + s * rpw + sub, I - 1);
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
        const uint32_t oq = rr * qrow + kb * 16;
        const uint32_t os = rr * srow + kb;
        if (kGate) {
          w[d][s][0][b] = ld_stream16(pf.q, oq);
          sc[d][s][0][b] = ld8(pf.s, os);
        }
        if (kUp) {
          w[d][s][1][b] = ld_stream16(pf.q, oq + up_q);
          sc[d][s][1][b] = ld8(pf.s, os + up_s);
        }
      }
    }
  };

  Current cur{-1, 0, 0, -1};
  uint4 xb[MT][BPL][4];

  auto consume = [&](int d) {
    const int item = ring_item[d];
    const int slot = uniform(item / tiles);
    const int tile = uniform(item - slot * tiles);
    if (slot != cur.slot) {  // new expert
      cur.slot = slot;
      cur.M = ring_m[d];
      cur.row0 = ring_r0[d];
      cur.a_m0 = -1;
    }
    const int n0 = tile * tile_rows;
    const bool full = n0 + tile_rows <= I;
    for (int m0 = 0; m0 < cur.M; m0 += MT) {
      const int mc = min(MT, cur.M - m0);
      if (m0 != cur.a_m0) {  // activation slices of this token chunk (LDS with STX, else L2 hits)
        cur.a_m0 = m0;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int row = cur.row0 + m0 + min(m, mc - 1);
          if constexpr (STX) {
            const int t = uniform(reinterpret_cast<const int32_t*>(x_stage + (size_t)T * H * 2)[row]);
            const uint8_t* xbase = x_stage + (size_t)t * H * 2;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
              const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
#pragma unroll
              for (int i = 0; i < 4; ++i) xb[m][b][i] = *reinterpret_cast<const uint4*>(xbase + kb * 64 + i * 16);
            }
          } else {
            const int t = uniform(Srt[row]) / k;
            const uint8_t* xbase = reinterpret_cast<const uint8_t*>(x + (size_t)t * H);
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
              const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
#pragma unroll
              for (int i = 0; i < 4; ++i) xb[m][b][i] = ld16(xbase, kb * 64 + i * 16);
            }
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
          if ((gu == 0 && !kGate) || (gu == 1 && !kUp)) continue;
#pragma unroll
          for (int b = 0; b < BPL; ++b) {
            float scale = e8m0_to_float(sc[d][s][gu][b]);
            if (!(full && k_exact) && !(n < I && q + lpr * b < NB)) scale = 0.0f;
            if (MT == 1 || mc == MT) {
              uint4 xs[MT][4];
#pragma unroll
              for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) xs[m][i] = xb[m][b][i];
              dot_block_bf16<MT>(w[d][s][gu][b], scale, xs, acc[s][gu]);
            } else {
              uint4 xs[1][4];
              float a1[1];
#pragma unroll
              for (int i = 0; i < 4; ++i) xs[0][i] = xb[0][b][i];
              a1[0] = acc[s][gu][0];
              dot_block_bf16<1>(w[d][s][gu][b], scale, xs, a1);
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
          float g = kGate ? segment_sum(acc[s][0][m], lpr) : 0.0f;
          float u = kUp ? segment_sum(acc[s][1][m], lpr) : 0.0f;
          if (q == lpr - 1 && n < I) {
            const size_t o = (size_t)(cur.row0 + m0 + m) * I + n;
            if (MODE == kGateOnly) {
              g_ws[o] = g;
            } else {
              if (MODE == kUpWithGate) g = g_ws[o];
              if (clamp > 0.0f) {
                g = clampf(g, clamp);
                u = clampf(u, clamp);
              }
              store_h_planes(h_hi, h_lo, o, silu_mul(g, u));
            }
          }
        }
      }
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) prefetch(d);
  // items are taken in increasing order, so the first entry past the range ends the wave's work
  // The loop leaves by a jump straight out of the unrolled ring walk: with a flag tested again at the
  // top, the control flow kept a path from a refill of entry d back to the consumption of entry d
  // with the other entry not refilled in between, and along it the compiler's wait before each
  // consumption covered every load in flight, the other entry's too (the ring drained at every item).
  for (;;) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (ring_item[d] >= ir.end) goto drained;
      consume(d);
      prefetch(d);
    }
  }
drained:;
}

// ---------------------------------------------------------------------------------------------
// down: an item is S rows of W2; activations h rebuilt in fp32 from its two bf16 planes.
//
// STAGED: the h rows of the experts in a workgroup's range form one contiguous block of the sorted
// rows when the list is the whole active list (ascending, and no expert between two listed ones has
// rows). The workgroup copies both planes of that block to LDS once, right after issuing its first
// weight loads, and its waves read their h blocks from there with LDS loads, which a wave waits for
// without waiting for its weight loads in flight; otherwise a wave fetches its rows from L2 at every
// change of expert and, the loads being in order, drains its weight ring there. The host enables it
// only when a bound on the rows of any range fits the LDS it allocates (down_stage_rows).

template <int BPL, int MT, int S, int D, int NW, bool STAGED>
__global__ __launch_bounds__(64 * NW, 1) void small_down_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ list, const int32_t* __restrict__ list_count, int list_cap, int H, int I,
    int tiles, int weighted, const uint8_t* __restrict__ w2_q, const uint8_t* __restrict__ w2_s,
    int lpr, const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo,
    float* __restrict__ y) {
  __shared__ int counter;
  __shared__ int range[2];
  extern __shared__ __attribute__((aligned(16))) uint8_t h_stage[];  // STAGED: hi plane, then lo plane
  ItemRange ir;
  if (threadIdx.x == 0) counter = 0;
  if (!my_items_wg(list, list_count, counts, list_cap, tiles, MT, weighted, range, ir)) return;

  const int lane = threadIdx.x & 63;
  const int lg = ilog2(lpr);
  const int q = lane & (lpr - 1);
  const int sub = lane >> lg;
  const int rpw = 64 >> lg;
  const int NB = I >> 5;
  const int tile_rows = S * rpw;
  const uint32_t qrow = (uint32_t)(I >> 1), srow = (uint32_t)NB;
  const size_t qexp = (size_t)H * qrow, sexp = (size_t)H * srow;

  // STAGED: the range's h rows [row_lo, row_hi)
  int row_lo = 0;
  uint32_t stage_plane = 0;  // bytes per plane
  if constexpr (STAGED) {
    const int e_last = uniform(list[(ir.end - 1) / tiles]);
    row_lo = uniform(offsets[uniform(list[ir.begin / tiles])]);
    const int row_hi = uniform(offsets[e_last]) + uniform(counts[e_last]);
    stage_plane = (uint32_t)(row_hi - row_lo) * (uint32_t)I * 2;
  }
  const bool k_exact = (NB % lpr) == 0;

  uint4 w[D][S][BPL];
  uint32_t sc[D][S][BPL];
  int ring_item[D];
  int ring_m[D], ring_r0[D];  // the entry's expert: row count and first row, read when its item is taken
  Prefetch pf{-1, w2_q, w2_s, 0, 0};

  auto prefetch = [&](int d) {
    ring_item[d] = take_item(&counter, ir);
    const int it = min(ring_item[d], ir.end - 1);
    const int slot = uniform(it / tiles);
    const int tile = uniform(it - slot * tiles);
    if (slot != pf.slot) {
      pf.slot = slot;
      const int e = uniform(list[slot]);
      pf.q = w2_q + (size_t)e * qexp;
      pf.s = w2_s + (size_t)e * sexp;
      pf.M = uniform(counts[e]);
      pf.row0 = uniform(offsets[e]);
    }
    ring_m[d] = pf.M;
    ring_r0[d] = pf.row0;
    const int n0 = tile * tile_rows;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t rr = (uint32_t)min(n0 + s * rpw + sub, H - 1);
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
        w[d][s][b] = ld_stream16(pf.q, rr * qrow + kb * 16);
        sc[d][s][b] = ld8(pf.s, rr * srow + kb);
      }
    }
  };

  Current cur{-1, 0, 0, -1};
  uint32_t hh[MT][BPL][16];  // h blocks as scaled fp16 pairs
  float hinv[MT][BPL];       // their inverse power-of-two scales

  auto consume = [&](int d) {
    const int item = ring_item[d];
    const int slot = uniform(item / tiles);
    const int tile = uniform(item - slot * tiles);
    if (slot != cur.slot) {
      cur.slot = slot;
      cur.M = ring_m[d];
      cur.row0 = ring_r0[d];
      cur.a_m0 = -1;
    }
    const int n0 = tile * tile_rows;
    const bool full = n0 + tile_rows <= H;
    for (int m0 = 0; m0 < cur.M; m0 += MT) {
      const int mc = min(MT, cur.M - m0);
      if (m0 != cur.a_m0) {
        cur.a_m0 = m0;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int row = cur.row0 + m0 + min(m, mc - 1);
          const uint8_t* hib = reinterpret_cast<const uint8_t*>(h_hi + (size_t)row * I);
          const uint8_t* lob = reinterpret_cast<const uint8_t*>(h_lo + (size_t)row * I);
          const uint32_t soff = (uint32_t)(row - row_lo) * (uint32_t)I * 2;
#pragma unroll
          for (int b = 0; b < BPL; ++b) {
            const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
            uint4 hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (STAGED) {
                hv[i] = *reinterpret_cast<const uint4*>(h_stage + soff + kb * 64 + i * 16);
                lv[i] = *reinterpret_cast<const uint4*>(h_stage + stage_plane + soff + kb * 64 + i * 16);
              } else {
                hv[i] = ld16(hib, kb * 64 + i * 16);
                lv[i] = ld16(lob, kb * 64 + i * 16);
              }
            }
            hinv[m][b] = h_planes_to_f16(hv, lv, hh[m][b]);
            // one block's planes in registers at a time
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int b = 0; b < BPL; ++b)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
              uint4 t = make_uint4(hh[m][b][i], hh[m][b][i + 1], hh[m][b][i + 2], hh[m][b][i + 3]);
              opaque(t);
              hh[m][b][i] = t.x, hh[m][b][i + 1] = t.y, hh[m][b][i + 2] = t.z, hh[m][b][i + 3] = t.w;
            }
      }
      float acc[S][MT];
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][m] = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = n0 + s * rpw + sub;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
          float scale = e8m0_to_float(sc[d][s][b]);
          if (!(full && k_exact) && !(n < H && q + lpr * b < NB)) scale = 0.0f;
          if (MT == 1 || mc == MT) {
            uint32_t hs[MT][16];
            float bs[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              bs[m] = scale * hinv[m][b];
#pragma unroll
              for (int i = 0; i < 16; ++i) hs[m][i] = hh[m][b][i];
            }
            dot_block_f16s<MT>(w[d][s][b], bs, hs, acc[s]);
          } else {
            uint32_t hs[1][16];
            float bs[1] = {scale * hinv[0][b]};
            float a1[1];
#pragma unroll
            for (int i = 0; i < 16; ++i) hs[0][i] = hh[0][b][i];
            a1[0] = acc[s][0];
            dot_block_f16s<1>(w[d][s][b], bs, hs, a1);
            acc[s][0] = a1[0];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = n0 + s * rpw + sub;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m >= mc) break;
          const float v = segment_sum(acc[s][m], lpr);
          if (q == lpr - 1 && n < H) y[(size_t)(cur.row0 + m0 + m) * H + n] = v;
        }
      }
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) prefetch(d);
  if constexpr (STAGED) {  // after the first weight loads, so both round trips overlap
    const uint32_t n16 = stage_plane >> 4;
    const uint4* src_hi = reinterpret_cast<const uint4*>(h_hi + (size_t)row_lo * I);
    const uint4* src_lo = reinterpret_cast<const uint4*>(h_lo + (size_t)row_lo * I);
    uint4* dst = reinterpret_cast<uint4*>(h_stage);
    for (uint32_t i = threadIdx.x; i < n16; i += blockDim.x) {
      const uint4 a = src_hi[i], c = src_lo[i];
      dst[i] = a;
      dst[n16 + i] = c;
    }
    __syncthreads();
  }
  // The loop leaves by a jump straight out of the unrolled ring walk: with a flag tested again at the
  // top, the control flow kept a path from a refill of entry d back to the consumption of entry d
  // with the other entry not refilled in between, and along it the compiler's wait before each
  // consumption covered every load in flight, the other entry's too (the ring drained at every item).
  for (;;) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (ring_item[d] >= ir.end) goto drained;
      consume(d);
      prefetch(d);
    }
  }
drained:;
}

// ---------------------------------------------------------------------------------------------
// down with the weighted combine folded in, for few routed pairs (P <= kCombinePairsMax, every active
// expert on these kernels, P rows of h within the LDS a workgroup can have). A workgroup owns whole
// tiles of output rows, for every pair: its items are (output-row tile, expert slot), tile outermost,
// and its range is a contiguous run of whole tiles. Every pair's h blocks are built once, at the start,
// into LDS in the down kernel's fp16 format (the same conversion, so the same values), the y values of
// the workgroup's rows stay in LDS, and at the end the workgroup sums topk_w[t, j] * y[pair_pos[t, j]]
// over j in order in fp32 and rounds once to bfloat16: the combine kernel's arithmetic, bit for bit.
// The layer then has one launch, and one round trip of y through memory, fewer.

template <int BPL, int MT, int S, int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void small_down_combine_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ list, const int32_t* __restrict__ list_count, int list_cap,
    const int32_t* __restrict__ pair_pos, const float* __restrict__ topk_w, int T, int k, int H, int I,
    int ntiles, const uint8_t* __restrict__ w2_q, const uint8_t* __restrict__ w2_s, int lpr,
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, uint16_t* __restrict__ out) {
  __shared__ int counter;
  __shared__ int s_n;
  __shared__ int32_t s_e[kCombinePairsMax], s_m[kCombinePairsMax], s_r0[kCombinePairsMax];
  __shared__ int32_t s_pp[kCombinePairsMax];
  __shared__ float s_w[kCombinePairsMax];
  // dynamic LDS: h blocks as fp16 pairs (P * NB * 64 bytes), their inverse scales [P][NB], y [P][NR]
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];

  const int P = T * k;
  const int G = gridDim.x, wg = blockIdx.x;
  const int nt0 = (int)((long)wg * ntiles / G), nt1 = (int)((long)(wg + 1) * ntiles / G);
  if (nt0 >= nt1) return;  // (uniform; the grid has at most ntiles workgroups)

  const int lane = threadIdx.x & 63;
  const int lg = ilog2(lpr);
  const int q = lane & (lpr - 1);
  const int sub = lane >> lg;
  const int rpw = 64 >> lg;
  const int NB = I >> 5;
  const int tile_rows = S * rpw;
  const int NR = (nt1 - nt0) * tile_rows;  // output rows of this workgroup (past H at the end: not used)
  const int nbase = nt0 * tile_rows;
  const uint32_t qrow = (uint32_t)(I >> 1), srow = (uint32_t)NB;
  const size_t qexp = (size_t)H * qrow, sexp = (size_t)H * srow;
  const bool k_exact = (NB % lpr) == 0;
  // quarter i of block kb of row r at h16[(r * 4 + i) * NB + kb]: the lanes of a wave read
  // consecutive 16-byte words
  uint4* h16 = reinterpret_cast<uint4*>(dyn);
  float* hinv_l = reinterpret_cast<float*>(dyn + (size_t)P * NB * 64);
  float* y_l = hinv_l + (size_t)P * NB;

  // the work list and each pair's weight and row, to LDS (n <= P <= kCombinePairsMax)
  if (threadIdx.x < 64) {
    // the list's entries are loaded with its length (entries past it are never used)
    const int e_pre = list[min(lane, list_cap - 1)];
    const int n = min(uniform(*list_count), kCombinePairsMax);  // (at most P, by the grouping)
    if (lane < n) {
      const int e = e_pre;
      s_e[lane] = e;
      s_m[lane] = counts[e];
      s_r0[lane] = offsets[e];
    }
    if (lane < P && lane < kCombinePairsMax) {
      s_pp[lane] = pair_pos[lane];
      s_w[lane] = topk_w[lane];
    }
    if (lane == 0) {
      s_n = n;
      counter = 0;
    }
  }
  __syncthreads();
  const int n = s_n;
  if (n <= 0) return;  // (uniform)
  const int nitems = (nt1 - nt0) * n;
  const ItemRange ir{0, nitems};

  uint4 w[D][S][BPL];
  uint32_t sc[D][S][BPL];
  int ring_item[D];

  auto prefetch = [&](int d) {
    ring_item[d] = take_item(&counter, ir);
    const int it = min(ring_item[d], nitems - 1);
    const int tl = uniform(it / n);
    const int slot = uniform(it - tl * n);
    const int e = uniform(s_e[slot]);
    const uint8_t* pq = w2_q + (size_t)e * qexp;
    const uint8_t* ps = w2_s + (size_t)e * sexp;
    const int n0 = (nt0 + tl) * tile_rows;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t rr = (uint32_t)min(n0 + s * rpw + sub, H - 1);
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
        w[d][s][b] = ld_stream16(pq, rr * qrow + kb * 16);
        sc[d][s][b] = ld8(ps, rr * srow + kb);
      }
    }
  };

  uint32_t hh[MT][BPL][16];  // h blocks as scaled fp16 pairs
  float hinv[MT][BPL];       // their inverse power-of-two scales

  auto consume = [&](int d) {
    const int item = ring_item[d];
    const int tl = uniform(item / n);
    const int slot = uniform(item - tl * n);
    const int M = uniform(s_m[slot]);
    const int row0 = uniform(s_r0[slot]);
    const int n0 = (nt0 + tl) * tile_rows;
    const bool full = n0 + tile_rows <= H;
    for (int m0 = 0; m0 < M; m0 += MT) {
      const int mc = min(MT, M - m0);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int row = row0 + m0 + min(m, mc - 1);
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
          const int kb = min(q + lpr * b, NB - 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = h16[((size_t)row * 4 + i) * NB + kb];
            hh[m][b][4 * i] = v.x, hh[m][b][4 * i + 1] = v.y, hh[m][b][4 * i + 2] = v.z, hh[m][b][4 * i + 3] = v.w;
          }
          hinv[m][b] = hinv_l[(size_t)row * NB + kb];
        }
      }
      float acc[S][MT];
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][m] = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int nn = n0 + s * rpw + sub;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
          float scale = e8m0_to_float(sc[d][s][b]);
          if (!(full && k_exact) && !(nn < H && q + lpr * b < NB)) scale = 0.0f;
          if (MT == 1 || mc == MT) {
            uint32_t hs[MT][16];
            float bs[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              bs[m] = scale * hinv[m][b];
#pragma unroll
              for (int i = 0; i < 16; ++i) hs[m][i] = hh[m][b][i];
            }
            dot_block_f16s<MT>(w[d][s][b], bs, hs, acc[s]);
          } else {
            uint32_t hs[1][16];
            float bs[1] = {scale * hinv[0][b]};
            float a1[1];
#pragma unroll
            for (int i = 0; i < 16; ++i) hs[0][i] = hh[0][b][i];
            a1[0] = acc[s][0];
            dot_block_f16s<1>(w[d][s][b], bs, hs, a1);
            acc[s][0] = a1[0];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int nn = n0 + s * rpw + sub;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m >= mc) break;
          const float v = segment_sum(acc[s][m], lpr);
          if (q == lpr - 1 && nn < H) y_l[(size_t)(row0 + m0 + m) * NR + (nn - nbase)] = v;
        }
      }
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) prefetch(d);
  // every pair's h blocks, as the down kernel builds them (after the first weight loads, so both
  // round trips overlap)
  for (int i = threadIdx.x; i < P * NB; i += blockDim.x) {
    const int row = i / NB, kb = i - row * NB;
    const uint8_t* hib = reinterpret_cast<const uint8_t*>(h_hi + (size_t)row * I) + kb * 64;
    const uint8_t* lob = reinterpret_cast<const uint8_t*>(h_lo + (size_t)row * I) + kb * 64;
    uint4 hv[4], lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hv[j] = ld16(hib, j * 16);
      lv[j] = ld16(lob, j * 16);
    }
    uint32_t blk[16];
    const float inv = h_planes_to_f16(hv, lv, blk);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      h16[((size_t)row * 4 + j) * NB + kb] = make_uint4(blk[4 * j], blk[4 * j + 1], blk[4 * j + 2], blk[4 * j + 3]);
    hinv_l[i] = inv;
  }
  __syncthreads();
  // (the ring walk leaves by a jump, as in the kernels above)
  for (;;) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (ring_item[d] >= nitems) goto drained;
      consume(d);
      prefetch(d);
    }
  }
drained:
  __syncthreads();
  // the weighted combine of this workgroup's output rows: out[t, n] = bf16(sum_j w[t, j] * y[pair, n])
  for (int i = threadIdx.x; i < T * NR; i += blockDim.x) {
    const int t = i / NR, nn = i - t * NR;
    const int nr = nbase + nn;
    if (nr >= H) continue;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc = fmaf(s_w[t * k + j], y_l[(size_t)s_pp[t * k + j] * NR + nn], acc);
    out[(size_t)t * H + nr] = f32_to_bf16_rne(acc);
  }
}

// x and the row tokens in LDS (STX) when they fit the staging bounds and there are at least 8 waves
// to copy them
bool gateup_stx(const SmallPlan& sp, int H) {
  return (size_t)sp.T * H * 2 <= (size_t)kXStageBytes && (size_t)sp.P * 4 <= (size_t)kTokStageBytes &&
         sp.gu_block >= 512 && (size_t)sp.T * H * 2 + (size_t)sp.P * 4 <= stage_limit();
}

template <int MODE>
hipError_t gateup_dispatch(const SmallPlan& sp, const Routed& r, const int32_t* list,
                           const int32_t* list_count, int H, int I, const uint8_t* wq,
                           const uint8_t* ws, float clamp, uint16_t* h_hi, uint16_t* h_lo,
                           float* g_ws, hipStream_t stream) {
  const dim3 grid(sp.gu_grid);
  const int lpr = sp.gu.lpr, tiles = sp.gu_tiles;
  const bool stx = gateup_stx(sp, H);
  const size_t lds = stx ? (size_t)sp.T * H * 2 + (size_t)sp.P * 4 : 0;
#define MOE_GU_K(BPL, MT, STX)                                                                           \
  {                                                                                                      \
    auto kern = small_gateup_kernel<BPL, MT, gateup_slots(BPL), gateup_ring(BPL), 4 * gu_waves(BPL, MT), \
                                    MODE, STX, 0>;                                                       \
    static std::atomic<bool> lds_attr_set{false};                                                        \
    if (STX && lds > 65536 && !lds_attr_set.load()) {                                                    \
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                                       \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageMaxBytes) !=        \
          hipSuccess)                                                                                    \
        return hipErrorInvalidValue;                                                                     \
      lds_attr_set.store(true);                                                                          \
    }                                                                                                    \
    kern<<<grid, 256 * gu_waves(BPL, MT), STX ? lds : 0, stream>>>(                                      \
        r.x, r.counts, r.offsets, r.sorted_pair, r.k, sp.T, list, list_count, sp.E, H, I, tiles,         \
        sp.weighted,                                                                                     \
        wq, ws, lpr, clamp, h_hi, h_lo, g_ws, RouteOut{});                                               \
  }
#define MOE_GU(BPL, MT)          \
  do {                           \
    if (stx && 4 * gu_waves(BPL, MT) >= 8) \
      MOE_GU_K(BPL, MT, true)    \
    else                         \
      MOE_GU_K(BPL, MT, false)   \
  } while (0)
#define MOE_GU_MT(BPL) \
  if (sp.mt_gu == 2)   \
    MOE_GU(BPL, 2);    \
  else                 \
    MOE_GU(BPL, 1);
  switch (sp.gu.bpl) {
    case 1: MOE_GU_MT(1) break;
    case 2: MOE_GU_MT(2) break;
    case 3: MOE_GU(3, 1); break;
    case 4: MOE_GU(4, 1); break;
    case 5: MOE_GU(5, 1); break;
    case 6: MOE_GU(6, 1); break;
    case 7: MOE_GU(7, 1); break;
    case 8: MOE_GU(8, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_GU_MT
#undef MOE_GU
#undef MOE_GU_K
  return hipGetLastError();
}

}  // namespace

bool gateup_routed_ok(const SmallPlan& sp, int H, int E) {
  return gateup_stx(sp, H) && sp.gu.bpl <= 2 && sp.gu_grid > 0 && sp.T >= 1 && sp.T <= sp.gu_block / 64 &&
         sp.P <= kRoutePairs && E >= 1 && E <= kRouteExperts;
}

hipError_t launch_small_gateup_routed(const SmallPlan& sp, const Routed& r, const RouteOut& ro, int H, int I,
                                      const uint8_t* w13_q, const uint8_t* w13_s, float clamp,
                                      uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream) {
  if (!gateup_routed_ok(sp, H, ro.E)) return hipErrorInvalidValue;
  const dim3 grid(sp.gu_grid);
  const int lpr = sp.gu.lpr, tiles = sp.gu_tiles;
  const size_t lds = (size_t)sp.T * H * 2 + (size_t)sp.P * 4;
#define MOE_GUR(BPL, MT, EPL)                                                                             \
  {                                                                                                       \
    auto kern = small_gateup_kernel<BPL, MT, gateup_slots(BPL), gateup_ring(BPL), 4 * gu_waves(BPL, MT),  \
                                    kGateUpFused, true, EPL>;                                             \
    static std::atomic<bool> lds_attr_set{false};                                                         \
    if (lds > 65536 && !lds_attr_set.load()) {                                                            \
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                                        \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageMaxBytes) != hipSuccess) \
        return hipErrorInvalidValue;                                                                      \
      lds_attr_set.store(true);                                                                           \
    }                                                                                                     \
    kern<<<grid, 256 * gu_waves(BPL, MT), lds, stream>>>(r.x, ro.counts, ro.offsets, ro.sorted_pair, r.k,  \
                                                         sp.T, ro.active, ro.n_active, sp.E, H, I, tiles,  \
                                                         sp.weighted, w13_q, w13_s, lpr, clamp, h_hi, h_lo, \
                                                         nullptr, ro);                                     \
  }
#define MOE_GUR_E(BPL, MT)          \
  if (ro.E <= 64)                   \
    MOE_GUR(BPL, MT, 1)             \
  else if (ro.E <= 128)             \
    MOE_GUR(BPL, MT, 2)             \
  else                              \
    MOE_GUR(BPL, MT, 4)
  if (sp.gu.bpl == 1) {
    if (sp.mt_gu == 2) {
      MOE_GUR_E(1, 2)
    } else {
      MOE_GUR_E(1, 1)
    }
  } else {
    if (sp.mt_gu == 2) {
      MOE_GUR_E(2, 2)
    } else {
      MOE_GUR_E(2, 1)
    }
  }
#undef MOE_GUR_E
#undef MOE_GUR
  return hipGetLastError();
}

SmallPlan plan_small(int T, int H, int I, int E, int k, int num_cus) {
  SmallPlan sp;
  sp.gu = choose_row_split(H);
  sp.dn = choose_row_split(I);
  const int rpw_gu = 64 / sp.gu.lpr, rpw_dn = 64 / sp.dn.lpr;
  sp.gu_tile = gateup_slots(sp.gu.bpl) * rpw_gu;
  sp.dn_tile = down_slots(sp.dn.bpl) * rpw_dn;
  sp.gu_tiles = (I + sp.gu_tile - 1) / sp.gu_tile;
  sp.dn_tiles = (H + sp.dn_tile - 1) / sp.dn_tile;
  const long P = (long)T * k;
  sp.slots = (int)(P < E ? P : E);
  sp.T = T;
  sp.P = (int)P;
  sp.E = E;
  sp.mt_gu = (T >= 2 && sp.gu.bpl <= 2) ? 2 : 1;
  sp.mt_dn = (T >= 2 && sp.dn.bpl <= 2) ? 2 : 1;
  // with T <= 2 every expert has one or two rows and costs about the same per item
  sp.weighted = T > 2;
  // one workgroup per CU (its waves share the CU's range of items), never more than there can
  // be items
  const long gu_items = (long)sp.slots * sp.gu_tiles, dn_items = (long)sp.slots * sp.dn_tiles;
  sp.gu_grid = (int)(gu_items < num_cus ? gu_items : num_cus);
  sp.dn_grid = (int)(dn_items < num_cus ? dn_items : num_cus);
  sp.fold_grid = sp.dn_tiles < num_cus ? sp.dn_tiles : num_cus;
  sp.gu_block = 256 * gu_waves(sp.gu.bpl, sp.mt_gu);
  sp.dn_block = 256 * dn_waves(sp.dn.bpl, sp.mt_dn);
  return sp;
}

hipError_t launch_small_gateup(const SmallPlan& sp, const Routed& r, const int32_t* list,
                               const int32_t* list_count, int H, int I, const uint8_t* w13_q,
                               const uint8_t* w13_s, float clamp, int mode, uint16_t* h_hi,
                               uint16_t* h_lo, float* g_ws, hipStream_t stream) {
  if (sp.gu_grid <= 0) return hipSuccess;
  switch (mode) {
    case kGateUpFused:
      return gateup_dispatch<kGateUpFused>(sp, r, list, list_count, H, I, w13_q, w13_s, clamp, h_hi, h_lo, g_ws,
                                           stream);
    case kGateOnly:
      return gateup_dispatch<kGateOnly>(sp, r, list, list_count, H, I, w13_q, w13_s, clamp, h_hi, h_lo, g_ws,
                                        stream);
    case kUpWithGate:
      return gateup_dispatch<kUpWithGate>(sp, r, list, list_count, H, I, w13_q, w13_s, clamp, h_hi, h_lo, g_ws,
                                          stream);
    default:
      return hipErrorInvalidValue;
  }
}

// Bound on the h rows of one down workgroup's range when the list is the whole active list. The
// grouping does not require a token's ids to be distinct, so one expert can hold every one of the
// P rows; a range of consecutive experts spans at most all of them. The bound is therefore P: the
// staged kernel runs only when all of h fits the LDS (decode at one or two tokens), whatever the
// routing.
int down_stage_rows(const SmallPlan& sp) { return sp.P; }


hipError_t launch_small_down(const SmallPlan& sp, const Routed& r, const int32_t* list,
                             const int32_t* list_count, bool list_is_active, int H, int I,
                             const uint8_t* w2_q, const uint8_t* w2_s, const uint16_t* h_hi,
                             const uint16_t* h_lo, float* y, hipStream_t stream) {
  if (sp.dn_grid <= 0) return hipSuccess;
  const dim3 grid(sp.dn_grid);
  const int lpr = sp.dn.lpr, tiles = sp.dn_tiles;
  const size_t stage_bytes = (size_t)down_stage_rows(sp) * I * 4;
  const bool staged = list_is_active && stage_bytes <= stage_limit();
#define MOE_DN_K(BPL, MT, ST)                                                                          \
  {                                                                                                   \
    auto kern = small_down_kernel<BPL, MT, down_slots(BPL), down_ring(BPL), 4 * dn_waves(BPL, MT), ST>; \
    const size_t lds = ST ? stage_bytes : 0;                                                          \
    static std::atomic<bool> lds_attr_set{false};                                                     \
    if (lds > 65536 && !lds_attr_set.load()) {                                                        \
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                                    \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageMaxBytes) !=     \
          hipSuccess)                                                                                 \
        return hipErrorInvalidValue;                                                                  \
      lds_attr_set.store(true);                                                                       \
    }                                                                                                 \
    kern<<<grid, 256 * dn_waves(BPL, MT), lds, stream>>>(r.counts, r.offsets, list, list_count, sp.E, H, I, \
                                                         tiles, sp.weighted, w2_q, w2_s, lpr, h_hi,    \
                                                         h_lo, y);                                     \
  }
#define MOE_DN(BPL, MT)        \
  do {                         \
    if (staged)                \
      MOE_DN_K(BPL, MT, true)  \
    else                       \
      MOE_DN_K(BPL, MT, false) \
  } while (0)
  switch (sp.dn.bpl) {
    case 1:
      if (sp.mt_dn == 2) MOE_DN(1, 2); else MOE_DN(1, 1);
      break;
    case 2:
      if (sp.mt_dn == 2) MOE_DN(2, 2); else MOE_DN(2, 1);
      break;
    case 3: MOE_DN(3, 1); break;
    case 4: MOE_DN(4, 1); break;
    case 5: MOE_DN(5, 1); break;
    case 6: MOE_DN(6, 1); break;
    case 7: MOE_DN(7, 1); break;
    case 8: MOE_DN(8, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_DN
#undef MOE_DN_K
  return hipGetLastError();
}

// LDS of the folded down + combine kernel: fp16 h blocks and their scales for every pair, and the y
// values of one workgroup's output rows for every pair.
size_t down_combine_lds(const SmallPlan& sp, int H, int I) {
  const int grid = sp.fold_grid;
  if (grid <= 0) return 0;
  const size_t rows = (size_t)((sp.dn_tiles + grid - 1) / grid) * sp.dn_tile;
  (void)H;
  return (size_t)sp.P * (I / 32) * 68 + (size_t)sp.P * rows * 4;
}

bool down_combine_fits(const SmallPlan& sp, int H, int I) {
  return sp.P >= 1 && sp.P <= kCombinePairsMax && sp.fold_grid > 0 &&
         down_combine_lds(sp, H, I) <= stage_limit();
}

hipError_t launch_small_down_combine(const SmallPlan& sp, const Routed& r, const int32_t* list,
                                     const int32_t* list_count, const int32_t* pair_pos,
                                     const float* topk_w, int H, int I, const uint8_t* w2_q,
                                     const uint8_t* w2_s, const uint16_t* h_hi, const uint16_t* h_lo,
                                     uint16_t* out, hipStream_t stream) {
  if (!down_combine_fits(sp, H, I)) return hipErrorInvalidValue;
  const dim3 grid(sp.fold_grid);
  const int lpr = sp.dn.lpr, ntiles = sp.dn_tiles;
  const size_t lds = down_combine_lds(sp, H, I);
#define MOE_DC(BPL, MT)                                                                              \
  {                                                                                                 \
    auto kern = small_down_combine_kernel<BPL, MT, down_slots(BPL), down_ring(BPL), 4 * dn_waves(BPL, MT)>; \
    static std::atomic<bool> lds_attr_set{false};                                                   \
    if (lds > 65536 && !lds_attr_set.load()) {                                                      \
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                                  \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageMaxBytes) !=   \
          hipSuccess)                                                                               \
        return hipErrorInvalidValue;                                                                \
      lds_attr_set.store(true);                                                                     \
    }                                                                                               \
    kern<<<grid, 256 * dn_waves(BPL, MT), lds, stream>>>(r.counts, r.offsets, list, list_count, sp.E, pair_pos, \
                                                         topk_w, sp.T, r.k, H, I, ntiles, w2_q, w2_s, lpr, \
                                                         h_hi, h_lo, out);                           \
  }
  switch (sp.dn.bpl) {
    case 1:
      if (sp.mt_dn == 2) MOE_DC(1, 2) else MOE_DC(1, 1)
      break;
    case 2:
      if (sp.mt_dn == 2) MOE_DC(2, 2) else MOE_DC(2, 1)
      break;
    case 3: MOE_DC(3, 1) break;
    case 4: MOE_DC(4, 1) break;
    case 5: MOE_DC(5, 1) break;
    case 6: MOE_DC(6, 1) break;
    case 7: MOE_DC(7, 1) break;
    case 8: MOE_DC(8, 1) break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_DC
  return hipGetLastError();
}

}  // namespace moe
