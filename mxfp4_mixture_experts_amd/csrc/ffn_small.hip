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
#include "kernels.hpp"

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

namespace {

// Row slots per item (one wave's share; gate_up slot = a gate row and its up row): with the ring of
// two items, about 8 block loads per lane in flight, so that 3-4 waves fit per SIMD.
constexpr int gateup_slots(int bpl) { return bpl >= 2 ? 1 : 2; }
constexpr int down_slots(int bpl) { return bpl >= 4 ? 1 : 4 / bpl; }
// Items in flight per wave (ring depth).
constexpr int gateup_ring(int bpl) { return 2; }
constexpr int down_ring(int bpl) { return 2; }

__device__ __forceinline__ int ilog2(int v) { return 31 - __clz(v); }

// Waves per SIMD each variant's registers allow without spilling (4 waves x 128 VGPRs, 3 x 168,
// 2 x 256, 1 x 512), read off the compiler's resource usage for these tile shapes; the workgroup
// (one per CU) has four times as many waves.
constexpr int gu_waves(int bpl, int mt) {
  return bpl == 1 ? 4 : bpl == 2 ? (mt == 1 ? 4 : 3) : bpl == 3 ? 3 : bpl <= 5 ? 2 : 1;
}
constexpr int dn_waves(int bpl, int mt) {
  return bpl == 1 ? 4 : bpl == 2 ? (mt == 1 ? 4 : 2) : bpl == 3 ? 4 : bpl <= 6 ? 2 : 1;
}

// The packed block is passed through an empty asm so the compiler cannot hoist its decode out of
// the token loop (that would keep up to 32 decoded registers per block alive and spill).
__device__ __forceinline__ void opaque(uint4& w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
}
__device__ __forceinline__ void opaque(float4& w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
}

// acc[m] += <decoded block, x block of token m> for MTC tokens (gate/up: bf16 dot2).
template <int MTC>
__device__ __forceinline__ void dot_block_bf16(uint4 w, float scale, const uint4 (&xb)[MTC][4],
                                               float (&acc)[MTC]) {
  opaque(w);
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const bf16x2_t p0 = fp4x2_to_bf16x2<0>(wd[d], scale);
    const bf16x2_t p1 = fp4x2_to_bf16x2<1>(wd[d], scale);
    const bf16x2_t p2 = fp4x2_to_bf16x2<2>(wd[d], scale);
    const bf16x2_t p3 = fp4x2_to_bf16x2<3>(wd[d], scale);
#pragma unroll
    for (int m = 0; m < MTC; ++m) {
      float a = acc[m];
      a = dot2_bf16(p0, as_bf16x2(xb[m][d].x), a);
      a = dot2_bf16(p1, as_bf16x2(xb[m][d].y), a);
      a = dot2_bf16(p2, as_bf16x2(xb[m][d].z), a);
      a = dot2_bf16(p3, as_bf16x2(xb[m][d].w), a);
      acc[m] = a;
    }
  }
}

// acc[m] += bs[m] * <codes of the block, h block of token m> for MTC tokens (down). The codes are
// decoded unscaled to fp16 and dotted with the token's fp16 h block by v_dot2_f32_f16 (fp32
// accumulation); bs[m] carries the block's E8M0 scale times the inverse of the h block's
// power-of-two scale.
template <int MTC>
__device__ __forceinline__ void dot_block_f16s(uint4 w, const float (&bs)[MTC],
                                               const uint32_t (&hh)[MTC][16], float (&acc)[MTC]) {
  opaque(w);
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float part[MTC];
#pragma unroll
  for (int m = 0; m < MTC; ++m) part[m] = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f16x2_t p0 = fp4x2_to_f16x2<0>(wd[d]);
    const f16x2_t p1 = fp4x2_to_f16x2<1>(wd[d]);
    const f16x2_t p2 = fp4x2_to_f16x2<2>(wd[d]);
    const f16x2_t p3 = fp4x2_to_f16x2<3>(wd[d]);
#pragma unroll
    for (int m = 0; m < MTC; ++m) {
      float a = part[m];
      a = dot2_f16(p0, as_f16x2(hh[m][4 * d + 0]), a);
      a = dot2_f16(p1, as_f16x2(hh[m][4 * d + 1]), a);
      a = dot2_f16(p2, as_f16x2(hh[m][4 * d + 2]), a);
      a = dot2_f16(p3, as_f16x2(hh[m][4 * d + 3]), a);
      part[m] = a;
    }
  }
#pragma unroll
  for (int m = 0; m < MTC; ++m) acc[m] = fmaf(part[m], bs[m], acc[m]);
}

// One lane's 32-value h block, given as its two bf16 planes (16 bytes x 4 of hi, of lo), as 16
// packed fp16 pairs: value j is hi_j + lo_j (exact in fp32), scaled by a power of two that puts the
// largest |hi_j| in [2^14, 2^15) (read from the bf16 exponent fields, so no fp32 copy of the block
// stays live). |hi + lo| <= |hi| (1 + 2^-8), so nothing overflows fp16 and every value keeps fp16's
// 11-bit precision relative to the block maximum. Returns the inverse scale.
__device__ __forceinline__ float h_planes_to_f16(const uint4 (&hv)[4], const uint4 (&lv)[4],
                                                 uint32_t (&hh)[16]) {
  // largest exponent field among the low and among the high bf16 halves
  uint32_t mx_lo = 0, mx_hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mx_lo = max(max(mx_lo, max(hv[i].x & 0x7F80u, hv[i].y & 0x7F80u)), max(hv[i].z & 0x7F80u, hv[i].w & 0x7F80u));
    mx_hi = max(max(mx_hi, max(hv[i].x & 0x7F800000u, hv[i].y & 0x7F800000u)),
                max(hv[i].z & 0x7F800000u, hv[i].w & 0x7F800000u));
  }
  const int eb = max((int)(mx_lo >> 7), (int)(mx_hi >> 23));  // biased exponent of max |hi|
  const int f = min(max(268 - eb, 1), 253);  // scale 2^(f - 127)
  const float sc = __builtin_bit_cast(float, (uint32_t)f << 23);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
    const uint32_t b[4] = {lv[i].x, lv[i].y, lv[i].z, lv[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v0 = bf16_lo_f32(a[j]) + bf16_lo_f32(b[j]);
      const float v1 = bf16_hi_f32(a[j]) + bf16_hi_f32(b[j]);
      hh[4 * i + j] = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)(v0 * sc), (_Float16)(v1 * sc)});
    }
  }
  return __builtin_bit_cast(float, (uint32_t)(254 - f) << 23);
}

// v plus a DPP lane permutation of v (lanes outside row_mask add 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over each aligned segment of `lpr` lanes (lpr a power of two); the total lands in the
// segment's last lane (lane % lpr == lpr - 1), which is the lane that writes the result.
__device__ __forceinline__ float segment_sum(float v, int lpr) {
  if (lpr >= 2) v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  if (lpr >= 4) v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  if (lpr >= 8) v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  if (lpr >= 16) v = dpp_add<0x140, 0xF>(v); // row_mirror
  if (lpr >= 32) v = dpp_add<0x142, 0xA>(v); // row_bcast15 into rows 1 and 3
  if (lpr >= 64) v = dpp_add<0x143, 0xC>(v); // row_bcast31 into rows 2 and 3
  return v;
}

struct ItemRange {
  int begin, end;  // items [begin, end) of this workgroup
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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
                                         const int32_t* counts, int tiles, int MT, int weighted,
                                         ItemRange& ir) {
  const int lane = threadIdx.x & 63;
  const int n = uniform(*count_ptr);
  if (n <= 0) return false;
  const int G = gridDim.x, b = blockIdx.x;
  if (!weighted) {  // every expert has the same row count: equal item counts, no count loads
    ir.begin = (int)((long)b * n * tiles / G);
    ir.end = (int)((long)(b + 1) * n * tiles / G);
    return ir.begin < ir.end;
  }
  // total cost
  long total = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int c = i < n ? item_cost(counts[list[i]], MT) : 0;
    total += (long)uniform(__shfl(wave_inclusive_scan(c, lane), 63, 64));
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
    run += (long)tiles * uniform(__shfl(scan, 63, 64));
  }
  ir.begin = begin;
  ir.end = end;
  return ir.begin < ir.end;
}

// The workgroup's range, computed by its first wave alone and passed to the others through LDS
// (every wave of the GPU loading the same few lines of the list and the counts at once would queue
// on those lines). Returns false, in every wave, for an empty range.
__device__ __forceinline__ bool my_items_wg(const int32_t* list, const int* count_ptr,
                                            const int32_t* counts, int tiles, int MT, int weighted,
                                            int* shared_range, ItemRange& ir) {
  if (threadIdx.x < 64) {
    ItemRange r{0, 0};
    if (!my_items(list, count_ptr, counts, tiles, MT, weighted, r)) r = ItemRange{0, 0};
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

// 16 bytes / 1 byte at a uniform base plus a 32-bit per-lane offset (lets the compiler use the
// scalar-base addressing form, one VGPR per address)
__device__ __forceinline__ uint4 ld16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint32_t ld8(const uint8_t* base, uint32_t off) { return base[off]; }

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
};

// Expert state of the item being consumed.
struct Current {
  int slot, e, M, row0, a_m0;
};

// Next item of the workgroup's range for this wave (uniform); >= ir.end once the range is drained.
__device__ __forceinline__ int take_item(int* counter, const ItemRange& ir) {
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(counter, 1);
  return ir.begin + uniform(__shfl(v, 0, 64));
}

// ---------------------------------------------------------------------------------------------
// gate_up: an item is S (gate row, up row) slot pairs.

template <int BPL, int MT, int S, int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, 1) void small_gateup_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, int k,
    const int32_t* __restrict__ list, const int32_t* __restrict__ list_count, int H, int I,
    int tiles, int weighted, const uint8_t* __restrict__ w13_q, const uint8_t* __restrict__ w13_s,
    int lpr, float clamp, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
    float* __restrict__ g_ws) {
  constexpr bool kGate = MODE != kUpWithGate;
  constexpr bool kUp = MODE != kGateOnly;
  __shared__ int counter;
  __shared__ int range[2];
  ItemRange ir;
  if (threadIdx.x == 0) counter = 0;
  if (!my_items_wg(list, list_count, counts, tiles, MT, weighted, range, ir)) return;

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
  Prefetch pf{-1, w13_q, w13_s};

  // take an item into ring entry d and issue its loads; rows of a partial last tile are clamped
  // (their results are never stored)
  auto prefetch = [&](int d) {
    ring_item[d] = take_item(&counter, ir);
    const int it = min(ring_item[d], ir.end - 1);
    const int slot = uniform(it / tiles);
    const int tile = uniform(it - slot * tiles);
    if (slot != pf.slot) {
      pf.slot = slot;
      const int e = uniform(list[slot]);
      pf.q = w13_q + (size_t)e * qexp;
      pf.s = w13_s + (size_t)e * sexp;
    }
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
          w[d][s][0][b] = ld16(pf.q, oq);
          sc[d][s][0][b] = ld8(pf.s, os);
        }
        if (kUp) {
          w[d][s][1][b] = ld16(pf.q, oq + up_q);
          sc[d][s][1][b] = ld8(pf.s, os + up_s);
        }
      }
    }
  };

  Current cur{-1, -1, 0, 0, -1};
  uint4 xb[MT][BPL][4];

  auto consume = [&](int d) {
    const int item = ring_item[d];
    const int slot = uniform(item / tiles);
    const int tile = uniform(item - slot * tiles);
    if (slot != cur.slot) {  // new expert
      cur.slot = slot;
      cur.e = uniform(list[slot]);
      cur.M = uniform(counts[cur.e]);
      cur.row0 = uniform(offsets[cur.e]);
      cur.a_m0 = -1;
    }
    const int n0 = tile * tile_rows;
    const bool full = n0 + tile_rows <= I;
    for (int m0 = 0; m0 < cur.M; m0 += MT) {
      const int mc = min(MT, cur.M - m0);
      if (m0 != cur.a_m0) {  // activation slices of this token chunk (L2 hits)
        cur.a_m0 = m0;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int t = uniform(sorted_pair[cur.row0 + m0 + min(m, mc - 1)]) / k;
          const uint8_t* xbase = reinterpret_cast<const uint8_t*>(x + (size_t)t * H);
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
  bool more = true;
  while (more) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (more) {
        if (ring_item[d] >= ir.end) {
          more = false;
        } else {
          consume(d);
          prefetch(d);
        }
      }
    }
  }
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
    const int32_t* __restrict__ list, const int32_t* __restrict__ list_count, int H, int I,
    int tiles, int weighted, const uint8_t* __restrict__ w2_q, const uint8_t* __restrict__ w2_s,
    int lpr, const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo,
    float* __restrict__ y) {
  __shared__ int counter;
  __shared__ int range[2];
  extern __shared__ __attribute__((aligned(16))) uint8_t h_stage[];  // STAGED: hi plane, then lo plane
  ItemRange ir;
  if (threadIdx.x == 0) counter = 0;
  if (!my_items_wg(list, list_count, counts, tiles, MT, weighted, range, ir)) return;

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
  Prefetch pf{-1, w2_q, w2_s};

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
    }
    const int n0 = tile * tile_rows;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t rr = (uint32_t)min(n0 + s * rpw + sub, H - 1);
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const uint32_t kb = (uint32_t)min(q + lpr * b, NB - 1);
        w[d][s][b] = ld16(pf.q, rr * qrow + kb * 16);
        sc[d][s][b] = ld8(pf.s, rr * srow + kb);
      }
    }
  };

  Current cur{-1, -1, 0, 0, -1};
  uint32_t hh[MT][BPL][16];  // h blocks as scaled fp16 pairs
  float hinv[MT][BPL];       // their inverse power-of-two scales

  auto consume = [&](int d) {
    const int item = ring_item[d];
    const int slot = uniform(item / tiles);
    const int tile = uniform(item - slot * tiles);
    if (slot != cur.slot) {
      cur.slot = slot;
      cur.e = uniform(list[slot]);
      cur.M = uniform(counts[cur.e]);
      cur.row0 = uniform(offsets[cur.e]);
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
  bool more = true;
  while (more) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (more) {
        if (ring_item[d] >= ir.end) {
          more = false;
        } else {
          consume(d);
          prefetch(d);
        }
      }
    }
  }
}

template <int MODE>
hipError_t gateup_dispatch(const SmallPlan& sp, const Routed& r, const int32_t* list,
                           const int32_t* list_count, int H, int I, const uint8_t* wq,
                           const uint8_t* ws, float clamp, uint16_t* h_hi, uint16_t* h_lo,
                           float* g_ws, hipStream_t stream) {
  const dim3 grid(sp.gu_grid);
  const int lpr = sp.gu.lpr, tiles = sp.gu_tiles;
#define MOE_GU(BPL, MT)                                                                          \
  small_gateup_kernel<BPL, MT, gateup_slots(BPL), gateup_ring(BPL), 4 * gu_waves(BPL, MT), MODE> \
      <<<grid, 256 * gu_waves(BPL, MT), 0, stream>>>(r.x, r.counts, r.offsets, r.sorted_pair, r.k,   \
                                                     list, list_count, H, I, tiles, sp.weighted, wq, \
                                                     ws, lpr, clamp, h_hi, h_lo, g_ws)
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
  return hipGetLastError();
}

}  // namespace

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
  sp.mt_gu = (T >= 2 && sp.gu.bpl <= 2) ? 2 : 1;
  sp.mt_dn = (T >= 2 && sp.dn.bpl <= 2) ? 2 : 1;
  // with T <= 2 every expert has one or two rows and costs about the same per item
  sp.weighted = T > 2;
  // one workgroup per CU (its waves share the CU's range of items), never more than there can
  // be items
  const long gu_items = (long)sp.slots * sp.gu_tiles, dn_items = (long)sp.slots * sp.dn_tiles;
  sp.gu_grid = (int)(gu_items < num_cus ? gu_items : num_cus);
  sp.dn_grid = (int)(dn_items < num_cus ? dn_items : num_cus);
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

// Bound on the h rows of one down workgroup's range when the list is the whole active list (every
// expert has at most T rows). Weighted ranges hold cost total/G, and an expert inside a range costs
// at least (rows + 3) per item over its items, so the experts wholly inside hold at most 4P/G + 1
// rows (the total cost is at most 4 per row); two more experts can overlap its ends. Equal-count
// ranges span at most ceil(P/G) + 2 experts.
int down_stage_rows(const SmallPlan& sp) {
  const long G = sp.dn_grid > 0 ? sp.dn_grid : 1;
  const long P = sp.P, T = sp.T;
  const long rows = sp.weighted ? 4 * P / G + 1 + 2 * T : ((P + G - 1) / G + 2) * T;
  return (int)(rows < P ? rows : P);
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
    kern<<<grid, 256 * dn_waves(BPL, MT), lds, stream>>>(r.counts, r.offsets, list, list_count, H, I,   \
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

}  // namespace moe
