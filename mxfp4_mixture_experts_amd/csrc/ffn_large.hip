// bf16-MFMA MXFP4 expert GEMMs for experts with many routed rows.
//
// Once an expert has tens of rows its GEMM is a real dense contraction, so it runs on the gfx950
// matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation). The weights stay MXFP4 in HBM and are
// decoded exactly to bf16 with the scaled FP4 conversion right before the MFMA:
//   - a workgroup owns one (expert, tile of up to 64 rows) pair and a block of output columns; its
//     eight waves (two per SIMD, so one wave's MFMAs cover the other's waits) split the columns,
//     every wave covers all rows of the tile;
//   - the activation tile (gathered x rows for gate_up, h rows for down) is staged in LDS, 128 K
//     elements per step, and read by all four waves as MFMA A operands;
//   - each lane loads one 32-element MX block (16 bytes + one scale byte) of one weight row per
//     column block and step, and its decoded 32 bf16 values feed four MFMAs directly as B operands.
//     The reduction order inside a step is a fixed permutation of K, applied identically to A and B,
//     which is all a dot product needs;
//   - gate columns i and up columns I+i of a wave land in the same lanes, so the clamp-SwiGLU
//     epilogue runs in registers; h is written as its two bf16 planes, like the weight-streaming
//     kernels do;
//   - the down GEMM feeds h to the bf16 MFMA as an exact-to-fp32 pair hi + lo (hi = bf16(h),
//     lo = bf16(h - hi)), two MFMAs per operand: a single bf16 rounding of h alone can cost up to
//     ~2% of the output's rms at small I or k (no averaging over many terms), while these medium-M
//     GEMMs are bound by the weight stream, so the extra MFMAs are free.
// Tile schedule: a one-wave kernel lists the (expert, row-tile) pairs of experts above small_m_max
// (and the remaining experts for the weight-streaming kernels) on the device, so the grids come from
// host bounds only and no launch needs a host synchronisation.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTileM = 64;      // rows per tile (4 MFMA row blocks of 16)
constexpr int kDenseRows = 256; // rows per tile of the dense kernels
constexpr int kKStep = 128;     // K elements per step (4 MX blocks)
constexpr int kLdsRow = 272;    // bytes per LDS activation row (256 + 16 padding)

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint4 ld16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint32_t ld8(const uint8_t* base, uint32_t off) { return base[off]; }

// One wave: split the active experts into those for the weight-streaming kernels (at most
// small_m_max rows), the 64-row tiles of those for the row-tile kernels and the 256-row tiles of
// those with at least dense_m_min rows for the dense kernels, in ascending expert order. Unused tail
// entries are -1, so consumers need not read the counts.
__global__ __launch_bounds__(64) void schedule_kernel(const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ active,
                                                      const int32_t* __restrict__ n_active, int E,
                                                      int small_m_max, int tile_slots, int dense_m_min,
                                                      int dense_slots, int32_t* __restrict__ small_list,
                                                      int32_t* __restrict__ n_small,
                                                      int32_t* __restrict__ tile_e,
                                                      int32_t* __restrict__ tile_m0,
                                                      int32_t* __restrict__ dense_e,
                                                      int32_t* __restrict__ dense_m0) {
  const int lane = threadIdx.x;
  const int na = *n_active;
  int ns = 0, nt = 0, nd = 0;
  for (int i0 = 0; i0 < na; i0 += 64) {
    const int i = i0 + lane;
    const int e = i < na ? active[i] : -1;
    const int c = e >= 0 ? counts[e] : 0;
    const bool small = e >= 0 && c <= small_m_max;
    const bool dense = e >= 0 && !small && c >= dense_m_min;
    const uint64_t sm = __ballot(small);
    if (small) small_list[ns + __popcll(sm & lanemask_lt(lane))] = e;
    ns += __popcll(sm);
    const int tiles = (e >= 0 && !small && !dense) ? (c + kTileM - 1) / kTileM : 0;
    const int incl = wave_inclusive_scan(tiles, lane);
    for (int t = 0; t < tiles; ++t) {
      const int slot = nt + incl - tiles + t;
      if (slot < tile_slots) {
        tile_e[slot] = e;
        tile_m0[slot] = t * kTileM;
      }
    }
    nt += wave_last(incl);
    const int dtiles = dense ? (c + kDenseRows - 1) / kDenseRows : 0;
    const int dincl = wave_inclusive_scan(dtiles, lane);
    for (int t = 0; t < dtiles; ++t) {
      const int slot = nd + dincl - dtiles + t;
      if (slot < dense_slots) {
        dense_e[slot] = e;
        dense_m0[slot] = t * kDenseRows;
      }
    }
    nd += wave_last(dincl);
  }
  for (int i = ns + lane; i < E; i += 64) small_list[i] = -1;
  for (int i = nt + lane; i < tile_slots; i += 64) tile_e[i] = -1;
  for (int i = nd + lane; i < dense_slots; i += 64) dense_e[i] = -1;
  if (lane == 0) *n_small = ns;
}

// Ring depth, in super-steps of two K-steps, by tile height: the fewer MFMAs a step holds, the more
// steps must be in flight to cover the memory latency with one workgroup per CU (as deep as the
// register file allows at two waves per SIMD).
constexpr int ring_depth(bool gateup, int msub) { return msub <= 3 ? 2 : 1; }

constexpr int kNW = 8;           // waves per workgroup (2 per SIMD)
constexpr int kThreads = 64 * kNW;

// Per-wave LDS buffer of one super-step's weights: CB column blocks x 16 rows x 128 bytes of codes
// (8 MX blocks), then the scale bytes: CB x 16 rows x 8 (one super-step), or with WIN, CB x 16 rows x
// 32 (a window of four super-steps).
template <int CB, bool WIN>
constexpr int wave_buf_bytes() { return CB * 2048 + CB * (WIN ? 512 : 128); }

// One (expert, row tile) x column block, with MSUB blocks of 16 rows fixed at compile time so the
// step is straight-line code (no per-row-block branches between MFMAs).
// Staging: gate_up stages MSUB*16 rows x 128 bf16 of gathered x per K-step (16-byte chunks, spread
// over the workgroup's threads; rows past the tile repeat its last row); down stages MSUB*16 rows x
// 128 of both bf16 planes of h (hi, lo) into two LDS tiles.
// Weights: the 16 weight rows of a column block are loaded per super-step (two K-steps, 8 MX blocks)
// as two 1 KB reads of 8 rows x 128 contiguous bytes (lane l: row 8h + l/8, block l%8), so every
// load instruction covers 8 whole cache lines; at use the wave passes them through its own LDS
// buffer into the MFMA lane layout (lane: row j16, block 4*step + g). Only the wave itself reads its
// buffer, so this needs no barrier.
// Scale bytes: without WIN a lane loads the one byte it writes to the buffer, per super-step, so each
// 32-byte sector of a row's scales is requested four times, a super-step apart, and the L2 serves
// few of those repeats (under the weight stream the counters showed the gate_up launch fetching 42%
// more than its weights and scales, and pointing every scale load at one sector took high_c4's
// gate_up from 1100 to 920 us). With WIN (K % 256 == 0) a lane loads 8 bytes of one row, and the
// wave the 32-byte windows of its 16 rows for four super-steps at once: every sector is fetched by
// one load.
template <bool GATEUP, int MSUB, int CB, bool WIN>
__device__ __forceinline__ void large_tile(const Routed& r, int H, int I, const uint8_t* __restrict__ qe,
                                           const uint8_t* __restrict__ se, int e, int m0, int xblk,
                                           float clamp, const uint16_t* __restrict__ h_hi_in,
                                           const uint16_t* __restrict__ h_lo_in,
                                           uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
                                           float* __restrict__ y_out, uint8_t* lds_a, uint8_t* lds_w) {
  constexpr int D = ring_depth(GATEUP, MSUB);
  constexpr int kATiles = GATEUP ? 1 : 2;  // bf16 x, or bf16 hi + lo of h
  constexpr int kTileBytes = kTileM * kLdsRow;
  // 16-byte chunks per thread and K-step: MSUB*16 rows of 16 (bf16 x) or 2 x 16 (h planes) chunks
  constexpr int NA = GATEUP ? (MSUB * 256 + kThreads - 1) / kThreads : (MSUB * 512 + kThreads - 1) / kThreads;

  const int rows = min(kTileM, uniform(r.counts[e]) - m0);
  const int row0 = uniform(r.offsets[e]) + m0;
  const int K = GATEUP ? H : I;  // reduction length
  const int NB = K >> 5;
  const uint32_t qrow = (uint32_t)(K >> 1), srow = (uint32_t)NB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j16 = lane & 15;  // MFMA column (weight row) / A row within a 16-block
  const int g = lane >> 4;    // K group: this lane's block within a step is 4*step + g

  // weight row (within the expert) of row j (0..15) of column block cb (gate_up: CB/2 gate blocks,
  // then the matching up blocks), and the column it gives; columns past the end are clamped
  auto col_of = [&](int cb, int j) {
    return GATEUP ? xblk * (kNW * 8 * CB) + wave * (8 * CB) + (cb % (CB / 2)) * 16 + j
                  : xblk * (kNW * 16 * CB) + wave * (16 * CB) + cb * 16 + j;
  };
  auto wrow_of = [&](int cb, int j) {
    const int c = col_of(cb, j);
    return GATEUP ? ((cb < CB / 2) ? min(c, I - 1) : I + min(c, I - 1)) : min(c, H - 1);
  };
  int col[CB];
  bool cval[CB];
  uint32_t cq[CB][2], cs[CB][2];  // offsets of the rows this lane loads (coalesced pattern)
  uint32_t cw[CB];                // WIN: scale-row offset of row lane / 4 of each column block
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    col[cb] = col_of(cb, j16);
    cval[cb] = col[cb] < (GATEUP ? I : H);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t wrow = (uint32_t)wrow_of(cb, 8 * h + (lane >> 3));
      cq[cb][h] = wrow * qrow;
      cs[cb][h] = wrow * srow;
    }
    cw[cb] = (uint32_t)wrow_of(cb, lane >> 2) * srow;
  }

  // activation rows this thread stages (rows past the tile repeat its last row: their results
  // are never written)
  const uint8_t* arow[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int ch = tid + kThreads * i;
    const int lr = min(GATEUP ? ch >> 4 : ch >> 5, rows - 1);
    if (GATEUP) {
      const int t = r.sorted_pair[row0 + lr] / r.k;
      arow[i] = reinterpret_cast<const uint8_t*>(r.x + (size_t)t * H);
    } else {
      const uint16_t* plane = ((ch >> 4) & 1) ? h_lo_in : h_hi_in;
      arow[i] = reinterpret_cast<const uint8_t*>(plane + (size_t)(row0 + lr) * I);
    }
  }

  const int nsteps = (NB + 3) >> 2;
  const int nss = (nsteps + 1) >> 1;  // super-steps
  // ring of D super-steps of loads in flight: weight blocks, scale bytes, activation slices
  uint4 rb[D][CB][2];
  uint32_t rs[D][CB][2];
  uint2 sw[CB];  // WIN: the next window's scale bytes
  uint4 ra[D][2][NA];

  // issue every load of super-step ss into ring slot `slot`. Block and element indices are clamped
  // into the row: a partial last step re-reads in-bounds data that is masked at use, and the steps
  // past the end re-read the last step (L2 hits spread over the channels; no branch around the loads).
  auto issue = [&](int slot, int ss) {
    const uint32_t blk = (uint32_t)min(ss * 8 + (lane & 7), NB - 1);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        rb[slot][cb][h] = ld16(qe, cq[cb][h] + blk * 16);
        if constexpr (!WIN) rs[slot][cb][h] = ld8(se, cs[cb][h] + blk);
      }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const uint32_t el = (uint32_t)min((2 * ss + st) * 128 + (tid & 15) * 8, K - 8);
        ra[slot][st][i] = ld16(arow[i], el * 2);
      }
  };

  // WIN: scale bytes of super-steps ss .. ss + 3 (blocks 8 ss .. 8 ss + 31; clamped into the row,
  // blocks past K are masked at use)
  auto issue_window = [&](int ss) {
    const uint32_t blk = (uint32_t)min(ss * 8 + (lane & 3) * 8, NB - 8);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sw[cb] = *reinterpret_cast<const uint2*>(se + cw[cb] + blk);
  };

  f32x4_t acc[MSUB][CB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[ms][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (WIN) issue_window(0);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);

  // this wave's buffer: row r of column block cb at cb*2048 + r*128, its 16-byte chunk c at position
  // c ^ (r % 8) (the 8 lanes writing a row, and the 8 lanes reading one chunk of 8 rows, hit
  // distinct banks); scale bytes at CB*2048 + cb*128 + r*8 + block
  uint8_t* wbuf = lds_w + wave * wave_buf_bytes<CB, WIN>();

  auto step_body = [&](int slot, int step, int st) {
    uint8_t* lb = lds_a + (step & 1) * (kATiles * kTileBytes);
    // the step's activation slice goes to LDS (zero past K), visible after the barrier
    const bool k_tail = (step * 4 + 4) > NB;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (GATEUP) {
        const int ch = tid + kThreads * i;
        const int lr = ch >> 4, c16 = ch & 15;
        uint4 v = ra[slot][st][i];
        if (k_tail && step * 128 + c16 * 8 >= K) v = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(lb + lr * kLdsRow + c16 * 16) = v;
      } else {
        const int ch = tid + kThreads * i;
        const int lr = ch >> 5, pl = (ch >> 4) & 1, c16 = ch & 15;
        uint4 v = ra[slot][st][i];
        if (k_tail && step * 128 + c16 * 8 >= K) v = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(lb + pl * kTileBytes + lr * kLdsRow + c16 * 16) = v;
      }
    }
    __syncthreads();
    // this lane's weight block of the step (row j16, block 4*st + g) from the wave's buffer
    uint4 wb[CB];
    float scale[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = 4 * st + g;
      wb[cb] = *reinterpret_cast<const uint4*>(wbuf + cb * 2048 + j16 * 128 + ((c ^ (j16 & 7)) << 4));
      const bool ok = cval[cb] && step * 4 + g < NB;
      const int so = WIN ? CB * 2048 + cb * 512 + j16 * 32 + ((step >> 1) & 3) * 8 + c
                         : CB * 2048 + cb * 128 + j16 * 8 + c;
      scale[cb] = ok ? e8m0_to_float(wbuf[so]) : 0.0f;
    }
    // decode the weight blocks straight into MFMA B operands (operand s = elements 8s..8s+7)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t aop[kATiles][MSUB];
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int at = 0; at < kATiles; ++at)
          aop[at][ms] = *reinterpret_cast<const bf16x8_t*>(lb + at * kTileBytes +
                                                            (ms * 16 + j16) * kLdsRow + g * 64 + s * 16);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t wd = s == 0 ? wb[cb].x : s == 1 ? wb[cb].y : s == 2 ? wb[cb].z : wb[cb].w;
        const bf16x2_t p0 = fp4x2_to_bf16x2<0>(wd, scale[cb]);
        const bf16x2_t p1 = fp4x2_to_bf16x2<1>(wd, scale[cb]);
        const bf16x2_t p2 = fp4x2_to_bf16x2<2>(wd, scale[cb]);
        const bf16x2_t p3 = fp4x2_to_bf16x2<3>(wd, scale[cb]);
        const bf16x8_t bop = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
          for (int at = 0; at < kATiles; ++at)
            acc[ms][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[at][ms], bop, acc[ms][cb], 0, 0, 0);
      }
      // keep the decode of the next operand group below these MFMAs (hoisting all of a step's
      // decodes ahead would hold 16 more B operands live and spill at two waves per SIMD)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // WINDOW_START: ss is the first super-step of a scale window (known at compile time below)
  auto super_step = [&](int slot, int ss, auto window_start, auto window_issue) {
    // the super-step's weights -> this wave's buffer (the wave finished reading the previous
    // super-step's; its LDS operations complete in order)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rr = 8 * h + (lane >> 3), c = lane & 7;
        *reinterpret_cast<uint4*>(wbuf + cb * 2048 + rr * 128 + ((c ^ (rr & 7)) << 4)) = rb[slot][cb][h];
        if constexpr (!WIN) wbuf[CB * 2048 + cb * 128 + rr * 8 + c] = (uint8_t)rs[slot][cb][h];
      }
    if constexpr (WIN && decltype(window_start)::value) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<uint2*>(wbuf + CB * 2048 + cb * 512 + (lane >> 2) * 32 + (lane & 3) * 8) = sw[cb];
    }
    step_body(slot, 2 * ss, 0);
    step_body(slot, 2 * ss + 1, 1);
    // the slot's registers are consumed: refill it with super-step ss + D (and, when that starts a
    // window, load the window)
    if constexpr (WIN && decltype(window_issue)::value) issue_window(ss + D);
    issue(slot, ss + D);
  };

  // the super-step count is padded to a multiple of 4 (of D, and of the scale window; padding steps
  // see zero activations and zero scales): a conditional tail would merge into the loop's control
  // flow and make the compiler count the newest ring slot's loads as needed by the oldest one
  const int nss_pad = (nss + 3) / 4 * 4;
  using T0 = std::integral_constant<bool, true>;
  using F0 = std::integral_constant<bool, false>;
  for (int ss = 0; ss < nss_pad; ss += 4) {
    super_step(0, ss, T0{}, std::integral_constant<bool, D == 4>{});
    super_step(1 % D, ss + 1, F0{}, std::integral_constant<bool, 1 + D == 4>{});
    super_step(2 % D, ss + 2, F0{}, std::integral_constant<bool, 2 + D == 4>{});
    super_step(3 % D, ss + 3, F0{}, std::integral_constant<bool, 3 + D == 4>{});
  }

  // epilogue: lane holds rows 4*g + i (i < 4) of each 16-row block, column j16 of each block
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = ms * 16 + g * 4 + i;
      if (lr >= rows) continue;
      const size_t orow = (size_t)(row0 + lr);
      if (GATEUP) {
#pragma unroll
        for (int cb = 0; cb < CB / 2; ++cb) {
          if (!cval[cb]) continue;
          float gv = acc[ms][cb][i];
          float uv = acc[ms][cb + CB / 2][i];
          if (clamp > 0.0f) {
            gv = clampf(gv, clamp);
            uv = clampf(uv, clamp);
          }
          store_h_planes(h_hi, h_lo, orow * I + col[cb], silu_mul(gv, uv));
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          if (cval[cb]) y_out[orow * H + col[cb]] = acc[ms][cb][i];
      }
    }
  }
}

// Grid: 8 * nx * ceil(tile_slots / 8) one-dimensional workgroups. Consecutive workgroups go to the
// 8 XCDs in turn, so workgroup b runs on XCD b % 8; the mapping below gives XCD x the row tiles
// y = x, x + 8, ... and dispatches all nx column blocks of one tile back to back on it, so a tile's
// activation rows are fetched into that XCD's L2 once and reused by every column block.
template <bool GATEUP, int CB, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void large_kernel(Routed r, int H, int I, int nx, int tile_slots,
                                                       const uint8_t* __restrict__ wq_all,
                                                       const uint8_t* __restrict__ ws_all,
                                                       const int32_t* __restrict__ tile_e,
                                                       const int32_t* __restrict__ tile_m0,
                                                       float clamp,
                                                       const uint16_t* __restrict__ h_hi_in,
                                                       const uint16_t* __restrict__ h_lo_in,
                                                       uint16_t* __restrict__ h_hi,
                                                       uint16_t* __restrict__ h_lo,
                                                       float* __restrict__ y_out) {
  constexpr int kATiles = GATEUP ? 1 : 2;
  // two LDS buffers (double-buffered across K-steps), each kATiles tiles
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * kATiles * kTileM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[kNW * wave_buf_bytes<CB, WIN>()];

  const int b = blockIdx.x;
  const int j = b >> 3;
  const int y = (b & 7) + 8 * (j / nx);
  const int xblk = j % nx;
  if (y >= tile_slots) return;
  const int te = tile_e[y];
  if (te < 0) return;
  const int e = uniform(te);
  const int m0 = uniform(tile_m0[y]);
  const int rows = min(kTileM, uniform(r.counts[e]) - m0);
  const int msub_n = (rows + 15) >> 4;

  const int K = GATEUP ? H : I;
  const size_t nrows_w = GATEUP ? (size_t)2 * I : (size_t)H;
  const uint8_t* qe = wq_all + (size_t)e * nrows_w * (size_t)(K >> 1);
  const uint8_t* se = ws_all + (size_t)e * nrows_w * (size_t)(K >> 5);
#define MOE_TILE(MS) \
  large_tile<GATEUP, MS, CB, WIN>(r, H, I, qe, se, e, m0, xblk, clamp, h_hi_in, h_lo_in, h_hi, h_lo, y_out, \
                                  lds_a, lds_w)
  switch (msub_n) {
    case 1: MOE_TILE(1); break;
    case 2: MOE_TILE(2); break;
    case 3: MOE_TILE(3); break;
    default: MOE_TILE(4); break;
  }
#undef MOE_TILE
}

constexpr int kGuCB = 4;  // gate_up: 4 column blocks per wave (2 gate + 2 up)
constexpr int kDnCB = 4;  // down: 4 column blocks per wave

}  // namespace

LargePlan plan_large(int T, int H, int I, int E, int k, int small_m_max) {
  LargePlan lp;
  lp.tile_m = kTileM;
  lp.gu_tile_n = kNW * 8 * kGuCB;
  lp.dn_tile_n = kNW * 16 * kDnCB;
  lp.gu_grid_x = (I + lp.gu_tile_n - 1) / lp.gu_tile_n;
  lp.dn_grid_x = (H + lp.dn_tile_n - 1) / lp.dn_tile_n;
  lp.tile_slots = tile_slots_bound(T, E, k, small_m_max);
  const int groups = (lp.tile_slots + 7) / 8;
  lp.gu_blocks = 8 * lp.gu_grid_x * groups;
  lp.dn_blocks = 8 * lp.dn_grid_x * groups;
  return lp;
}

int tile_slots_bound(int T, int E, int k, int small_m_max) {
  // sum over experts above the threshold of ceil(M_e / 64) <= P/64 + (number of such experts)
  const long P = (long)T * k;
  long n_large = P / ((long)small_m_max + 1);
  if (n_large > E) n_large = E;
  return (int)((P + kTileM - 1) / kTileM + n_large);
}

hipError_t launch_schedule(const Routed& r, int E, int small_m_max, int tile_slots, int dense_m_min,
                           int dense_slots, int32_t* small_list, int32_t* n_small, int32_t* tile_e,
                           int32_t* tile_m0, int32_t* dense_e, int32_t* dense_m0, hipStream_t stream) {
  schedule_kernel<<<1, 64, 0, stream>>>(r.counts, r.active, r.n_active, E, small_m_max, tile_slots,
                                        dense_m_min, dense_slots, small_list, n_small, tile_e, tile_m0,
                                        dense_e, dense_m0);
  return hipGetLastError();
}

hipError_t launch_large_gateup(const LargePlan& lp, const Routed& r, int H, int I,
                               const uint8_t* w13_q, const uint8_t* w13_s, const int32_t* tile_e,
                               const int32_t* tile_m0, float clamp, uint16_t* h_hi, uint16_t* h_lo,
                               hipStream_t stream) {
  if (lp.tile_slots <= 0) return hipSuccess;
  if (H % 256 == 0)
    large_kernel<true, kGuCB, true><<<lp.gu_blocks, kThreads, 0, stream>>>(
        r, H, I, lp.gu_grid_x, lp.tile_slots, w13_q, w13_s, tile_e, tile_m0, clamp, nullptr, nullptr, h_hi,
        h_lo, nullptr);
  else
    large_kernel<true, kGuCB, false><<<lp.gu_blocks, kThreads, 0, stream>>>(
        r, H, I, lp.gu_grid_x, lp.tile_slots, w13_q, w13_s, tile_e, tile_m0, clamp, nullptr, nullptr, h_hi,
        h_lo, nullptr);
  return hipGetLastError();
}

hipError_t launch_large_down(const LargePlan& lp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* tile_e, const int32_t* tile_m0,
                             const uint16_t* h_hi, const uint16_t* h_lo, float* y, hipStream_t stream) {
  if (lp.tile_slots <= 0) return hipSuccess;
  if (I % 256 == 0)
    large_kernel<false, kDnCB, true><<<lp.dn_blocks, kThreads, 0, stream>>>(
        r, H, I, lp.dn_grid_x, lp.tile_slots, w2_q, w2_s, tile_e, tile_m0, 0.0f, h_hi, h_lo, nullptr, nullptr,
        y);
  else
    large_kernel<false, kDnCB, false><<<lp.dn_blocks, kThreads, 0, stream>>>(
        r, H, I, lp.dn_grid_x, lp.tile_slots, w2_q, w2_s, tile_e, tile_m0, 0.0f, h_hi, h_lo, nullptr, nullptr,
        y);
  return hipGetLastError();
}

}  // namespace moe
