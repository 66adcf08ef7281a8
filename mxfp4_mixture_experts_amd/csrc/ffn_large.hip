// bf16-MFMA MXFP4 expert GEMMs for experts with many routed rows.
//
// Once an expert has tens of rows its GEMM is a real dense contraction, so it runs on the gfx950
// matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation). The weights stay MXFP4 in HBM and are
// decoded exactly to bf16 with the scaled FP4 conversion right before the MFMA:
//   - a workgroup owns one (expert, tile of up to 64 rows) pair and a block of output columns; the
//     four waves split the columns, every wave covers all rows of the tile;
//   - the activation tile (gathered x rows for gate_up, h rows for down) is staged in LDS, 128 K
//     elements per step, and read by all four waves as MFMA A operands;
//   - each lane loads one 32-element MX block (16 bytes + one scale byte) of one weight row per
//     column block and step, and its decoded 32 bf16 values feed four MFMAs directly as B operands.
//     The reduction order inside a step is a fixed permutation of K, applied identically to A and B,
//     which is all a dot product needs;
//   - gate columns i and up columns I+i of a wave land in the same lanes, so the clamp-SwiGLU
//     epilogue runs in registers; h is written in fp32, like the weight-streaming kernels do;
//   - the down GEMM feeds h to the bf16 MFMA as an exact-to-fp32 pair hi + lo (hi = bf16(h),
//     lo = bf16(h - hi)), two MFMAs per operand: a single bf16 rounding of h alone can cost up to
//     ~2% of the output's rms at small I or k (no averaging over many terms), while these medium-M
//     GEMMs are bound by the weight stream, so the extra MFMAs are free.
// Tile schedule: a one-wave kernel lists the (expert, row-tile) pairs of experts above small_m_max
// (and the remaining experts for the weight-streaming kernels) on the device, so the grids come from
// host bounds only and no launch needs a host synchronisation.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTileM = 64;      // rows per tile (4 MFMA row blocks of 16)
constexpr int kKStep = 128;     // K elements per step (4 MX blocks)
constexpr int kLdsRow = 272;    // bytes per LDS activation row (256 + 16 padding)
constexpr int kColBlocks = 4;   // 16-column MFMA blocks per wave

// One wave: split the active experts into those for the weight-streaming kernels (at most
// small_m_max rows) and the row tiles of the others, in ascending expert order. Unused tail entries
// are -1, so consumers need not read the counts.
__global__ __launch_bounds__(64) void schedule_kernel(const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ active,
                                                      const int32_t* __restrict__ n_active, int E,
                                                      int small_m_max, int tile_slots,
                                                      int32_t* __restrict__ small_list,
                                                      int32_t* __restrict__ n_small,
                                                      int32_t* __restrict__ tile_e,
                                                      int32_t* __restrict__ tile_m0) {
  const int lane = threadIdx.x;
  const int na = *n_active;
  int ns = 0, nt = 0;
  for (int i0 = 0; i0 < na; i0 += 64) {
    const int i = i0 + lane;
    const int e = i < na ? active[i] : -1;
    const int c = e >= 0 ? counts[e] : 0;
    const bool small = e >= 0 && c <= small_m_max;
    const uint64_t sm = __ballot(small);
    if (small) small_list[ns + __popcll(sm & lanemask_lt(lane))] = e;
    ns += __popcll(sm);
    const int tiles = (e >= 0 && !small) ? (c + kTileM - 1) / kTileM : 0;
    const int incl = wave_inclusive_scan(tiles, lane);
    for (int t = 0; t < tiles; ++t) {
      const int slot = nt + incl - tiles + t;
      if (slot < tile_slots) {
        tile_e[slot] = e;
        tile_m0[slot] = t * kTileM;
      }
    }
    nt += __shfl(incl, 63, 64);
  }
  for (int i = ns + lane; i < E; i += 64) small_list[i] = -1;
  for (int i = nt + lane; i < tile_slots; i += 64) tile_e[i] = -1;
  if (lane == 0) *n_small = ns;
}

template <bool GATEUP>
__global__ __launch_bounds__(256) void large_kernel(Routed r, int H, int I,
                                                    const uint8_t* __restrict__ wq_all,
                                                    const uint8_t* __restrict__ ws_all,
                                                    const int32_t* __restrict__ tile_e,
                                                    const int32_t* __restrict__ tile_m0, float clamp,
                                                    const float* __restrict__ h_in,
                                                    float* __restrict__ h_out,
                                                    float* __restrict__ y_out) {
  // gate_up: one bf16 tile of gathered x rows; down: h split into a hi and a lo bf16 tile
  constexpr int kATiles = GATEUP ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kATiles * kTileM * kLdsRow];

  struct {
    int e, m0, rows;
  } tr;
  tr.e = tile_e[blockIdx.y];
  if (tr.e < 0) return;
  tr.m0 = tile_m0[blockIdx.y];
  tr.rows = min(kTileM, r.counts[tr.e] - tr.m0);
  const int row0 = r.offsets[tr.e] + tr.m0;
  const int msub_n = (tr.rows + 15) >> 4;

  const int K = GATEUP ? H : I;      // reduction length
  const int NB = K >> 5;
  const int NCOL = GATEUP ? I : H;   // output columns (gate columns for gate_up)
  const size_t qrow = (size_t)(K >> 1), srow = (size_t)NB;
  const size_t nrows_w = GATEUP ? (size_t)2 * I : (size_t)H;
  const uint8_t* qe = wq_all + (size_t)tr.e * nrows_w * qrow;
  const uint8_t* se = ws_all + (size_t)tr.e * nrows_w * srow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j16 = lane & 15;   // MFMA column / row within a 16-block
  const int g = lane >> 4;     // K group: block (4*step + g)

  // output columns of this wave's four column blocks, and the weight row each lane loads for them
  int col[kColBlocks];
  int wrow[kColBlocks];
  bool cval[kColBlocks];
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb) {
    if (GATEUP) {
      const int gc = blockIdx.x * 128 + wave * 32 + (cb & 1) * 16 + j16;  // gate column
      col[cb] = gc;
      cval[cb] = gc < I;
      const int gcc = min(gc, I - 1);
      wrow[cb] = (cb < 2) ? gcc : I + gcc;
    } else {
      const int c = blockIdx.x * 256 + wave * 64 + cb * 16 + j16;
      col[cb] = c;
      cval[cb] = c < H;
      wrow[cb] = min(c, H - 1);
    }
  }

  // activation rows this thread stages. gate_up: idx = tid + 256*i (i < 4) -> row idx/16, 8 bf16 of
  // x at column chunk idx%16; down: idx = tid + 256*i (i < 8) -> row idx/32, 4 fp32 of h at idx%32.
  constexpr int kStage = GATEUP ? 4 : 8;
  const uint16_t* xrow[kStage];
  const float* hrow[kStage];
  bool aval[kStage];
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int lr = GATEUP ? (tid + 256 * i) >> 4 : (tid + 256 * i) >> 5;
    aval[i] = lr < tr.rows;
    const int lrc = min(lr, tr.rows - 1);
    if (GATEUP) {
      xrow[i] = r.x + (size_t)(r.sorted_pair[row0 + lrc] / r.k) * (size_t)H;
      hrow[i] = nullptr;
    } else {
      hrow[i] = h_in + (size_t)(row0 + lrc) * (size_t)I;
      xrow[i] = nullptr;
    }
  }

  f32x4_t acc[4][kColBlocks];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) acc[ms][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (NB + 3) >> 2;
  uint4 wnext[kColBlocks];
  uint32_t snext[kColBlocks];
  auto load_b = [&](int step) {
    const int kb_raw = step * 4 + g;
    const int kb = min(kb_raw, NB - 1);  // unconditional in-bounds loads, zeroed below if unused
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      wnext[cb] = *reinterpret_cast<const uint4*>(qe + (size_t)wrow[cb] * qrow + (size_t)kb * 16);
      snext[cb] = (uint32_t)se[(size_t)wrow[cb] * srow + kb];
    }
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb)
      if (!(cval[cb] && kb_raw < NB)) wnext[cb] = make_uint4(0, 0, 0, 0);
  };
  load_b(0);

  for (int step = 0; step < nsteps; ++step) {
    // stage the activation tile(s) of this step
    __syncthreads();
    if (GATEUP) {
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        const int idx = tid + 256 * i;
        const int lr = idx >> 4, c16 = idx & 15;
        const int kelem = step * kKStep + c16 * 8;
        uint4 v = *reinterpret_cast<const uint4*>(xrow[i] + min(kelem, K - 8));
        if (!(aval[i] && kelem < K)) v = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(lds_a + lr * kLdsRow + c16 * 16) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        const int idx = tid + 256 * i;
        const int lr = idx >> 5, c4 = idx & 31;
        const int kelem = step * kKStep + c4 * 4;
        float4 v = *reinterpret_cast<const float4*>(hrow[i] + min(kelem, K - 4));
        if (!(aval[i] && kelem < K)) v = make_float4(0.f, 0.f, 0.f, 0.f);
        const uint16_t h0 = f32_to_bf16_rne(v.x), h1 = f32_to_bf16_rne(v.y);
        const uint16_t h2 = f32_to_bf16_rne(v.z), h3 = f32_to_bf16_rne(v.w);
        auto up = [](uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); };
        uint2 hi, lo;
        hi.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
        hi.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
        lo.x = pack_bf16x2(v.x - up(h0), v.y - up(h1));
        lo.y = pack_bf16x2(v.z - up(h2), v.w - up(h3));
        *reinterpret_cast<uint2*>(lds_a + lr * kLdsRow + c4 * 8) = hi;
        *reinterpret_cast<uint2*>(lds_a + kTileM * kLdsRow + lr * kLdsRow + c4 * 8) = lo;
      }
    }
    uint4 wcur[kColBlocks];
    uint32_t scur[kColBlocks];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      wcur[cb] = wnext[cb];
      scur[cb] = snext[cb];
    }
    if (step + 1 < nsteps) load_b(step + 1);
    __syncthreads();

    // decode this step's weight blocks into MFMA B operands: operand s = elements 8s..8s+7
    bf16x8_t bop[kColBlocks][4];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const float scale = e8m0_to_float(scur[cb]);
      const uint32_t wd[4] = {wcur[cb].x, wcur[cb].y, wcur[cb].z, wcur[cb].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x2_t p0 = fp4x2_to_bf16x2<0>(wd[s], scale);
        const bf16x2_t p1 = fp4x2_to_bf16x2<1>(wd[s], scale);
        const bf16x2_t p2 = fp4x2_to_bf16x2<2>(wd[s], scale);
        const bf16x2_t p3 = fp4x2_to_bf16x2<3>(wd[s], scale);
        bop[cb][s] = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    }
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      if (ms >= msub_n) break;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int at = 0; at < kATiles; ++at) {
          const bf16x8_t aop = *reinterpret_cast<const bf16x8_t*>(
              lds_a + at * kTileM * kLdsRow + (ms * 16 + j16) * kLdsRow + g * 64 + s * 16);
#pragma unroll
          for (int cb = 0; cb < kColBlocks; ++cb)
            acc[ms][cb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[cb][s], acc[ms][cb], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: lane holds rows 4*g + i (i < 4) of each 16-row block, column j16 of each column block
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    if (ms >= msub_n) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = ms * 16 + g * 4 + i;
      if (lr >= tr.rows) continue;
      const size_t orow = (size_t)(row0 + lr);
      if (GATEUP) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          if (!cval[cb]) continue;
          float gv = acc[ms][cb][i];
          float uv = acc[ms][cb + 2][i];
          if (clamp > 0.0f) {
            gv = clampf(gv, clamp);
            uv = clampf(uv, clamp);
          }
          h_out[orow * I + col[cb]] = silu_mul(gv, uv);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb)
          if (cval[cb]) y_out[orow * H + col[cb]] = acc[ms][cb][i];
      }
    }
  }
}

}  // namespace

LargePlan plan_large(int T, int H, int I, int E, int k, int small_m_max) {
  LargePlan lp;
  lp.tile_m = kTileM;
  lp.gu_tile_n = 128;
  lp.dn_tile_n = 256;
  lp.gu_grid_x = (I + lp.gu_tile_n - 1) / lp.gu_tile_n;
  lp.dn_grid_x = (H + lp.dn_tile_n - 1) / lp.dn_tile_n;
  lp.tile_slots = tile_slots_bound(T, E, k, small_m_max);
  return lp;
}

int tile_slots_bound(int T, int E, int k, int small_m_max) {
  // sum over experts above the threshold of ceil(M_e / 64) <= P/64 + (number of such experts)
  const long P = (long)T * k;
  long n_large = P / ((long)small_m_max + 1);
  if (n_large > E) n_large = E;
  return (int)((P + kTileM - 1) / kTileM + n_large);
}

hipError_t launch_schedule(const Routed& r, int E, int small_m_max, int tile_slots, int32_t* small_list,
                           int32_t* n_small, int32_t* tile_e, int32_t* tile_m0, hipStream_t stream) {
  schedule_kernel<<<1, 64, 0, stream>>>(r.counts, r.active, r.n_active, E, small_m_max, tile_slots,
                                        small_list, n_small, tile_e, tile_m0);
  return hipGetLastError();
}

hipError_t launch_large_gateup(const LargePlan& lp, const Routed& r, int H, int I,
                               const uint8_t* w13_q, const uint8_t* w13_s, const int32_t* tile_e,
                               const int32_t* tile_m0, float clamp, float* h, hipStream_t stream) {
  if (lp.tile_slots <= 0) return hipSuccess;
  const dim3 grid(lp.gu_grid_x, lp.tile_slots), block(256);
  large_kernel<true><<<grid, block, 0, stream>>>(r, H, I, w13_q, w13_s, tile_e, tile_m0, clamp,
                                                 nullptr, h, nullptr);
  return hipGetLastError();
}

hipError_t launch_large_down(const LargePlan& lp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* tile_e, const int32_t* tile_m0,
                             const float* h, float* y, hipStream_t stream) {
  if (lp.tile_slots <= 0) return hipSuccess;
  const dim3 grid(lp.dn_grid_x, lp.tile_slots), block(256);
  large_kernel<false><<<grid, block, 0, stream>>>(r, H, I, w2_q, w2_s, tile_e, tile_m0, 0.0f, h,
                                                  nullptr, y);
  return hipGetLastError();
}

}  // namespace moe
