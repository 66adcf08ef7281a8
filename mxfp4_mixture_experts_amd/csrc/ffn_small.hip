// Weight-streaming MXFP4 expert GEMMs for experts with few routed rows (decode).
//
// At small per-expert M the expert GEMMs are bound by HBM bandwidth ("Chunk 8.0": the small
// per-expert GEMMs are memory-bandwidth-bound; "MTP1 Post-Portfolio Eager-Cycle Profile": the compact
// routed MXFP4 GEMM is the largest open kernel family at M=2). Every weight byte is used by at most
// a handful of rows, so these kernels are organised around streaming the expert's packed weights
// once, at full width:
//   - each lane loads whole 32-element MX blocks: 16 bytes of E2M1 codes (one 128-bit load, a wave
//     load covering up to 1 KB of consecutive bytes of a row) and the block's E8M0 scale byte;
//   - a row of K elements is split over `lpr` lanes (in-wave split-K), each owning fixed blocks, so
//     the lane's slice of the activations is loaded into registers once and reused for every row;
//   - the codes are decoded in registers with the gfx950 scaled FP4 conversion (two codes and the
//     scale per instruction) and consumed by bf16 dot2 (gate/up; products exact in fp32) or fp32 FMA
//     (down, whose activations h are fp32);
//   - partial sums are reduced across the row's lanes with a butterfly, deterministically;
//   - gate row i and up row I+i are handled by the same lanes, so SwiGLU (with the optional clamp) is
//     applied in registers and only h is written (gate_up fusion as in vllm.cpp PR #52; clamp-SwiGLU
//     epilogue per the routed clamp-SwiGLU row of the Post-Portfolio Device Attribution table).
// Grid: x = row tiles of the expert, y = active-expert slot. Slots past n_active and experts with more
// than small_m_max rows exit at once; the grid is sized from host-known bounds only.
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

constexpr int gateup_slots(int bpl) { return bpl >= 8 ? 1 : 8 / bpl; }
constexpr int down_slots(int bpl) { return bpl >= 16 ? 1 : 16 / bpl; }

__device__ __forceinline__ int ilog2(int v) { return 31 - __clz(v); }

// acc[m] += <decoded block, x block of token m> for MTC tokens (gate/up: bf16 dot2).
// The packed block is passed through an empty asm so the compiler cannot hoist its decode out of
// the token loop (that would keep up to 32 decoded registers per block alive and spill).
__device__ __forceinline__ void opaque(uint4& w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
}

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

// acc[m] += <decoded block, h block of token m> for MTC tokens (down: fp32 FMA).
template <int MTC>
__device__ __forceinline__ void dot_block_f32(uint4 w, float scale, const float4 (&hb)[MTC][8],
                                              float (&acc)[MTC]) {
  opaque(w);
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2_t p0 = fp4x2_to_f32x2<0>(wd[d], scale);
    const f32x2_t p1 = fp4x2_to_f32x2<1>(wd[d], scale);
    const f32x2_t p2 = fp4x2_to_f32x2<2>(wd[d], scale);
    const f32x2_t p3 = fp4x2_to_f32x2<3>(wd[d], scale);
#pragma unroll
    for (int m = 0; m < MTC; ++m) {
      const float4 h0 = hb[m][2 * d];
      const float4 h1 = hb[m][2 * d + 1];
      float a = acc[m];
      a = fmaf(p0[0], h0.x, a);
      a = fmaf(p0[1], h0.y, a);
      a = fmaf(p1[0], h0.z, a);
      a = fmaf(p1[1], h0.w, a);
      a = fmaf(p2[0], h1.x, a);
      a = fmaf(p2[1], h1.y, a);
      a = fmaf(p3[0], h1.z, a);
      a = fmaf(p3[1], h1.w, a);
      acc[m] = a;
    }
  }
}

__device__ __forceinline__ float reduce_row(float v, int lpr) {
  for (int off = lpr >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int BPL, int MT, int MODE>
__global__ __launch_bounds__(256) void small_gateup_kernel(
    Routed r, int H, int I, const uint8_t* __restrict__ w13_q, const uint8_t* __restrict__ w13_s,
    int lpr, int small_m_max, int check_m, float clamp, float* __restrict__ h_out,
    float* __restrict__ g_ws) {
  constexpr int S = gateup_slots(BPL);
  constexpr bool kGate = MODE != kUpWithGate;
  constexpr bool kUp = MODE != kGateOnly;

  // active[] holds -1 past n_active, and the grid has at most E slots: no n_active read needed
  const int e = r.active[blockIdx.y];
  if (e < 0) return;
  if (check_m && r.counts[e] > small_m_max) return;  // that expert runs on the MFMA kernels

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = ilog2(lpr);
  const int q = lane & (lpr - 1);
  const int sub = lane >> lg;
  const int rpw = 64 >> lg;
  const int NB = H >> 5;
  const int tile = 4 * S * rpw;
  const size_t qrow = (size_t)(H >> 1), srow = (size_t)NB;
  const uint8_t* qe = w13_q + (size_t)e * 2 * I * qrow;
  const uint8_t* se = w13_s + (size_t)e * 2 * I * srow;

  // Every load below is unconditional at a clamped, in-bounds address, and out-of-range lanes are
  // zeroed afterwards: a load under a branch would have to complete before the branch joins, which
  // serialises the loads instead of keeping them all in flight.
  int n[S];
  uint4 wq[S][2][BPL];
  uint32_t sc[S][2][BPL];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    n[s] = blockIdx.x * tile + (wave * S + s) * rpw + sub;
    const int nc = min(n[s], I - 1);
#pragma unroll
    for (int gu = 0; gu < 2; ++gu) {
      if ((gu == 0 && !kGate) || (gu == 1 && !kUp)) continue;
      const size_t row = (size_t)(gu ? I + nc : nc);
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const int kb = min(q + lpr * b, NB - 1);
        wq[s][gu][b] = *reinterpret_cast<const uint4*>(qe + row * qrow + (size_t)kb * 16);
        sc[s][gu][b] = (uint32_t)se[row * srow + kb];
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int gu = 0; gu < 2; ++gu)
#pragma unroll
      for (int b = 0; b < BPL; ++b)
        if (!(n[s] < I && q + lpr * b < NB)) wq[s][gu][b] = make_uint4(0, 0, 0, 0);

  const int M = r.counts[e];
  const int row0 = r.offsets[e];
  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mc = min(MT, M - m0);
    uint4 xb[MT][BPL][4];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = r.sorted_pair[row0 + m0 + min(m, mc - 1)] / r.k;
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const int kb = min(q + lpr * b, NB - 1);
        const uint4* xp = reinterpret_cast<const uint4*>(r.x + (size_t)t * H + (size_t)kb * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[m][b][i] = xp[i];
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int b = 0; b < BPL; ++b)
        if (!(m < mc && q + lpr * b < NB))
#pragma unroll
          for (int i = 0; i < 4; ++i) xb[m][b][i] = make_uint4(0, 0, 0, 0);

    float acc[S][2][MT];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int gu = 0; gu < 2; ++gu)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][gu][m] = 0.0f;

#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int gu = 0; gu < 2; ++gu) {
        if ((gu == 0 && !kGate) || (gu == 1 && !kUp)) continue;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
          const float scale = e8m0_to_float(sc[s][gu][b]);
          if (MT == 1 || mc == MT) {
            uint4 xs[MT][4];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int i = 0; i < 4; ++i) xs[m][i] = xb[m][b][i];
            dot_block_bf16<MT>(wq[s][gu][b], scale, xs, acc[s][gu]);
          } else {
            // fewer tokens left than MT: skip the empty ones (uniform branch)
            uint4 xs[1][4];
            float a1[1];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m >= mc) break;
#pragma unroll
              for (int i = 0; i < 4; ++i) xs[0][i] = xb[m][b][i];
              a1[0] = acc[s][gu][m];
              dot_block_bf16<1>(wq[s][gu][b], scale, xs, a1);
              acc[s][gu][m] = a1[0];
            }
          }
          // keep each block's decode next to its use (bounds the decoded values' live range)
          __builtin_amdgcn_sched_barrier(0);
        }
      }

#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float g = kGate ? reduce_row(acc[s][0][m], lpr) : 0.0f;
        float u = kUp ? reduce_row(acc[s][1][m], lpr) : 0.0f;
        if (q == 0 && m < mc && n[s] < I) {
          const size_t o = (size_t)(row0 + m0 + m) * I + n[s];
          if (MODE == kGateOnly) {
            g_ws[o] = g;
          } else {
            if (MODE == kUpWithGate) g = g_ws[o];
            if (clamp > 0.0f) {
              g = clampf(g, clamp);
              u = clampf(u, clamp);
            }
            h_out[o] = silu_mul(g, u);
          }
        }
      }
    }
  }
}

template <int BPL, int MT>
__global__ __launch_bounds__(256) void small_down_kernel(Routed r, int H, int I,
                                                         const uint8_t* __restrict__ w2_q,
                                                         const uint8_t* __restrict__ w2_s, int lpr,
                                                         int small_m_max, int check_m,
                                                         const float* __restrict__ h,
                                                         float* __restrict__ y) {
  constexpr int S = down_slots(BPL);
  const int e = r.active[blockIdx.y];
  if (e < 0) return;
  if (check_m && r.counts[e] > small_m_max) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = ilog2(lpr);
  const int q = lane & (lpr - 1);
  const int sub = lane >> lg;
  const int rpw = 64 >> lg;
  const int NB = I >> 5;
  const int tile = 4 * S * rpw;
  const size_t qrow = (size_t)(I >> 1), srow = (size_t)NB;
  const uint8_t* qe = w2_q + (size_t)e * H * qrow;
  const uint8_t* se = w2_s + (size_t)e * H * srow;

  int n[S];
  uint4 wq[S][BPL];
  uint32_t sc[S][BPL];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    n[s] = blockIdx.x * tile + (wave * S + s) * rpw + sub;
    const size_t nc = (size_t)min(n[s], H - 1);
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int kb = min(q + lpr * b, NB - 1);
      wq[s][b] = *reinterpret_cast<const uint4*>(qe + nc * qrow + (size_t)kb * 16);
      sc[s][b] = (uint32_t)se[nc * srow + kb];
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int b = 0; b < BPL; ++b)
      if (!(n[s] < H && q + lpr * b < NB)) wq[s][b] = make_uint4(0, 0, 0, 0);

  const int M = r.counts[e];
  const int row0 = r.offsets[e];

  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mc = min(MT, M - m0);
    float4 hb[MT][BPL][8];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const int kb = min(q + lpr * b, NB - 1);
        const float4* hp = reinterpret_cast<const float4*>(h + (size_t)(row0 + m0 + min(m, mc - 1)) * I +
                                                           (size_t)kb * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) hb[m][b][i] = hp[i];
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int b = 0; b < BPL; ++b)
        if (!(m < mc && q + lpr * b < NB))
#pragma unroll
          for (int i = 0; i < 8; ++i) hb[m][b][i] = make_float4(0.f, 0.f, 0.f, 0.f);
    float acc[S][MT];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[s][m] = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const float scale = e8m0_to_float(sc[s][b]);
        if (MT == 1 || mc == MT) {
          float4 hs[MT][8];
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) hs[m][i] = hb[m][b][i];
          dot_block_f32<MT>(wq[s][b], scale, hs, acc[s]);
        } else {
          float4 hs[1][8];
          float a1[1];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m >= mc) break;
#pragma unroll
            for (int i = 0; i < 8; ++i) hs[0][i] = hb[m][b][i];
            a1[0] = acc[s][m];
            dot_block_f32<1>(wq[s][b], scale, hs, a1);
            acc[s][m] = a1[0];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float v = reduce_row(acc[s][m], lpr);
        if (q == 0 && m < mc && n[s] < H) y[(size_t)(row0 + m0 + m) * H + n[s]] = v;
      }
  }
}

template <int MODE>
hipError_t gateup_dispatch(const SmallPlan& sp, const Routed& r, int H, int I, const uint8_t* wq,
                           const uint8_t* ws, int small_m_max, int check_m, float clamp, float* h,
                           float* g_ws, hipStream_t stream) {
  const dim3 grid(sp.gu_grid_x, sp.slots), block(256);
  const int lpr = sp.gu.lpr;
#define MOE_GU(BPL, MT)                                                                           \
  small_gateup_kernel<BPL, MT, MODE><<<grid, block, 0, stream>>>(r, H, I, wq, ws, lpr, small_m_max, \
                                                                 check_m, clamp, h, g_ws)
#define MOE_GU_MT(BPL)   \
  if (sp.mt_gu == 2)     \
    MOE_GU(BPL, 2);      \
  else                   \
    MOE_GU(BPL, 1);
  switch (sp.gu.bpl) {
    case 1: MOE_GU_MT(1) break;
    case 2: MOE_GU_MT(2) break;
    case 3: MOE_GU_MT(3) break;
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

SmallPlan plan_small(int T, int H, int I, int E, int k) {
  SmallPlan sp;
  sp.gu = choose_row_split(H);
  sp.dn = choose_row_split(I);
  const int rpw_gu = 64 / sp.gu.lpr, rpw_dn = 64 / sp.dn.lpr;
  sp.gu_tile = 4 * gateup_slots(sp.gu.bpl) * rpw_gu;
  sp.dn_tile = 4 * down_slots(sp.dn.bpl) * rpw_dn;
  sp.gu_grid_x = (I + sp.gu_tile - 1) / sp.gu_tile;
  sp.dn_grid_x = (H + sp.dn_tile - 1) / sp.dn_tile;
  const long P = (long)T * k;
  sp.slots = (int)(P < E ? P : E);
  sp.mt_gu = (T >= 2 && sp.gu.bpl <= 3) ? 2 : 1;
  sp.mt_dn = (T >= 2 && sp.dn.bpl <= 2) ? 2 : 1;
  return sp;
}

hipError_t launch_small_gateup(const SmallPlan& sp, const Routed& r, int H, int I,
                               const uint8_t* w13_q, const uint8_t* w13_s, int small_m_max,
                               int check_m, float clamp, int mode, float* h, float* g_ws,
                               hipStream_t stream) {
  switch (mode) {
    case kGateUpFused:
      return gateup_dispatch<kGateUpFused>(sp, r, H, I, w13_q, w13_s, small_m_max, check_m, clamp, h, g_ws,
                                       stream);
    case kGateOnly:
      return gateup_dispatch<kGateOnly>(sp, r, H, I, w13_q, w13_s, small_m_max, check_m, clamp, h, g_ws,
                                       stream);
    case kUpWithGate:
      return gateup_dispatch<kUpWithGate>(sp, r, H, I, w13_q, w13_s, small_m_max, check_m, clamp, h, g_ws,
                                       stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_small_down(const SmallPlan& sp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, int small_m_max, int check_m, const float* h,
                             float* y, hipStream_t stream) {
  const dim3 grid(sp.dn_grid_x, sp.slots), block(256);
  const int lpr = sp.dn.lpr;
#define MOE_DN(BPL, MT) \
  small_down_kernel<BPL, MT><<<grid, block, 0, stream>>>(r, H, I, w2_q, w2_s, lpr, small_m_max, \
                                                         check_m, h, y)
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
  return hipGetLastError();
}

}  // namespace moe
