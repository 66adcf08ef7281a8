// Dense MFMA MXFP4 expert GEMMs for experts with hundreds of routed rows (compute-bound).
//
// With M in the hundreds per expert the expert GEMMs are compute-bound, and what limits the row-tile
// kernels there is the FP4 decode: each wave decodes its own weight columns, one conversion per
// MFMA. Here a workgroup stages both operands of a K-step in LDS and the weights are decoded once per
// workgroup:
//   - a workgroup owns 256 rows of one expert x 256 weight rows (gate_up: 128 gate columns and the
//     matching 128 up columns; down: 256 output columns); its eight waves (two per SIMD) each
//     compute 64 rows x 128 weight rows with 16x16x32 MFMAs (32 accumulator blocks);
//   - per K-step of 64 every thread loads 16-byte chunks of the activation rows and one MX block of
//     one weight row (16 bytes of E2M1 codes + the E8M0 scale), decodes the block exactly with the
//     scaled FP4 conversion and writes both to LDS; the loads of the next K-step are in flight in
//     registers meanwhile;
//   - LDS rows are padded to 16 bytes past a multiple of 64 so the MFMA operand reads (16 rows x
//     16 bytes per lane group) hit 64 distinct banks; two LDS buffers alternate, one barrier per
//     K-step.
// gate_up multiplies bf16 x with bf16 weights (E2M1 x E8M0 is exact in bf16). Gate columns and the
// matching up columns land in the same lanes of a wave, so the clamp-SwiGLU epilogue runs in
// registers; it writes h as its two bf16 planes and, per row and 64-column segment, the biased
// exponent of the largest |hi| (no atomics: each segment has one writer).
// down runs one fp16 MFMA per operand pair instead of one bf16 MFMA per h plane:
//   - each h row is rebuilt as hi + lo (exact in fp32) and scaled by a power of two chosen from the
//     row's largest |hi| (the maximum of its segment exponents) so that its largest magnitude lands
//     in [2^14, 2^15), then rounded to fp16: 11 significant bits per value, as in the weight-
//     streaming down kernel, and no overflow since |hi + lo| <= |hi| (1 + 2^-8);
//   - each weight column (output column) is decoded as code x 2^(s - c + 13) in fp16, with c the
//     largest scale byte of that column: the largest block reaches at most 6 x 2^13, and every
//     block whose scale byte is within 36 of the column's largest is exact;
//   - the epilogue multiplies the fp32 sum by 2^((127 - f) + (c - 140)) with one ldexp, which
//     undoes both scalings exactly (within fp32 range).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kDM = 256;              // rows per tile
constexpr int kDN = 256;              // weight rows per workgroup
constexpr int kDW = 8;                // waves: 4 row groups x 2 column groups
constexpr int kWM = kDM / (kDW / 2);  // rows per wave (64)
constexpr int kMS = kWM / 16;         // MFMA row blocks per wave
constexpr int kDThreads = 64 * kDW;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint4 ld16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint32_t ld8(const uint8_t* base, uint32_t off) { return base[off]; }

__device__ __forceinline__ uint32_t max_byte4(uint32_t w) {
  return max(max(w & 0xFFu, (w >> 8) & 0xFFu), max((w >> 16) & 0xFFu, w >> 24));
}

// Largest of n bytes at p: 16-byte loads when `vec` (p 16-byte aligned, n a multiple of 16).
__device__ __forceinline__ uint32_t max_bytes(const uint8_t* p, int n, bool vec) {
  uint32_t m = 0;
  if (vec) {
    for (int j = 0; j < n; j += 16) {
      const uint4 v = ld16(p, (uint32_t)j);
      m = max(m, max(max(max_byte4(v.x), max_byte4(v.y)), max(max_byte4(v.z), max_byte4(v.w))));
    }
  } else {
    for (int j = 0; j < n; ++j) m = max(m, ld8(p, (uint32_t)j));
  }
  return m;
}

// v and its rotations within each 16-lane row: every lane ends with its row's maximum.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));  // row_ror:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

template <bool GATEUP>
struct DenseShape {
  static constexpr int kBK = 64;                        // K elements per step (two MX blocks)
  static constexpr int kBlocks = kBK / 32;              // MX blocks per weight row and step
  static constexpr int kPlanes = GATEUP ? 1 : 2;        // global planes per activation: x, or hi + lo
  static constexpr int kRow = kBK * 2 + 16;             // LDS bytes per row (16-bit values + padding)
  static constexpr int kATileBytes = kDM * kRow;
  static constexpr int kBTileBytes = kDN * kRow;
  static constexpr int kStage = kATileBytes + kBTileBytes;
  // LDS bytes past the two stages: down keeps the row and column exponents there
  static constexpr int kExtra = GATEUP ? 0 : (kDM + kDN) * 4;
  static constexpr int kLds = 2 * kStage + kExtra;
  // 16-byte LDS chunks per activation row and step, per thread and step (each chunk is one global
  // 16-byte load per plane), and weight-block chunks per thread and step
  static constexpr int kCpr = kBK * 2 / 16;
  static constexpr int kAChunks = kDM * kCpr / kDThreads;
  static constexpr int kBChunks = (kDN * kBlocks + kDThreads - 1) / kDThreads;
  static constexpr int kD = 1;                          // K-steps of loads in flight
};

// Weight row (within the expert) streamed as LDS B-tile row n of column tile xblk.
//   gate_up: n in [0,64) gate of wave column 0, [64,128) its up rows, [128,192) gate of column 1,
//            [192,256) its up rows (so a wave's gate and up blocks share lanes);
//   down: n is the output column offset.
template <bool GATEUP>
__device__ __forceinline__ int dense_weight_row(int xblk, int n, int I, int H) {
  if (GATEUP) {
    const int c = min(xblk * 128 + (n >> 7) * 64 + (n & 63), I - 1);
    return (n & 64) ? I + c : c;
  }
  return min(xblk * kDN + n, H - 1);
}

template <bool GATEUP>
__global__ __launch_bounds__(kDThreads, 1) void dense_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, int k, int H, int I,
    int nx, int dense_slots, const uint8_t* __restrict__ wq_all, const uint8_t* __restrict__ ws_all,
    const int32_t* __restrict__ dense_e, const int32_t* __restrict__ dense_m0, float clamp,
    const uint16_t* __restrict__ h_hi_in, const uint16_t* __restrict__ h_lo_in,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo, uint8_t* __restrict__ rexp, int nseg,
    float* __restrict__ y_out) {
  using S = DenseShape<GATEUP>;
  using op_t = typename std::conditional<GATEUP, bf16x8_t, f16x8_t>::type;
  constexpr int D = S::kD;
  constexpr int NA = S::kAChunks;
  constexpr int NP = S::kPlanes;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int* s_rowe = reinterpret_cast<int*>(lds + 2 * S::kStage);  // down: 127 - f per tile row
  int* s_colc = s_rowe + kDM;                                  // down: c per B-tile row

  // XCD-interleaved tile order (workgroup b runs on XCD b % 8): XCD x gets row tiles x, x + 8, ...
  // with all their column tiles back to back
  const int b = blockIdx.x;
  const int jb = b >> 3;
  const int y = (b & 7) + 8 * (jb / nx);
  const int xblk = jb % nx;
  if (y >= dense_slots) return;
  const int te = dense_e[y];
  if (te < 0) return;
  const int e = uniform(te);
  const int m0 = uniform(dense_m0[y]);
  const int rows = min(kDM, uniform(counts[e]) - m0);
  const int row0 = uniform(offsets[e]) + m0;

  const int K = GATEUP ? H : I;
  const int N = GATEUP ? I : H;
  const int NB = K >> 5;
  const int nsteps = (NB + S::kBlocks - 1) / S::kBlocks;
  const uint32_t qrow = (uint32_t)(K >> 1), srow = (uint32_t)NB;
  const size_t nrows_w = GATEUP ? (size_t)2 * I : (size_t)H;
  const uint8_t* qe = wq_all + (size_t)e * nrows_w * qrow;
  const uint8_t* se = ws_all + (size_t)e * nrows_w * srow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int j16 = lane & 15;
  const int g = lane >> 4;
  const int wr = wave % (kDW / 2);  // row group: rows wr*kWM .. +kWM
  const int wc = wave / (kDW / 2);  // column group: B-tile rows wc*128 .. +128

  // ---- staging assignments
  // activations: chunk c = tid + kDThreads * i covers elements 8 (c % kCpr) .. +8 of row c / kCpr
  // (of x for gate_up; of both h planes for down)
  constexpr int kCpr = S::kCpr;
  const uint8_t* arow[NA][NP];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int c = tid + kDThreads * i;
    const int lr = min(c / kCpr, rows - 1);
    if (GATEUP) {
      const int t = sorted_pair[row0 + lr] / k;
      arow[i][0] = reinterpret_cast<const uint8_t*>(x + (size_t)t * H);
    } else {
      arow[i][0] = reinterpret_cast<const uint8_t*>(h_hi_in + (size_t)(row0 + lr) * I);
      arow[i][NP - 1] = reinterpret_cast<const uint8_t*>(h_lo_in + (size_t)(row0 + lr) * I);
    }
  }
  // weights: chunk q = tid + kDThreads * j is block (q % kBlocks) of B-tile row (q / kBlocks)
  constexpr int NBW = S::kBChunks;
  const int bblk = tid % S::kBlocks;  // the same for every j (kDThreads is a multiple of kBlocks)
  int bn[NBW];
  uint32_t bq[NBW], bs[NBW];
#pragma unroll
  for (int jw = 0; jw < NBW; ++jw) {
    bn[jw] = ((tid + kDThreads * jw) / S::kBlocks) % kDN;
    const uint32_t wrow = (uint32_t)dense_weight_row<GATEUP>(xblk, bn[jw], I, H);
    bq[jw] = wrow * qrow;
    bs[jw] = wrow * srow;
  }

  uint4 ra[D][NA][NP];
  uint4 rb[D][NBW];
  uint32_t rs[D][NBW];

  auto issue = [&](int slot, int step) {
    const int st = min(step, nsteps - 1);  // steps past the end re-load the last one (never used)
    const uint32_t blk = (uint32_t)min(st * S::kBlocks + bblk, NB - 1);
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      rb[slot][jw] = ld16(qe, bq[jw] + blk * 16);
      rs[slot][jw] = ld8(se, bs[jw] + blk);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + kDThreads * i;
      const int el = st * S::kBK + (c % kCpr) * 8;  // first element of the chunk
      const int elc = min(el, K - 8);
#pragma unroll
      for (int p = 0; p < NP; ++p) ra[slot][i][p] = ld16(arow[i][p], (uint32_t)elc * 2);
    }
  };

  f32x4_t acc[kMS][8];
#pragma unroll
  for (int ms = 0; ms < kMS; ++ms)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[ms][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);

  // down: the row scales of this tile (from the segment exponents gate_up wrote) and the column
  // shifts of this column tile; each staging thread keeps the scales of its activation rows
  float asc[NA];
  int ccol[NBW];
  if (!GATEUP) {
    if (tid < kDM) {
      const int lr = min(tid, rows - 1);
      const uint8_t* p = rexp + (size_t)(row0 + lr) * nseg;
      const int eb = (int)max_bytes(p, nseg, (nseg & 15) == 0);  // biased exponent of max |hi|
      const int f = min(max(268 - eb, 1), 253);                  // row scale 2^(f - 127)
      s_rowe[tid] = 127 - f;
    }
    const bool svec = (NB & 15) == 0 && (reinterpret_cast<uintptr_t>(se) & 15) == 0;
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      ccol[jw] = (int)max_bytes(se + bs[jw], NB, svec);
      if (tid + kDThreads * jw < kDN * S::kBlocks) s_colc[bn[jw]] = ccol[jw];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int lr = (tid + kDThreads * i) / kCpr;
      asc[i] = __builtin_bit_cast(float, (uint32_t)(127 - s_rowe[lr]) << 23);
    }
  }

  auto step_body = [&](int slot, int step) {
    uint8_t* st_a = lds + (step & 1) * S::kStage;
    uint8_t* st_b = st_a + S::kATileBytes;
    // activations of this step -> LDS (zero past K); down: hi + lo, scaled, as fp16
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + kDThreads * i;
      const int lr = c / kCpr, cc = c % kCpr;
      uint4 v;
      if (GATEUP) {
        v = ra[slot][i][0];
      } else {
        const uint4 hv = ra[slot][i][0], lv = ra[slot][i][NP - 1];
        const uint32_t a[4] = {hv.x, hv.y, hv.z, hv.w};
        const uint32_t l[4] = {lv.x, lv.y, lv.z, lv.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v0 = bf16_lo_f32(a[j]) + bf16_lo_f32(l[j]);
          const float v1 = bf16_hi_f32(a[j]) + bf16_hi_f32(l[j]);
          o[j] = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)(v0 * asc[i]), (_Float16)(v1 * asc[i])});
        }
        v = make_uint4(o[0], o[1], o[2], o[3]);
      }
      if (step * S::kBK + cc * 8 >= K) v = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(st_a + lr * S::kRow + cc * 16) = v;
    }
    // weight blocks of this step -> 32 16-bit values each in LDS (a zero scale past K): bf16 with
    // the block scale for gate_up, fp16 with the block scale relative to the column's for down
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      if (tid + kDThreads * jw >= kDN * S::kBlocks) break;  // a repeated chunk: written by its owner
      const bool ok = step * S::kBlocks + bblk < NB;
      const uint32_t wd[4] = {rb[slot][jw].x, rb[slot][jw].y, rb[slot][jw].z, rb[slot][jw].w};
      uint8_t* dst = st_b + bn[jw] * S::kRow + bblk * 64;
      if (GATEUP) {
        const float scale = ok ? e8m0_to_float(rs[slot][jw]) : 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x2_t p0 = fp4x2_to_bf16x2<0>(wd[d], scale);
          const bf16x2_t p1 = fp4x2_to_bf16x2<1>(wd[d], scale);
          const bf16x2_t p2 = fp4x2_to_bf16x2<2>(wd[d], scale);
          const bf16x2_t p3 = fp4x2_to_bf16x2<3>(wd[d], scale);
          *reinterpret_cast<bf16x8_t*>(dst + d * 16) =
              bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
      } else {
        // 2^(s - c + 13); blocks 140 or more below the column's largest scale byte decode to zero
        const int ex = (int)rs[slot][jw] + 140 - ccol[jw];
        const float scale = ok ? __builtin_bit_cast(float, (uint32_t)max(ex, 0) << 23) : 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f16x2_t p0 = fp4x2_to_f16x2_scaled<0>(wd[d], scale);
          const f16x2_t p1 = fp4x2_to_f16x2_scaled<1>(wd[d], scale);
          const f16x2_t p2 = fp4x2_to_f16x2_scaled<2>(wd[d], scale);
          const f16x2_t p3 = fp4x2_to_f16x2_scaled<3>(wd[d], scale);
          *reinterpret_cast<f16x8_t*>(dst + d * 16) =
              f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
      }
    }
    __syncthreads();
    // refill the slot with step + D while this step computes
    issue(slot, step + D);
    // MFMAs: per 32-wide K slice, A operands of the wave's 4 row blocks and B operands of its 8
    // column blocks (lane: row / column j16, K elements 8g .. 8g+7 of the slice)
#pragma unroll
    for (int kk = 0; kk < S::kBlocks; ++kk) {
      op_t bop[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
        bop[cb] = *reinterpret_cast<const op_t*>(st_b + (wc * 128 + cb * 16 + j16) * S::kRow + kk * 64 + g * 16);
      // A operands one row block ahead; the barrier keeps the compiler from hoisting every read of
      // the step (which would not fit next to the 256 accumulator registers)
      auto read_a = [&](int ms) {
        return *reinterpret_cast<const op_t*>(st_a + (wr * kWM + ms * 16 + j16) * S::kRow + kk * 64 + g * 16);
      };
      op_t aop[2];
      aop[0] = read_a(0);
#pragma unroll
      for (int ms = 0; ms < kMS; ++ms) {
        if (ms < kMS - 1) aop[(ms + 1) & 1] = read_a(ms + 1);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          if constexpr (GATEUP)
            acc[ms][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[ms & 1], bop[cb], acc[ms][cb], 0, 0, 0);
          else
            acc[ms][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[ms & 1], bop[cb], acc[ms][cb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // the step count is padded to a multiple of D (padding steps see zero activations and zero
  // scales), so the loop body has no conditional MFMA block and the accumulators stay in place
  const int nsteps_pad = (nsteps + D - 1) / D * D;
  for (int step = 0; step < nsteps_pad; step += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step_body(d, step + d);
  }

  // epilogue: lane holds rows 4g+i of each 16-row block, column j16 of each column block
  if (GATEUP) {
    uint32_t mx[kMS][4];  // largest |hi| bit pattern of the row over the wave's 64 columns
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx[ms][i] = 0;
        const int lr = wr * kWM + ms * 16 + g * 4 + i;
        if (lr >= rows) continue;
        const size_t orow = (size_t)(row0 + lr);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int col = xblk * 128 + wc * 64 + cb * 16 + j16;
          if (col >= N) continue;
          float gv = acc[ms][cb][i];
          float uv = acc[ms][cb + 4][i];
          if (clamp > 0.0f) {
            gv = clampf(gv, clamp);
            uv = clampf(uv, clamp);
          }
          const uint16_t hb = store_h_planes(h_hi, h_lo, orow * I + col, silu_mul(gv, uv));
          mx[ms][i] = max(mx[ms][i], (uint32_t)(hb & 0x7FFFu));
        }
      }
    }
    // one byte per row and segment: the biased exponent of the segment's largest |hi|
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t m = row16_max(mx[ms][i]);
        const int lr = wr * kWM + ms * 16 + g * 4 + i;
        if (j16 == 0 && lr < rows) rexp[(size_t)(row0 + lr) * nseg + xblk * 2 + wc] = (uint8_t)(m >> 7);
      }
    }
  } else {
    int ecol[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) ecol[cb] = s_colc[wc * 128 + cb * 16 + j16] - 140;
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = wr * kWM + ms * 16 + g * 4 + i;
        if (lr >= rows) continue;
        const size_t orow = (size_t)(row0 + lr);
        const int erow = s_rowe[lr];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const int col = xblk * kDN + wc * 128 + cb * 16 + j16;
          if (col < N) y_out[orow * H + col] = __builtin_amdgcn_ldexpf(acc[ms][cb][i], erow + ecol[cb]);
        }
      }
    }
  }
}

}  // namespace

int dense_slots_bound(int T, int E, int k, int dense_m_min) {
  // sum over experts with at least dense_m_min rows of ceil(M_e / 256) <= P/256 + their number
  const long P = (long)T * k;
  long n_dense = P / (dense_m_min > 0 ? dense_m_min : 1);
  if (n_dense > E) n_dense = E;
  return (int)((P + kDM - 1) / kDM + n_dense);
}

// gate_up column tiles are 128 h columns, two 64-column segments (one per wave column group)
int dense_row_segments(int I) { return 2 * ((I + 127) / 128); }

DensePlan plan_dense(int T, int H, int I, int E, int k, int dense_m_min) {
  DensePlan dp;
  dp.tile_m = kDM;
  dp.gu_grid_x = (I + 127) / 128;
  dp.dn_grid_x = (H + kDN - 1) / kDN;
  dp.slots = dense_slots_bound(T, E, k, dense_m_min);
  const int groups = (dp.slots + 7) / 8;
  dp.gu_blocks = 8 * dp.gu_grid_x * groups;
  dp.dn_blocks = 8 * dp.dn_grid_x * groups;
  return dp;
}

hipError_t launch_dense_gateup(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w13_q,
                               const uint8_t* w13_s, const int32_t* dense_e, const int32_t* dense_m0,
                               float clamp, uint16_t* h_hi, uint16_t* h_lo, uint8_t* rexp,
                               hipStream_t stream) {
  if (dp.slots <= 0) return hipSuccess;
  constexpr int lds = DenseShape<true>::kLds;
  static const bool attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<true>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   lds) == hipSuccess;
  (void)attr_set;
  dense_kernel<true><<<dp.gu_blocks, kDThreads, lds, stream>>>(
      r.x, r.counts, r.offsets, r.sorted_pair, r.k, H, I, dp.gu_grid_x, dp.slots, w13_q, w13_s, dense_e,
      dense_m0, clamp, nullptr, nullptr, h_hi, h_lo, rexp, dense_row_segments(I), nullptr);
  return hipGetLastError();
}

hipError_t launch_dense_down(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* dense_e, const int32_t* dense_m0,
                             const uint16_t* h_hi, const uint16_t* h_lo, const uint8_t* rexp, float* y,
                             hipStream_t stream) {
  if (dp.slots <= 0) return hipSuccess;
  constexpr int lds = DenseShape<false>::kLds;
  static const bool attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<false>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   lds) == hipSuccess;
  (void)attr_set;
  dense_kernel<false><<<dp.dn_blocks, kDThreads, lds, stream>>>(
      r.x, r.counts, r.offsets, r.sorted_pair, r.k, H, I, dp.dn_grid_x, dp.slots, w2_q, w2_s, dense_e,
      dense_m0, 0.0f, h_hi, h_lo, nullptr, nullptr, const_cast<uint8_t*>(rexp), dense_row_segments(I), y);
  return hipGetLastError();
}

}  // namespace moe
