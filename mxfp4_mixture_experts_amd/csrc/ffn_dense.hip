// Dense bf16-MFMA MXFP4 expert GEMMs for experts with hundreds of routed rows (compute-bound).
//
// With M in the hundreds per expert the expert GEMMs are compute-bound (the M=1024 MFMA target of
// the layer), and what limits the row-tile kernels there is the FP4 decode: each wave decodes its
// own weight columns, one conversion per MFMA. Here a workgroup stages both operands of a K-step in
// LDS and the weights are decoded once per workgroup:
//   - a workgroup owns 256 rows of one expert x 256 weight rows (gate_up: 128 gate columns and the
//     matching 128 up columns; down: 256 output columns); its eight waves (two per SIMD) each
//     compute 64 rows x 128 weight rows with v_mfma_f32_16x16x32_bf16 (32 accumulator blocks);
//   - per K-step every thread loads 16-byte chunks of the activation rows (gathered x rows for
//     gate_up; for down, h rows of both of its bf16 planes, hi and lo) and one MX block of one
//     weight row (16 bytes of E2M1 codes + the E8M0 scale), decodes the block exactly to 32 bf16
//     with the scaled FP4 conversion and writes both to LDS; the loads of the next K-steps are in
//     flight in registers meanwhile;
//   - LDS rows are padded to 16 bytes past a multiple of 64 so the MFMA operand reads (16 rows x
//     16 bytes per lane group) hit 64 distinct banks; two LDS buffers alternate, one barrier per
//     K-step;
//   - gate columns and the matching up columns land in the same lanes of a wave, so the
//     clamp-SwiGLU epilogue runs in registers; down adds the hi and lo products (two MFMAs per A
//     operand), as the row-tile kernels do.
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

template <bool GATEUP>
struct DenseShape {
  static constexpr int kBK = GATEUP ? 64 : 32;          // K elements per step (MX blocks x 32)
  static constexpr int kBlocks = kBK / 32;              // MX blocks per weight row and step
  static constexpr int kATiles = GATEUP ? 1 : 2;        // x, or h hi + lo
  static constexpr int kRow = kBK * 2 + 16;             // LDS bytes per row (bf16 + padding)
  static constexpr int kATileBytes = kDM * kRow;
  static constexpr int kBTileBytes = kDN * kRow;
  static constexpr int kStage = kATiles * kATileBytes + kBTileBytes;
  // 16-byte global chunks per activation row and step (bf16 x: kBK*2 bytes; h: kBK*2 bytes of each
  // plane), per thread and step, and weight-block chunks per thread and step
  static constexpr int kCpr = kATiles * kBK * 2 / 16;
  static constexpr int kAChunks = kDM * kCpr / kDThreads;
  static constexpr int kBChunks = (kDN * kBlocks + kDThreads - 1) / kDThreads;
  static constexpr int kD = GATEUP ? 1 : 2;             // K-steps of loads in flight
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
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo, float* __restrict__ y_out) {
  using S = DenseShape<GATEUP>;
  constexpr int D = S::kD;
  constexpr int NA = S::kAChunks;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

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
  // activations: chunk c = tid + kDThreads * i covers 8 elements of row (c / kCpr): for down, of
  // plane (c % kCpr) / (kBK / 8), for gate_up of x
  constexpr int kCpr = S::kCpr;
  constexpr int kCpp = S::kBK / 8;  // chunks per row and plane
  const uint8_t* arow[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int c = tid + kDThreads * i;
    const int lr = min(c / kCpr, rows - 1);
    if (GATEUP) {
      const int t = sorted_pair[row0 + lr] / k;
      arow[i] = reinterpret_cast<const uint8_t*>(x + (size_t)t * H);
    } else {
      const uint16_t* plane = ((c % kCpr) / kCpp) ? h_lo_in : h_hi_in;
      arow[i] = reinterpret_cast<const uint8_t*>(plane + (size_t)(row0 + lr) * I);
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

  uint4 ra[D][NA];
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
      const int el = st * S::kBK + (c % kCpp) * 8;  // first element of the chunk
      const int elc = min(el, K - 8);
      ra[slot][i] = ld16(arow[i], (uint32_t)elc * 2);
    }
  };

  f32x4_t acc[kMS][8];
#pragma unroll
  for (int ms = 0; ms < kMS; ++ms)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[ms][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);

  auto step_body = [&](int slot, int step) {
    uint8_t* st_a = lds + (step & 1) * S::kStage;
    uint8_t* st_b = st_a + S::kATiles * S::kATileBytes;
    // activations of this step -> LDS (zero past K)
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + kDThreads * i;
      const int lr = c / kCpr, pl = (c % kCpr) / kCpp, cc = c % kCpp;
      uint4 v = ra[slot][i];
      if (step * S::kBK + cc * 8 >= K) v = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(st_a + pl * S::kATileBytes + lr * S::kRow + cc * 16) = v;
    }
    // weight blocks of this step -> 32 bf16 each in LDS (a zero scale past K)
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      if (tid + kDThreads * jw >= kDN * S::kBlocks) break;  // a repeated chunk: written by its owner
      const bool ok = step * S::kBlocks + bblk < NB;
      const float scale = ok ? e8m0_to_float(rs[slot][jw]) : 0.0f;
      const uint32_t wd[4] = {rb[slot][jw].x, rb[slot][jw].y, rb[slot][jw].z, rb[slot][jw].w};
      uint8_t* dst = st_b + bn[jw] * S::kRow + bblk * 64;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x2_t p0 = fp4x2_to_bf16x2<0>(wd[d], scale);
        const bf16x2_t p1 = fp4x2_to_bf16x2<1>(wd[d], scale);
        const bf16x2_t p2 = fp4x2_to_bf16x2<2>(wd[d], scale);
        const bf16x2_t p3 = fp4x2_to_bf16x2<3>(wd[d], scale);
        *reinterpret_cast<bf16x8_t*>(dst + d * 16) =
            bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    }
    __syncthreads();
    // refill the slot with step + D while this step computes
    issue(slot, step + D);
    // MFMAs: per 32-wide K slice, A operands of the wave's 4 row blocks and B operands of its 8
    // column blocks (lane: row / column j16, K elements 8g .. 8g+7 of the slice)
#pragma unroll
    for (int kk = 0; kk < S::kBlocks; ++kk) {
      bf16x8_t bop[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
        bop[cb] = *reinterpret_cast<const bf16x8_t*>(st_b + (wc * 128 + cb * 16 + j16) * S::kRow + kk * 64 +
                                                     g * 16);
      // A operands one row block ahead; the barrier keeps the compiler from hoisting every read of
      // the step (which would not fit next to the 256 accumulator registers)
      auto read_a = [&](int ms, bf16x8_t (&a)[S::kATiles]) {
#pragma unroll
        for (int at = 0; at < S::kATiles; ++at)
          a[at] = *reinterpret_cast<const bf16x8_t*>(st_a + at * S::kATileBytes +
                                                     (wr * kWM + ms * 16 + j16) * S::kRow + kk * 64 + g * 16);
      };
      bf16x8_t aop[2][S::kATiles];
      read_a(0, aop[0]);
#pragma unroll
      for (int ms = 0; ms < kMS; ++ms) {
        if (ms < kMS - 1) read_a(ms + 1, aop[(ms + 1) & 1]);
#pragma unroll
        for (int at = 0; at < S::kATiles; ++at) {
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
            acc[ms][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[ms & 1][at], bop[cb], acc[ms][cb], 0, 0, 0);
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
#pragma unroll
  for (int ms = 0; ms < kMS; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = wr * kWM + ms * 16 + g * 4 + i;
      if (lr >= rows) continue;
      const size_t orow = (size_t)(row0 + lr);
      if (GATEUP) {
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
          store_h_planes(h_hi, h_lo, orow * I + col, silu_mul(gv, uv));
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const int col = xblk * kDN + wc * 128 + cb * 16 + j16;
          if (col < N) y_out[orow * H + col] = acc[ms][cb][i];
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
                               float clamp, uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream) {
  if (dp.slots <= 0) return hipSuccess;
  constexpr int lds = 2 * DenseShape<true>::kStage;
  static const bool attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<true>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   lds) == hipSuccess;
  (void)attr_set;
  dense_kernel<true><<<dp.gu_blocks, kDThreads, lds, stream>>>(
      r.x, r.counts, r.offsets, r.sorted_pair, r.k, H, I, dp.gu_grid_x, dp.slots, w13_q, w13_s, dense_e,
      dense_m0, clamp, nullptr, nullptr, h_hi, h_lo, nullptr);
  return hipGetLastError();
}

hipError_t launch_dense_down(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* dense_e, const int32_t* dense_m0,
                             const uint16_t* h_hi, const uint16_t* h_lo, float* y, hipStream_t stream) {
  if (dp.slots <= 0) return hipSuccess;
  constexpr int lds = 2 * DenseShape<false>::kStage;
  static const bool attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<false>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   lds) == hipSuccess;
  (void)attr_set;
  dense_kernel<false><<<dp.dn_blocks, kDThreads, lds, stream>>>(
      r.x, r.counts, r.offsets, r.sorted_pair, r.k, H, I, dp.dn_grid_x, dp.slots, w2_q, w2_s, dense_e,
      dense_m0, 0.0f, h_hi, h_lo, nullptr, nullptr, y);
  return hipGetLastError();
}

}  // namespace moe
