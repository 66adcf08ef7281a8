// Dense MFMA MXFP4 expert GEMMs for experts with hundreds of routed rows (compute-bound).
//
// With M in the hundreds per expert the expert GEMMs are compute-bound, and what limits the row-tile
// kernels there is the FP4 decode: each wave decodes its own weight columns, one conversion per
// MFMA. Here a workgroup stages both operands of a K-step in LDS and the weights are decoded once per
// workgroup:
//   - a workgroup owns 256 rows of one expert x 256 weight rows (gate_up: 128 gate columns and the
//     matching 128 up columns; down: 256 or 224 output columns, whichever fills the compute units
//     in fewer, fuller rounds); its eight waves (two per SIMD) each compute 64 rows x 128 (or 112)
//     weight rows with 16x16x32 MFMAs (32 or 28 accumulator blocks);
//   - per K-step of 64 the activation rows go straight from memory to LDS (direct loads) and every
//     thread loads one MX block of one weight row (16 bytes of E2M1 codes + the E8M0 scale), decodes
//     it exactly with the scaled FP4 conversion and writes it to LDS; the loads of step s + 1 are
//     issued while step s runs its MFMAs;
//   - weight rows in LDS are padded to 16 bytes past a multiple of 64 and activation rows have their
//     16-byte chunks permuted, so the MFMA operand reads (16 rows x 16 bytes per lane group) hit 64
//     distinct banks; two LDS buffers alternate, one barrier per K-step.
// gate_up multiplies bf16 x with bf16 weights (E2M1 x E8M0 is exact in bf16). Gate columns and the
// matching up columns land in the same lanes of a wave, so the clamp-SwiGLU epilogue runs in
// registers; it writes h as its two bf16 planes.
// down runs one fp16 MFMA per operand pair instead of one bf16 MFMA per h plane:
//   - between the two GEMMs one wave per row rebuilds the row as hi + lo (exact in fp32), scales it
//     by a power of two chosen from the row's largest |hi| so that its largest magnitude lands in
//     [2^14, 2^15), rounds it to fp16 (11 significant bits per value, as in the weight-streaming
//     down kernel; no overflow since |hi + lo| <= |hi| (1 + 2^-8)) and writes it over the hi plane,
//     with the scale's exponent in one byte per row; the down workgroups then stage it unchanged;
//   - each weight column (output column) is decoded as code x 2^(s - c + 13) in fp16, with c the
//     largest scale byte of that column: the largest block reaches at most 6 x 2^13, and every
//     block whose scale byte is within 36 of the column's largest is exact;
//   - the epilogue multiplies the fp32 sum by 2^((127 - f) + (c - 140)) with one ldexp, which
//     undoes both scalings exactly (within fp32 range).
// Only the dense down GEMM reads the rows of dense experts, so their hi plane can be overwritten.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace moe {

namespace {

constexpr int kDM = 256;              // rows per tile
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

template <bool GATEUP, int NCB>
struct DenseShape {
  static constexpr int kNW = 16 * NCB;
  static constexpr int kTN = 2 * kNW;
  static constexpr int kBK = 64;                        // K elements per step (two MX blocks)
  static constexpr int kBlocks = kBK / 32;              // MX blocks per weight row and step
  static constexpr int kRow = kBK * 2 + 16;             // LDS bytes per weight row (16-bit values + padding)
  static constexpr int kARow = kBK * 2;                 // LDS bytes per activation row (chunks permuted)
  static constexpr int kATileBytes = kDM * kARow;
  static constexpr int kBTileBytes = kTN * kRow;
  static constexpr int kStage = kATileBytes + kBTileBytes;
  // LDS bytes past the two stages: down keeps the row and column exponents there
  static constexpr int kExtra = GATEUP ? 0 : (kDM + kTN) * 4;
  static constexpr int kLds = 2 * kStage + kExtra;
  // 16-byte LDS chunks per activation row and step, direct loads per wave and step (each puts 1 KB,
  // eight rows, into LDS), and weight-block chunks per thread and step
  static constexpr int kCpr = kBK * 2 / 16;
  static constexpr int kAChunks = kATileBytes / (kDW * 1024);
  static constexpr int kBChunks = (kTN * kBlocks + kDThreads - 1) / kDThreads;
};

// Weight row (within the expert) streamed as LDS B-tile row n of column tile xblk.
//   gate_up: n in [0,64) gate of wave column 0, [64,128) its up rows, [128,192) gate of column 1,
//            [192,256) its up rows (so a wave's gate and up blocks share lanes);
//   down: n is the output column offset (kTN columns per tile).
template <bool GATEUP, int kTN>
__device__ __forceinline__ int dense_weight_row(int xblk, int n, int I, int H) {
  if (GATEUP) {
    const int c = min(xblk * 128 + (n >> 7) * 64 + (n & 63), I - 1);
    return (n & 64) ? I + c : c;
  }
  return min(xblk * kTN + n, H - 1);
}

template <bool GATEUP, int NCB>
__global__ __launch_bounds__(kDThreads, 1) void dense_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, int k, int H, int I,
    int nx, int dense_slots, const uint8_t* __restrict__ wq_all, const uint8_t* __restrict__ ws_all,
    const int32_t* __restrict__ dense_e, const int32_t* __restrict__ dense_m0, float clamp,
    const uint16_t* __restrict__ h16_in, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
    const uint8_t* __restrict__ rowf,
    float* __restrict__ y_out) {
  using S = DenseShape<GATEUP, NCB>;
  static_assert(!GATEUP || NCB == 8, "gate_up pairs gate blocks 0..3 with up blocks 4..7");
  static_assert(NCB >= 2 + kMS, "the next slice's A operands are read during passes 2 .. 1 + kMS");
  constexpr int kNW = S::kNW, kTN = S::kTN;
  using op_t = typename std::conditional<GATEUP, bf16x8_t, f16x8_t>::type;
  constexpr int NA = S::kAChunks;
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
  const int wc = wave / (kDW / 2);  // column group: B-tile rows wc*kNW .. +kNW

  // ---- staging assignments
  // activations (x for gate_up, the fp16 h rows for down) go straight from memory to LDS: direct load
  // i of wave w fills LDS kilobyte w * NA + i of the tile, lane l the 16 bytes at 16 l, i.e. position
  // l % 8 of tile row r = 8 (w * NA + i) + l / 8. Rows are unpadded and a row's chunk c sits at position
  // c ^ ((r >> 1) & 7), so the operand reads of 16 consecutive rows (one chunk each) hit 64 distinct
  // banks; the lane therefore fetches the chunk that belongs at its position.
  constexpr int kCpr = S::kCpr;
  static_assert(kCpr == 8, "activation rows of 128 bytes");
  const uint8_t* arow[NA];
  int achunk[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = 8 * (wave * NA + i) + lane / 8;
    achunk[i] = (lane & 7) ^ ((r >> 1) & 7);
    const int lr = min(r, rows - 1);
    if (GATEUP) {
      const int t = sorted_pair[row0 + lr] / k;
      arow[i] = reinterpret_cast<const uint8_t*>(x + (size_t)t * H);
    } else {
      arow[i] = reinterpret_cast<const uint8_t*>(h16_in + (size_t)(row0 + lr) * I);
    }
  }
  // weights: chunk q = tid + kDThreads * j is block (q % kBlocks) of B-tile row (q / kBlocks)
  constexpr int NBW = S::kBChunks;
  const int bblk = tid % S::kBlocks;  // the same for every j (kDThreads is a multiple of kBlocks)
  int bn[NBW];
  uint32_t bq[NBW], bs[NBW];
#pragma unroll
  for (int jw = 0; jw < NBW; ++jw) {
    bn[jw] = ((tid + kDThreads * jw) / S::kBlocks) % kTN;
    const uint32_t wrow = (uint32_t)dense_weight_row<GATEUP, kTN>(xblk, bn[jw], I, H);
    bq[jw] = wrow * qrow;
    bs[jw] = wrow * srow;
  }

  // one register set of loads: the weight block(s) of one K-step
  uint4 rb[NBW];
  uint32_t rs[NBW];

  // activations of K-step `step` -> LDS buffer step & 1 (direct loads, waited for by the caller). Past K
  // (a last step of 32 when K is not a multiple of 64) a chunk repeats the row's last eight finite
  // values: the weights there decode with a zero scale, so those products are exact zeros and no
  // masking is needed.
  auto dma_a = [&](int step) {
    uint8_t* st_a = lds + (step & 1) * S::kStage;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int elc = min(step * S::kBK + achunk[i] * 8, K - 8);  // first element of the chunk
      lds_dma16(arow[i] + (size_t)elc * 2, st_a + (wave * NA + i) * 1024);
    }
  };
  // VMEM instructions of one load_b (a 16-byte code load and a scale byte per block)
  constexpr int kBOps = 2 * NBW;
  auto load_b = [&](int step) {
    const int st = min(step, nsteps - 1);
    const uint32_t blk = (uint32_t)min(st * S::kBlocks + bblk, NB - 1);
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      rb[jw] = ld16(qe, bq[jw] + blk * 16);
      rs[jw] = ld8(se, bs[jw] + blk);
    }
  };

  f32x4_t acc[kMS][NCB];
#pragma unroll
  for (int ms = 0; ms < kMS; ++ms)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[ms][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  dma_a(0);
  load_b(0);

  // down: the row scales of this tile and the column shifts of this column tile
  int ccol[NBW];
  if (!GATEUP) {
    if (tid < kDM) s_rowe[tid] = 127 - (int)rowf[row0 + min(tid, rows - 1)];  // row scale 2^(f - 127)
    const bool svec = (NB & 15) == 0 && (reinterpret_cast<uintptr_t>(se) & 15) == 0;
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      ccol[jw] = (int)max_bytes(se + bs[jw], NB, svec);
      if (tid + kDThreads * jw < kTN * S::kBlocks) s_colc[bn[jw]] = ccol[jw];
    }
    __syncthreads();
  }

  // weight blocks of K-step `step` -> 32 16-bit values each in LDS buffer step & 1 (a zero scale
  // past K): bf16 with the block scale for gate_up, fp16 with the block scale relative to the
  // column's for down
  auto stage_b = [&](int step) {
    uint8_t* st_b = lds + (step & 1) * S::kStage + S::kATileBytes;
#pragma unroll
    for (int jw = 0; jw < NBW; ++jw) {
      // a repeated chunk (only when the tile has fewer blocks than threads): written by its owner
      if (kTN * S::kBlocks < kDThreads * NBW && tid + kDThreads * jw >= kTN * S::kBlocks) break;
      const bool ok = step * S::kBlocks + bblk < NB;
      const uint32_t wd[4] = {rb[jw].x, rb[jw].y, rb[jw].z, rb[jw].w};
      uint8_t* dst = st_b + bn[jw] * S::kRow + bblk * 64;
      if (GATEUP) {
        const float scale = ok ? e8m0_to_float(rs[jw]) : 0.0f;
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
        const int ex = (int)rs[jw] + 140 - ccol[jw];
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
  };

  // software pipeline: step 0 staged and step 1's weights in flight before the loop. Step s opens by
  // issuing the activation loads of step s + 1 into buffer (s + 1) & 1 (last read in step s - 1,
  // before the barrier that opened step s); its MFMA passes read buffer s & 1; its last pass decodes
  // the weights of step s + 1 into buffer (s + 1) & 1 and refills their registers with step s + 2.
  // Every load has about a step to arrive. One barrier per step, after the wait for the activations.
  stage_b(0);
  load_b(1);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(kBOps));  // step 0's activations (step 1's weights may fly)
  __syncthreads();

  // operand reads from LDS (lane: row / column j16, K elements 8g .. 8g+7 of 32-wide slice kk)
  auto read_a = [&](const uint8_t* st_a, int kk, int ms) {
    const int r = wr * kWM + ms * 16 + j16;
    return *reinterpret_cast<const op_t*>(st_a + r * S::kARow + (((kk * 4 + g) ^ ((r >> 1) & 7)) * 16));
  };
  auto read_b = [&](const uint8_t* st_b, int kk, int cb) {
    return *reinterpret_cast<const op_t*>(st_b + (wc * kNW + cb * 16 + j16) * S::kRow + kk * 64 + g * 16);
  };
  constexpr int kQ = S::kBlocks * NCB;  // column-block passes per step (slice-major)

  for (int step = 0; step < nsteps; ++step) {
    if (step + 1 < nsteps) dma_a(step + 1);
    const uint8_t* st_a = lds + (step & 1) * S::kStage;
    const uint8_t* st_b = st_a + S::kATileBytes;
    // Column-block-major passes: pass q = 8 kk + cb multiplies the slice's four A operands (held in
    // registers) with one B operand. B operands stream through a three-entry register ring read two
    // passes ahead, and the next slice's A operands are read during the current slice, so LDS reads
    // are spread over the step instead of arriving in one burst per slice.
    op_t acur[kMS], anxt[kMS], bring[3];
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) acur[ms] = read_a(st_a, 0, ms);
    bring[0] = read_b(st_b, 0, 0);
    bring[1] = read_b(st_b, 0, 1);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int kk = q / NCB, cb = q % NCB;
      if (q + 2 < kQ) bring[(q + 2) % 3] = read_b(st_b, (q + 2) / NCB, (q + 2) % NCB);
      if (kk + 1 < S::kBlocks && cb >= 2 && cb < 2 + kMS) anxt[cb - 2] = read_a(st_a, kk + 1, cb - 2);
#pragma unroll
      for (int ms = 0; ms < kMS; ++ms) {
        if constexpr (GATEUP)
          acc[ms][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur[ms], bring[q % 3], acc[ms][cb], 0, 0, 0);
        else
          acc[ms][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[ms], bring[q % 3], acc[ms][cb], 0, 0, 0);
      }
      // the weights of the next step in the last pass, as late as possible behind the activation loads
      // (the compiler's wait for their registers also waits for those)
      if (q == kQ - 1) {
        stage_b(step + 1);
        load_b(step + 2);
      }
      if (cb == NCB - 1) {
#pragma unroll
        for (int ms = 0; ms < kMS; ++ms) acur[ms] = anxt[ms];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(kBOps));  // the activations of step + 1 have landed
    __syncthreads();
  }

  // epilogue: lane holds rows 4g+i of each 16-row block, column j16 of each column block
  if (GATEUP) {
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
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
          store_h_planes(h_hi, h_lo, orow * I + col, silu_mul(gv, uv));
        }
      }
    }
  } else {
    int ecol[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) ecol[cb] = s_colc[wc * kNW + cb * 16 + j16] - 140;
#pragma unroll
    for (int ms = 0; ms < kMS; ++ms) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = wr * kWM + ms * 16 + g * 4 + i;
        if (lr >= rows) continue;
        const size_t orow = (size_t)(row0 + lr);
        const int erow = s_rowe[lr];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int col = xblk * kTN + wc * kNW + cb * 16 + j16;
          if (col < N) y_out[orow * H + col] = __builtin_amdgcn_ldexpf(acc[ms][cb][i], erow + ecol[cb]);
        }
      }
    }
  }
}

// Rows of dense experts, between the two GEMMs: one wave per row rebuilds h as hi + lo, scales it by
// 2^(f - 127) with f = clamp(268 - biased exponent of the row's largest |hi|, 1, 253) and writes it
// as fp16 over the hi plane; rowf[row] = f. Both passes read the row in groups of four 16-byte
// chunks per lane (the second finds the hi plane in L2).
constexpr int kH16Waves = 4;  // rows per workgroup

__global__ __launch_bounds__(64 * kH16Waves) void dense_h16_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int I, int dense_slots,
    const int32_t* __restrict__ dense_e, const int32_t* __restrict__ dense_m0, uint16_t* h_hi,
    const uint16_t* __restrict__ h_lo, uint8_t* __restrict__ rowf) {
  constexpr int kSub = kDM / kH16Waves;  // workgroups per row tile
  const int y = blockIdx.x / kSub;
  if (y >= dense_slots) return;
  const int te = dense_e[y];
  if (te < 0) return;
  const int e = uniform(te);
  const int m0 = uniform(dense_m0[y]);
  const int rows = min(kDM, uniform(counts[e]) - m0);
  const int lr = (blockIdx.x % kSub) * kH16Waves + uniform((int)(threadIdx.x >> 6));
  if (lr >= rows) return;
  const size_t row = (size_t)(uniform(offsets[e]) + m0 + lr);
  uint8_t* hi = reinterpret_cast<uint8_t*>(h_hi + row * I);
  const uint8_t* lo = reinterpret_cast<const uint8_t*>(h_lo + row * I);
  const int lane = threadIdx.x & 63;
  const int nch = I >> 3;  // 16-byte chunks per row and plane
  const uint4 zero = make_uint4(0, 0, 0, 0);

  // largest exponent field among the low and among the high bf16 halves of the hi plane
  uint32_t mx_lo = 0, mx_hi = 0;
  for (int c0 = 0; c0 < nch; c0 += 256) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u + lane;
      v[u] = c < nch ? ld16(hi, (uint32_t)c * 16) : zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mx_lo = max(mx_lo, max(max(v[u].x & 0x7F80u, v[u].y & 0x7F80u), max(v[u].z & 0x7F80u, v[u].w & 0x7F80u)));
      mx_hi = max(mx_hi, max(max(v[u].x & 0x7F800000u, v[u].y & 0x7F800000u),
                             max(v[u].z & 0x7F800000u, v[u].w & 0x7F800000u)));
    }
  }
  int eb = max((int)(mx_lo >> 7), (int)(mx_hi >> 23));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) eb = max(eb, __shfl_xor(eb, off));
  const int f = min(max(268 - eb, 1), 253);
  const float sc = __builtin_bit_cast(float, (uint32_t)f << 23);

  for (int c0 = 0; c0 < nch; c0 += 256) {
    uint4 hv[4], lv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u + lane;
      hv[u] = c < nch ? ld16(hi, (uint32_t)c * 16) : zero;
      lv[u] = c < nch ? ld16(lo, (uint32_t)c * 16) : zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u + lane;
      const uint32_t a[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
      const uint32_t l[4] = {lv[u].x, lv[u].y, lv[u].z, lv[u].w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = bf16_lo_f32(a[j]) + bf16_lo_f32(l[j]);
        const float v1 = bf16_hi_f32(a[j]) + bf16_hi_f32(l[j]);
        o[j] = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)(v0 * sc), (_Float16)(v1 * sc)});
      }
      if (c < nch) *reinterpret_cast<uint4*>(hi + (size_t)c * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if (lane == 0) rowf[row] = (uint8_t)f;
}

}  // namespace

int dense_slots_bound(int T, int E, int k, int dense_m_min) {
  // sum over experts with at least dense_m_min rows of ceil(M_e / 256) <= P/256 + their number
  const long P = (long)T * k;
  long n_dense = P / (dense_m_min > 0 ? dense_m_min : 1);
  if (n_dense > E) n_dense = E;
  return (int)((P + kDM - 1) / kDM + n_dense);
}

DensePlan plan_dense(int T, int H, int I, int E, int k, int dense_m_min, int num_cus, int force_ncb) {
  DensePlan dp;
  dp.tile_m = kDM;
  dp.gu_grid_x = (I + 127) / 128;
  // down column tile: with one workgroup per compute unit (LDS), the layer takes
  // ceil(tiles / CUs) rounds of work proportional to the tile width; expect ceil(P / 256) row tiles
  // (every pair in a dense expert) and take the width with the smaller product (ties: the wider)
  const long rt = ((long)T * k + kDM - 1) / kDM;
  const int cus = num_cus > 0 ? num_cus : 1;
  long best = -1;
  for (int ncb = 8; ncb >= 7; --ncb) {
    const int width = 32 * ncb;
    const long tiles = rt * ((H + width - 1) / width);
    const long cost = (tiles + cus - 1) / cus * width;
    if (best < 0 || cost < best) {
      best = cost;
      dp.dn_ncb = ncb;
    }
  }
  if (force_ncb == 7 || force_ncb == 8) dp.dn_ncb = force_ncb;
  dp.dn_grid_x = (H + 32 * dp.dn_ncb - 1) / (32 * dp.dn_ncb);
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
  constexpr int lds = DenseShape<true, 8>::kLds;
  static const bool attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<true, 8>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   lds) == hipSuccess;
  (void)attr_set;
  dense_kernel<true, 8><<<dp.gu_blocks, kDThreads, lds, stream>>>(
      r.x, r.counts, r.offsets, r.sorted_pair, r.k, H, I, dp.gu_grid_x, dp.slots, w13_q, w13_s, dense_e,
      dense_m0, clamp, nullptr, h_hi, h_lo, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_dense_h16(const DensePlan& dp, const Routed& r, int I, const int32_t* dense_e,
                            const int32_t* dense_m0, uint16_t* h_hi, const uint16_t* h_lo, uint8_t* rowf,
                            hipStream_t stream) {
  if (dp.slots <= 0) return hipSuccess;
  dense_h16_kernel<<<dp.slots * (kDM / kH16Waves), 64 * kH16Waves, 0, stream>>>(
      r.counts, r.offsets, I, dp.slots, dense_e, dense_m0, h_hi, h_lo, rowf);
  return hipGetLastError();
}

template <int NCB>
hipError_t launch_dense_down_ncb(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w2_q,
                                 const uint8_t* w2_s, const int32_t* dense_e, const int32_t* dense_m0,
                                 const uint16_t* h16, const uint8_t* rowf, float* y, hipStream_t stream) {
  constexpr int lds = DenseShape<false, NCB>::kLds;
  static const bool attr_set = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<false, NCB>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   lds) == hipSuccess;
  (void)attr_set;
  dense_kernel<false, NCB><<<dp.dn_blocks, kDThreads, lds, stream>>>(
      r.x, r.counts, r.offsets, r.sorted_pair, r.k, H, I, dp.dn_grid_x, dp.slots, w2_q, w2_s, dense_e,
      dense_m0, 0.0f, h16, nullptr, nullptr, rowf, y);
  return hipGetLastError();
}

hipError_t launch_dense_down(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* dense_e, const int32_t* dense_m0,
                             const uint16_t* h16, const uint8_t* rowf, float* y, hipStream_t stream) {
  if (dp.slots <= 0) return hipSuccess;
  if (dp.dn_ncb == 7)
    return launch_dense_down_ncb<7>(dp, r, H, I, w2_q, w2_s, dense_e, dense_m0, h16, rowf, y, stream);
  return launch_dense_down_ncb<8>(dp, r, H, I, w2_q, w2_s, dense_e, dense_m0, h16, rowf, y, stream);
}

}  // namespace moe
