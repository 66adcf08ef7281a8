// Activation-quantised expert GEMMs (W4A8 / W4A4): the activations of both GEMMs are quantised to
// OCP MX blocks (32 values along the reduction axis sharing an E8M0 scale; MXFP8 E4M3 or MXFP4 E2M1
// elements) and multiplied with the packed MXFP4 weights by the gfx950 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), which takes codes and scale bytes as they are: no weight is
// decoded anywhere.
//
//   quantise x   four lanes per 32-value block of a token's x: amax, the scale byte
//                (biased exponent of amax minus the element format's largest exponent, at least 0),
//                the codes (nearest-even, saturating), written as [T, H] (E4M3) or [T, H/2] (E2M1)
//                plus [T, H/32] scale bytes;
//   gate_up      256 rows of one expert x 128 h columns (their 128 gate and 128 up weight rows) per
//                workgroup; the clamp-SwiGLU epilogue computes h in fp32 and quantises it per
//                32-column block in registers (the block's 32 values sit in the 32 lanes of a
//                half-wave), writing h's codes [P, I] (or [P, I/2]) and scales [P, I/32] in sorted-row
//                order;
//   down         256 rows x 256 output columns per workgroup, h codes as A, y in fp32 [P, H];
//   combine      the common weighted combine.
//
// GEMM tiling: eight waves (4 row groups x 2 column groups), each 64 rows x 128 weight rows as
// 2 x 4 blocks of 32x32 accumulators. A K-step of 128 stages the activation tile (256 rows x 128
// bytes E4M3 or 64 bytes E2M1), the weight tile (256 rows x 64 bytes) and one scale dword per row
// of each in LDS; two LDS buffers alternate, one barrier per step, and each thread's global loads
// for step s + 2 are issued while step s + 1 is being multiplied. LDS rows are padded by 16 bytes so
// the 16-byte operand reads of 16 consecutive rows fall in distinct banks.
//
// MFMA operand layout (32x32x64, lane l: r = l % 32, g = l / 32; checked on the hardware):
//   E2M1 operand: row r, K [32g, 32g + 32) of the 64, 16 bytes in dwords 0..3;
//   E4M3 operand: row r, K [16g, 16g + 16) in dwords 0..3 and K [32 + 16g, 48 + 16g) in dwords 4..7;
//   scale: lane (g, r) supplies the byte of row r's K block g (K [32g, 32g + 32));
//   result: lane l holds column r, rows 8 * (i / 4) + 4 * g + i % 4 in element i.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace moe {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kMxThreads = 512;
constexpr int kMxBK = 128;  // K per step

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) that
// waits for every vector memory operation and nothing else.
constexpr int kVmcntWaitAll = (7 << 4) | (15 << 8);

// E4M3 code of a non-negative binary32 a: nearest-even, saturating at 448 (the sign is the caller's).
__device__ __forceinline__ uint32_t e4m3_mag(float a) {
  if (a >= 448.0f) return 0x7Eu;
  const uint32_t u = __builtin_bit_cast(uint32_t, a);
  if (u < 0x3C800000u)  // below 2^-6: the subnormal grid of spacing 2^-9 (code 8 is 2^-6 itself)
    return (uint32_t)__builtin_rintf(a * 512.0f);
  // normal: keep three mantissa bits, nearest-even on the rest, and rebias the exponent (127 -> 7)
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
  return r - ((127u - 7u) << 3);
}

// E2M1 code of a non-negative binary32 a: nearest-even on the grids 0.5 / 1 / 2, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  if (a >= 6.0f) return 7u;
  if (a < 2.0f) return (uint32_t)__builtin_rintf(a * 2.0f);
  if (a < 4.0f) return (uint32_t)__builtin_rintf(a) + 2u;
  return (uint32_t)__builtin_rintf(a * 0.5f) + 4u;
}

// Scale byte of a block whose largest magnitude is amax: floor(log2 amax) - emax + 127, i.e. the
// biased exponent of amax minus emax (8 for E4M3, 2 for E2M1), at least 0 (also for a zero block).
template <int AF>
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
  return (uint32_t)max(e - (AF == kActFp8 ? 8 : 2), 0);
}

// 2^(127 - byte): the factor that maps a block onto its element grid (exact scaling).
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) {
  return __builtin_bit_cast(float, (254u - byte) << 23);
}

template <int AF>
__device__ __forceinline__ uint32_t mx_code(float v, float mult) {
  const uint32_t sign = __builtin_bit_cast(uint32_t, v) >> 31;
  const float a = fabsf(v) * mult;
  return AF == kActFp8 ? ((sign << 7) | e4m3_mag(a)) : ((sign << 3) | e2m1_mag(a));
}

// ---- x quantisation ---------------------------------------------------------------------------

// Four consecutive lanes hold one 32-value block, 8 values (16 bytes) each, so a wave's loads and
// stores are contiguous; the block maximum is a two-step shuffle max within the four lanes.
template <int AF>
__global__ __launch_bounds__(256) void mx_quant_x_kernel(const uint16_t* __restrict__ x, int nchunks,
                                                         uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 8-value chunk, over T * H / 8 (a multiple of 4)
  const bool valid = i < nchunks;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (valid) v = *reinterpret_cast<const uint4*>(x + (size_t)i * 8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo_f32(w[j])), fabsf(bf16_hi_f32(w[j]))));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const uint32_t sb = mx_scale_byte<AF>(amax);
  const float mult = mx_inv_scale(sb);
  if (!valid) return;
  if ((i & 3) == 0) xs[i >> 2] = (uint8_t)sb;
  if (AF == kActFp8) {
    uint32_t o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t a = w[2 * j], b = w[2 * j + 1];
      o[j] = mx_code<AF>(bf16_lo_f32(a), mult) | (mx_code<AF>(bf16_hi_f32(a), mult) << 8) |
             (mx_code<AF>(bf16_lo_f32(b), mult) << 16) | (mx_code<AF>(bf16_hi_f32(b), mult) << 24);
    }
    *reinterpret_cast<uint2*>(xq + (size_t)i * 8) = make_uint2(o[0], o[1]);
  } else {
    uint32_t d = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      d |= (mx_code<AF>(bf16_lo_f32(w[q]), mult) | (mx_code<AF>(bf16_hi_f32(w[q]), mult) << 4)) << (8 * q);
    *reinterpret_cast<uint32_t*>(xq + (size_t)i * 4) = d;
  }
}

// ---- tile list --------------------------------------------------------------------------------

// (expert, first row) of every 256-row tile, experts in index order; -1 past the last tile.
__global__ __launch_bounds__(512) void mx_schedule_kernel(const int32_t* __restrict__ counts, int E, int slots,
                                                          int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_m0) {
  __shared__ int s[512];
  const int t = threadIdx.x;
  const int c = t < E ? counts[t] : 0;
  const int n = (max(c, 0) + kMxTileM - 1) / kMxTileM;
  s[t] = n;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int v = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  const int start = s[t] - n;
  for (int j = 0; j < n; ++j)
    if (start + j < slots) {
      tile_e[start + j] = t;
      tile_m0[start + j] = j * kMxTileM;
    }
  for (int i = s[511] + t; i < slots; i += 512) tile_e[i] = -1;
}

// ---- GEMMs ------------------------------------------------------------------------------------

template <int AF>
struct MxShape {
  static constexpr int kABytes = AF == kActFp8 ? kMxBK : kMxBK / 2;  // activation bytes per row and step
  static constexpr int kCpr = kABytes / 16;                          // 16-byte chunks per activation row
  static constexpr int kATile = kMxTileM * kABytes;
  static constexpr int kBTile = kMxTileN * (kMxBK / 2);
  static constexpr int kScales = (kMxTileM + kMxTileN) * 4;  // one scale dword per row and step
  static constexpr int kStage = kATile + kBTile + kScales;
  static constexpr int kALoads = kATile / (kMxThreads * 16);  // 16-byte direct loads per thread and step
  static constexpr int kBLoads = kBTile / (kMxThreads * 16);
};

// LDS position of 16-byte chunk c of row r: rows are unpadded and the chunks of a row permuted so
// that the operand reads of 16 consecutive rows (one chunk each) hit 64 distinct banks: a 128-byte
// row spans 32 banks, so rows alternate between the two halves and (r >> 1) picks one of 8
// positions; a 64-byte row spans 16 banks, (r & 3) picks the quarter and (r >> 2) the position.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return CPR == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
}

// Weight row (within the expert) of B-tile row n for column tile xblk.
//   gate_up: the wave column group wc = n / 128 owns h columns xblk*128 + wc*64 + [0, 64): B rows
//            [0, 64) of the group are their gate rows, [64, 128) their up rows;
//   down: output column xblk*256 + n (clamped; columns past H are computed and not stored).
template <bool GATEUP>
__device__ __forceinline__ int mx_weight_row(int xblk, int n, int I, int H) {
  if (GATEUP) {
    const int c = xblk * 128 + (n >> 7) * 64 + (n & 63);
    return (n & 64) ? I + c : c;
  }
  return min(xblk * kMxTileN + n, H - 1);
}

// Global sources of one thread's direct loads (advanced by the step offset at each load).
template <int AF>
struct MxSrc {
  const uint8_t* a[MxShape<AF>::kALoads];
  const uint8_t* b[MxShape<AF>::kBLoads];
  const uint8_t* s;
};

// Scale bytes of 512 rows (the tile's activation rows, then its weight rows) for four steps: 16 bytes
// per row, so one load per thread and four steps instead of one dword per thread and step (each a
// separate cache line). Used when K is a multiple of 512.
constexpr int kScaleGroupSteps = 4;
constexpr int kScaleGroupBytes = (kMxTileM + kMxTileN) * 16;

// Direct global -> LDS loads of step s into one stage: one instruction puts the wave's 64 x 16 bytes at
// 1 KB of consecutive LDS, lane l at 16 l. Load j of wave w fills kilobyte w * loads + j of its tile.
// With scale groups (SG) the scales of steps s .. s + 3 go to `sgrp` when s is a multiple of four;
// otherwise each step's scale dword goes to its stage.
template <int AF, bool SG>
__device__ __forceinline__ void mx_gload(const MxSrc<AF>& src, int s, int wave, uint8_t* __restrict__ base,
                                         uint8_t* __restrict__ sgrp) {
  using S = MxShape<AF>;
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j)
    lds_dma16(src.a[j] + (size_t)s * S::kABytes, base + (wave * S::kALoads + j) * 1024);
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j)
    lds_dma16(src.b[j] + (size_t)s * (kMxBK / 2), base + S::kATile + (wave * S::kBLoads + j) * 1024);
  if (SG) {
    if ((s & (kScaleGroupSteps - 1)) == 0)
      lds_dma16(src.s + (size_t)s * (kMxBK / 32), sgrp + wave * 1024);
  } else {
    lds_dma4(src.s + (size_t)s * (kMxBK / 32), base + S::kATile + S::kBTile + wave * 256);
  }
}

// One K-step of one wave: 64 rows x 128 weight rows, K = 128 as two halves of 64 (16 MFMAs). Two LDS
// stages alternate. At step s every wave waits for its own loads of step s (issued during step s - 1)
// and one barrier makes all of them visible; the wave then at once issues the loads of step s + 1 into
// `next`, which every wave finished reading before the barrier (its reads of it had returned: its MFMAs
// of step s - 1 consumed them), and reads the operands of step s from `cur`, each MFMA waiting only for
// its own operands. So the loads of step s + 1 have the whole step to arrive, and no read of a stage
// ever waits on loads into it that are still in flight (the loads are inline assembly, so the compiler
// adds no wait for them before the reads). The barrier carries no memory fence; the empty asm
// statements keep the compiler from moving LDS accesses across it. (With the loads issued after the
// reads, as built-ins, every MFMA of the step waited for all of the step's reads: W4A8 gate_up 248-251
// against 237-238 us, W4A4 216 against 202 us at m1024, same box, two alternations.)
template <int AF, bool SG>
__device__ __forceinline__ void mx_step(const MxSrc<AF>& src, int s, int nsteps, int wave, int wr, int wc, int g,
                                        int r, const uint8_t* cur, uint8_t* next, uint8_t* sg0, uint8_t* sg1,
                                        v16f_t (&acc)[2][4]) {
  using S = MxShape<AF>;
  __builtin_amdgcn_s_waitcnt(kVmcntWaitAll);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (s + 1 < nsteps) mx_gload<AF, SG>(src, s + 1, wave, next, (((s + 1) >> 2) & 1) ? sg1 : sg0);

  const uint8_t* A = cur;
  const uint8_t* B = A + S::kATile;
  // the step's scale dword of row i: SG: word s % 4 of the row's 16 bytes in the current group
  const uint8_t* sgc = ((s >> 2) & 1) ? sg1 : sg0;
  const uint32_t* SA = SG ? reinterpret_cast<const uint32_t*>(sgc) + (s & 3)
                          : reinterpret_cast<const uint32_t*>(B + S::kBTile);
  const int sstride = SG ? 4 : 1;  // dwords per row
  const uint32_t* SB = SA + kMxTileM * sstride;
  uint32_t sa[2], sb[4];
  uint4 alo[2][2], ahi[2][2], bv[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) sa[mi] = SA[(wr * 64 + mi * 32 + r) * sstride];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) sb[ni] = SB[(wc * 128 + ni * 32 + r) * sstride];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int row = wr * 64 + mi * 32 + r;
      const uint8_t* p = A + row * S::kABytes;
      if (AF == kActFp8) {
        alo[ks][mi] = *reinterpret_cast<const uint4*>(p + swz<8>(row, ks * 4 + g) * 16);
        ahi[ks][mi] = *reinterpret_cast<const uint4*>(p + swz<8>(row, ks * 4 + 2 + g) * 16);
      } else {
        alo[ks][mi] = *reinterpret_cast<const uint4*>(p + swz<4>(row, ks * 2 + g) * 16);
      }
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = wc * 128 + ni * 32 + r;
      bv[ks][ni] = *reinterpret_cast<const uint4*>(B + n * (kMxBK / 2) + swz<4>(n, ks * 2 + g) * 16);
    }
  }

#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int sh = 8 * (2 * ks + g);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const uint4 v = bv[ks][ni];
      const v8i_t bq = v8i_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint4 lo = alo[ks][mi];
        const uint4 hi = AF == kActFp8 ? ahi[ks][mi] : make_uint4(0, 0, 0, 0);
        const v8i_t af = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            af, bq, acc[mi][ni], AF == kActFp8 ? 0 : 4, 4, 0, (int)(sa[mi] >> sh), 0, (int)(sb[ni] >> sh));
      }
    }
  }
}

template <bool GATEUP, int AF, bool SG>
__global__ __launch_bounds__(kMxThreads, 1) void mx_gemm_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, int k, int H, int I, int nx,
    int slots, const int32_t* __restrict__ tile_e, const int32_t* __restrict__ tile_m0,
    const uint8_t* __restrict__ wq_all, const uint8_t* __restrict__ ws_all, float clamp,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, float* __restrict__ y) {
  using S = MxShape<AF>;
  __shared__ __attribute__((aligned(16))) uint8_t st0[SG ? S::kStage - S::kScales : S::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SG ? S::kStage - S::kScales : S::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t sg0[SG ? kScaleGroupBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sg1[SG ? kScaleGroupBytes : 16];

  // XCD-interleaved order (workgroup b runs on XCD b % 8): XCD x takes row tiles x, x + 8, ... with
  // all their column tiles back to back, so a row tile's activations stay in one L2
  const int b = blockIdx.x;
  const int jb = b >> 3;
  const int ys = (b & 7) + 8 * (jb / nx);
  const int xblk = jb % nx;
  if (ys >= slots) return;
  const int te = tile_e[ys];
  if (te < 0) return;
  const int e = uniform_i(te);
  const int m0 = uniform_i(tile_m0[ys]);
  const int rows = min(kMxTileM, uniform_i(counts[e]) - m0);
  const int row0 = uniform_i(offsets[e]) + m0;
  if (rows <= 0) return;

  const int K = GATEUP ? H : I;
  const int nsteps = K / kMxBK;
  const size_t arow_bytes = AF == kActFp8 ? (size_t)K : (size_t)K / 2;
  const int nbk = K >> 5;  // scale bytes per row
  const size_t nrows_w = GATEUP ? (size_t)2 * I : (size_t)H;
  const uint8_t* qe = wq_all + (size_t)e * nrows_w * (size_t)(K >> 1);
  const uint8_t* se = ws_all + (size_t)e * nrows_w * (size_t)nbk;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // activation row of tile row r (rows past the expert's last repeat its last row; never stored)
  auto act_row = [&](int r) -> size_t {
    const int rr = row0 + min(r, rows - 1);
    return GATEUP ? (size_t)(sorted_pair[rr] / k) : (size_t)rr;
  };

  // Lane l of load j of wave w writes 16 bytes at 16 l of LDS kilobyte w * loads + j of its tile: it
  // takes the row and swizzled position that place holds and fetches the chunk that belongs there.
  constexpr int CPR = S::kCpr, NA = S::kALoads, NB = S::kBLoads;
  const uint8_t* a_src[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = (wave * NA + j) * (1024 / S::kABytes) + lane / CPR;
    a_src[j] = aq + act_row(r) * arow_bytes + swz<CPR>(r, lane % CPR) * 16;
  }
  const uint8_t* b_src[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = (wave * NB + j) * 16 + lane / 4;
    b_src[j] = qe + (size_t)mx_weight_row<GATEUP>(xblk, n, I, H) * (size_t)(K >> 1) + swz<4>(n, lane % 4) * 16;
  }
  // scales: waves 0-3 the activation rows (row = tid), waves 4-7 the weight rows (row = tid - 256)
  const uint8_t* s_src = tid < kMxTileM
                             ? as + act_row(tid) * (size_t)nbk
                             : se + (size_t)mx_weight_row<GATEUP>(xblk, tid - kMxTileM, I, H) * (size_t)nbk;

  MxSrc<AF> src;
#pragma unroll
  for (int jj = 0; jj < NA; ++jj) src.a[jj] = a_src[jj];
#pragma unroll
  for (int jj = 0; jj < NB; ++jj) src.b[jj] = b_src[jj];
  src.s = s_src;

  const int wr = wave >> 1, wc = wave & 1;
  const int g = lane >> 5, r = lane & 31;
  v16f_t acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

  mx_gload<AF, SG>(src, 0, wave, st0, sg0);
  for (int s = 0; s < nsteps; s += 2) {
    mx_step<AF, SG>(src, s, nsteps, wave, wr, wc, g, r, st0, st1, sg0, sg1, acc);
    if (s + 1 < nsteps) mx_step<AF, SG>(src, s + 1, nsteps, wave, wr, wc, g, r, st1, st0, sg0, sg1, acc);
  }
  __builtin_amdgcn_s_waitcnt(kVmcntWaitAll);  // no load into LDS outlives the loop

  if (GATEUP) {
    // h = silu(g) * u per element, then each row's 32-column block quantised: the block is column r
    // of the 32 lanes of one half-wave
    const size_t hrow_bytes = AF == kActFp8 ? (size_t)I : (size_t)I / 2;
    const int nbi = I >> 5;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nh = 0; nh < 2; ++nh) {
        const int col = xblk * 128 + wc * 64 + nh * 32 + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float gv = acc[mi][nh][i], uv = acc[mi][nh + 2][i];
          if (clamp > 0.0f) {
            gv = clampf(gv, clamp);
            uv = clampf(uv, clamp);
          }
          const float h = silu_mul(gv, uv);
          float m = fabsf(h);
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
          const uint32_t sbyte = mx_scale_byte<AF>(m);
          const uint32_t code = mx_code<AF>(h, mx_inv_scale(sbyte));
          const uint32_t partner = AF == kActFp8 ? 0u : (uint32_t)__shfl_xor((int)code, 1, kWave);
          const int rl = wr * 64 + mi * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (rl < rows) {
            const size_t R = (size_t)(row0 + rl);
            if (AF == kActFp8) {
              hq[R * hrow_bytes + col] = (uint8_t)code;
            } else if ((r & 1) == 0) {
              hq[R * hrow_bytes + (col >> 1)] = (uint8_t)(code | (partner << 4));
            }
            if (r == 0) hs[R * (size_t)nbi + (col >> 5)] = (uint8_t)sbyte;
          }
        }
      }
  } else {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int col = xblk * kMxTileN + wc * 128 + ni * 32 + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = wr * 64 + mi * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (rl < rows && col < H) y[(size_t)(row0 + rl) * H + col] = acc[mi][ni][i];
        }
      }
  }
}

template <bool GATEUP, int AF, bool SG>
hipError_t launch_mx_gemm_sg(const MxPlan& mp, const uint8_t* aq, const uint8_t* as, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pair, int k, int H, int I,
                          const int32_t* tile_e, const int32_t* tile_m0, const uint8_t* wq, const uint8_t* ws,
                          float clamp, uint8_t* hq, uint8_t* hs, float* y, hipStream_t stream) {
  auto kern = &mx_gemm_kernel<GATEUP, AF, SG>;
  const int nx = GATEUP ? mp.gu_grid_x : mp.dn_grid_x;
  const int blocks = GATEUP ? mp.gu_blocks : mp.dn_blocks;
  kern<<<blocks, kMxThreads, 0, stream>>>(aq, as, counts, offsets, sorted_pair, k, H, I, nx, mp.slots,
                                                 tile_e, tile_m0, wq, ws, clamp, hq, hs, y);
  return hipGetLastError();
}

// Scale groups of four steps when K is a multiple of 512 (every group's 16 bytes then lie inside its row).
template <bool GATEUP, int AF>
hipError_t launch_mx_gemm(const MxPlan& mp, const uint8_t* aq, const uint8_t* as, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pair, int k, int H, int I,
                          const int32_t* tile_e, const int32_t* tile_m0, const uint8_t* wq, const uint8_t* ws,
                          float clamp, uint8_t* hq, uint8_t* hs, float* y, hipStream_t stream) {
  const int K = GATEUP ? H : I;
  if (K % (kMxBK * kScaleGroupSteps) == 0)
    return launch_mx_gemm_sg<GATEUP, AF, true>(mp, aq, as, counts, offsets, sorted_pair, k, H, I, tile_e, tile_m0, wq,
                                               ws, clamp, hq, hs, y, stream);
  return launch_mx_gemm_sg<GATEUP, AF, false>(mp, aq, as, counts, offsets, sorted_pair, k, H, I, tile_e, tile_m0, wq,
                                              ws, clamp, hq, hs, y, stream);
}

}  // namespace

int mx_slots_bound(int T, int E, int k) {
  const long P = (long)T * k;
  return (int)(P / kMxTileM + (E < P ? (long)E : P) + 1);
}

MxPlan plan_mx(int T, int H, int I, int E, int k) {
  MxPlan mp;
  mp.slots = mx_slots_bound(T, E, k);
  mp.gu_grid_x = I / 128;
  mp.dn_grid_x = (H + kMxTileN - 1) / kMxTileN;
  const int slot_groups = (mp.slots + 7) / 8;
  mp.gu_blocks = slot_groups * 8 * mp.gu_grid_x;
  mp.dn_blocks = slot_groups * 8 * mp.dn_grid_x;
  return mp;
}

hipError_t launch_mx_schedule(const int32_t* counts, int E, const MxPlan& mp, int32_t* tile_e, int32_t* tile_m0,
                              hipStream_t stream) {
  mx_schedule_kernel<<<1, 512, 0, stream>>>(counts, E, mp.slots, tile_e, tile_m0);
  return hipGetLastError();
}

hipError_t launch_mx_quant_x(const uint16_t* x, int T, int H, int act, uint8_t* xq, uint8_t* xs,
                             hipStream_t stream) {
  const int nchunks = T * (H / 8);
  const int grid = (nchunks + 255) / 256;
  if (act == kActFp8)
    mx_quant_x_kernel<kActFp8><<<grid, 256, 0, stream>>>(x, nchunks, xq, xs);
  else
    mx_quant_x_kernel<kActFp4><<<grid, 256, 0, stream>>>(x, nchunks, xq, xs);
  return hipGetLastError();
}

hipError_t launch_mx_gateup(const MxPlan& mp, int act, const uint8_t* xq, const uint8_t* xs, const int32_t* counts,
                            const int32_t* offsets, const int32_t* sorted_pair, int k, int H, int I,
                            const int32_t* tile_e, const int32_t* tile_m0, const uint8_t* w13_q,
                            const uint8_t* w13_s, float clamp, uint8_t* hq, uint8_t* hs, hipStream_t stream) {
  if (act == kActFp8)
    return launch_mx_gemm<true, kActFp8>(mp, xq, xs, counts, offsets, sorted_pair, k, H, I, tile_e, tile_m0, w13_q,
                                         w13_s, clamp, hq, hs, nullptr, stream);
  return launch_mx_gemm<true, kActFp4>(mp, xq, xs, counts, offsets, sorted_pair, k, H, I, tile_e, tile_m0, w13_q,
                                       w13_s, clamp, hq, hs, nullptr, stream);
}

hipError_t launch_mx_down(const MxPlan& mp, int act, const uint8_t* hq, const uint8_t* hs, const int32_t* counts,
                          const int32_t* offsets, int k, int H, int I, const int32_t* tile_e,
                          const int32_t* tile_m0, const uint8_t* w2_q, const uint8_t* w2_s, float* y,
                          hipStream_t stream) {
  if (act == kActFp8)
    return launch_mx_gemm<false, kActFp8>(mp, hq, hs, counts, offsets, nullptr, k, H, I, tile_e, tile_m0, w2_q,
                                          w2_s, 0.0f, nullptr, nullptr, y, stream);
  return launch_mx_gemm<false, kActFp4>(mp, hq, hs, counts, offsets, nullptr, k, H, I, tile_e, tile_m0, w2_q, w2_s,
                                        0.0f, nullptr, nullptr, y, stream);
}

}  // namespace moe
