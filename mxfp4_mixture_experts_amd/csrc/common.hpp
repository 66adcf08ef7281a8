// Device helpers shared by the gfx950 kernels of the routed MXFP4 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// E8M0 scale byte s -> the binary32 2^(s-127), built from its exponent field. Exact for s in
// [1, 254]; the library's contract covers s in [2, 254] (decoded values stay normal binary32).
__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  return __builtin_bit_cast(float, s << 23);
}

// Round a binary32 to bfloat16, nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// h of a routed pair as two bfloat16 planes: hi = bf16(v), lo = bf16(v - hi). hi + lo is exact in
// fp32 and equals v to about 2^-17 relative. Returns the hi bits.
__device__ __forceinline__ uint16_t store_h_planes(uint16_t* hi, uint16_t* lo, size_t o, float v) {
  const uint16_t h = f32_to_bf16_rne(v);
  hi[o] = h;
  lo[o] = f32_to_bf16_rne(v - __builtin_bit_cast(float, (uint32_t)h << 16));
  return h;
}

// The two bf16 halves of a dword as floats (element 0 in the low half).
__device__ __forceinline__ float bf16_lo_f32(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// Two E2M1 codes (byte `sel` of `w`: low nibble = even element) times `scale` -> two bf16 in one
// dword, the even element in the low half. Exact for normal results.
template <int sel>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, sel);
}

// Two E2M1 codes (byte `sel` of `w`) as fp16 values, unscaled (E2M1 values are exact in fp16).
template <int sel>
__device__ __forceinline__ f16x2_t fp4x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, sel);
}

// Two E2M1 codes (byte `sel` of `w`) times `scale` -> two fp16 (nearest-even; the even element in
// the low half). Exact while the results are fp16 normals or multiples of 2^-24 below 65504.
template <int sel>
__device__ __forceinline__ f16x2_t fp4x2_to_f16x2_scaled(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, sel);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }
__device__ __forceinline__ f16x2_t as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2_t, v); }

// acc + a.lo*b.lo + a.hi*b.hi in fp32 (products of two fp16 are exact in fp32).
__device__ __forceinline__ float dot2_f16(f16x2_t a, f16x2_t b, float acc) {
  return __builtin_amdgcn_fdot2(a, b, acc, false);
}

// acc + a.lo*b.lo + a.hi*b.hi in fp32 (products of two bf16 are exact in fp32).
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

// silu(g) * u = g * u / (1 + exp(-g)), with the hardware exp2 and reciprocal (each about 1 ulp);
// exp(-g) overflowing to +inf for very negative g gives the correct limit -0.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float clampf(float v, float c) { return fminf(fmaxf(v, -c), c); }

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Lane 63's value, uniform (a scalar read of the lane, no LDS traffic); every lane must be active.
__device__ __forceinline__ int wave_last(int v) { return __builtin_amdgcn_readlane(v, 63); }

// v plus a DPP-moved copy of v; lanes whose source is outside the row or the row mask add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_i32(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave (all active), in registers: within each row of 16 lanes by
// shifts of 1, 2, 4 and 8 lanes (row_shr), then the last lane of row 0 into row 1 and of row 2 into
// row 3 (row_bcast:15), then the last lane of row 1 into rows 2 and 3 (row_bcast:31). `lane` is
// unused (kept for the call sites).
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
  (void)lane;
  v = dpp_add_i32<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add_i32<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add_i32<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add_i32<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add_i32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add_i32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Lanes of the wave holding the same key (keys in [0, 1024)), restricted to lanes with `valid`.
__device__ __forceinline__ uint64_t match_key(int key, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    bool bit = (key >> b) & 1;
    uint64_t ones = __ballot(bit);
    m &= bit ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

}  // namespace moe
