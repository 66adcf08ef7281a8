// Device code shared by the weight-streaming MXFP4 kernels (small per-expert M) and the single-launch
// decode layer: block dot products of decoded E2M1 codes against activations, the fp16 block format
// of the down GEMM's activations, segmented DPP reductions and load helpers.
#pragma once

#include "common.hpp"

namespace moe {
namespace stream_dev {

__device__ __forceinline__ int ilog2(int v) { return 31 - __clz(v); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 16 bytes / 1 byte at a uniform base plus a 32-bit per-lane offset (lets the compiler use the
// scalar-base addressing form, one VGPR per address)
__device__ __forceinline__ uint4 ld16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint32_t ld8(const uint8_t* base, uint32_t off) { return base[off]; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 code bytes of a weight row, loaded non-temporal (the nt cache-policy bit): the weight-streaming
// kernels read each byte of their experts' codes once per launch, and each 128-byte line of codes is
// requested by exactly one load, so the lines need not stay in the caches. On MI355X a load-only probe
// of the decode access patterns streamed 10-13% faster this way (gate_up layout 5.5 -> 6.2 TB/s, down
// 4.9 -> 5.5 TB/s), and the decode layer at M=2 / M=8 ran 2% / 7% faster. The scale bytes keep
// ordinary loads, since several loads share each line of scales. The row-tile MFMA kernels and the
// single-launch layer measured slower with nt code loads and do not use them.
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* base, uint32_t off) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + off));
  return make_uint4(v.x, v.y, v.z, v.w);
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

}  // namespace stream_dev
}  // namespace moe
