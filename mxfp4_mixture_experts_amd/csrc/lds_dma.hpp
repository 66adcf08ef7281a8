// Direct global -> LDS loads for the MFMA kernels.
#pragma once

#include "common.hpp"

namespace moe {

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) that
// waits until at most n vector memory operations are outstanding (0 <= n < 64), nothing else.
constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// One direct load of 16 bytes a lane from global memory into LDS: lane l's bytes land at lds + 16 l
// (lds wave-uniform, given to M0, one wait state before the load uses it). Written as inline assembly
// so that the compiler, which cannot tell the LDS such a load writes apart from the LDS a kernel reads,
// adds no wait for it before every later LDS read: the kernel waits for it itself (s_waitcnt vmcnt and
// a barrier) before any wave reads what it wrote. The load has no register result.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0v) : "memory");
}

// The same with 4 bytes a lane (lane l's dword at lds + 4 l).
__device__ __forceinline__ void lds_dma4(const void* g, void* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0v) : "memory");
}

}  // namespace moe
