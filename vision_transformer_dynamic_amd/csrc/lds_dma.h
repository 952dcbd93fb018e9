// Direct-to-LDS loads and the waits that track them (gfx950), shared by the
// kernels that stage every routed key of a head in LDS.
#pragma once

#include "attn_common.h"

namespace bra {

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maximum
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most n of the wave's vector memory loads are outstanding
// (n clamped to 15: waiting for more of them is always safe).
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  switch (n < 15 ? n : 15) {
#define BRA_W(k) case k: wait_vmcnt<k>(); break;
    BRA_W(0) BRA_W(1) BRA_W(2) BRA_W(3) BRA_W(4) BRA_W(5) BRA_W(6) BRA_W(7)
    BRA_W(8) BRA_W(9) BRA_W(10) BRA_W(11) BRA_W(12) BRA_W(13) BRA_W(14)
#undef BRA_W
    default: wait_vmcnt<15>(); break;
  }
}

typedef __attribute__((address_space(3))) shortx4 lds_s4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// One direct-to-LDS load: 16 bytes per lane from gptr into the wave's 1 KB
// block at LDS byte offset lds_off (uniform), lane l at lds_off + 16 l. The
// instruction's address registers are read when it issues and it writes no
// register, so nothing of it is pending in registers afterwards; its
// completion is tracked by the wave's vector-memory counter only, which the
// kernels' phase loops wait on explicitly (wait_vmcnt) before any read of the
// block. (The compiler cannot count these loads across the runtime-length
// issue loops, so its own wait would be for all of them.)
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_off) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((const lds_u8*)p));
}

}  // namespace bra
