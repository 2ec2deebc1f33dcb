// lds_dma.h -- global memory straight into LDS (buffer_load ... lds).
//
// A wave's buffer_load_dword{,x4} ... lds writes lane i's 4 (16) bytes at
// LDS byte address m0 + 4 i (16 i), from whatever buffer offset the lane
// names; no register receives data.  The GEMMs that stage tiles this way wait
// for the loads themselves (vmcnt) before the barrier that publishes a stage.
#pragma once

#include "gemv_core.h"

namespace moe {

typedef int i32x4r_t __attribute__((ext_vector_type(4)));

// buffer resource words for a byte range (as make_rsrc), for the asm below
__device__ __forceinline__ i32x4r_t rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return (i32x4r_t){(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)bytes,
                    (int)kBufDword3};
}

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}

// Written as asm so that the compiler, which cannot tell which LDS buffer
// such a load writes, does not make every later LDS read wait for it.  lds:
// a wave-uniform LDS byte address; vo: this lane's buffer offset.
__device__ __forceinline__ void lds_load16(i32x4r_t r, uint32_t lds, uint32_t vo) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(vo), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(i32x4r_t r, uint32_t lds, uint32_t vo) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(vo), "s"(r)
               : "memory", "m0");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt n (n < 16), the other counters
// not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8); }

}  // namespace moe
