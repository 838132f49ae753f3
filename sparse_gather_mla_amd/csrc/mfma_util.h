// Matrix-core and LDS-DMA helpers for gfx950 (wave64): operand vector types,
// explicit vector-memory waits and direct global-to-LDS loads.
#pragma once

#include "device_util.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_cvoid_t;

// s_waitcnt (gfx9 encoding) until at most N vector-memory operations of this
// wave are outstanding; the other counters are left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Direct global->LDS load of 16 bytes per lane: lane l's bytes land at
// lds_base + 16*l (lds_base is wave-uniform).  Issued from asm so that the
// compiler does not tie later LDS reads of other ring buffers to it; the ring
// waits on vmcnt explicitly instead.  The load is non-temporal: on this chip a
// stream of cached loads tops out at well under half the HBM rate that the
// same stream reaches with the nt policy.
__device__ __forceinline__ void dma16(const void* src, const void* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(m0), "v"(src) : "memory", "m0");
}

}  // namespace mla
