// Device helpers shared by the MLA gather-decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint16_t bf16_t;

constexpr int kBlock = 256;  // threads per workgroup for every kernel (4 waves)
constexpr int kWave = 64;

// bf16 <-> fp32.  A bf16 word is the top half of an fp32 word.
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ void unpack8(const uint4 v, float* w) {
  w[0] = bf16lo(v.x); w[1] = bf16hi(v.x);
  w[2] = bf16lo(v.y); w[3] = bf16hi(v.y);
  w[4] = bf16lo(v.z); w[5] = bf16hi(v.z);
  w[6] = bf16lo(v.w); w[7] = bf16hi(v.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over the workgroup; every thread gets the result.  `scratch` holds >= 4 floats
// and must not be in use by the caller across this call.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / kWave; ++i) s += scratch[i];
  return s;
}

}  // namespace mla
