// Skinny GEMV building blocks (VALU, few tokens) and deterministic split-K reduction.
#pragma once

#include "device_util.h"

namespace mla {

constexpr int kTile = 512;  // output columns per GEMV tile: 64 lanes x 8 bf16
constexpr int kTT = 8;      // tokens per pass of the VALU GEMV
constexpr int kUnroll = 8;  // 16-byte weight loads in flight per lane

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte weight load that does not allocate in the caches on the way.
__device__ __forceinline__ u32x4 ld_stream(const bf16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void unpack8v(const u32x4 v, float* w) {
  w[0] = bf16lo(v[0]); w[1] = bf16hi(v[0]);
  w[2] = bf16lo(v[1]); w[3] = bf16hi(v[1]);
  w[4] = bf16lo(v[2]); w[5] = bf16hi(v[2]);
  w[6] = bf16lo(v[3]); w[7] = bf16hi(v[3]);
}

// dst[i] = sum_{s < S} src[s*sstride + (i / w)*tstride + (i % w)] for i < n.
// Deterministic: part sp of nsp sums s = sp, sp+nsp, ... in order, then the parts
// are added in order.  dst and scratch are LDS; scratch holds 256 floats.
// Every thread of the workgroup must call it.
__device__ __forceinline__ void reduce_parts(const float* __restrict__ src, size_t sstride, int S, int n, int w,
                                             size_t tstride, float* dst, float* scratch) {
  const int tid = threadIdx.x;
  int nsp = (n > 0) ? kBlock / n : 1;
  nsp = max(1, min(nsp, 16));
  float* out = (nsp == 1) ? dst : scratch;
  for (int idx = tid; idx < n * nsp; idx += kBlock) {
    const int i = idx % n, sp = idx / n;
    const float* s0 = src + (size_t)(i / w) * tstride + (i % w);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int s = sp;
    for (; s + 3 * nsp < S; s += 4 * nsp) {
      a0 += s0[(size_t)s * sstride];
      a1 += s0[(size_t)(s + nsp) * sstride];
      a2 += s0[(size_t)(s + 2 * nsp) * sstride];
      a3 += s0[(size_t)(s + 3 * nsp) * sstride];
    }
    for (; s < S; s += nsp) a0 += s0[(size_t)s * sstride];
    out[sp * n + i] = (a0 + a1) + (a2 + a3);
  }
  __syncthreads();
  if (nsp > 1) {
    for (int i = tid; i < n; i += kBlock) {
      float a = 0.f;
      for (int sp = 0; sp < nsp; ++sp) a += scratch[sp * n + i];
      dst[i] = a;
    }
    __syncthreads();
  }
}

// One GEMV tile for up to kTT tokens:
//   out[tt*ldo + c0 + c] = sum_{r < ks} xs[tt*xstride + r] * W[(k0 + r)*N + c0 + c],  c < nc <= 512.
// W is [K, N] row-major bf16 (N and nc multiples of 8), xs is LDS.  Lanes of a
// wave cover one row with lpr lanes (8 columns each) and 64/lpr rows at once;
// the four waves take interleaved rows; kUnroll loads per lane are in flight.
// Partial sums are combined across lanes by shuffles and across waves in LDS
// (`red`: 3*kTT*512 floats).
__device__ __forceinline__ void gemv_tile(const bf16_t* __restrict__ W, int N, int k0, int ks, int c0, int nc,
                                          const float* xs, int xstride, int nt, float* __restrict__ out,
                                          size_t ldo, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ngroups = nc >> 3;
  int lpr = 64;
  while (lpr > 8 && (lpr >> 1) >= ngroups) lpr >>= 1;
  const int rpi = 64 / lpr;
  const int cg = lane % lpr, rsub = lane / lpr;
  const bool active = cg < ngroups;
  const int rstep = 4 * rpi;
  float acc[kTT][8];
#pragma unroll
  for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[tt][i] = 0.f;
  const bf16_t* wp = W + (size_t)k0 * N + c0 + 8 * cg;
  for (int r0 = wv * rpi + rsub; r0 < ks; r0 += rstep * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int r = r0 + u * rstep;
      if (active && r < ks) v[u] = ld_stream(wp + (size_t)r * N);
      else v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int r = min(r0 + u * rstep, ks - 1);  // out-of-range rows carry zero weights
      float w[8];
      unpack8v(v[u], w);
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) {
        if (tt < nt) {
          const float xv = xs[tt * xstride + r];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[tt][i] = fmaf(xv, w[i], acc[tt][i]);
        }
      }
    }
  }
  for (int off = lpr; off < 64; off <<= 1)
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
      if (tt < nt)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[tt][i] += __shfl_xor(acc[tt][i], off, kWave);
  if (wv > 0 && rsub == 0 && active) {
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
      if (tt < nt)
#pragma unroll
        for (int i = 0; i < 8; ++i) red[((wv - 1) * kTT + tt) * kTile + 8 * cg + i] = acc[tt][i];
  }
  __syncthreads();
  if (wv == 0 && rsub == 0 && active) {
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      if (tt < nt) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          o[i] = acc[tt][i] + red[(0 * kTT + tt) * kTile + 8 * cg + i] + red[(1 * kTT + tt) * kTile + 8 * cg + i] +
                 red[(2 * kTT + tt) * kTile + 8 * cg + i];
        float4* dst = reinterpret_cast<float4*>(out + (size_t)tt * ldo + c0 + 8 * cg);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
  __syncthreads();
}

}  // namespace mla
