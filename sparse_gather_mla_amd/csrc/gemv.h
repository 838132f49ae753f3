// Skinny GEMV building blocks (VALU, few tokens) and deterministic split-K reduction.
#pragma once

#include "device_util.h"
#include "handoff.h"

namespace mla {

constexpr int kTile = 512;  // output columns per GEMV tile: 64 lanes x 8 bf16
constexpr int kTT = 4;      // most tokens per pass of the VALU GEMV (the GEMV path takes up to 3)

// 16-byte weight loads in flight per lane: a one-token pass holds few
// accumulators, so it keeps twice as many loads in flight.
__host__ __device__ constexpr int gemv_unroll(int ntt) { return ntt == 1 ? 16 : 8; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte weight load (non-temporal: the weight is read once).
__device__ __forceinline__ u32x4 ld_stream(const bf16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// fp16 words of a 32-bit pair
__device__ __forceinline__ float f16lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

// eight fp16 values of a 16-byte piece
__device__ __forceinline__ void unpack8vh(const u32x4 v, float* w) {
  w[0] = f16lo(v[0]); w[1] = f16hi(v[0]);
  w[2] = f16lo(v[1]); w[3] = f16hi(v[1]);
  w[4] = f16lo(v[2]); w[5] = f16hi(v[2]);
  w[6] = f16lo(v[3]); w[7] = f16hi(v[3]);
}

__device__ __forceinline__ void unpack8v(const u32x4 v, float* w) {
  w[0] = bf16lo(v[0]); w[1] = bf16hi(v[0]);
  w[2] = bf16lo(v[1]); w[3] = bf16hi(v[1]);
  w[4] = bf16lo(v[2]); w[5] = bf16hi(v[2]);
  w[6] = bf16lo(v[3]); w[7] = bf16hi(v[3]);
}

// dst[i] = sum_{s < S} src[s*sstride + (i / w)*tstride + (i % w)] for i < n (floats).
// Deterministic: part sp of nsp sums s = sp, sp+nsp, ... in order (loaded
// eight at a time, so that up to 8*nsp slabs take one round trip), then the
// parts are added in order.  dst and scratch (256 floats) are LDS.  Every
// thread of the workgroup must call it.  `sy` loads the partials (handoff.h).
template <class Sy = HandoffNone>
__device__ __forceinline__ void reduce_parts(const float* __restrict__ src, size_t sstride, int S, int n, int w,
                                             size_t tstride, float* dst, float* scratch, const Sy& sy = Sy()) {
  const int tid = threadIdx.x;
  int nsp = (n > 0) ? kBlock / n : 1;
  nsp = max(1, min(nsp, 16));
  float* out = (nsp == 1) ? dst : scratch;
  for (int idx = tid; idx < n * nsp; idx += kBlock) {
    const int i = idx % n, sp = idx / n;
    const float* s0 = src + (size_t)(i / w) * tstride + (i % w);
    float a = 0.f;
    for (int s = sp; s < S; s += 8 * nsp) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (s + u * nsp < S) ? sy.ld(s0 + (size_t)(s + u * nsp) * sstride) : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) a += v[u];
    }
    out[sp * n + i] = a;
  }
  __syncthreads();
  if (nsp > 1) {
    for (int i = tid; i < n; i += kBlock) {
      float acc = 0.f;
      for (int sp = 0; sp < nsp; ++sp) acc += scratch[sp * n + i];
      dst[i] = acc;
    }
    __syncthreads();
  }
}

// As reduce_parts for groups of 4 floats: items are float4 at element offset
// (i / w4)*tstride + 4*(i % w4); tstride and the source must be 16-byte
// aligned.  scratch holds 256 float4.
template <class Sy = HandoffNone>
__device__ __forceinline__ void reduce_parts4(const float* __restrict__ src, size_t sstride, int S, int n4, int w4,
                                              size_t tstride, float* dst, float* scratch, const Sy& sy = Sy()) {
  const int tid = threadIdx.x;
  int nsp = (n4 > 0) ? kBlock / n4 : 1;
  nsp = max(1, min(nsp, 16));
  float4* out = reinterpret_cast<float4*>((nsp == 1) ? dst : scratch);
  for (int idx = tid; idx < n4 * nsp; idx += kBlock) {
    const int i = idx % n4, sp = idx / n4;
    const float* s0 = src + (size_t)(i / w4) * tstride + 4 * (i % w4);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = sp; s < S; s += 8 * nsp) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = (s + u * nsp < S) ? sy.ld4(s0 + (size_t)(s + u * nsp) * sstride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a.x += v[u].x; a.y += v[u].y; a.z += v[u].z; a.w += v[u].w;
      }
    }
    out[sp * n4 + i] = a;
  }
  __syncthreads();
  if (nsp > 1) {
    const float4* sc = reinterpret_cast<const float4*>(scratch);
    float4* d = reinterpret_cast<float4*>(dst);
    for (int i = tid; i < n4; i += kBlock) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int sp = 0; sp < nsp; ++sp) {
        const float4 v = sc[sp * n4 + i];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      d[i] = acc;
    }
    __syncthreads();
  }
}

// Lane geometry of one GEMV tile: a row of nc columns is covered by lpr lanes
// (8 columns each), a wave covers 64/lpr rows at once, the four waves take
// interleaved rows.
struct GemvGeom {
  int lpr, rpi, cg, rsub, rstep, r0;
  bool active;
};
__device__ __forceinline__ GemvGeom gemv_geom(int nc) {
  GemvGeom g;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ngroups = nc >> 3;
  g.lpr = 64;
  while (g.lpr > 8 && (g.lpr >> 1) >= ngroups) g.lpr >>= 1;
  g.rpi = 64 / g.lpr;
  g.cg = lane % g.lpr;
  g.rsub = lane / g.lpr;
  g.active = g.cg < ngroups;
  g.rstep = 4 * g.rpi;
  g.r0 = wv * g.rpi + g.rsub;
  return g;
}

// The first UNR weight loads of a tile, issued before the activations are ready.
template <int UNR>
__device__ __forceinline__ void gemv_first(const bf16_t* __restrict__ W, int N, int k0, int ks, int c0, int nc,
                                           u32x4* v) {
  const GemvGeom g = gemv_geom(nc);
  const bf16_t* wp = W + (size_t)k0 * N + c0 + 8 * g.cg;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int r = g.r0 + u * g.rstep;
    if (g.active && r < ks) v[u] = ld_stream(wp + (size_t)r * N);
    else v[u] = u32x4{0u, 0u, 0u, 0u};
  }
}

// One GEMV tile for up to NTT tokens:
//   out[tt*ldo + c0 + c] = sum_{r < ks} xs[tt*xstride + r] * W[(k0 + r)*N + c0 + c],  c < nc <= 512.
// W is [K, N] row-major bf16 (N and nc multiples of 8), xs is LDS.  `v` holds
// the loads of gemv_first<UNR>.  Lanes of equal column combine by shuffles,
// waves through LDS (`red`: 3*NTT*512 floats).  The output goes out through
// the hand-off policy `sy` (handoff.h).  kHalf: W holds fp16 instead of bf16.
template <int NTT, int UNR, class Sy = HandoffNone, bool kHalf = false>
__device__ __forceinline__ void gemv_tile(const bf16_t* __restrict__ W, int N, int k0, int ks, int c0, int nc,
                                          const float* xs, int xstride, int nt, float* __restrict__ out,
                                          size_t ldo, float* red, u32x4* v, const Sy& sy = Sy()) {
  const GemvGeom g = gemv_geom(nc);
  const int wv = threadIdx.x >> 6;
  float acc[NTT][8];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[tt][i] = 0.f;
  const bf16_t* wp = W + (size_t)k0 * N + c0 + 8 * g.cg;
  for (int r0 = g.r0; r0 < ks; r0 += g.rstep * UNR) {
    if (r0 != g.r0) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + u * g.rstep;
        if (g.active && r < ks) v[u] = ld_stream(wp + (size_t)r * N);
        else v[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int r = min(r0 + u * g.rstep, ks - 1);  // rows past the slab carry zero weights
      float w[8];
      if constexpr (kHalf) unpack8vh(v[u], w);
      else unpack8v(v[u], w);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        if (tt < nt) {
          const float xv = xs[tt * xstride + r];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[tt][i] = fmaf(xv, w[i], acc[tt][i]);
        }
      }
    }
  }
  for (int off = g.lpr; off < 64; off <<= 1)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
      if (tt < nt)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[tt][i] += __shfl_xor(acc[tt][i], off, kWave);
  if (wv > 0 && g.rsub == 0 && g.active) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
      if (tt < nt)
#pragma unroll
        for (int i = 0; i < 8; ++i) red[((wv - 1) * NTT + tt) * kTile + 8 * g.cg + i] = acc[tt][i];
  }
  __syncthreads();
  if (wv == 0 && g.rsub == 0 && g.active) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      if (tt < nt) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          o[i] = acc[tt][i] + red[(0 * NTT + tt) * kTile + 8 * g.cg + i] + red[(1 * NTT + tt) * kTile + 8 * g.cg + i] +
                 red[(2 * NTT + tt) * kTile + 8 * g.cg + i];
        float* dst = out + (size_t)tt * ldo + c0 + 8 * g.cg;
        sy.st4(dst, make_float4(o[0], o[1], o[2], o[3]));
        sy.st4(dst + 4, make_float4(o[4], o[5], o[6], o[7]));
      }
    }
  }
  __syncthreads();
}

}  // namespace mla
