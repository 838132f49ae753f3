// Fused RMSNorm + MoE router top-K for gfx950: the single-device part of the
// "RMSNorm Router Top-K A2AV Kernel API Reference" page ("API Reference";
// "Notes": top-K on the raw logits, the activation on the selected experts).
//
// Two kernels:
//   k_rt_partial  split-K GEMV over router_weights with the RMSNorm scale folded
//                 out: workgroup (64-expert tile, slab of hidden, group of 8
//                 tokens) loads its weight slab (16-byte non-temporal loads)
//                 while it stages its tokens' activations, and writes partial
//                 logits of (x * gamma) @ W and, on tile 0, partial sums of x^2;
//   k_rt_select   one workgroup per token: 1/rms from the partial sums, the
//                 normalised bf16 row, logits = (1/rms) * sum of partials + bias
//                 (the slabs summed in a fixed order, many loads in flight),
//                 top-K by K rounds of a block-wide argmax (ties to the lower
//                 expert), the activation on the selected logits, and the
//                 indices and masked affinities.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../csrc/gemv.h"
#include "rmsnorm_router_topk.h"

namespace rt {
using namespace mla;

constexpr int kTW = 64;      // experts per GEMV tile (128-byte weight row segments)
constexpr int kMaxKs = 256;  // slab rows: one batch of weight loads per lane at 64 columns
constexpr int kNtt = 8;      // tokens per GEMV pass
constexpr int kMaxT = 128, kMaxH = 65536, kMaxE = 1024, kMaxK = 32;
constexpr int kTargetWG = 112;  // GEMV workgroups before token groups: few slabs keep the select reduction short

struct RtPlan {
  int ntile, s, ks;
};

int cdiv(int a, int b) { return (a + b - 1) / b; }

RtPlan rt_plan(int T, int H, int E) {
  RtPlan pl;
  pl.ntile = cdiv(E, kTW);
  int s = std::max(cdiv(H, kMaxKs), cdiv(kTargetWG, pl.ntile));
  // many tokens: keep the partial logits (written and read once) near the weight's size
  s = std::min(s, std::max(cdiv(H, kMaxKs), H / (2 * T)));
  s = std::min(s, std::max(1, H / 16));
  int ks = cdiv(H, s);
  ks = std::min(kMaxKs, (ks + 7) / 8 * 8);  // whole 16-byte activation pieces
  pl.ks = ks;
  pl.s = cdiv(H, ks);
  return pl;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int shape_code(int T, int H, int E) {
  if (T < 1 || H < 1 || E < 1) return RT_E_INVAL;
  if (T > kMaxT || H % 128 || H > kMaxH || E % 8 || E > kMaxE) return RT_E_UNSUPPORTED;
  return RT_OK;
}

__global__ __launch_bounds__(kBlock) void k_rt_partial(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                                                      const bf16_t* __restrict__ W, int T, int H, int E, int ks,
                                                      int ntile, int s, float* __restrict__ part,
                                                      float* __restrict__ ssq) {
  __shared__ float xs[kNtt * kMaxKs];
  __shared__ float red[3 * kNtt * kTile];
  __shared__ float sq8[kBlock];
  const int tile = blockIdx.x % ntile, slab = (blockIdx.x / ntile) % s, tg = blockIdx.x / (ntile * s);
  const int c0 = tile * kTW, nc = min(kTW, E - c0);
  const int k0 = slab * ks, kss = min(ks, H - k0);
  // the slab fits one batch of loads: gemv_tile issues no further weight loads
  u32x4 v[gemv_unroll(kNtt)];
  gemv_first<gemv_unroll(kNtt)>(W, E, k0, kss, c0, nc, v);
  {
    const int t0 = tg * kNtt, nt = min(kNtt, T - t0);
    // one 16-byte piece of x and of gamma per thread (nt * kss / 8 <= 256 pieces)
    const int g8 = kss / 8;
    const int tt = threadIdx.x / g8, r8 = threadIdx.x % g8;
    float q = 0.f;
    if (tt < nt) {
      float xv[8], gv[8];
      unpack8(*reinterpret_cast<const uint4*>(x + (size_t)(t0 + tt) * H + k0 + 8 * r8), xv);
      unpack8(*reinterpret_cast<const uint4*>(gamma + k0 + 8 * r8), gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xs[tt * kMaxKs + 8 * r8 + i] = xv[i] * gv[i];
        q = fmaf(xv[i], xv[i], q);
      }
    }
    sq8[threadIdx.x] = q;
    __syncthreads();
    if (tile == 0 && (int)threadIdx.x < nt) {  // sum of x^2 over the slab, pieces in order
      float a = 0.f;
      for (int i = 0; i < g8; ++i) a += sq8[threadIdx.x * g8 + i];
      ssq[(size_t)slab * T + t0 + threadIdx.x] = a;
    }
    gemv_tile<kNtt, gemv_unroll(kNtt)>(W, E, k0, kss, c0, nc, xs, kMaxKs, nt,
                                       part + ((size_t)slab * T + t0) * E, (size_t)E, red, v);
  }
}

__global__ __launch_bounds__(kBlock) void k_rt_select(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                                                     const float* __restrict__ bias, int T, int H, int E, int K,
                                                     int s, float eps, int act, const float* __restrict__ part,
                                                     const float* __restrict__ ssq, bf16_t* __restrict__ normed,
                                                     int32_t* __restrict__ idx, bf16_t* __restrict__ aff) {
  __shared__ __attribute__((aligned(16))) float zl[kMaxE];  // float4 stores of the partial reduction
  __shared__ unsigned char taken[kMaxE];
  __shared__ float wv[kBlock / kWave];
  __shared__ int we[kBlock / kWave];
  __shared__ int sel[kMaxK];
  __shared__ float val[kMaxK];
  __shared__ float scratch[kBlock / kWave];
  __shared__ float4 rscratch[kBlock];
  const int t = blockIdx.x, tid = threadIdx.x;

  float sq = 0.f;
  for (int i = tid; i < s; i += kBlock) sq += ssq[(size_t)i * T + t];
  sq = block_sum(sq, scratch);
  const float inv = 1.f / sqrtf(sq / (float)H + eps);
  // the normalised row, 16-byte pieces, four per thread in flight
  const int nv = H / 8;
  for (int i0 = tid; i0 < nv; i0 += 4 * kBlock) {
    uint4 xv[4], gv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + u * kBlock, nv - 1);
      xv[u] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + 8 * i);
      gv[u] = *reinterpret_cast<const uint4*>(gamma + 8 * i);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kBlock;
      if (i >= nv) continue;
      float a[8], b[8];
      unpack8(xv[u], a);
      unpack8(gv[u], b);
      uint4 o;
      o.x = (uint32_t)f32_to_bf16(a[0] * inv * b[0]) | ((uint32_t)f32_to_bf16(a[1] * inv * b[1]) << 16);
      o.y = (uint32_t)f32_to_bf16(a[2] * inv * b[2]) | ((uint32_t)f32_to_bf16(a[3] * inv * b[3]) << 16);
      o.z = (uint32_t)f32_to_bf16(a[4] * inv * b[4]) | ((uint32_t)f32_to_bf16(a[5] * inv * b[5]) << 16);
      o.w = (uint32_t)f32_to_bf16(a[6] * inv * b[6]) | ((uint32_t)f32_to_bf16(a[7] * inv * b[7]) << 16);
      *reinterpret_cast<uint4*>(normed + (size_t)t * H + 8 * i) = o;
    }
  }
  reduce_parts4(part + (size_t)t * E, (size_t)T * E, s, E / 4, E / 4, 0, zl, reinterpret_cast<float*>(rscratch));
  for (int e = tid; e < E; e += kBlock) {
    zl[e] = zl[e] * inv + (bias ? bias[e] : 0.f);
    taken[e] = 0;
  }
  __syncthreads();

  // K rounds of a block-wide argmax over the untaken experts (NaN ranks as -inf,
  // so every round finds an expert)
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
    for (int e = tid; e < E; e += kBlock) {
      if (taken[e]) continue;
      float z = zl[e];
      if (z != z) z = -INFINITY;
      if (z > bv || (z == bv && e < be)) { bv = z; be = e; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oe = __shfl_xor(be, off, kWave);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if ((tid & 63) == 0) { wv[tid >> 6] = bv; we[tid >> 6] = be; }
    __syncthreads();
    if (tid == 0) {
      float b = wv[0];
      int e0 = we[0];
      for (int w = 1; w < kBlock / kWave; ++w)
        if (wv[w] > b || (wv[w] == b && we[w] < e0)) { b = wv[w]; e0 = we[w]; }
      sel[k] = e0;
      taken[e0] = 1;
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (act == RT_ACT_SIGMOID) {
      for (int k = 0; k < K; ++k) val[k] = 1.f / (1.f + expf(-zl[sel[k]]));
    } else {  // softmax over the selected logits; sel[0] holds the largest
      const float m = zl[sel[0]];
      float sum = 0.f;
      for (int k = 0; k < K; ++k) {
        val[k] = expf(zl[sel[k]] - m);
        sum += val[k];
      }
      for (int k = 0; k < K; ++k) val[k] /= sum;
    }
  }
  __syncthreads();
  if (tid < K) idx[(size_t)t * K + tid] = sel[tid];
  for (int e = tid; e < E; e += kBlock) zl[e] = 0.f;
  __syncthreads();
  if (tid < K) zl[sel[tid]] = val[tid];
  __syncthreads();
  for (int e = tid; e < E; e += kBlock) aff[(size_t)t * E + e] = f32_to_bf16(zl[e]);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace rt

extern "C" {

size_t rmsnorm_router_topk_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_experts) {
  if (rt::shape_code(n_tokens, hidden, n_experts) != RT_OK) return 0;
  const rt::RtPlan pl = rt::rt_plan(n_tokens, hidden, n_experts);
  return rt::align256((size_t)pl.s * n_tokens * n_experts * sizeof(float)) +
         rt::align256((size_t)pl.s * n_tokens * sizeof(float));
}

int rmsnorm_router_topk(const void* hidden_states, const void* gamma, const void* router_weights,
                        const float* router_bias, int32_t n_tokens, int32_t hidden, int32_t n_experts,
                        int32_t top_k, float eps, int32_t act, void* normed_out, int32_t* topk_indices,
                        void* affinities, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace rt;
  if (!hidden_states || !gamma || !router_weights || !normed_out || !topk_indices || !affinities || !workspace)
    return RT_E_INVAL;
  const int sc = shape_code(n_tokens, hidden, n_experts);
  if (sc != RT_OK) return sc;
  if (top_k < 1 || top_k > std::min(n_experts, kMaxK) || (act != RT_ACT_SIGMOID && act != RT_ACT_SOFTMAX) ||
      !(eps >= 0.f) || eps > 1e30f)
    return RT_E_INVAL;
  const void* a16[] = {hidden_states, gamma, router_weights, normed_out, affinities, workspace};
  for (const void* q : a16) if (!aligned(q, 16)) return RT_E_ALIGN;
  if (!aligned(topk_indices, 4) || (router_bias && !aligned(router_bias, 4))) return RT_E_ALIGN;
  if (workspace_bytes < rmsnorm_router_topk_workspace_size(n_tokens, hidden, n_experts)) return RT_E_WORKSPACE;

  const RtPlan pl = rt_plan(n_tokens, hidden, n_experts);
  float* part = static_cast<float*>(workspace);
  float* ssq = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256((size_t)pl.s * n_tokens * n_experts * sizeof(float)));
  hipStream_t s = (hipStream_t)stream;
  const int ntg = (n_tokens + kNtt - 1) / kNtt;
  hipLaunchKernelGGL(k_rt_partial, dim3(pl.ntile * pl.s * ntg), dim3(kBlock), 0, s, (const bf16_t*)hidden_states,
                     (const bf16_t*)gamma, (const bf16_t*)router_weights, n_tokens, hidden, n_experts, pl.ks, pl.ntile,
                     pl.s, part, ssq);
  if (hipGetLastError() != hipSuccess) return RT_E_HIP;
  hipLaunchKernelGGL(k_rt_select, dim3(n_tokens), dim3(kBlock), 0, s, (const bf16_t*)hidden_states,
                     (const bf16_t*)gamma, router_bias, n_tokens, hidden, n_experts, top_k, pl.s, eps, act, part,
                     ssq, (bf16_t*)normed_out, topk_indices, (bf16_t*)affinities);
  if (hipGetLastError() != hipSuccess) return RT_E_HIP;
  return RT_OK;
}

}  // extern "C"
