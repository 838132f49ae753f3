// Fused RMSNorm + MoE router top-K for gfx950: the single-device part of the
// "RMSNorm Router Top-K A2AV Kernel API Reference" page ("API Reference";
// "Notes": top-K on the raw logits, the activation on the selected experts).
//
// Two kernels, each templated on the input type (bf16 or fp16, the page's two);
// a single token runs both in one launch, k_rt_one_token (below):
//   k_rt_partial  split-K GEMV over router_weights with the RMSNorm scale folded
//                 out: workgroup (64-expert tile, slab of hidden, group of 8
//                 tokens) loads its weight slab (16-byte non-temporal loads)
//                 while it stages its tokens' activations x * gamma, and writes
//                 partial logits of (x * gamma) @ W;
// From 9 tokens on (bf16 inputs) the logits run on the matrix cores instead:
//   k_rt_partial_m  split-K GEMM (x * gamma) @ W on v_mfma_f32_16x16x32_bf16,
//                 partial logits per K slab.  Each k-step's x and gamma
//                 pieces ride in the same register pipeline as its weight
//                 pieces; x * gamma is formed in fp32 and split into bf16 hi
//                 and lo halves as it is written to LDS in fragment order, and
//                 both halves meet the weight (gemm_mfma.h: about 16
//                 significant bits).
//   k_rt_select   one workgroup per token.  Its loads go out together (the x
//                 and gamma row, the bias and the partial logits, many in
//                 flight), then 1/rms from the row it holds, the logits
//                 (1/rms) * sum of partials + bias (slabs in a fixed order).
//                 Wave 0 then runs top-K on registers (E/64 keys a lane, a DPP
//                 argmax per round, ties to the lower expert, no barriers) and
//                 the activation of the selected logits, lane by lane, while
//                 the other waves write the normalised row.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../csrc/core_mfma.h"
#include "../csrc/gemm_mfma.h"
#include "../csrc/gemv.h"
#include "rmsnorm_router_topk.h"

namespace rt {
using namespace mla;

constexpr int kTW = 64;      // experts per GEMV tile (128-byte weight row segments)
constexpr int kMaxKs = 256;  // slab rows: one batch of weight loads per lane at 64 columns
constexpr int kNtt = 8;      // tokens per GEMV pass
constexpr int kMaxT = 128, kMaxH = 65536, kMaxE = 1024, kMaxK = 32;
constexpr int kTargetWG = 112;  // GEMV workgroups before token groups: few slabs keep the select reduction short
constexpr int kEPL = kMaxE / kWave;  // logits per lane of the top-K wave
constexpr int kXPre = 4;             // 16-byte pieces of x (and gamma) per thread loaded with the partials
constexpr size_t kCounterBytes = 256;  // workspace head: the one-token launch's arrival counter

struct RtPlan {
  int ntile, s, ks;
};

// Matrix-core plan: token blocks of kMtb m-tiles (32 tokens), 128-expert
// tiles, K slabs of ks k-steps (at least 8 where that still gives 512
// workgroups).
constexpr int kMtb = 2;
constexpr int kRtMinKs = 8;  // 4 (twice the workgroups and partials) measured slower at 128 tokens
constexpr int kMfmaMinT = 9;
struct RtPlanM {
  int ntile, ntb, kt, ks, s;
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

RtPlanM rt_plan_m(int T, int H, int E) {
  RtPlanM pl;
  pl.ntile = cdiv(E, mg_cols(kMtb));
  pl.ntb = cdiv(T, 16 * kMtb);
  pl.kt = H / kMgK;
  const int s = std::max(1, std::min(512 / (pl.ntile * pl.ntb), std::max(1, pl.kt / kRtMinKs)));
  pl.ks = cdiv(pl.kt, s);
  pl.s = cdiv(pl.kt, pl.ks);
  return pl;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }


int shape_code(int T, int H, int E) {
  if (T < 1 || H < 1 || E < 1) return RT_E_INVAL;
  if (T > kMaxT || H % 128 || H > kMaxH || E % 8 || E > kMaxE) return RT_E_UNSUPPORTED;
  return RT_OK;
}

// eight input values of a 16-byte piece, and their rounding back
template <bool F16>
__device__ __forceinline__ void unpack8in(const uint4 v, float* w) {
  if constexpr (F16) {
    unpack8vh(u32x4{v.x, v.y, v.z, v.w}, w);
  } else {
    unpack8(v, w);
  }
}
template <bool F16>
__device__ __forceinline__ uint32_t pack2out(float a, float b) {
  if constexpr (F16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
  } else {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  }
}

// NTT: tokens per pass (and the width of the LDS stages).
template <bool F16, int NTT = kNtt, class Sy = HandoffNone>
__device__ __forceinline__ void rt_partial(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                           const uint16_t* __restrict__ W, int T, int H, int E, int ks, int ntile,
                                           int s, float* __restrict__ part, const Sy& sy = Sy()) {
  __shared__ float xs[NTT * kMaxKs];
  __shared__ float red[3 * NTT * kTile];
  const int tile = blockIdx.x % ntile, slab = (blockIdx.x / ntile) % s, tg = blockIdx.x / (ntile * s);
  const int c0 = tile * kTW, nc = min(kTW, E - c0);
  const int k0 = slab * ks, kss = min(ks, H - k0);
  // the slab fits one batch of loads: gemv_tile issues no further weight loads
  u32x4 v[gemv_unroll(NTT)];
  gemv_first<gemv_unroll(NTT)>(W, E, k0, kss, c0, nc, v);
  const int t0 = tg * NTT, nt = min(NTT, T - t0);
  // one 16-byte piece of x and of gamma per thread (nt * kss / 8 <= 256 pieces)
  const int g8 = kss / 8;
  const int tt = threadIdx.x / g8, r8 = threadIdx.x % g8;
  if (tt < nt) {
    float xv[8], gv[8];
    unpack8in<F16>(*reinterpret_cast<const uint4*>(x + (size_t)(t0 + tt) * H + k0 + 8 * r8), xv);
    unpack8in<F16>(*reinterpret_cast<const uint4*>(gamma + k0 + 8 * r8), gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[tt * kMaxKs + 8 * r8 + i] = xv[i] * gv[i];
  }
  __syncthreads();
  gemv_tile<NTT, gemv_unroll(NTT), Sy, F16>(W, E, k0, kss, c0, nc, xs, kMaxKs, nt,
                                             part + ((size_t)slab * T + t0) * E, (size_t)E, red, v, sy);
}

template <bool F16>
__global__ __launch_bounds__(kBlock) void k_rt_partial(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                      const uint16_t* __restrict__ W, int T, int H, int E, int ks,
                                                      int ntile, int s, float* __restrict__ part) {
  rt_partial<F16>(x, gamma, W, T, H, E, ks, ntile, s, part);
}

// Sixteen zero bytes for the GEMM's padding loads (never written).
__device__ __attribute__((aligned(16))) uint16_t g_zero16[8] = {};

// Partial logits of one (128-expert tile, K slab, 32-token block).  Per
// k-step each thread loads two 16-byte weight pieces and four k of one token's
// x and gamma (tokens past T and k-steps past the slab read zeros).
__global__ __launch_bounds__(kBlock) void k_rt_partial_m(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                        const uint16_t* __restrict__ W, int T, int H, int E, int ntile,
                                                        int ntb, int kt, int ks, int s, float* __restrict__ part) {
  using S = Mg<kMtb, mg_cols(kMtb), 4>;
  constexpr int NC = mg_cols(kMtb);
  static_assert(S::kBPieces == 2 && kMtb * 16 * kMgK == 4 * kBlock, "one x piece per thread and k-step");
  __shared__ __attribute__((aligned(16))) char stage[S::kStage];
  int u, tb;
  if (!mg_unit(blockIdx.x, ntile * s, ntb, u, tb)) return;
  const int tile = u % ntile, slab = u / ntile, tid = threadIdx.x;
  const int c0 = tile * NC, k0 = slab * ks * kMgK, nks = min(ks, kt - slab * ks);
  const int t0 = tb * kMtb * 16, tt = tid >> 3, k4 = 4 * (tid & 7);
  const bool row_ok = t0 + tt < T;
  const uint16_t* xs = x + (size_t)(row_ok ? t0 + tt : 0) * H + k0 + k4;
  const uint16_t* gs = gamma + k0 + k4;
  const BTileSrc<NC> bs = btile_src<NC>(W, H, E, k0, c0);
  f32x4_t acc[S::MTW][S::NTW];
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  mg_pipe<3, S::kAhead>(
      nks, stage, S::kStep,
      [&](int st) {
        Pieces<3> r;
        const bool live = st < nks;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint16_t* src = g_zero16;
          if (live && bs.p[i]) src = bs.p[i] + bs.step * st;
          r.v[i] = load16_nt(src);
        }
        const uint2 xa = *reinterpret_cast<const uint2*>(live && row_ok ? xs + kMgK * st : g_zero16);
        const uint2 ga = *reinterpret_cast<const uint2*>(live ? gs + kMgK * st : g_zero16);
        r.v[2] = u32x4_t{xa.x, xa.y, ga.x, ga.y};
        return r;
      },
      [&](const Pieces<3>& r, char* buf) {
        const u32x4_t v = r.v[2];
        const float a[4] = {bf16lo(v[0]) * bf16lo(v[2]), bf16hi(v[0]) * bf16hi(v[2]), bf16lo(v[1]) * bf16lo(v[3]),
                            bf16hi(v[1]) * bf16hi(v[3])};
        put_a4_lds<true>(buf, kMtb, tt, k4, a);
#pragma unroll
        for (int i = 0; i < 2; ++i) store16(buf + S::kABytes + (i * kBlock + tid) * 16, r.v[i]);
      },
      [&](int, const char* buf) { mg_step<kMtb, NC, 4>(buf, buf + S::kABytes, acc); });
  float* out = part + (size_t)slab * T * E;
  mg_for_outputs4<kMtb, NC, 4>(acc, t0, c0, [&](int t, int c, const f32x4_t& v) {
    if (t < T) store_f32x4(out + (size_t)t * E, c, E, v);
  });
}

// Top-K keys: the logit mapped to an unsigned number of the same order (NaN
// ranks as -inf, -0 as +0); 0 is below every expert's key and marks an empty
// slot.  A round takes the largest key of the wave and, among lanes holding
// it, the lowest expert: two reductions on 32-bit values (v_max_u32 /
// v_min_u32 after DPP moves within rows of 16 and lane swaps across them),
// with no LDS round trips.
__device__ __forceinline__ unsigned order_key(float v) {
  if (v != v) v = -INFINITY;
  if (v == 0.f) v = 0.f;
  const unsigned u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// lanes l and l^16 (K32 false) or l and l^32 (true) both get (lower lane's
// value, upper lane's value), as in core_mfma.h's lane_pair
template <bool K32>
__device__ __forceinline__ void pair_u(unsigned a, unsigned& lo, unsigned& hi) {
  unsigned b = a;
  asm volatile("" : "+v"(b));
  const auto r = K32 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                     : __builtin_amdgcn_permlane16_swap(a, b, false, false);
  lo = r[0];
  hi = r[1];
  asm volatile("" : "+v"(lo), "+v"(hi));
}
template <bool kMax>
__device__ __forceinline__ unsigned wave_reduce_u(unsigned v) {
  auto op = [](unsigned a, unsigned b) { return kMax ? max(a, b) : min(a, b); };
  v = op(v, dpp_u<kDppQuadXor1>(v));
  v = op(v, dpp_u<kDppQuadXor2>(v));
  v = op(v, dpp_u<kDppRowHalfMirror>(v));
  v = op(v, dpp_u<kDppRowMirror>(v));
  unsigned lo, hi;
  pair_u<false>(v, lo, hi);
  v = op(lo, hi);
  pair_u<true>(v, lo, hi);
  return op(lo, hi);
}

template <bool F16, class Sy = HandoffNone>
__device__ __forceinline__ void rt_select(int t, const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                          const float* __restrict__ bias, int T, int H, int E, int K, int s,
                                          float eps, int act, const float* __restrict__ part,
                                          uint16_t* __restrict__ normed, int32_t* __restrict__ idx,
                                          uint16_t* __restrict__ aff, const Sy& sy = Sy()) {
  __shared__ __attribute__((aligned(16))) float zl[kMaxE];  // float4 stores of the partial reduction
  __shared__ float scratch[kBlock / kWave];
  __shared__ float4 rscratch[kBlock];
  static_assert(kBlock * 8 + (kBlock / kWave) * kMaxK * 8 + kMaxK * 8 <= sizeof(float4) * kBlock, "top-K scratch");
  const int tid = threadIdx.x, lane = tid & 63;
  const uint16_t* xr = x + (size_t)t * H;
  const int nv = H / 8;  // 16-byte pieces of the row

  // the first kXPre pieces of x and gamma per thread and the bias, issued
  // before the partial logits so that all of them share one round trip
  uint4 xv[kXPre], gv[kXPre];
#pragma unroll
  for (int u = 0; u < kXPre; ++u) {
    const int i = min(tid + u * kBlock, nv - 1);
    xv[u] = *reinterpret_cast<const uint4*>(xr + 8 * i);
    gv[u] = *reinterpret_cast<const uint4*>(gamma + 8 * i);
  }
  float bz[kMaxE / kBlock];
#pragma unroll
  for (int u = 0; u < kMaxE / kBlock; ++u) {
    const int e = tid + u * kBlock;
    bz[u] = (bias && e < E) ? bias[e] : 0.f;
  }
  reduce_parts4(part + (size_t)t * E, (size_t)T * E, s, E / 4, E / 4, 0, zl, reinterpret_cast<float*>(rscratch), sy);

  // sum of x^2 over the row (pieces past the first kXPre per thread loaded now)
  float sq = 0.f;
#pragma unroll
  for (int u = 0; u < kXPre; ++u) {
    if (tid + u * kBlock < nv) {
      float a[8];
      unpack8in<F16>(xv[u], a);
#pragma unroll
      for (int k = 0; k < 8; ++k) sq = fmaf(a[k], a[k], sq);
    }
  }
  for (int i = tid + kXPre * kBlock; i < nv; i += kBlock) {
    float a[8];
    unpack8in<F16>(*reinterpret_cast<const uint4*>(xr + 8 * i), a);
#pragma unroll
    for (int k = 0; k < 8; ++k) sq = fmaf(a[k], a[k], sq);
  }
  sq = block_sum(sq, scratch);  // its barriers also make zl visible
  const float inv = 1.f / sqrtf(sq / (float)H + eps);
#pragma unroll
  for (int u = 0; u < kMaxE / kBlock; ++u) {
    const int e = tid + u * kBlock;
    if (e < E) zl[e] = zl[e] * inv + bz[u];
  }
  __syncthreads();  // the logits
  // the normalised row: each thread its own pieces (H % 8 == 0); wave 0
  // writes its pieces after the top-K, so that no store of its own is in
  // flight while it ranks (the compiler waits for outstanding stores there)
  auto put = [&](int i, const uint4& xa, const uint4& ga) {
    float a[8], b[8];
    unpack8in<F16>(xa, a);
    unpack8in<F16>(ga, b);
    uint4 o;
    o.x = pack2out<F16>(a[0] * inv * b[0], a[1] * inv * b[1]);
    o.y = pack2out<F16>(a[2] * inv * b[2], a[3] * inv * b[3]);
    o.z = pack2out<F16>(a[4] * inv * b[4], a[5] * inv * b[5]);
    o.w = pack2out<F16>(a[6] * inv * b[6], a[7] * inv * b[7]);
    *reinterpret_cast<uint4*>(normed + (size_t)t * H + 8 * i) = o;
  };
  auto put_mine = [&]() {
#pragma unroll
    for (int u = 0; u < kXPre; ++u)
      if (tid + u * kBlock < nv) put(tid + u * kBlock, xv[u], gv[u]);
    for (int i = tid + kXPre * kBlock; i < nv; i += kBlock)
      put(i, *reinterpret_cast<const uint4*>(xr + 8 * i), *reinterpret_cast<const uint4*>(gamma + 8 * i));
  };
  if (E <= kBlock) {
    // Two levels by rank, one expert per thread.  A key is the 64-bit (order
    // key of the logit, kMaxE - 1 - expert), unique per expert, so ranks need
    // no tie rule; 0 marks no expert.  Each expert is first ranked within its
    // wave's 64 (the number of larger keys there); the K best of each wave are
    // the candidates, which hold the global top K.  Wave 0 then ranks the 4K
    // candidates; those of rank < K are the selection, in order.  Every LDS
    // read of a pass is issued before its compares (one wave per SIMD: a
    // read's latency is not hidden by another wave).  (Keys, candidates and
    // selection reuse the reduction's scratch.)
    unsigned long long* ck = reinterpret_cast<unsigned long long*>(rscratch);   // [kBlock] keys
    unsigned long long* cand = ck + kBlock;                                     // [waves * K]
    float* selz = reinterpret_cast<float*>(cand + (kBlock / kWave) * kMaxK);
    int* sele = reinterpret_cast<int*>(selz + kMaxK);
    const int wv = tid >> 6;
    const unsigned long long key =
        tid < E ? ((unsigned long long)order_key(zl[tid]) << 32) | (unsigned)(kMaxE - 1 - tid) : 0ull;
    ck[tid] = key;
    if (tid < (kBlock / kWave) * K) cand[tid] = 0ull;
    __syncthreads();
    // rank of this expert within its wave
    {
      const ulonglong2* w = reinterpret_cast<const ulonglong2*>(ck + kWave * wv);
      int lr = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ulonglong2 c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = w[16 * h + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) lr += (c[u].x > key ? 1 : 0) + (c[u].y > key ? 1 : 0);
      }
      if (lr < K) cand[wv * K + lr] = key;  // a wave with fewer than K experts leaves zero keys
    }
    __syncthreads();
    const int nc = (kBlock / kWave) * K;  // <= 128, even
    const unsigned long long mine = tid < nc && tid < kWave * 2 ? cand[tid] : 0ull;
    int rank = 0;
    if (tid < kWave * 2) {  // waves 0 and 1 (nc <= 128)
      for (int j0 = 0; j0 < nc; j0 += 32) {
        ulonglong2 c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = j0 + 2 * u < nc ? reinterpret_cast<const ulonglong2*>(cand + j0)[u]
                                                             : ulonglong2{0ull, 0ull};
#pragma unroll
        for (int u = 0; u < 16; ++u) rank += (c[u].x > mine ? 1 : 0) + (c[u].y > mine ? 1 : 0);
      }
    }
    if (mine != 0ull && rank < K) {
      const int e = kMaxE - 1 - (int)(unsigned)(mine & 0xffffffffu);
      selz[rank] = zl[e];
      sele[rank] = e;
    }
    __syncthreads();
    if (tid < E) zl[tid] = 0.f;  // the affinity row, selected entries filled in below
    __syncthreads();
    if (tid < kWave) {
      // the activations, lane k for the k-th selected expert; the masked
      // affinity row through LDS (this wave's LDS accesses run in order)
      const bool on = lane < K;
      const float z = on ? selz[lane] : -INFINITY;
      const int e = on ? sele[lane] : 0;
      float a;
      if (act == RT_ACT_SIGMOID) {
        a = 1.f / (1.f + expf(-z));
      } else {
        const float zmax = wave_max_dpp(z);
        const float ex = on ? expf(z - zmax) : 0.f;
        a = ex * (1.f / wave_sum_dpp(ex));
      }
      if (on) {
        zl[e] = a;
        idx[(size_t)t * K + lane] = e;
      }
      for (int e0 = 2 * lane; e0 < E; e0 += 2 * kWave)
        *reinterpret_cast<uint32_t*>(aff + (size_t)t * E + e0) =
            (uint32_t)f32_to_bf16(zl[e0]) | ((uint32_t)f32_to_bf16(zl[e0 + 1]) << 16);
    }
    put_mine();
    return;
  }
  if (tid >= kWave) {
    put_mine();
    return;
  }

  // more than kBlock experts: top-K in one wave: lane l holds the keys of experts l + 64 j (j < kEPL),
  // 0 past E, so every round finds a real expert (K <= E).  Each lane keeps
  // its best untaken (key, expert); only the lane whose expert a round takes
  // looks for its next best.
  unsigned kh[kEPL];
#pragma unroll
  for (int j = 0; j < kEPL; ++j) {
    const int e = lane + kWave * j;
    kh[j] = e < E ? order_key(zl[e]) : 0u;
  }
  unsigned taken = 0u, bv = 0u, be = 0xffffffffu;
  auto lane_best = [&]() {
    bv = 0u;
    be = 0xffffffffu;
#pragma unroll
    for (int j = kEPL - 1; j >= 0; --j)  // downwards: among equal keys the lower expert stays
      if (!((taken >> j) & 1u) && kh[j] != 0u && kh[j] >= bv) {
        bv = kh[j];
        be = (unsigned)(lane + kWave * j);
      }
  };
  lane_best();
  int my_sel = 0;
  for (int k = 0; k < K; ++k) {
    const unsigned vmax = wave_reduce_u<true>(bv);
    const int e = (int)wave_reduce_u<false>(bv == vmax ? be : 0xffffffffu);
    if (lane == k) my_sel = e;
    if ((e & 63) == lane) {
      taken |= 1u << (e >> 6);
      lane_best();
    }
  }
  // the activation of every selected logit, by the lane that holds it:
  // sigmoid on its own; softmax against the largest selected logit, divided
  // by the sum over the selected (wave reductions)
  float zmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < kEPL; ++j)
    if ((taken >> j) & 1u) zmax = fmaxf(zmax, zl[lane + kWave * j]);
  zmax = wave_max_dpp(zmax);
  float ex[kEPL];
  float esum = 0.f;
#pragma unroll
  for (int j = 0; j < kEPL; ++j) {
    ex[j] = 0.f;
    if ((taken >> j) & 1u) {
      const float zj = zl[lane + kWave * j];
      ex[j] = act == RT_ACT_SIGMOID ? 1.f / (1.f + expf(-zj)) : expf(zj - zmax);
      esum += ex[j];
    }
  }
  if (act != RT_ACT_SIGMOID) {
    const float r = 1.f / wave_sum_dpp(esum);
#pragma unroll
    for (int j = 0; j < kEPL; ++j) ex[j] *= r;
  }
  // the masked affinity row through LDS (this wave alone: its LDS accesses
  // run in order), written as pairs of bf16
#pragma unroll
  for (int j = 0; j < kEPL; ++j)
    if (lane + kWave * j < E) zl[lane + kWave * j] = ex[j];
  for (int e0 = 2 * lane; e0 < E; e0 += 2 * kWave)
    *reinterpret_cast<uint32_t*>(aff + (size_t)t * E + e0) =
        (uint32_t)f32_to_bf16(zl[e0]) | ((uint32_t)f32_to_bf16(zl[e0 + 1]) << 16);
  if (lane < K) idx[(size_t)t * K + lane] = my_sel;
  put_mine();
}

template <bool F16>
__global__ __launch_bounds__(kBlock) void k_rt_select(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                     const float* __restrict__ bias, int T, int H, int E, int K,
                                                     int s, float eps, int act, const float* __restrict__ part,
                                                     uint16_t* __restrict__ normed, int32_t* __restrict__ idx,
                                                     uint16_t* __restrict__ aff) {
  rt_select<F16>(blockIdx.x, x, gamma, bias, T, H, E, K, s, eps, act, part, normed, idx, aff);
}

// k_rt_select with the DeepSeek-V3 router's sizes as compile-time constants
// (hidden 7168, 256 experts, top 8, 28 slabs of partial logits); the token
// count stays an argument.
template <bool F16>
__global__ __launch_bounds__(kBlock) void k_rt_select_ds(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ gamma,
                                                        const float* __restrict__ bias, int T, float eps, int act,
                                                        const float* __restrict__ part, uint16_t* __restrict__ normed,
                                                        int32_t* __restrict__ idx, uint16_t* __restrict__ aff) {
  rt_select<F16>(blockIdx.x, x, gamma, bias, T, 7168, 256, 8, 28, eps, act, part, normed, idx, aff);
}

// Partial logits read back by the last workgroup of the same launch:
// device-scope loads (they bypass this XCD's L2, which may hold stale lines).
struct DevLoads {
  static constexpr bool kWeightsFirst = false;
  __device__ __forceinline__ void wait() const {}
  __device__ __forceinline__ float ld(const float* p) const { return ld_dev(p); }
  __device__ __forceinline__ float4 ld4(const float* p) const { return ld_dev4(p); }
};

// One token in one launch.  Every workgroup computes its tile and slab of the
// partial logits (as k_rt_partial) and stores them with device scope, waits
// for those stores, then counts itself in the arrival counter (a device-scope
// atomic); the last to arrive resets the counter to zero and runs the select
// of the token (as k_rt_select), reading the partials with device-scope loads.
// The partials are added in slab order whichever workgroup is last, so the
// result is the two-kernel path's, bit for bit.
template <bool F16>
__global__ __launch_bounds__(kBlock) void k_rt_one_token(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                        const uint16_t* __restrict__ W, const float* __restrict__ bias,
                                                        int H, int E, int K, int ks, int ntile, int s, float eps,
                                                        int act, float* __restrict__ part, unsigned* __restrict__ cnt,
                                                        uint16_t* __restrict__ normed, int32_t* __restrict__ idx,
                                                        uint16_t* __restrict__ aff) {
  __shared__ unsigned arrived;
  rt_partial<F16, 1>(x, gamma, W, 1, H, E, ks, ntile, s, part, HandoffDevStores());
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();  // this workgroup's partial stores are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) arrived = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (arrived != (unsigned)(ntile * s) - 1u) return;
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  rt_select<F16>(0, x, gamma, bias, 1, H, E, K, s, eps, act, part, normed, idx, aff, DevLoads());
}

// The same launch with the DeepSeek-V3 router's sizes as compile-time
// constants (hidden 7168, 256 experts, top 8; the plan rt_plan gives them:
// 64-expert tiles, 28 slabs of 256 rows), so the index arithmetic folds.
constexpr int kDsH = 7168, kDsE = 256, kDsK = 8, kDsKs = 256, kDsTiles = 4, kDsSlabs = 28;
template <bool F16>
__global__ __launch_bounds__(kBlock) void k_rt_one_token_ds(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ gamma,
                                                           const uint16_t* __restrict__ W,
                                                           const float* __restrict__ bias, float eps, int act,
                                                           float* __restrict__ part, unsigned* __restrict__ cnt,
                                                           uint16_t* __restrict__ normed, int32_t* __restrict__ idx,
                                                           uint16_t* __restrict__ aff) {
  __shared__ unsigned arrived;
  rt_partial<F16, 1>(x, gamma, W, 1, kDsH, kDsE, kDsKs, kDsTiles, kDsSlabs, part, HandoffDevStores());
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) arrived = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (arrived != (unsigned)(kDsTiles * kDsSlabs) - 1u) return;
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  rt_select<F16>(0, x, gamma, bias, 1, kDsH, kDsE, kDsK, kDsSlabs, eps, act, part, normed, idx, aff, DevLoads());
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace rt

extern "C" {

size_t rmsnorm_router_topk_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_experts) {
  if (rt::shape_code(n_tokens, hidden, n_experts) != RT_OK) return 0;
  const rt::RtPlan pl = rt::rt_plan(n_tokens, hidden, n_experts);
  size_t b = rt::align256((size_t)pl.s * n_tokens * n_experts * sizeof(float));
  if (n_tokens >= rt::kMfmaMinT) {  // the matrix-core plan (bf16 inputs)
    const rt::RtPlanM pm = rt::rt_plan_m(n_tokens, hidden, n_experts);
    b = std::max(b, rt::align256((size_t)pm.s * n_tokens * n_experts * sizeof(float)));
  }
  return rt::kCounterBytes + b;
}

int rmsnorm_router_topk_typed(int32_t dtype, const void* hidden_states, const void* gamma, const void* router_weights,
                              const float* router_bias, int32_t n_tokens, int32_t hidden, int32_t n_experts,
                              int32_t top_k, float eps, int32_t act, void* normed_out, int32_t* topk_indices,
                              void* affinities, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace rt;
  if (dtype != RT_DTYPE_BF16 && dtype != RT_DTYPE_FP16) return RT_E_INVAL;
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

  hipStream_t s = (hipStream_t)stream;
  const bool f16 = dtype == RT_DTYPE_FP16;
  const auto* xh = (const uint16_t*)hidden_states;
  const auto* gh = (const uint16_t*)gamma;
  const auto* wh = (const uint16_t*)router_weights;
  unsigned* cnt = static_cast<unsigned*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
  if (n_tokens == 1) {
    const RtPlan pl = rt_plan(1, hidden, n_experts);
    if (hidden == kDsH && n_experts == kDsE && top_k == kDsK && pl.ks == kDsKs && pl.ntile == kDsTiles &&
        pl.s == kDsSlabs) {
      hipLaunchKernelGGL(f16 ? k_rt_one_token_ds<true> : k_rt_one_token_ds<false>, dim3(kDsTiles * kDsSlabs),
                         dim3(kBlock), 0, s, xh, gh, wh, router_bias, eps, act, part, cnt, (uint16_t*)normed_out,
                         topk_indices, (uint16_t*)affinities);
      return hipGetLastError() == hipSuccess ? RT_OK : RT_E_HIP;
    }
    hipLaunchKernelGGL(f16 ? k_rt_one_token<true> : k_rt_one_token<false>, dim3(pl.ntile * pl.s), dim3(kBlock), 0, s,
                       xh, gh, wh, router_bias, hidden, n_experts, top_k, pl.ks, pl.ntile, pl.s, eps, act, part, cnt,
                       (uint16_t*)normed_out, topk_indices, (uint16_t*)affinities);
    return hipGetLastError() == hipSuccess ? RT_OK : RT_E_HIP;
  }
  int slabs;
  if (!f16 && n_tokens >= kMfmaMinT) {
    const RtPlanM pm = rt_plan_m(n_tokens, hidden, n_experts);
    const int nwg = cdiv(pm.ntile * pm.s, 8) * 8 * pm.ntb;
    hipLaunchKernelGGL(k_rt_partial_m, dim3(nwg), dim3(kBlock), 0, s, xh, gh, wh, n_tokens, hidden, n_experts, pm.ntile,
                       pm.ntb, pm.kt, pm.ks, pm.s, part);
    slabs = pm.s;
  } else {
    const RtPlan pl = rt_plan(n_tokens, hidden, n_experts);
    const int ntg = (n_tokens + kNtt - 1) / kNtt;
    hipLaunchKernelGGL(f16 ? k_rt_partial<true> : k_rt_partial<false>, dim3(pl.ntile * pl.s * ntg), dim3(kBlock), 0,
                       s, xh, gh, wh, n_tokens, hidden, n_experts, pl.ks, pl.ntile, pl.s, part);
    slabs = pl.s;
  }
  if (hipGetLastError() != hipSuccess) return RT_E_HIP;
  if (hidden == kDsH && n_experts == kDsE && top_k == kDsK && slabs == kDsSlabs) {
    hipLaunchKernelGGL(f16 ? k_rt_select_ds<true> : k_rt_select_ds<false>, dim3(n_tokens), dim3(kBlock), 0, s, xh, gh,
                       router_bias, n_tokens, eps, act, part, (uint16_t*)normed_out, topk_indices,
                       (uint16_t*)affinities);
    return hipGetLastError() == hipSuccess ? RT_OK : RT_E_HIP;
  }
  hipLaunchKernelGGL(f16 ? k_rt_select<true> : k_rt_select<false>, dim3(n_tokens), dim3(kBlock), 0, s, xh, gh,
                     router_bias, n_tokens, hidden, n_experts, top_k, slabs, eps, act, part, (uint16_t*)normed_out,
                     topk_indices, (uint16_t*)affinities);
  if (hipGetLastError() != hipSuccess) return RT_E_HIP;
  return RT_OK;
}

int rmsnorm_router_topk(const void* hidden_states, const void* gamma, const void* router_weights,
                        const float* router_bias, int32_t n_tokens, int32_t hidden, int32_t n_experts,
                        int32_t top_k, float eps, int32_t act, void* normed_out, int32_t* topk_indices,
                        void* affinities, void* workspace, size_t workspace_bytes, void* stream) {
  return rmsnorm_router_topk_typed(RT_DTYPE_BF16, hidden_states, gamma, router_weights, router_bias, n_tokens, hidden,
                                   n_experts, top_k, eps, act, normed_out, topk_indices, affinities, workspace,
                                   workspace_bytes, stream);
}

}  // extern "C"
