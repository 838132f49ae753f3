// Phases of the matrix-core path, used when a step carries more than a few
// tokens.  The operations and their order are those of the GEMV path
// (phases.h); the projections become hi/lo bf16 GEMMs on the matrix cores
// (gemm_mfma.h).  Each producer writes the next GEMM's activation already in
// fragment order, so the GEMM kernels stream both operands with plain 16-byte
// loads:
//   k_prep    index build; A1 = x * g_in; partial sums of x^2
//   k_down    split-K partials of A1 @ [wq_a | wkv_a]
//   k_qa      reduce them: A2 = acc_q * g_q and partial sums of acc_q^2 per
//             column chunk; per token, kv-latent RMSNorm, RoPE, cache-row write
//   k_qup     split-K partials of A2 @ wq_b
//   k_absorb  q_lat = (beta * q_nope) @ q_absorb_w[h], beta = alpha * inv_q;
//             RoPE of q_pe -> Qcat
//   k_core    (shared with the GEMV path)
//   k_oabsorb combine the core's splits into o_lat; o_v = out_absorb_w[h] . o_lat -> A5
//   k_oproj   split-K partials of A5 @ o_proj_w
//   k_out     (shared) reduction to the bf16 output
// Rows of a token block past the last token carry unspecified values; they
// only reach output rows that are never stored.  K padding is written as zeros.
#pragma once

#include <type_traits>

#include "device_util.h"
#include "gemm_mfma.h"
#include "phases.h"
#include "step_params.h"

namespace mla {

constexpr int kPrepChunk = 4 * kBlock * 2;  // hidden columns per k_prep workgroup
constexpr int kQaChunk = 4 * kBlock;        // q_lora_rank columns per k_qa workgroup

// ---------------------------------------------------------------------------
// k_prep: index build (first n_idx_wg workgroups); then workgroup (token t,
// chunk of kPrepChunk hidden columns): A1 = x * g_in in fragment order (K
// padded with zeros) and the chunk's sum of x^2.
// ---------------------------------------------------------------------------
__device__ void phase_prep(const StepParams& p, int b, float* lds) {
  const Plan& pl = p.pl;
  clear_zero_region(p, b);
  if (b < pl.n_idx_wg) {
    index_build(p, b * kBlock + threadIdx.x);
    return;
  }
  const int t = (b - pl.n_idx_wg) / pl.nxc, ch = (b - pl.n_idx_wg) % pl.nxc;
  const int KP = pl.kt1 * kMgK;
  const bf16_t* xr = p.x + (size_t)t * p.H;
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kPrepChunk / (4 * kBlock); ++u) {
    const int k = ch * kPrepChunk + u * 4 * kBlock + 4 * threadIdx.x;
    if (k >= KP) break;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (k < p.H) {  // H % 8 == 0: a group of four is wholly inside or outside
      const uint2 v = *reinterpret_cast<const uint2*>(xr + k);
      const float xv[4] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ss = fmaf(xv[i], xv[i], ss);
        a[i] = xv[i] * p.g_in[k + i];
      }
    }
    put_a4(p.a1, pl.mt_pad, t, k, a);
  }
  ss = block_sum(ss, lds);
  if (threadIdx.x == 0) p.ssx[(size_t)ch * pl.T + t] = ss;
}

// sum of n floats at p, p + stride, ... in index order; the loads of four
// terms go out together
// sum_{c < n} p[c*stride] in order, eight loads at a time (an index past the
// last reloads the last and is dropped), n >= 1
__device__ __forceinline__ float sum_strided(const float* p, size_t stride, int n) {
  float s = 0.f;
  for (int c = 0; c < n; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(size_t)min(c + u, n - 1) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c + u < n) s += v[u];
  }
  return s;
}

// alpha = 1/rms(x) of token t from the chunk sums (fixed order)
__device__ __forceinline__ float mfma_alpha(const StepParams& p, int t) {
  return inv_rms(sum_strided(p.ssx + t, p.pl.T, p.pl.nxc), p.H, p.eps);
}

// beta = alpha / rms(alpha * acc_q) of token t: the scale of the wq_b output
// (both chunk-sum lists are loaded before either is added)
__device__ __forceinline__ float mfma_beta(const StepParams& p, int t) {
  const Plan& pl = p.pl;
  if (pl.nxc <= 8 && pl.nqc <= 8) {
    float vx[8], vq[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      vx[u] = p.ssx[(size_t)min(u, pl.nxc - 1) * pl.T + t];
      vq[u] = p.ssq[(size_t)min(u, pl.nqc - 1) * pl.T + t];
    }
    float sx = 0.f, sq = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < pl.nxc) sx += vx[u];
      if (u < pl.nqc) sq += vq[u];
    }
    const float a = inv_rms(sx, p.H, p.eps);
    return a / sqrtf(a * a * sq / (float)p.Q + p.eps);
  }
  const float a = mfma_alpha(p, t);
  const float s = sum_strided(p.ssq + t, pl.T, pl.nqc);
  return a / sqrtf(a * a * s / (float)p.Q + p.eps);
}

// ---------------------------------------------------------------------------
// k_down: split-K partials of A1 @ [wq_a | wkv_a] (wq_a's tiles first)
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_down_m(const StepParams& p, int b, char* stage) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, pl.nt1m * pl.s1, pl.ntb, u, tb)) return;
  const int tile = u % pl.nt1m, slab = u / pl.nt1m;
  const bool is_q = tile < pl.ntq1m;
  const bf16_t* W = is_q ? p.wq_a : p.wkv_a;
  const int N = is_q ? p.Q : p.KVR;
  constexpr int NC = mg_cols(MTB);
  const int c0 = (is_q ? tile : tile - pl.ntq1m) * NC;
  const int k0 = slab * pl.ks1m * kMgK;
  const int nks = min(pl.ks1m, pl.kt1 - slab * pl.ks1m);
  f32x4_t acc[Mg<MTB>::MTW][Mg<MTB>::NTW];
  mgemm<MTB>(p.a1, pl.mt_pad, tb * MTB, W, p.H, N, k0, nks, c0, reinterpret_cast<const bf16_t*>(p.zero16), stage, acc);
  const int N1 = p.Q + p.KVR, T = pl.T;
  float* out = p.part1 + (size_t)slab * T * N1 + (is_q ? 0 : p.Q);
  mg_for_outputs4<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, const f32x4_t& v) {
    if (t < T) store_f32x4(out + (size_t)t * N1, c, N, v);
  });
}

// ---------------------------------------------------------------------------
// k_qa: workgroup (token t, w).  w < nqc: columns [w*kQaChunk, ...) of the
// query latent, reduced over the down-projection's slabs (fixed order):
// A2 = acc_q * g_q in fragment order (the chunks cover the K padding, which
// gets zeros) and the chunk's sum of acc_q^2.  w == nqc: the kv row,
// y = alpha * acc_kv, RMSNorm of its latent part, RoPE of its rotary part,
// bf16 row at slot_mapping[t].
// ---------------------------------------------------------------------------
// Sums over S split-K slabs, in slab order, of partials written by the
// previous kernel.  G slabs' loads go out together, so a reduction costs
// ceil(S/G) memory round trips; slabs past S - 1 are not loaded (the
// condition is the same in every lane).
template <int G>
__device__ __forceinline__ float4 sum_slabs4(const float* src, size_t stride, int S) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; s += G) {
    float4 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u)
      v[u] = s + u < S ? *reinterpret_cast<const float4*>(src + (size_t)(s + u) * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s + u < S) {
        a.x += v[u].x; a.y += v[u].y; a.z += v[u].z; a.w += v[u].w;
      }
  }
  return a;
}

// acc[i] = sum over S slabs (in slab order) of the float4 at src[i] + s*stride,
// for NI items at once: G slabs' loads of all NI items go out together.
// Items with a null source give zeros.
template <int NI, int G>
__device__ __forceinline__ void sum_slabs4_n(const float* const (&src)[NI], size_t stride, int S, float4 (&acc)[NI]) {
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; s += G) {
    float4 v[G][NI];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const size_t o = (size_t)(s + u) * stride;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        v[u][i] = (src[i] && s + u < S) ? *reinterpret_cast<const float4*>(src[i] + o) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s + u < S)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          acc[i].x += v[u][i].x; acc[i].y += v[u][i].y; acc[i].z += v[u][i].z; acc[i].w += v[u][i].w;
        }
  }
}

__device__ void phase_qa(const StepParams& p, int b, float* lds) {
  const Plan& pl = p.pl;
  const int T = pl.T, tid = threadIdx.x;
  const int t = b / (pl.nqc + 1), w = b % (pl.nqc + 1);
  const int N1 = p.Q + p.KVR;
  const size_t sstride = (size_t)T * N1;
  const float* src = p.part1 + (size_t)t * N1;
  if (w < pl.nqc) {
    const int k = w * kQaChunk + 4 * tid;
    const int KP = pl.kt2 * kMgK;
    float ss = 0.f;
    if (k < KP) {
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      if (k < p.Q) {  // Q % 8 == 0
        const float4 v = sum_slabs4<16>(src + k, sstride, pl.s1);
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss = fmaf(vv[i], vv[i], ss);
          a[i] = vv[i] * p.g_q[k + i];
        }
      }
      put_a4(p.a2, pl.mt_pad, t, k, a);
    }
    ss = block_sum(ss, lds);
    if (tid == 0) p.ssq[(size_t)w * T + t] = ss;
    return;
  }
  float* y = lds;                            // [KVR]
  float* scratch = lds + ((p.KVR + 63) & ~63);
  const float alpha = mfma_alpha(p, t);
  for (int c4 = tid; c4 < p.KVR / 4; c4 += kBlock) {
    const float4 v = sum_slabs4<16>(src + p.Q + 4 * c4, sstride, pl.s1);
    y[4 * c4 + 0] = alpha * v.x;
    y[4 * c4 + 1] = alpha * v.y;
    y[4 * c4 + 2] = alpha * v.z;
    y[4 * c4 + 3] = alpha * v.w;
  }
  __syncthreads();
  float sk = 0.f;
  for (int c = tid; c < p.R; c += kBlock) sk = fmaf(y[c], y[c], sk);
  sk = block_sum(sk, scratch);
  const float inv = inv_rms(sk, p.R, p.eps);
  if (!slot_ok(p, t)) return;
  bf16_t* crow = p.cache + (size_t)p.slot[t] * p.KVR;
  for (int c = tid; c < p.R; c += kBlock) crow[c] = f32_to_bf16(y[c] * inv * p.g_kv[c]);
  const int half = p.DR / 2;
  for (int i = tid; i < half; i += kBlock) {
    const float x0 = y[p.R + 2 * i], x1 = y[p.R + 2 * i + 1];
    const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
    crow[p.R + 2 * i] = f32_to_bf16(x0 * cs - x1 * sn);
    crow[p.R + 2 * i + 1] = f32_to_bf16(x0 * sn + x1 * cs);
  }
}

// ---------------------------------------------------------------------------
// k_qup: split-K partials of A2 @ wq_b
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_qup_m(const StepParams& p, int b, char* stage) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, pl.nt2m * pl.s2, pl.ntb, u, tb)) return;
  const int tile = u % pl.nt2m, slab = u / pl.nt2m;
  constexpr int NC = mg_cols(MTB);
  const int c0 = tile * NC;
  const int k0 = slab * pl.ks2m * kMgK;
  const int nks = min(pl.ks2m, pl.kt2 - slab * pl.ks2m);
  f32x4_t acc[Mg<MTB>::MTW][Mg<MTB>::NTW];
  mgemm<MTB>(p.a2, pl.mt_pad, tb * MTB, p.wq_b, p.Q, p.N2, k0, nks, c0, reinterpret_cast<const bf16_t*>(p.zero16), stage, acc);
  const int T = pl.T;
  float* out = p.part2 + (size_t)slab * T * p.N2;
  mg_for_outputs4<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, const f32x4_t& v) {
    if (t < T) store_f32x4(out + (size_t)t * p.N2, c, p.N2, v);
  });
}

// ---------------------------------------------------------------------------
// k_absorb: workgroup (head h, group of tpw3 NCA-column tiles of kv_lora_rank,
// token block).  The pipeline streams the group's tiles of q_absorb_w[h]
// (ceil(DN/32) k-steps each); its first loads go out before A3 = beta * q_nope
// (wq_b slabs summed in order) is written to LDS in fragment order, once for
// all the group's tiles.  Each tile's q_lat lands in Qcat as bf16, pre-scaled
// by softmax_scale * log2(e); q_pe is roped into Qcat too.
// NCA = 128 where kv_lora_rank allows (each weight row segment is 256 bytes), else 64.
// LDS: stages (2 x NCA/16 KB) | beta (512 B) | A3 (ceil(DN/32) x MTB x 2 KB).
// ---------------------------------------------------------------------------
constexpr int kAbsorbBetaBytes = 512;  // beta of up to 128 tokens

// interleaved RoPE of rotary pair i of the (pre-scaled) query of token t, head h, into Qcat
__device__ __forceinline__ void rope_q(const StepParams& p, int t, int h, int i, float x0, float x1) {
  const int half = p.DR / 2;
  const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
  bf16_t* q = p.qcat + ((size_t)t * p.NH + h) * p.KVR + p.R;
  q[2 * i] = f32_to_bf16(x0 * cs - x1 * sn);
  q[2 * i + 1] = f32_to_bf16(x0 * sn + x1 * cs);
}

template <int MTB, int NCA>
__device__ void phase_absorb_m(const StepParams& p, int b, char* lds) {
  using S = Mg<MTB, NCA, 4>;  // four waves: the loads below index by kBlock
  constexpr int NV = NCA / 64;  // 16-byte weight pieces per lane per step
  const Plan& pl = p.pl;
  const int ngrp = pl.nct3 / pl.tpw3;
  int u, tb;
  if (!mg_unit(b, p.NH * ngrp, pl.ntb3, u, tb)) return;
  const int h = u / ngrp, j0 = (u % ngrp) * pl.tpw3;
  const int T = pl.T, tid = threadIdx.x;
  const int t0 = tb * MTB * 16;
  const int KS = (p.DN + kMgK - 1) / kMgK;
  const int nsteps = pl.tpw3 * KS;
  static_assert(MTB * 16 * 4 <= kAbsorbBetaBytes, "beta region");
  char* stage = lds;
  float* beta = reinterpret_cast<float*>(lds + 2 * S::kBBytes);
  char* ares = lds + 2 * S::kBBytes + kAbsorbBetaBytes;
  // this lane's pieces of a 32 x NCA weight tile: piece q = 256 i + tid is
  // row q / (NCA/8), swizzled 16-byte column piece
  const bf16_t* W = p.w_qabs + (size_t)h * p.DN * p.R;
  int pr[NV], ppc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int qq = i * kBlock + tid;
    pr[i] = qq / (NCA / 8);
    ppc[i] = bswz(qq % (NCA / 8), pr[i]);
  }
  auto load = [&](int st) {
    Pieces<NV> q;
    const int j = j0 + st / KS, ks = st % KS;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int row = ks * kMgK + pr[i];
      const bf16_t* src = reinterpret_cast<const bf16_t*>(p.zero16);
      if (st < nsteps && row < p.DN) src = W + (size_t)row * p.R + j * NCA + 8 * ppc[i];
      q.v[i] = load16_nt(src);
    }
    return q;
  };
  constexpr int P = NV == 1 ? 8 : (NV == 2 ? 6 : 2);  // k-steps of weight pieces loaded ahead
  Pieces<NV> q[P];
  mg_pipe_prologue(q, load);
  if (tid < MTB * 16) beta[tid] = (t0 + tid < T) ? mfma_beta(p, t0 + tid) : 0.f;
  __syncthreads();
  // float4 items (token, 4 columns of q_nope), NI per thread per pass, with
  // the loads of GS slabs issued together (fewer registers for the largest
  // token blocks, whose pipeline holds more)
  constexpr int NI = MTB <= 2 ? 4 : 8;
  constexpr int GS = MTB <= 2 ? 8 : 2;
  const int n_items = MTB * 16 * KS * 8;
  for (int base = 0; base < n_items; base += NI * kBlock) {
    const float* src[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = base + i * kBlock + tid;
      const int tt = idx / (KS * 8), k = 4 * (idx % (KS * 8)), t = t0 + tt;
      src[i] = (idx < n_items && t < T && k < p.DN)  // DN % 8 == 0
                   ? p.part2 + (size_t)t * p.N2 + (size_t)h * p.QKH + k
                   : nullptr;
    }
    float4 v[NI];
    sum_slabs4_n<NI, GS>(src, (size_t)T * p.N2, pl.s2, v);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = base + i * kBlock + tid;
      if (idx >= n_items) continue;
      const int tt = idx / (KS * 8), k = 4 * (idx % (KS * 8));
      const float bt = beta[tt];
      const float a[4] = {bt * v[i].x, bt * v[i].y, bt * v[i].z, bt * v[i].w};
      put_a4_lds<true>(ares, MTB, tt, k, a);
    }
  }
  __syncthreads();
  f32x4_t acc[S::MTW][S::NTW];
  auto zero = [&]() {
#pragma unroll
    for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < S::NTW; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  zero();
  mg_pipe_loop(
      q, nsteps, stage, S::kBBytes, load,
      [&](const Pieces<NV>& v, char* buf) {
#pragma unroll
        for (int i = 0; i < NV; ++i) store16(buf + (i * kBlock + tid) * 16, v.v[i]);
      },
      [&](int st, const char* buf) {
        const int j = j0 + st / KS, ks = st % KS;
        mg_step<MTB, NCA, 4>(ares + ks * S::kABytes, buf, acc);
        if (ks == KS - 1) {  // tile j complete
          mg_for_outputs4<MTB, NCA, 4>(acc, t0, j * NCA, [&](int t, int c, const f32x4_t& v) {
            if (t < T) {  // four bf16 in one 8-byte store (KVR % 8 == 0, c % 4 == 0)
              const float sl = p.scale_log2;
              const uint2 w = make_uint2(pack_bf16x2(f32_to_bf16(v[0] * sl), f32_to_bf16(v[1] * sl)),
                                         pack_bf16x2(f32_to_bf16(v[2] * sl), f32_to_bf16(v[3] * sl)));
              *reinterpret_cast<uint2*>(p.qcat + ((size_t)t * p.NH + h) * p.KVR + c) = w;
            }
          });
          zero();
        }
      });
  if (j0 != 0) return;  // the first tile group also ropes q_pe
  const int half = p.DR / 2;
  constexpr int NQ = MTB <= 2 ? 4 : 8;  // (token, rotary pair) items per thread per pass
  constexpr int GQ = MTB <= 2 ? 8 : 1;  // slabs whose loads go out together
  for (int base = 0; base < MTB * 16 * half; base += NQ * kBlock) {
    float2 x[NQ];
    const float* src[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      x[j] = make_float2(0.f, 0.f);
      const int idx = base + j * kBlock + tid;
      const int tt = idx / half, i = idx % half, t = t0 + tt;
      src[j] = (idx < MTB * 16 * half && t < T) ? p.part2 + (size_t)t * p.N2 + (size_t)h * p.QKH + p.DN + 2 * i
                                                 : nullptr;
    }
    for (int s2 = 0; s2 < pl.s2; s2 += GQ) {
      float2 v[GQ][NQ];
#pragma unroll
      for (int u = 0; u < GQ; ++u) {
        const size_t o = (size_t)(s2 + u) * T * p.N2;
#pragma unroll
        for (int j = 0; j < NQ; ++j)
          v[u][j] = (src[j] && s2 + u < pl.s2) ? *reinterpret_cast<const float2*>(src[j] + o) : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < GQ; ++u)
        if (s2 + u < pl.s2)
#pragma unroll
          for (int j = 0; j < NQ; ++j) {
            x[j].x += v[u][j].x;
            x[j].y += v[u][j].y;
          }
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int idx = base + j * kBlock + tid;
      const int tt = idx / half, i = idx % half, t = t0 + tt;
      if (idx >= MTB * 16 * half || t >= T) continue;
      const float bq = beta[tt] * p.scale_log2;  // the query tile is stored pre-scaled
      rope_q(p, t, h, i, x[j].x * bq, x[j].y * bq);
    }
  }
}


// ---------------------------------------------------------------------------
// k_oabsorb: workgroup (head h, token block).  o_lat, the core's split
// partials combined (weights w_s = 2^(m_s - M) over the splits, L = sum_s w_s
// l_s, o_lat = (sum_s w_s o_s) / L in split order; a token with no valid entry
// gets zeros), goes to LDS as hi/lo fragments in the plain order and meets
// out_absorb_w[h] ([DV, R], k-contiguous: B fragments load straight from
// memory, every k-step of two output tiles at once).  o_v goes to A5 in
// fragment order; the last head's workgroups write A5's K padding.
// LDS: split weights [16*MTB][nsplit] | 1/L [16*MTB] | A4 (R/32 x MTB x 2 KB).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int oabsorb_hdr_bytes(int mtb, int nsplit) {
  return (16 * mtb * (nsplit + 1) * 4 + 255) / 256 * 256;
}
constexpr int kOabsMaxKs = 16;  // kv_lora_rank <= 512

// Activation halves the o-projection reads (gemm_mfma.h): blocks of 32 to
// 128 tokens take o_v as plain bf16 (its hi half).  There the hi/lo products
// and the second half's loads cost more than the weight stream can hide
// (at 128 tokens the doubled matrix work alone outweighs it), and o_v is the
// path's last activation: its rounding reaches the output only through the
// sum over n_heads * v_head_dim products.
__host__ __device__ constexpr int oproj_ah(int mtb) { return mtb >= 2 ? 1 : 2; }

// Q5 output tiles per wave.  With nq5 > 1 parts per (head, token block) each
// workgroup takes 4*Q5 of the 16-row output tiles (and combines the splits
// itself), so few heads and tokens still fill the chip.
template <int MTB, int Q5, bool PO16>
__device__ void phase_oabsorb_m(const StepParams& p, int b, char* lds) {
  using ElemT = std::conditional_t<PO16, _Float16, float>;  // the core's partials (pl.po16)
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, p.NH * pl.nq5, pl.ntb5, u, tb)) return;
  const int h = u / pl.nq5, pq = u % pl.nq5;
  const int T = pl.T, R = p.R, tid = threadIdx.x, NSP = pl.nsplit;
  const int t0 = tb * MTB * 16;
  const int nt = min(MTB * 16, T - t0);
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int KS = R / kMgK;
  const int ndt = (p.DV + 15) / 16;
  const int nlo = pl.nq5 == 1 ? 0 : pq * 4 * Q5;
  const int nhi = pl.nq5 == 1 ? ndt : min(ndt, nlo + 4 * Q5);
  // this wave's tiles n0 + 4q: every B fragment straight from the k-contiguous weight
  bf16x8_t bfr[Q5][kOabsMaxKs];
  auto load_b = [&](int n0) {
#pragma unroll
    for (int q = 0; q < Q5; ++q) {
      const int d = 16 * (n0 + 4 * q) + l16;
      const bool dok = n0 + 4 * q < nhi && d < p.DV;
      const bf16_t* wrow = p.w_oabs + ((size_t)h * p.DV + (dok ? d : 0)) * R + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kOabsMaxKs; ++ks) {
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (dok && ks < KS) v = load16_nt(wrow + kMgK * ks);
        bfr[q][ks] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  };
  // one tile per wave: its fragments load before the combine (two would hold
  // too many registers across it)
  const int nfirst = nlo + wave;
  if (Q5 == 1 && nfirst < nhi) load_b(nfirst);
  float* wsp = reinterpret_cast<float*>(lds);  // [16*MTB][NSP]
  float* linv = wsp + 16 * MTB * NSP;           // [16*MTB]
  char* ares = lds + oabsorb_hdr_bytes(MTB, NSP);
  // split weights and 1/L: a wave per token (tokens wave + 4j), a lane per
  // split (NSP <= 64), every token's loads issued together; the butterfly
  // sums leave the same value in every lane
  constexpr int TPW = MTB * 16 / (kBlock / kWave);
  float mj[TPW], lj[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tt = wave + j * (kBlock / kWave);
    const bool ok = tt < nt && lane < NSP;
    const size_t q = ((size_t)(t0 + (ok ? tt : 0)) * NSP + (ok ? lane : 0)) * p.NH + h;
    mj[j] = ok ? p.pm[q] : -INFINITY;
    lj[j] = ok ? p.pden[q] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tt = wave + j * (kBlock / kWave);
    if (tt >= nt) continue;  // wave-uniform
    const float m = mj[j], l = lj[j];
    const float M = wave_max_dpp(m);
    const float w = (M == -INFINITY || lane >= NSP) ? 0.f : exp2f(m - M);
    const float L = wave_sum_dpp(l * w);
    // normalised fp16 partials (o / l) weigh in with w * l
    if (lane < NSP) wsp[tt * NSP + lane] = PO16 ? w * l : w;
    if (lane == 0) linv[tt] = (L > 0.f) ? 1.f / L : 0.f;
  }
  __syncthreads();
  // o_lat float4 items (token, 4 columns), eight per thread per pass; the
  // loads of G splits go out together (splits past the last are not loaded).  Two tiles per wave keep G = 1: the registers
  // of four splits cost more than the round trips they save.  Partials in
  // fp16 (PO16) are four halves, 8 bytes, per item.
  {
    using VT = std::conditional_t<PO16, f16x4_t, float4>;
    constexpr int NI = 8;
    constexpr int G = Q5 == 1 ? 4 : (PO16 ? 2 : 1);
    const int n_items = MTB * 16 * (R / 4);
    for (int base = 0; base < n_items; base += NI * kBlock) {
      float4 o[NI];
      const VT* src[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int idx = base + i * kBlock + tid;
        const int tt = idx / (R / 4), c = 4 * (idx % (R / 4));
        src[i] = (idx < n_items && tt < nt)
                     ? reinterpret_cast<const VT*>(reinterpret_cast<const ElemT*>(p.po) +
                                                   ((size_t)(t0 + tt) * NSP * p.NH + h) * R + c)
                     : nullptr;
      }
      for (int s = 0; s < NSP; s += G) {
        VT v[G][NI];
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const size_t off = (size_t)(s + u) * p.NH * R / 4;  // in items
#pragma unroll
          for (int i = 0; i < NI; ++i) v[u][i] = (src[i] && s + u < NSP) ? src[i][off] : VT{};
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
          if (s + u >= NSP) continue;  // uniform
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const int idx = base + i * kBlock + tid;
            const int tt = idx / (R / 4);
            const float w = src[i] ? wsp[tt * NSP + s + u] : 0.f;
            o[i].x = fmaf(w, (float)v[u][i].x, o[i].x);
            o[i].y = fmaf(w, (float)v[u][i].y, o[i].y);
            o[i].z = fmaf(w, (float)v[u][i].z, o[i].z);
            o[i].w = fmaf(w, (float)v[u][i].w, o[i].w);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int idx = base + i * kBlock + tid;
        if (idx >= n_items) continue;
        const int tt = idx / (R / 4), c = 4 * (idx % (R / 4));
        const float li = tt < nt ? linv[tt] : 0.f;
        const float a[4] = {o[i].x * li, o[i].y * li, o[i].z * li, o[i].w * li};
        put_a4_lds<false>(ares, MTB, tt, c, a);
      }
    }
  }
  __syncthreads();
  const int K5 = p.NH * p.DV;
  const bool a5_lo = oproj_ah(pl.mtb) == 2;  // the o-projection reads A5's lo half
  for (int n0 = nfirst; n0 < nhi; n0 += 4 * Q5) {
    if (Q5 != 1 || n0 != nfirst) load_b(n0);
#pragma unroll
    for (int q = 0; q < Q5; ++q) {
      const int n = n0 + 4 * q;
      if (n >= nhi) continue;  // wave-uniform
      f32x4_t acc[MTB];
#pragma unroll
      for (int mt = 0; mt < MTB; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kOabsMaxKs; ++ks) {
        if (ks >= KS) continue;  // uniform
        const char* blk = ares + (size_t)(ks * MTB) * 2 * (kAFragElems * 2);
#pragma unroll
        for (int mt = 0; mt < MTB; ++mt) {
          const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t*>(blk + ((mt * 2) * 64 + lane) * 16);
          const bf16x8_t alo = *reinterpret_cast<const bf16x8_t*>(blk + ((mt * 2 + 1) * 64 + lane) * 16);
          // transposed product: lane (g, l16) gets o_v columns 4g..4g+3 of token l16
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[q][ks], ahi, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[q][ks], alo, acc[mt], 0, 0, 0);
        }
      }
      const int d0 = 16 * n + 4 * g;
#pragma unroll
      for (int mt = 0; mt < MTB; ++mt) {
        const int t = t0 + 16 * mt + l16;
        if (t >= T) continue;
        const float a[4] = {acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]};
        if ((p.DV & 3) == 0 && d0 + 3 < p.DV) {
          put_a4(p.a5, pl.mt_pad, t, h * p.DV + d0, a, a5_lo);  // one 8-byte run per half
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (d0 + i >= p.DV) continue;
            const bf16_t hi = f32_to_bf16(a[i]);
            const size_t e = abuf_index(t, h * p.DV + d0 + i, pl.mt_pad);
            p.a5[e] = hi;
            p.a5[e + kAFragElems] = f32_to_bf16(a[i] - bf16_to_f32(hi));
          }
        }
      }
    }
  }
  if (h == p.NH - 1 && pq == 0) {
    const int KP = pl.kt6 * kMgK;
    for (int idx = tid; idx < nt * (KP - K5); idx += kBlock) {
      const int t = t0 + idx / (KP - K5), k = K5 + idx % (KP - K5);
      const size_t e = abuf_index(t, k, pl.mt_pad);
      p.a5[e] = 0;
      p.a5[e + kAFragElems] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// k_oproj: split-K partials of A5 @ o_proj_w (oproj_ah(MTB) halves of A5)
// ---------------------------------------------------------------------------

template <int MTB>
__device__ void phase_oproj_m(const StepParams& p, int b, char* stage) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, pl.nt6m * pl.s6, pl.ntb, u, tb)) return;
  const int tile = u % pl.nt6m, slab = u / pl.nt6m;
  constexpr int NC = mg_cols(MTB);
  const int c0 = tile * NC;
  const int k0 = slab * pl.ks6m * kMgK;
  const int nks = min(pl.ks6m, pl.kt6 - slab * pl.ks6m);
  f32x4_t acc[Mg<MTB>::MTW][Mg<MTB>::NTW];
  mgemm<MTB, mg_cols(MTB), mg_waves(MTB), oproj_ah(MTB)>(p.a5, pl.mt_pad, tb * MTB, p.w_o, p.NH * p.DV, p.H, k0, nks,
                                                        c0, reinterpret_cast<const bf16_t*>(p.zero16), stage, acc);
  const int T = pl.T;
  float* out = p.part6 + (size_t)slab * T * p.H;
  mg_for_outputs4<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, const f32x4_t& v) {
    if (t < T) store_f32x4(out + (size_t)t * p.H, c, p.H, v);
  });
}

}  // namespace mla
