// Phases of the matrix-core path, used when a step carries more than a few
// tokens.  The operations and their order are those of the GEMV path
// (phases.h); the projections become hi/lo bf16 GEMMs on the matrix cores
// (gemm_mfma.h).  Each producer writes the next GEMM's activation already in
// fragment order, so the GEMM kernels stream both operands with direct
// global->LDS loads:
//   k_prep    index build; A1 = x * g_in; partial sums of x^2
//   k_down    split-K partials of A1 @ [wq_a | wkv_a]
//   k_qa      reduce them: A2 = acc_q * g_q and partial sums of acc_q^2 per
//             column chunk; per token, kv-latent RMSNorm, RoPE, cache-row write
//   k_qup     split-K partials of A2 @ wq_b
//   k_absorb  q_lat = (beta * q_nope) @ q_absorb_w[h], beta = alpha * inv_q;
//             RoPE of q_pe -> Qcat
//   k_core    (shared with the GEMV path)
//   k_combine the core's split partials -> normalised o_lat (only with splits)
//   k_oabsorb o_v = out_absorb_w[h] . o_lat -> A5
//   k_oproj   split-K partials of A5 @ o_proj_w
//   k_out     (shared) reduction to the bf16 output
// Rows of a token block past the last token carry unspecified values; they
// only reach output rows that are never stored.  K padding is written as zeros.
#pragma once

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

// alpha = 1/rms(x) of token t from the chunk sums (fixed order)
__device__ __forceinline__ float mfma_alpha(const StepParams& p, int t) {
  float s = 0.f;
  for (int c = 0; c < p.pl.nxc; ++c) s += p.ssx[(size_t)c * p.pl.T + t];
  return inv_rms(s, p.H, p.eps);
}

// beta = alpha / rms(alpha * acc_q) of token t: the scale of the wq_b output
__device__ __forceinline__ float mfma_beta(const StepParams& p, int t) {
  const float a = mfma_alpha(p, t);
  float s = 0.f;
  for (int c = 0; c < p.pl.nqc; ++c) s += p.ssq[(size_t)c * p.pl.T + t];
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
  mg_for_outputs<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, float v) {
    if (t < T && c < N) out[(size_t)t * N1 + c] = v;
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
__device__ __forceinline__ float4 sum_slabs4(const float* src, size_t stride, int S) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(src + (size_t)(s + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a.x += v[u].x; a.y += v[u].y; a.z += v[u].z; a.w += v[u].w;
    }
  }
  for (; s < S; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(src + (size_t)s * stride);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  return a;
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
        const float4 v = sum_slabs4(src + k, sstride, pl.s1);
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
    const float4 v = sum_slabs4(src + p.Q + 4 * c4, sstride, pl.s1);
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
  mg_for_outputs<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, float v) {
    if (t < T && c < p.N2) out[(size_t)t * p.N2 + c] = v;
  });
}

// ---------------------------------------------------------------------------
// k_absorb: workgroup (head h, group of tpw3 64-column tiles of kv_lora_rank,
// token block).  The pipeline streams the group's tiles of q_absorb_w[h]
// (ceil(DN/32) k-steps each); its first loads go out before A3 = beta * q_nope
// (wq_b slabs summed in order) is written to LDS in fragment order, once for
// all the group's tiles.  Each tile's q_lat lands in Qcat as bf16, pre-scaled
// by softmax_scale * log2(e); q_pe is roped into Qcat too.
// LDS: stages (2 x 4 KB) | beta (512 B) | A3 (ceil(DN/32) x MTB x 2 KB).
// ---------------------------------------------------------------------------
constexpr int kAbsorbBetaBytes = 512;  // beta of up to 128 tokens

template <int MTB>
__device__ void phase_absorb_m(const StepParams& p, int b, char* lds) {
  using S = Mg<MTB, kMgCols>;
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
  // this lane's piece of a 32 x 64 weight tile (row r, swizzled 16-byte piece pc)
  const bf16_t* W = p.w_qabs + (size_t)h * p.DN * p.R;
  const int r = tid >> 3, pc = (tid & 7) ^ (r & 7);
  auto load = [&](int st) {
    Pieces<1> q;
    const int j = j0 + st / KS, ks = st % KS;
    const int row = ks * kMgK + r;
    const bf16_t* src = reinterpret_cast<const bf16_t*>(p.zero16);
    if (st < nsteps && row < p.DN) src = W + (size_t)row * p.R + j * kMgCols + 8 * pc;
    q.v[0] = load16_nt(src);
    return q;
  };
  constexpr int P = 8;
  Pieces<1> q[P];
  mg_pipe_prologue(q, load);
  if (tid < MTB * 16) beta[tid] = (t0 + tid < T) ? mfma_beta(p, t0 + tid) : 0.f;
  __syncthreads();
  for (int idx = tid; idx < MTB * 16 * KS * 8; idx += kBlock) {
    const int tt = idx / (KS * 8), k = 4 * (idx % (KS * 8));
    const int t = t0 + tt;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < T && k < p.DN) {  // DN % 8 == 0
      const float4 v = sum_slabs4(p.part2 + (size_t)t * p.N2 + (size_t)h * p.QKH + k, (size_t)T * p.N2, pl.s2);
      const float bt = beta[tt];
      a[0] = bt * v.x; a[1] = bt * v.y; a[2] = bt * v.z; a[3] = bt * v.w;
    }
    put_a4_lds<true>(ares, MTB, tt, k, a);
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
      q, nsteps, stage, S::kBBytes, load, [&](const Pieces<1>& v, char* buf) { store16(buf + tid * 16, v.v[0]); },
      [&](int st, const char* buf) {
        const int j = j0 + st / KS, ks = st % KS;
        mg_step<MTB, kMgCols>(ares + ks * S::kABytes, buf, acc);
        if (ks == KS - 1) {  // tile j complete
          mg_for_outputs<MTB, kMgCols>(acc, t0, j * kMgCols, [&](int t, int c, float v) {
            if (t < T) p.qcat[((size_t)t * p.NH + h) * p.KVR + c] = f32_to_bf16(v * p.scale_log2);
          });
          zero();
        }
      });
  if (j0 != 0) return;  // the first tile group also ropes q_pe
  const int half = p.DR / 2;
  for (int idx = tid; idx < MTB * 16 * half; idx += kBlock) {
    const int tt = idx / half, i = idx % half, t = t0 + tt;
    if (t >= T) continue;
    const float* src = p.part2 + (size_t)t * p.N2 + (size_t)h * p.QKH + p.DN + 2 * i;
    float x0 = 0.f, x1 = 0.f;
    for (int s2 = 0; s2 < pl.s2; ++s2) {
      x0 += src[(size_t)s2 * T * p.N2];
      x1 += src[(size_t)s2 * T * p.N2 + 1];
    }
    x0 *= beta[tt] * p.scale_log2;  // the query tile is stored pre-scaled
    x1 *= beta[tt] * p.scale_log2;
    const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
    bf16_t* q = p.qcat + ((size_t)t * p.NH + h) * p.KVR + p.R;
    q[2 * i] = f32_to_bf16(x0 * cs - x1 * sn);
    q[2 * i + 1] = f32_to_bf16(x0 * sn + x1 * cs);
  }
}

// ---------------------------------------------------------------------------
// k_combine (when the core splits the selected rows): one thread per
// (token, head, 4 latent columns).  Weights w_s = 2^(m_s - M) over the splits,
// L = sum_s w_s * l_s, o_lat = sum_s w_s * o_s / L in split order; a token
// with no valid entry (L = 0) gets zeros.
// ---------------------------------------------------------------------------
__device__ void phase_combine(const StepParams& p, int b) {
  const Plan& pl = p.pl;
  const int R4 = p.R / 4, NSP = pl.nsplit;
  const int i = b * kBlock + threadIdx.x;
  if (i >= pl.T * p.NH * R4) return;
  const int c4 = i % R4, th = i / R4, h = th % p.NH, t = th / p.NH;
  const float* pm = p.pm + (size_t)t * NSP * p.NH + h;
  const float* pd = p.pden + (size_t)t * NSP * p.NH + h;
  float M = -INFINITY;
  for (int s = 0; s < NSP; ++s) M = fmaxf(M, pm[(size_t)s * p.NH]);
  float L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
    const float* po = p.po + ((size_t)t * NSP * p.NH + h) * p.R + 4 * c4;
    for (int s = 0; s < NSP; ++s) {
      const float w = exp2f(pm[(size_t)s * p.NH] - M);
      L = fmaf(pd[(size_t)s * p.NH], w, L);
      const float4 v = *reinterpret_cast<const float4*>(po + (size_t)s * p.NH * p.R);
      o.x = fmaf(w, v.x, o.x); o.y = fmaf(w, v.y, o.y); o.z = fmaf(w, v.z, o.z); o.w = fmaf(w, v.w, o.w);
    }
  }
  const float li = (L > 0.f) ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(p.olat + (size_t)th * p.R + 4 * c4) = make_float4(o.x * li, o.y * li, o.z * li, o.w * li);
}

// ---------------------------------------------------------------------------
// k_oabsorb: workgroup (head h, token block).  o_lat (from k_combine, or the
// core's single split divided by its denominator) goes to LDS as hi/lo
// fragments in the plain order and meets out_absorb_w[h] ([DV, R],
// k-contiguous: B fragments load straight from memory).  o_v goes to A5 in
// fragment order; the last head's workgroups write A5's K padding.
// LDS: 1/L [16*MTB] (256 B) | A4 (R/32 x MTB x 2 KB).
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_oabsorb_m(const StepParams& p, int b, char* lds) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, p.NH, pl.ntb5, u, tb)) return;
  const int h = u;
  const int T = pl.T, R = p.R, tid = threadIdx.x;
  const int t0 = tb * MTB * 16;
  const int nt = min(MTB * 16, T - t0);
  const bool split = pl.nsplit > 1;
  float* linv = reinterpret_cast<float*>(lds);  // [16*MTB]
  char* ares = lds + 256;
  if (tid < nt) {
    float li = 1.f;
    if (!split) {
      const float L = p.pden[(size_t)(t0 + tid) * p.NH + h];
      li = (L > 0.f) ? 1.f / L : 0.f;
    }
    linv[tid] = li;
  }
  __syncthreads();
  const float* src = split ? p.olat : p.po;  // both [T][NH][R] here
  for (int idx = tid; idx < MTB * 16 * (R / 4); idx += kBlock) {
    const int tt = idx / (R / 4), c = 4 * (idx % (R / 4));
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (tt < nt) {
      const float4 v = *reinterpret_cast<const float4*>(src + ((size_t)(t0 + tt) * p.NH + h) * R + c);
      const float li = linv[tt];
      a[0] = v.x * li; a[1] = v.y * li; a[2] = v.z * li; a[3] = v.w * li;
    }
    put_a4_lds<false>(ares, MTB, tt, c, a);
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int KS = R / kMgK;
  const int ndt = (p.DV + 15) / 16;
  const int K5 = p.NH * p.DV;
  for (int n = wave; n < ndt; n += 4) {
    f32x4_t acc[MTB];
#pragma unroll
    for (int mt = 0; mt < MTB; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int d = 16 * n + l16;
    const bool dok = d < p.DV;
    const bf16_t* wrow = p.w_oabs + ((size_t)h * p.DV + (dok ? d : 0)) * R + 8 * g;
    for (int ks = 0; ks < KS; ks += 4) {
      bf16x8_t bfr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (dok && ks + q < KS) v = load16_nt(wrow + kMgK * (ks + q));
        bfr[q] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (ks + q >= KS) break;
        const char* blk = ares + (size_t)((ks + q) * MTB) * 2 * (kAFragElems * 2);
#pragma unroll
        for (int mt = 0; mt < MTB; ++mt) {
          const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t*>(blk + ((mt * 2) * 64 + lane) * 16);
          const bf16x8_t alo = *reinterpret_cast<const bf16x8_t*>(blk + ((mt * 2 + 1) * 64 + lane) * 16);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfr[q], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfr[q], acc[mt], 0, 0, 0);
        }
      }
    }
    if (dok) {
      const int k = h * p.DV + d;
#pragma unroll
      for (int mt = 0; mt < MTB; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * mt + 4 * g + i;
          if (t < T) {
            const float v = acc[mt][i];
            const bf16_t hi = f32_to_bf16(v);
            const size_t e = abuf_index(t, k, pl.mt_pad);
            p.a5[e] = hi;
            p.a5[e + kAFragElems] = f32_to_bf16(v - bf16_to_f32(hi));
          }
        }
    }
  }
  if (h == p.NH - 1) {
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
// k_oproj: split-K partials of A5 @ o_proj_w
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
  mgemm<MTB>(p.a5, pl.mt_pad, tb * MTB, p.w_o, p.NH * p.DV, p.H, k0, nks, c0, reinterpret_cast<const bf16_t*>(p.zero16), stage, acc);
  const int T = pl.T;
  float* out = p.part6 + (size_t)slab * T * p.H;
  mg_for_outputs<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, float v) {
    if (t < T && c < p.H) out[(size_t)t * p.H + c] = v;
  });
}

}  // namespace mla
