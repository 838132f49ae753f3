// Phases of the matrix-core path, used when a step carries more than a few
// tokens.  The operations and their order are those of the GEMV path
// (phases.h); the projections become hi/lo bf16 GEMMs on the matrix cores
// (gemm_mfma.h).  Each producer writes the next GEMM's activation already in
// fragment order, so the GEMM kernels stream both operands with direct
// global->LDS loads:
//   k_prep    index build; A1 = x * g_in; sums of x^2
//   k_down    split-K partials of A1 @ [wq_a | wkv_a]
//   k_qa      per token: reduce them; A2 = acc_q * g_q; beta = alpha * inv_q;
//             kv-latent RMSNorm, RoPE and the cache-row write
//   k_qup     split-K partials of A2 @ wq_b
//   k_absorb  q_lat = (beta * q_nope) @ q_absorb_w[h]; RoPE of q_pe -> Qcat
//   k_core    (shared with the GEMV path)
//   k_oabsorb split combine; o_v = out_absorb_w[h] . o_lat -> A5
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

// ---------------------------------------------------------------------------
// k_prep: index build (first n_idx_wg workgroups); then one workgroup per
// token: A1 = x * g_in in fragment order (K padded with zeros) and sum of x^2.
// ---------------------------------------------------------------------------
__device__ void phase_prep(const StepParams& p, int b, float* lds) {
  const Plan& pl = p.pl;
  if (b < pl.n_idx_wg) {
    index_build(p, b * kBlock + threadIdx.x);
    return;
  }
  const int t = b - pl.n_idx_wg;
  const int KP = pl.kt1 * kMgK;
  const bf16_t* xr = p.x + (size_t)t * p.H;
  float ss = 0.f;
  for (int k = 4 * threadIdx.x; k < KP; k += 4 * kBlock) {
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
  if (threadIdx.x == 0) p.ssx[t] = ss;
}

// ---------------------------------------------------------------------------
// k_down: split-K partials of A1 @ [wq_a | wkv_a] (wq_a's tiles first)
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_down_m(const StepParams& p, int b, char* ring, char* sink) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, pl.nt1m * pl.s1, pl.ntb, u, tb)) return;
  const int tile = u % pl.nt1m, slab = u / pl.nt1m;
  const bool is_q = tile < pl.ntq1m;
  const bf16_t* W = is_q ? p.wq_a : p.wkv_a;
  const int N = is_q ? p.Q : p.KVR;
  const int c0 = (is_q ? tile : tile - pl.ntq1m) * kMgCols;
  const int k0 = slab * pl.ks1m * kMgK;
  const int nks = min(pl.ks1m, pl.kt1 - slab * pl.ks1m);
  f32x4_t acc[Mg<MTB>::MTW][Mg<MTB>::NTW];
  mgemm<MTB>(p.a1, pl.mt_pad, tb * MTB, W, p.H, N, k0, nks, c0, p.zero16, ring, sink, acc);
  const int N1 = p.Q + p.KVR, T = pl.T;
  float* out = p.part1 + (size_t)slab * T * N1 + (is_q ? 0 : p.Q);
  mg_for_outputs<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, float v) {
    if (t < T && c < N) out[(size_t)t * N1 + c] = v;
  });
}

// ---------------------------------------------------------------------------
// k_qa: one workgroup per token.  Reduces the down-projection over its slabs
// (fixed order); alpha = 1/rms(x); A2 = acc_q * g_q in fragment order;
// beta = alpha / rms(alpha * acc_q); and the kv branch: y = alpha * acc_kv,
// RMSNorm of its latent part, RoPE of its rotary part, bf16 row at slot_mapping[t].
// ---------------------------------------------------------------------------
__device__ void phase_qa(const StepParams& p, int b, float* lds) {
  const Plan& pl = p.pl;
  const int T = pl.T, t = b, tid = threadIdx.x;
  const int N1 = p.Q + p.KVR;
  float* row = lds;                           // [N1]
  float* scratch = lds + ((N1 + 63) & ~63);   // block_sum scratch
  for (int c4 = tid; c4 < N1 / 4; c4 += kBlock) {
    const float* src = p.part1 + (size_t)t * N1 + 4 * c4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < pl.s1; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(src + (size_t)s * T * N1);
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    *reinterpret_cast<float4*>(row + 4 * c4) = a;
  }
  __syncthreads();
  const float alpha = inv_rms(p.ssx[t], p.H, p.eps);
  const int KP = pl.kt2 * kMgK;
  float ss = 0.f;
  for (int k = 4 * tid; k < KP; k += 4 * kBlock) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (k < p.Q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = row[k + i];
        ss = fmaf(v, v, ss);
        a[i] = v * p.g_q[k + i];
      }
    }
    put_a4(p.a2, pl.mt_pad, t, k, a);
  }
  ss = block_sum(ss, scratch);
  const float iq = 1.f / sqrtf(alpha * alpha * ss / (float)p.Q + p.eps);
  if (tid == 0) p.beta[t] = alpha * iq;
  const float* kv = row + p.Q;
  float sk = 0.f;
  for (int c = tid; c < p.R; c += kBlock) {
    const float y = alpha * kv[c];
    sk = fmaf(y, y, sk);
  }
  sk = block_sum(sk, scratch);
  const float inv = inv_rms(sk, p.R, p.eps);
  bf16_t* crow = p.cache + (size_t)p.slot[t] * p.KVR;
  for (int c = tid; c < p.R; c += kBlock) crow[c] = f32_to_bf16(alpha * kv[c] * inv * p.g_kv[c]);
  const int half = p.DR / 2;
  for (int i = tid; i < half; i += kBlock) {
    const float x0 = alpha * kv[p.R + 2 * i], x1 = alpha * kv[p.R + 2 * i + 1];
    const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
    crow[p.R + 2 * i] = f32_to_bf16(x0 * cs - x1 * sn);
    crow[p.R + 2 * i + 1] = f32_to_bf16(x0 * sn + x1 * cs);
  }
}

// ---------------------------------------------------------------------------
// k_qup: split-K partials of A2 @ wq_b
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_qup_m(const StepParams& p, int b, char* ring, char* sink) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, pl.nt2m * pl.s2, pl.ntb, u, tb)) return;
  const int tile = u % pl.nt2m, slab = u / pl.nt2m;
  const int c0 = tile * kMgCols;
  const int k0 = slab * pl.ks2m * kMgK;
  const int nks = min(pl.ks2m, pl.kt2 - slab * pl.ks2m);
  f32x4_t acc[Mg<MTB>::MTW][Mg<MTB>::NTW];
  mgemm<MTB>(p.a2, pl.mt_pad, tb * MTB, p.wq_b, p.Q, p.N2, k0, nks, c0, p.zero16, ring, sink, acc);
  const int T = pl.T;
  float* out = p.part2 + (size_t)slab * T * p.N2;
  mg_for_outputs<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, float v) {
    if (t < T && c < p.N2) out[(size_t)t * p.N2 + c] = v;
  });
}

// ---------------------------------------------------------------------------
// k_absorb: workgroup (head h, 64-column tile of kv_lora_rank, token block).
// A3 = beta * q_nope (wq_b slabs summed in order) goes to LDS in fragment
// order; the weight tile streams through the ring; q_lat lands in Qcat as
// bf16.  The tile-0 workgroups also rope q_pe into Qcat.
// LDS: ring (kMgDepth x 4 KB) | sink (1 KB) | A3 (ceil(DN/32) x MTB x 2 KB).
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_absorb_m(const StepParams& p, int b, char* lds) {
  using S = Mg<MTB>;
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, p.NH * pl.nct3, pl.ntb3, u, tb)) return;
  const int h = u / pl.nct3, j = u % pl.nct3;
  const int T = pl.T, tid = threadIdx.x;
  const int t0 = tb * MTB * 16;
  const int KS = (p.DN + kMgK - 1) / kMgK;
  char* ring = lds;
  char* sink = lds + kMgDepth * S::kBBytes;
  char* ares = sink + 1024;
  for (int idx = tid; idx < MTB * 16 * KS * 8; idx += kBlock) {
    const int tt = idx / (KS * 8), k = 4 * (idx % (KS * 8));
    const int t = t0 + tt;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < T && k < p.DN) {  // DN % 8 == 0
      const float* src = p.part2 + (size_t)t * p.N2 + (size_t)h * p.QKH + k;
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < pl.s2; ++s) {
        const float4 v = *reinterpret_cast<const float4*>(src + (size_t)s * T * p.N2);
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
      }
      const float bt = p.beta[t];
      a[0] = bt * sum.x; a[1] = bt * sum.y; a[2] = bt * sum.z; a[3] = bt * sum.w;
    }
    put_a4_lds<true>(ares, MTB, tt, k, a);
  }
  __syncthreads();
  f32x4_t acc[S::MTW][S::NTW];
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int c0 = j * kMgCols;
  const BTileSrc bs = btile_src(p.w_qabs + (size_t)h * p.DN * p.R, p.DN, p.R, 0, c0);
  mg_ring<1>(
      KS, ring, S::kBBytes,
      [&](int st, char* buf) { issue_btile(bs, st, st < KS, buf, p.zero16); },
      [&](int st, const char* buf) { mg_step<MTB>(ares + st * S::kABytes, buf, acc); });
  mg_for_outputs<MTB>(acc, t0, c0, [&](int t, int c, float v) {
    if (t < T) p.qcat[((size_t)t * p.NH + h) * p.KVR + c] = f32_to_bf16(v);
  });
  if (j == 0) {
    const int half = p.DR / 2;
    for (int idx = tid; idx < MTB * 16 * half; idx += kBlock) {
      const int t = t0 + idx / half, i = idx % half;
      if (t >= T) continue;
      const float* src = p.part2 + (size_t)t * p.N2 + (size_t)h * p.QKH + p.DN + 2 * i;
      float x0 = 0.f, x1 = 0.f;
      for (int s = 0; s < pl.s2; ++s) {
        x0 += src[(size_t)s * T * p.N2];
        x1 += src[(size_t)s * T * p.N2 + 1];
      }
      const float bt = p.beta[t];
      x0 *= bt;
      x1 *= bt;
      const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
      bf16_t* q = p.qcat + ((size_t)t * p.NH + h) * p.KVR + p.R;
      q[2 * i] = f32_to_bf16(x0 * cs - x1 * sn);
      q[2 * i + 1] = f32_to_bf16(x0 * sn + x1 * cs);
    }
  }
}

// ---------------------------------------------------------------------------
// k_oabsorb: workgroup (head h, token block).  Combines the core's split
// partials into o_lat (softmax normalisation; no valid entry gives zeros),
// stores it in LDS as hi/lo fragments in the plain order, and multiplies by
// out_absorb_w[h] ([DV, R], k-contiguous: B fragments load straight from
// memory).  o_v goes to A5 in fragment order; the last head's workgroups
// write A5's K padding.
// LDS: split weights [16*MTB][nsplit] | 1/L [16*MTB] | A4 (R/32 x MTB x 2 KB).
// ---------------------------------------------------------------------------
template <int MTB>
__device__ void phase_oabsorb_m(const StepParams& p, int b, char* lds) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, p.NH, pl.ntb5, u, tb)) return;
  const int h = u;
  const int T = pl.T, NSP = pl.nsplit, R = p.R, tid = threadIdx.x;
  const int t0 = tb * MTB * 16;
  const int nt = min(MTB * 16, T - t0);
  float* wsp = reinterpret_cast<float*>(lds);  // [16*MTB][NSP]
  float* plv = wsp + MTB * 16 * NSP;           // [16*MTB][NSP] denominators
  float* linv = plv + MTB * 16 * NSP;          // [16*MTB]
  char* ares = lds + ((size_t)(2 * MTB * 16 * NSP + MTB * 16) * 4 + 255) / 256 * 256;
  for (int idx = tid; idx < nt * NSP; idx += kBlock) {
    const int tt = idx / NSP, s = idx % NSP;
    const size_t q = ((size_t)(t0 + tt) * NSP + s) * p.NH + h;
    wsp[idx] = p.pm[q];
    plv[idx] = p.pden[q];
  }
  __syncthreads();
  if (tid < nt) {
    float M = -INFINITY;
    for (int s = 0; s < NSP; ++s) M = fmaxf(M, wsp[tid * NSP + s]);
    float L = 0.f;
    for (int s = 0; s < NSP; ++s) {
      const float w = (M == -INFINITY) ? 0.f : exp2f(wsp[tid * NSP + s] - M);
      wsp[tid * NSP + s] = w;
      L = fmaf(plv[tid * NSP + s], w, L);
    }
    linv[tid] = (L > 0.f) ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < MTB * 16 * (R / 4); idx += kBlock) {
    const int tt = idx / (R / 4), c = 4 * (idx % (R / 4));
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (tt < nt) {
      const float* src = p.po + ((size_t)(t0 + tt) * NSP * p.NH + h) * R + c;
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < NSP; ++s) {
        const float w = wsp[tt * NSP + s];
        const float4 v = *reinterpret_cast<const float4*>(src + (size_t)s * p.NH * R);
        o.x = fmaf(w, v.x, o.x); o.y = fmaf(w, v.y, o.y); o.z = fmaf(w, v.z, o.z); o.w = fmaf(w, v.w, o.w);
      }
      const float li = linv[tt];
      a[0] = o.x * li; a[1] = o.y * li; a[2] = o.z * li; a[3] = o.w * li;
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
        if (dok && ks + q < KS) v = *reinterpret_cast<const u32x4_t*>(wrow + kMgK * (ks + q));
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
__device__ void phase_oproj_m(const StepParams& p, int b, char* ring, char* sink) {
  const Plan& pl = p.pl;
  int u, tb;
  if (!mg_unit(b, pl.nt6m * pl.s6, pl.ntb, u, tb)) return;
  const int tile = u % pl.nt6m, slab = u / pl.nt6m;
  const int c0 = tile * kMgCols;
  const int k0 = slab * pl.ks6m * kMgK;
  const int nks = min(pl.ks6m, pl.kt6 - slab * pl.ks6m);
  f32x4_t acc[Mg<MTB>::MTW][Mg<MTB>::NTW];
  mgemm<MTB>(p.a5, pl.mt_pad, tb * MTB, p.w_o, p.NH * p.DV, p.H, k0, nks, c0, p.zero16, ring, sink, acc);
  const int T = pl.T;
  float* out = p.part6 + (size_t)slab * T * p.H;
  mg_for_outputs<MTB>(acc, tb * MTB * 16, c0, [&](int t, int c, float v) {
    if (t < T && c < p.H) out[(size_t)t * p.H + c] = v;
  });
}

}  // namespace mla
