// Phases of one MLA gather-decode step.  Each phase is a device function over
// "virtual workgroups" b in [0, n); a kernel runs one phase with one
// workgroup per b.  Operation order follows the parameter list of the MLA
// attention block gather decode API page: index build; input RMSNorm and the
// wq_a / wkv_a down-projections; query-latent RMSNorm and wq_b; kv-latent
// RMSNorm, RoPE and the cache-row write; q absorption and RoPE of q_pe; the
// gather-attention core; output absorption; o-projection.
#pragma once

#include "device_util.h"
#include "step_params.h"

namespace mla {

constexpr int kTile = 512;     // output columns per GEMV tile: 64 lanes x 8 bf16
constexpr int kGemvTT = 4;     // tokens per pass of the VALU GEMV
constexpr int kHeadGroup = 16; // heads per attention-core workgroup
constexpr int kChunk = 16;     // gathered rows staged per core iteration
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// split-K GEMV tile: part[t][c0 + c] = sum_{k in [k0,k1)} (X[t][k] * gamma[k]) * W[k][c0 + c]
// for c < nc <= 512, all T tokens.  W is [K, N] row-major bf16, read once per
// token pass with 16-byte loads; wave w takes rows k0+w, k0+w+4, ...; the four
// waves are summed through LDS.  X is fp32 (Xf) or bf16 (Xb) with leading
// dimension ldx.  `lds` holds 4*kGemvTT*512 floats.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gemv_tile(const bf16_t* __restrict__ W, int N, int k0, int k1, int c0,
                                          int nc, const float* __restrict__ Xf,
                                          const bf16_t* __restrict__ Xb, int ldx,
                                          const float* __restrict__ gamma, int T,
                                          float* __restrict__ part, int ldp, float* lds) {
  const int tid = threadIdx.x, cg = tid & 63, wv = tid >> 6;
  const bool active = 8 * cg < nc;
  for (int t0 = 0; t0 < T; t0 += kGemvTT) {
    float acc[kGemvTT][8];
#pragma unroll
    for (int tt = 0; tt < kGemvTT; ++tt)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[tt][i] = 0.f;
#pragma unroll 4
    for (int k = k0 + wv; k < k1; k += 4) {
      float w[8];
      if (active) {
        const uint4 v = *reinterpret_cast<const uint4*>(W + (size_t)k * N + c0 + 8 * cg);
        unpack8(v, w);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.f;
      }
      const float g = gamma ? gamma[k] : 1.f;
#pragma unroll
      for (int tt = 0; tt < kGemvTT; ++tt) {
        const int t = t0 + tt;
        float xv = 0.f;
        if (t < T) xv = (Xf ? Xf[(size_t)t * ldx + k] : bf16_to_f32(Xb[(size_t)t * ldx + k])) * g;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[tt][i] = fmaf(xv, w[i], acc[tt][i]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < kGemvTT; ++tt)
#pragma unroll
      for (int i = 0; i < 8; ++i) lds[(wv * kGemvTT + tt) * kTile + 8 * cg + i] = acc[tt][i];
    __syncthreads();
    for (int idx = tid; idx < kGemvTT * kTile; idx += kBlock) {
      const int tt = idx / kTile, c = idx % kTile, t = t0 + tt;
      if (c < nc && t < T) {
        float s = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) s += lds[(w4 * kGemvTT + tt) * kTile + c];
        part[(size_t)t * ldp + c0 + c] = s;
      }
    }
    __syncthreads();
  }
}

// sum_{k in [k0,k1)} X[t][k]^2 for every token, one thread per token
__device__ __forceinline__ void slab_sumsq(const float* __restrict__ Xf, const bf16_t* __restrict__ Xb,
                                           int ldx, int k0, int k1, int T, float* __restrict__ ss) {
  for (int t = threadIdx.x; t < T; t += kBlock) {
    float s = 0.f;
    for (int k = k0; k < k1; ++k) {
      const float v = Xf ? Xf[(size_t)t * ldx + k] : bf16_to_f32(Xb[(size_t)t * ldx + k]);
      s = fmaf(v, v, s);
    }
    ss[t] = s;
  }
}

// ---------------------------------------------------------------------------
// phase 1: index build + input RMSNorm folded into the wq_a / wkv_a down-projection.
// The norm's 1/rms is a per-token scalar, so the GEMV runs on x*gamma and the
// reducer of each column tile multiplies by 1/rms from the slabs' sums of squares.
// ---------------------------------------------------------------------------
__device__ void phase_down(const StepParams& p, int b, float* lds, int* flag) {
  const Plan& pl = p.pl;
  const int T = pl.T;
  const int n_gemv = pl.nt1 * pl.s1;
  if (b >= n_gemv) {
    // index build: selected position -> flat cache row, -1 where causally masked.
    const int idx = (b - n_gemv) * kBlock + threadIdx.x;
    if (idx < T * p.P) {
      const int t = idx / p.P;
      const int g = p.gidx[idx];
      const int ps = p.pos[t];
      int row = -1;
      if (g >= 0 && g <= ps) row = p.btab[(size_t)t * p.MB + g / p.BS] * p.BS + g % p.BS;
      p.rows[idx] = row;
      if (p.rows_out) p.rows_out[idx] = row;
    }
    return;
  }
  const int tile = b / pl.s1, slab = b % pl.s1;
  const bool is_q = tile < pl.nt_q;
  const bf16_t* W = is_q ? p.wq_a : p.wkv_a;
  const int N = is_q ? p.Q : p.KVR;
  const int c0 = (is_q ? tile : tile - pl.nt_q) * kTile;
  const int nc = min(kTile, N - c0);
  const int N1 = p.Q + p.KVR;
  const int k0 = slab * pl.ks1, k1 = min(p.H, k0 + pl.ks1);
  float* part = p.part1 + (size_t)slab * T * N1 + (is_q ? 0 : p.Q);
  gemv_tile(W, N, k0, k1, c0, nc, nullptr, p.x, p.H, p.g_in, T, part, N1, lds);
  slab_sumsq(nullptr, p.x, p.H, k0, k1, T, p.ss1 + ((size_t)tile * pl.s1 + slab) * T);
  if (!arrive_last(p.cnt + pl.cnt1 + tile, pl.s1, flag)) return;
  // reducer for this column tile
  float* inv = lds;  // [T]
  for (int t = threadIdx.x; t < T; t += kBlock) {
    float ss = 0.f;
    for (int s = 0; s < pl.s1; ++s) ss += p.ss1[((size_t)tile * pl.s1 + s) * T + t];
    inv[t] = 1.f / sqrtf(ss / (float)p.H + p.eps);
  }
  __syncthreads();
  const int base = is_q ? c0 : p.Q + c0;
  for (int idx = threadIdx.x; idx < T * nc; idx += kBlock) {
    const int t = idx / nc, c = idx % nc;
    float y = 0.f;
    for (int s = 0; s < pl.s1; ++s) y += p.part1[((size_t)s * T + t) * N1 + base + c];
    y *= inv[t];
    if (is_q) p.qa[(size_t)t * p.Q + c0 + c] = y;
    else p.kvb[(size_t)t * p.KVR + c0 + c] = y;
  }
}

// ---------------------------------------------------------------------------
// phase 2: query-latent RMSNorm folded into wq_b (same scheme as phase 1), and
// in extra workgroups the kv branch: kv-latent RMSNorm, interleaved RoPE of the
// rotary part, bf16 write of the row at slot_mapping[t].
// ---------------------------------------------------------------------------
__device__ void phase_qup(const StepParams& p, int b, float* lds, int* flag) {
  const Plan& pl = p.pl;
  const int T = pl.T;
  const int n_gemv = pl.nt2 * pl.s2;
  if (b >= n_gemv) {
    const int t = b - n_gemv;
    const float* kv = p.kvb + (size_t)t * p.KVR;
    float ss = 0.f;
    for (int c = threadIdx.x; c < p.R; c += kBlock) ss = fmaf(kv[c], kv[c], ss);
    ss = block_sum(ss, lds);
    const float inv = 1.f / sqrtf(ss / (float)p.R + p.eps);
    bf16_t* row = p.cache + (size_t)p.slot[t] * p.KVR;
    for (int c = threadIdx.x; c < p.R; c += kBlock) row[c] = f32_to_bf16(kv[c] * inv * p.g_kv[c]);
    const int half = p.DR / 2;
    for (int i = threadIdx.x; i < half; i += kBlock) {
      const float x0 = kv[p.R + 2 * i], x1 = kv[p.R + 2 * i + 1];
      const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
      row[p.R + 2 * i] = f32_to_bf16(x0 * cs - x1 * sn);
      row[p.R + 2 * i + 1] = f32_to_bf16(x0 * sn + x1 * cs);
    }
    return;
  }
  const int tile = b / pl.s2, slab = b % pl.s2;
  const int c0 = tile * kTile, nc = min(kTile, p.N2 - c0);
  const int k0 = slab * pl.ks2, k1 = min(p.Q, k0 + pl.ks2);
  gemv_tile(p.wq_b, p.N2, k0, k1, c0, nc, p.qa, nullptr, p.Q, p.g_q, T,
            p.part2 + (size_t)slab * T * p.N2, p.N2, lds);
  slab_sumsq(p.qa, nullptr, p.Q, k0, k1, T, p.ss2 + ((size_t)tile * pl.s2 + slab) * T);
  if (!arrive_last(p.cnt + pl.cnt2 + tile, pl.s2, flag)) return;
  float* inv = lds;
  for (int t = threadIdx.x; t < T; t += kBlock) {
    float ss = 0.f;
    for (int s = 0; s < pl.s2; ++s) ss += p.ss2[((size_t)tile * pl.s2 + s) * T + t];
    inv[t] = 1.f / sqrtf(ss / (float)p.Q + p.eps);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * nc; idx += kBlock) {
    const int t = idx / nc, c = idx % nc;
    float y = 0.f;
    for (int s = 0; s < pl.s2; ++s) y += p.part2[((size_t)s * T + t) * p.N2 + c0 + c];
    p.q[(size_t)t * p.N2 + c0 + c] = y * inv[t];
  }
}

// ---------------------------------------------------------------------------
// phase 3: q_lat[t,h,:] = q_nope[t,h,:] @ q_absorb_w[h]; RoPE of q_pe[t,h,:].
// ---------------------------------------------------------------------------
__device__ void phase_absorb(const StepParams& p, int b, float* lds) {
  const Plan& pl = p.pl;
  const int T = pl.T;
  const int h = b / pl.nt_r, rt = b % pl.nt_r;
  const int c0 = rt * kTile, nc = min(kTile, p.R - c0);
  gemv_tile(p.w_qabs + (size_t)h * p.DN * p.R, p.R, 0, p.DN, c0, nc, p.q + (size_t)h * p.QKH, nullptr,
            p.N2, nullptr, T, p.qlat + (size_t)h * p.R, p.NH * p.R, lds);
  if (rt != 0) return;
  const int half = p.DR / 2;
  for (int idx = threadIdx.x; idx < T * half; idx += kBlock) {
    const int t = idx / half, i = idx % half;
    const float* qh = p.q + (size_t)t * p.N2 + (size_t)h * p.QKH + p.DN;
    const float x0 = qh[2 * i], x1 = qh[2 * i + 1];
    const float cs = p.cos_t[(size_t)t * half + i], sn = p.sin_t[(size_t)t * half + i];
    float* o = p.qpe + ((size_t)t * p.NH + h) * p.DR;
    o[2 * i] = x0 * cs - x1 * sn;
    o[2 * i + 1] = x0 * sn + x1 * cs;
  }
}

// ---------------------------------------------------------------------------
// phase 4: gather-attention core.  Workgroup (t, head group, split) walks its
// share of the selected entries 16 rows at a time: stage the gathered rows in
// LDS, scores = scale*(q_lat . row[:R] + q_pe . row[R:]) with masked entries
// at -inf, online softmax (running max m, sum l, output o in the log2
// domain).  The last split of a (t, head group) to finish combines the
// splits' (m, l, o) into o_lat; a token with no valid entry gets zeros.
// ---------------------------------------------------------------------------
// LDS floats of the core: q_lat [16][R+4], q_pe [16][DR+4], rows [kChunk][KVR+4] bf16,
// scores [16][kChunk], row ids [kChunk]; sized for R <= 512, DR <= 128.
constexpr int kCoreLds = 16 * (512 + 4) + 16 * (128 + 4) + (kChunk * (640 + 4)) / 2 + 16 * kChunk + kChunk;

__device__ void phase_core(const StepParams& p, int b, float* lds, int* flag) {
  const Plan& pl = p.pl;
  const int R = p.R, DR = p.DR, KVR = p.KVR;
  const int per_t = pl.nhg * pl.nsplit;
  const int t = b / per_t, rem = b % per_t, hg = rem / pl.nsplit, s = rem % pl.nsplit;
  const int h0 = hg * kHeadGroup, nhl = min(kHeadGroup, p.NH - h0);
  const int j0 = s * pl.ps, j1 = min(p.P, j0 + pl.ps);
  const int RQ = R + 4, DQ = DR + 4, KP = KVR + 4;  // padded LDS pitches
  float* q_s = lds;                                  // [16][RQ]
  float* qp_s = q_s + 16 * RQ;                       // [16][DQ]
  bf16_t* k_s = reinterpret_cast<bf16_t*>(qp_s + 16 * DQ);  // [kChunk][KP]
  float* sc = reinterpret_cast<float*>(k_s + kChunk * KP);  // [16][kChunk]
  int* ri = reinterpret_cast<int*>(sc + 16 * kChunk);       // [kChunk]
  const int tid = threadIdx.x;

  for (int idx = tid; idx < 16 * R; idx += kBlock) {
    const int hl = idx / R, c = idx % R;
    q_s[hl * RQ + c] = hl < nhl ? p.qlat[((size_t)t * p.NH + h0 + hl) * R + c] : 0.f;
  }
  for (int idx = tid; idx < 16 * DR; idx += kBlock) {
    const int hl = idx / DR, c = idx % DR;
    qp_s[hl * DQ + c] = hl < nhl ? p.qpe[((size_t)t * p.NH + h0 + hl) * DR + c] : 0.f;
  }
  const int hl = tid / 16, cb = tid % 16;  // accumulator ownership: head hl, column block cb
  const int RC = R / 16;                   // columns per thread (<= 32)
  float o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int nvec = KVR / 8;

  for (int jc = j0; jc < j1; jc += kChunk) {
    const int nr = min(kChunk, j1 - jc);
    __syncthreads();  // previous chunk fully consumed
    if (tid < kChunk) ri[tid] = tid < nr ? p.rows[(size_t)t * p.P + jc + tid] : -1;
    __syncthreads();
    for (int v = tid; v < kChunk * nvec; v += kBlock) {
      const int rr = v / nvec, q8 = v % nvec;
      const int row = ri[rr];
      uint4 val = make_uint4(0, 0, 0, 0);
      if (row >= 0) val = *reinterpret_cast<const uint4*>(p.cache + (size_t)row * KVR + 8 * q8);
      uint32_t* dst = reinterpret_cast<uint32_t*>(k_s + rr * KP + 8 * q8);
      dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
    }
    __syncthreads();
    {
      const int hs = tid / kChunk, js = tid % kChunk;
      float sv = -INFINITY;
      if (hs < nhl && js < nr && ri[js] >= 0) {
        const bf16_t* kr = k_s + js * KP;
        const float* qr = q_s + hs * RQ;
        float acc = 0.f;
        for (int c = 0; c < R; c += 2) {
          const uint32_t kk = *reinterpret_cast<const uint32_t*>(kr + c);
          acc = fmaf(qr[c], bf16lo(kk), acc);
          acc = fmaf(qr[c + 1], bf16hi(kk), acc);
        }
        const float* qpr = qp_s + hs * DQ;
        for (int c = 0; c < DR; c += 2) {
          const uint32_t kk = *reinterpret_cast<const uint32_t*>(kr + R + c);
          acc = fmaf(qpr[c], bf16lo(kk), acc);
          acc = fmaf(qpr[c + 1], bf16hi(kk), acc);
        }
        sv = acc * p.scale_log2;
      }
      sc[hs * kChunk + js] = sv;
    }
    __syncthreads();
    float cmax = -INFINITY;
    for (int j = 0; j < nr; ++j) cmax = fmaxf(cmax, sc[hl * kChunk + j]);
    const float m_new = fmaxf(m, cmax);
    if (m_new != -INFINITY) {
      const float alpha = exp2f(m - m_new);  // m = -inf gives 0
      l *= alpha;
      for (int i = 0; i < RC; ++i) o[i] *= alpha;
      for (int j = 0; j < nr; ++j) {
        const float sj = sc[hl * kChunk + j];
        if (sj == -INFINITY) continue;
        const float pj = exp2f(sj - m_new);
        l += pj;
        const bf16_t* kr = k_s + j * KP + cb * RC;
        for (int i = 0; i < RC; ++i) o[i] = fmaf(pj, bf16_to_f32(kr[i]), o[i]);
      }
      m = m_new;
    }
  }
  // this split's partial result
  const size_t pbase = ((size_t)t * pl.nsplit + s) * p.NH;
  if (hl < nhl) {
    float* co = p.co + (pbase + h0 + hl) * R + cb * RC;
    for (int i = 0; i < RC; ++i) co[i] = o[i];
    if (cb == 0) {
      p.cm[pbase + h0 + hl] = m;
      p.cl[pbase + h0 + hl] = l;
    }
  }
  if (!arrive_last(p.cnt + pl.cnt3 + t * pl.nhg + hg, pl.nsplit, flag)) return;
  for (int idx = tid; idx < nhl * R; idx += kBlock) {
    const int hh = h0 + idx / R, c = idx % R;
    float M = -INFINITY;
    for (int sp = 0; sp < pl.nsplit; ++sp) M = fmaxf(M, p.cm[((size_t)t * pl.nsplit + sp) * p.NH + hh]);
    float res = 0.f;
    if (M != -INFINITY) {
      float L = 0.f, O = 0.f;
      for (int sp = 0; sp < pl.nsplit; ++sp) {
        const size_t pb = ((size_t)t * pl.nsplit + sp) * p.NH + hh;
        const float ms = p.cm[pb];
        if (ms == -INFINITY) continue;
        const float wgt = exp2f(ms - M);
        L = fmaf(p.cl[pb], wgt, L);
        O = fmaf(p.co[pb * R + c], wgt, O);
      }
      res = O / L;
    }
    p.olat[((size_t)t * p.NH + hh) * R + c] = res;
  }
}

// ---------------------------------------------------------------------------
// phase 5: o_v[t, h*dv + d] = out_absorb_w[h, d, :] . o_lat[t, h, :]; one wave per (h, d).
// ---------------------------------------------------------------------------
__device__ void phase_oabsorb(const StepParams& p, int b) {
  const int T = p.pl.T;
  const int lane = threadIdx.x & 63;
  const int rr = b * 4 + (threadIdx.x >> 6);
  if (rr >= p.NH * p.DV) return;
  const int h = rr / p.DV;
  const int c = 8 * lane;
  float w[8];
  if (c < p.R) {
    unpack8(*reinterpret_cast<const uint4*>(p.w_oabs + (size_t)rr * p.R + c), w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0.f;
  }
  for (int t = 0; t < T; ++t) {
    float acc = 0.f;
    if (c < p.R) {
      const float* ol = p.olat + ((size_t)t * p.NH + h) * p.R + c;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(w[i], ol[i], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) p.ov[(size_t)t * p.NH * p.DV + rr] = acc;
  }
}

// ---------------------------------------------------------------------------
// phase 6: out[t,:] = o_v[t,:] @ o_proj_w (this rank's partial); bf16 output.
// ---------------------------------------------------------------------------
__device__ void phase_oproj(const StepParams& p, int b, float* lds, int* flag) {
  const Plan& pl = p.pl;
  const int T = pl.T;
  const int K = p.NH * p.DV;
  const int tile = b / pl.s5, slab = b % pl.s5;
  const int c0 = tile * kTile, nc = min(kTile, p.H - c0);
  const int k0 = slab * pl.ks5, k1 = min(K, k0 + pl.ks5);
  gemv_tile(p.w_o, p.H, k0, k1, c0, nc, p.ov, nullptr, K, nullptr, T,
            p.part5 + (size_t)slab * T * p.H, p.H, lds);
  if (!arrive_last(p.cnt + pl.cnt5 + tile, pl.s5, flag)) return;
  for (int idx = threadIdx.x; idx < T * nc; idx += kBlock) {
    const int t = idx / nc, c = idx % nc;
    float y = 0.f;
    for (int s = 0; s < pl.s5; ++s) y += p.part5[((size_t)s * T + t) * p.H + c0 + c];
    p.out[(size_t)t * p.H + c0 + c] = f32_to_bf16(y);
  }
}

}  // namespace mla
