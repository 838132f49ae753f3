// Gather-attention core on the matrix cores (gfx950, wave64).
//
// For one token, every head attends over the rows its selected positions
// resolve to.  Scores and the latent output are two dense contractions over
// the gathered rows, shared by all heads (MLA keeps one latent KV head):
//   S^T[row, head] = sum_k K[row, k] * Qcat[head, k]        (k over kv_row = latent | rope)
//   O[head, c]    += sum_row P[head, row] * K[row, c]         (c over the latent width)
// Both run as 16x16 MFMA tiles: a wave owns 16 heads ("head group") and takes
// 16 gathered rows per step.  The score tile's output layout (lane l holds rows
// 4*(l/16)+i of head l%16) is exactly the A-operand layout of the 16x16x16
// product, so the probabilities never leave registers; the value operand is
// read from the LDS copy of the rows with the transposing LDS read, which hands
// lane l four consecutive rows of column l%16.
#pragma once

#include "device_util.h"
#include "step_params.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ i16x4_t pack4_bf16(float a, float b, float c, float d) {
  i16x4_t r;
  r[0] = (short)f32_to_bf16(a);
  r[1] = (short)f32_to_bf16(b);
  r[2] = (short)f32_to_bf16(c);
  r[3] = (short)f32_to_bf16(d);
  return r;
}

// LDS bytes of the core for a given row pitch (bf16 elements) and row streams.
__host__ __device__ constexpr int core_lds_bytes(int rp, int rs) { return rs * 16 * rp * 2 + rs * 16 * 4; }

// NT: latent width / 16.  HG: head groups (of 16) per workgroup.  NW: waves.
// Row streams RS = NW / HG; stream s walks 16-row chunks s, s+RS, ... of the
// split, and each stream writes its own partial result (m, l, o).
template <int NT, int HG, int NW>
__device__ void core_phase(const StepParams& p, int b, char* lds_raw) {
  constexpr int RS = NW / HG;
  constexpr int KSMAX = NT / 2 + 2;  // 32-wide k-steps over kv_row = 16*NT + DR, DR <= 64
  constexpr int LS = 64 * HG;        // lanes loading one stream's chunk
  constexpr int PSTRIDE = LS / 16;   // 16-byte pieces of a row taken per lane step
  constexpr int PFMAX = (2 * NT + 8 + PSTRIDE - 1) / PSTRIDE;  // pieces per lane (kv_row/8 <= 2*NT+8)
  const Plan& pl = p.pl;
  const int KVR = p.KVR;
  const int ks = (KVR + 31) >> 5;
  const int RP = ks * 32 + 8;  // padded LDS row pitch in bf16
  const int npieces = KVR >> 3;

  const int per_t = pl.nsplit * pl.core_nhb;
  const int t = b / per_t;
  const int rem = b % per_t;
  const int hb = rem / pl.nsplit, split = rem % pl.nsplit;
  const int j0 = split * pl.ps, j1 = min(p.P, j0 + pl.ps);
  const int nchunks = (j1 - j0 + 15) >> 4;
  const int iters = (nchunks + RS - 1) / RS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave % HG, rs = wave / HG;
  const int g = lane >> 4, l16 = lane & 15;
  const int head = (hb * HG + hg) * 16 + l16;  // this lane's head for Q / softmax state

  bf16_t* buf = reinterpret_cast<bf16_t*>(lds_raw) + rs * 16 * RP;
  int* valid = reinterpret_cast<int*>(lds_raw + RS * 16 * RP * 2) + rs * 16;

  // zero the padded columns once (never overwritten by row data)
  for (int i = tid; i < RS * 16 * (RP - KVR); i += NW * 64) {
    const int row = i / (RP - KVR), c = KVR + i % (RP - KVR);
    reinterpret_cast<bf16_t*>(lds_raw)[row * RP + c] = 0;
  }

  // Q fragments (B operand of the score product): lane l holds Qcat[head][32*kk + 8*g .. +8]
  bf16x8_t qf[KSMAX];
#pragma unroll
  for (int kk = 0; kk < KSMAX; ++kk) {
    const int k = 32 * kk + 8 * g;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (kk < ks && head < p.NH && k < KVR)
      v = *reinterpret_cast<const u32x4_t*>(p.qcat + ((size_t)t * p.NH + head) * KVR + k);
    qf[kk] = __builtin_bit_cast(bf16x8_t, v);
  }

  f32x4_t o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // chunk loader: this lane's stream-local index, row within the chunk and first piece
  const int sl = hg * 64 + lane;  // 0 .. LS-1
  const int lrow = sl & 15, lp0 = sl >> 4;
  u32x4_t pf[PFMAX];
  int prow = -1;
  auto prefetch = [&](int it) {
    const int chunk = it * RS + rs;
    const int j = j0 + 16 * chunk + lrow;
    prow = (chunk < nchunks && j < j1) ? p.rows[(size_t)t * p.P + j] : -1;
#pragma unroll
    for (int u = 0; u < PFMAX; ++u) {
      const int pc = lp0 + u * PSTRIDE;
      pf[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (prow >= 0 && pc < npieces)
        pf[u] = *reinterpret_cast<const u32x4_t*>(p.cache + (size_t)prow * KVR + 8 * pc);
    }
  };

  if (iters > 0) prefetch(0);
  for (int it = 0; it < iters; ++it) {
    const int chunk = it * RS + rs;
    __syncthreads();  // the previous chunk is fully consumed
#pragma unroll
    for (int u = 0; u < PFMAX; ++u) {
      const int pc = lp0 + u * PSTRIDE;
      if (pc < npieces) *reinterpret_cast<u32x4_t*>(buf + lrow * RP + 8 * pc) = pf[u];
    }
    if (lp0 == 0) valid[lrow] = prow >= 0;
    __syncthreads();
    if (it + 1 < iters) prefetch(it + 1);
    if (chunk >= nchunks) continue;  // wave-uniform: this stream has no chunk this round

    // scores S^T[row 4g+i][head l16]
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSMAX; ++kk) {
      if (kk < ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(buf + l16 * RP + 32 * kk + 8 * g);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc, 0, 0, 0);
      }
    }
    float s[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = valid[4 * g + i] ? sacc[i] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f, pr[4] = {0.f, 0.f, 0.f, 0.f};
    if (m_new != -INFINITY) {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = exp2f(s[i] - m_new);  // -inf -> 0
    }
    float ps = (pr[0] + pr[1]) + (pr[2] + pr[3]);
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // rescale the accumulators: lane l holds heads 4g+i of each output tile
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= ai[i];
    // O[head][c] += P[head][rows] * V[rows][c]
    const i16x4_t pa = pack4_bf16(pr[0], pr[1], pr[2], pr[3]);
    const bf16_t* vbase = buf + (4 * g + (l16 >> 2)) * RP + 4 * (l16 & 3);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vbase + 16 * n));
      o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[n], 0, 0, 0);
    }
  }

  const size_t pb = ((size_t)t * pl.nsplit + split) * p.NH;
  const int hbase = (hb * HG + hg) * 16;
  if constexpr (RS == 1) {
    // one stream: its (m, l, o) is this split's partial result
    if (g == 0 && head < p.NH) {
      p.pm[pb + head] = m_run;
      p.pden[pb + head] = l_run;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hbase + 4 * g + i;
        if (h < p.NH) p.po[(pb + h) * (16 * NT) + 16 * n + l16] = o[n][i];
      }
  } else {
    // HG == 1: merge the RS streams (same 16 heads) in LDS, in stream order
    float* ml = reinterpret_cast<float*>(lds_raw);      // [RS][16] m, then [RS][16] l
    float* acc = ml + 2 * RS * 16;                      // [16][16*NT]
    __syncthreads();                                    // row buffers are free now
    if (g == 0) {
      ml[rs * 16 + l16] = m_run;
      ml[RS * 16 + rs * 16 + l16] = l_run;
    }
    __syncthreads();
    // this lane's heads 4g+i: merged max and the stream's weight
    float wi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * g + i;
      float M = -INFINITY;
#pragma unroll
      for (int s2 = 0; s2 < RS; ++s2) M = fmaxf(M, ml[s2 * 16 + hh]);
      wi[i] = (M == -INFINITY) ? 0.f : exp2f(ml[rs * 16 + hh] - M);
    }
    for (int s2 = 0; s2 < RS; ++s2) {
      if (rs == s2) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* a = acc + (4 * g + i) * (16 * NT) + 16 * n + l16;
            const float v = o[n][i] * wi[i];
            *a = (s2 == 0) ? v : *a + v;
          }
      }
      __syncthreads();
    }
    if (rs == 0) {
      if (g == 0 && head < p.NH) {
        float M = -INFINITY;
        for (int s2 = 0; s2 < RS; ++s2) M = fmaxf(M, ml[s2 * 16 + l16]);
        float L = 0.f;
        if (M != -INFINITY)
          for (int s2 = 0; s2 < RS; ++s2) L += ml[RS * 16 + s2 * 16 + l16] * exp2f(ml[s2 * 16 + l16] - M);
        p.pm[pb + head] = M;
        p.pden[pb + head] = L;
      }
      for (int idx = lane; idx < 16 * 16 * NT; idx += 64) {
        const int h = hbase + idx / (16 * NT);
        if (h < p.NH) p.po[(pb + h) * (16 * NT) + idx % (16 * NT)] = acc[idx];
      }
    }
  }
}

}  // namespace mla
