// Phases of one MLA gather-decode step.  Each phase is a device function over
// workgroup index b; one kernel runs one phase.  The operation order follows
// the parameter list of the MLA attention block gather decode API page:
// index build; input RMSNorm folded into the wq_a / wkv_a down-projection;
// query-latent RMSNorm folded into wq_b; kv-latent RMSNorm, interleaved RoPE
// and the cache-row write; absorption of q_nope into the latent and RoPE of
// q_pe; the gather-attention core; output absorption; o-projection.
//
// Split-K partial sums are plain stores; the consuming phase reduces them in
// a fixed order (no atomics, no arrival counters), so a step is bitwise
// reproducible for a given n_tokens.  Each GEMV workgroup issues its first
// weight loads before it reduces its activations, so the two latencies overlap.
//
// Every RMSNorm's 1/rms is a per-token scalar, so it is factored out of the
// GEMV that follows the norm and applied where the reduced sums are consumed:
//   q_a   = alpha * acc_a,      alpha = 1/sqrt(mean(x^2) + eps)
//   c_q   = q_a * inv_q * g_q,  inv_q = 1/sqrt(alpha^2 * mean(acc_a^2) + eps)
//   q     = (alpha * inv_q) * ((acc_a * g_q) @ wq_b)
#pragma once

#include "core_mfma.h"
#include "mfma_util.h"
#include "device_util.h"
#include "gemv.h"
#include "handoff.h"
#include "step_params.h"
#include "mla_gather_decode.h"

namespace MLA_PHASE_NS {
using namespace ::mla;

// LDS of a GEMV phase that passes over NTT tokens at a time (floats):
// xs [NTT][512], red [3][NTT][512], scratch [1024], aux [1024]
template <int NTT>
struct GemvLds {
  static constexpr int xs = 0;
  static constexpr int red = NTT * kTile;
  static constexpr int scratch = red + 3 * NTT * kTile;
  static constexpr int aux = scratch + 1024;
  static constexpr int floats = aux + 1024;
};
constexpr int kGemvLdsFloats = GemvLds<kTT>::floats;  // the largest (kTT tokens per pass)
// k_oabsorb's LDS layout (floats): split weights and maxima | o_lat [8][R] | scratch
constexpr int kOabsOl = kTT * kTile;
constexpr int kOabsScratch = kOabsOl + 4096;
constexpr int kKvSlice = 64;  // kv-row columns reduced per kv-branch workgroup

__device__ __forceinline__ float inv_rms(float sumsq, int n, float eps) {
  return 1.f / sqrtf(sumsq / (float)n + eps);
}

// Index build for entry idx = t*P + j: selected position -> flat cache row,
// -1 where causally masked.  Masked entries touch neither the block table nor
// the cache.  Token t resolves through block-table row token_seq[t] (row t
// without token_seq).  With the debug checks, an entry whose sequence,
// block-table column or block id is out of range is masked too, and reported.
template <class Sy = HandoffNone>
__device__ __forceinline__ void index_build(const StepParams& p, int idx, const Sy& sy = Sy()) {
  if (idx >= MLA_PL(T) * p.P) return;
  const int t = idx / p.P;
  const int g = p.gidx[idx];
  const int ps = p.pos[t];
  int row = -1;
  if (g >= 0 && g <= ps) {
    const int col = g / p.BS;
    const int sq = p.tseq ? p.tseq[t] : t;
    if (p.dbg && (unsigned)sq >= (unsigned)MLA_PL(T)) {
      atomicOr(p.err, MLA_GD_CHECK_SEQ_RANGE);
    } else if (p.dbg && col >= p.MB) {
      atomicOr(p.err, MLA_GD_CHECK_TABLE_COLUMN);
    } else {
      const int blk = p.btab[(size_t)sq * p.MB + col];
      if (p.dbg && (unsigned)blk >= (unsigned)p.NBLK) atomicOr(p.err, MLA_GD_CHECK_BLOCK_RANGE);
      else row = blk * p.BS + g % p.BS;
    }
  }
  sy.st(p.rows + idx, row);
  if (p.rows_out) p.rows_out[idx] = row;
}

// The workspace's 256-byte zero region (the source of padding loads) must
// read as zeros.  Workgroup 0 of a step's first kernel rewrites it, so a
// workspace whose earlier contents are unknown (a reused buffer, the static
// scratch of the allocation-free entry point) needs no separate clearing; no
// workgroup of a first kernel reads the region.
__device__ __forceinline__ void clear_zero_region(const StepParams& p, int b) {
  if (b == 0 && threadIdx.x < 64) const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(p.zero16))[threadIdx.x] = 0u;
}

// Whether token t's cache row may be written: always without the debug
// checks; with them, when slot_mapping[t] lies in the pool (a slot shared
// with another token is reported and still written).  Every thread of the
// workgroup calls it.
__device__ __forceinline__ bool slot_ok(const StepParams& p, int t) {
  if (!p.dbg) return true;
  const int s = p.slot[t];
  const bool in_range = (unsigned)s < (unsigned)p.NBLK * (unsigned)p.BS;
  int shared = 0;
  for (int u = threadIdx.x; u < MLA_PL(T); u += blockDim.x) shared |= (u != t && p.slot[u] == s);
  shared = __syncthreads_or(shared);
  if (threadIdx.x == 0) {
    if (!in_range) atomicOr(p.err, MLA_GD_CHECK_SLOT_RANGE);
    if (shared) atomicOr(p.err, MLA_GD_CHECK_SLOT_SHARED);
  }
  return in_range;
}

// ---------------------------------------------------------------------------
// Counters of the fused variant.  A producer workgroup publishes its stores
// with a device-scope release and one atomic increment; a consumer polls with
// relaxed device-scope loads (bounded: after kSpinLimit polls it sets
// MLA_GD_CHECK_WAIT_TIMEOUT in the error word and goes on, so no wait can
// hang) and then fences before reading.
// Producers always have lower workgroup indices than their consumers and never
// wait themselves, so in-order dispatch guarantees progress.
// ---------------------------------------------------------------------------
constexpr int kSyncStride = 16;  // counters 64 bytes apart
constexpr int kSpinLimit = 1 << 20;

// The barrier completes every wave's stores; one device-scope fence then
// writes the XCD's L2 back (it is shared by the workgroup's waves).
__device__ __forceinline__ void count_done(unsigned* c) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Polls with relaxed device-scope loads (an acquire load would invalidate the
// caches on every poll); the caller fences once after the wait.
__device__ __forceinline__ void wait_count(const unsigned* c, unsigned target, unsigned* err) {
  for (int it = 0; __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++it) {
    if (it >= kSpinLimit) {
      atomicOr(err, MLA_GD_CHECK_WAIT_TIMEOUT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// ---------------------------------------------------------------------------
// k_down: index build; (x * g_in) @ [wq_a | wkv_a] split-K partials; sums of x^2
// ---------------------------------------------------------------------------
template <int NTT, class Sy = HandoffNone>
__device__ __attribute__((always_inline)) void phase_down(const StepParams& p, int b, float* lds, const Sy& sy = Sy()) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T);
  const int n_gemv = pl.nt1 * MLA_PL(s1);
  if (b >= n_gemv) {
    index_build(p, (b - n_gemv) * kBlock + threadIdx.x);
    return;
  }
  const int slab = b / pl.nt1, tile = b % pl.nt1;
  const bool is_q = tile < pl.nt_q;
  const bf16_t* W = is_q ? p.wq_a : p.wkv_a;
  const int N = is_q ? MLA_D(Q) : MLA_D(KVR);
  const int c0 = (is_q ? tile : tile - pl.nt_q) * MLA_PL(tw1);
  const int nc = min(MLA_PL(tw1), N - c0);
  const int N1 = MLA_D(Q) + MLA_D(KVR);
  const int k0 = slab * MLA_PL(ks1), ks = min(MLA_PL(ks1), MLA_D(H) - k0);
  float* xs = lds + GemvLds<NTT>::xs;
  float* red = lds + GemvLds<NTT>::red;
  for (int t0 = 0; t0 < T; t0 += NTT) {
    const int nt = min(NTT, T - t0);
    u32x4 v[gemv_unroll(NTT)];
    gemv_first<gemv_unroll(NTT)>(W, N, k0, ks, c0, nc, v);
    for (int idx = threadIdx.x; idx < nt * ks; idx += kBlock) {
      const int tt = idx / ks, r = idx % ks;
      xs[tt * kTile + r] = bf16_to_f32(p.x[(size_t)(t0 + tt) * MLA_D(H) + k0 + r]) * p.g_in[k0 + r];
    }
    if (tile == 0) {
      // sum of x^2 over this slab, one 32-lane group per token
      const int tt = threadIdx.x >> 5, rp = threadIdx.x & 31;
      float s = 0.f;
      if (tt < nt)
        for (int r = rp; r < ks; r += 32) {
          const float xv = bf16_to_f32(p.x[(size_t)(t0 + tt) * MLA_D(H) + k0 + r]);
          s = fmaf(xv, xv, s);
        }
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
      if (tt < nt && rp == 0) sy.st(p.ssx + (size_t)slab * T + t0 + tt, s);
    }
    __syncthreads();
    float* part = p.part1 + ((size_t)slab * T + t0) * N1 + (is_q ? 0 : MLA_D(Q));
    gemv_tile<NTT, gemv_unroll(NTT)>(W, N, k0, ks, c0, nc, xs, kTile, nt, part, N1, red, v, sy);
  }
}

// ---------------------------------------------------------------------------
// k_qup: (acc_a * g_q) @ wq_b split-K partials and sums of acc_a^2.  Extra
// workgroups (token t, 64-column slice) reduce the kv row: kvr = alpha * acc_kv
// and partial sums of squares of its latent columns.
// ---------------------------------------------------------------------------
template <int NTT, class Sy = HandoffNone>
__device__ __attribute__((always_inline)) void phase_qup(const StepParams& p, int b, float* lds, const Sy& sy = Sy()) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T);
  const int N1 = MLA_D(Q) + MLA_D(KVR);
  const int n_gemv = pl.nt2 * MLA_PL(s2);
  float* xs = lds + GemvLds<NTT>::xs;
  float* red = lds + GemvLds<NTT>::red;
  float* scratch = lds + GemvLds<NTT>::scratch;
  if (b >= n_gemv) {
    const int t = (b - n_gemv) / MLA_PL(nkv), sl = (b - n_gemv) % MLA_PL(nkv);
    const int c0 = sl * kKvSlice, nc = min(kKvSlice, MLA_D(KVR) - c0);
    float* kv = xs;  // [64]
    float* sx = xs + kKvSlice;
    sy.wait();
    reduce_parts4(p.part1 + (size_t)t * N1 + MLA_D(Q) + c0, (size_t)T * N1, MLA_PL(s1), nc / 4, nc / 4, 0, kv, scratch, sy);
    reduce_parts(p.ssx + t, T, MLA_PL(s1), 1, 1, 0, sx, scratch, sy);
    const float alpha = inv_rms(sx[0], MLA_D(H), p.eps);
    float ss = 0.f;
    for (int c = threadIdx.x; c < nc; c += kBlock) {
      const float y = alpha * kv[c];
      sy.st(p.kvr + (size_t)t * MLA_D(KVR) + c0 + c, y);
      if (c0 + c < MLA_D(R)) ss = fmaf(y, y, ss);
    }
    ss = block_sum(ss, scratch);
    if (threadIdx.x == 0) sy.st(p.kvss + (size_t)t * MLA_PL(nkv) + sl, ss);
    return;
  }
  const int slab = b / pl.nt2, tile = b % pl.nt2;
  const int c0 = tile * MLA_PL(tw2), nc = min(MLA_PL(tw2), MLA_D(N2) - c0);
  const int k0 = slab * MLA_PL(ks2), ks = min(MLA_PL(ks2), MLA_D(Q) - k0);
  for (int t0 = 0; t0 < T; t0 += NTT) {
    const int nt = min(NTT, T - t0);
    u32x4 v[gemv_unroll(NTT)];
    gemv_first<gemv_unroll(NTT)>(p.wq_b, MLA_D(N2), k0, ks, c0, nc, v);
    // g_q of this thread's columns r = tid + 256k, before the partials (an
    // input, so before any wait too)
    float gq[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = threadIdx.x + k * kBlock;
      gq[k] = r < ks ? p.g_q[k0 + r] : 0.f;
    }
    sy.wait();
    // acc_a[t][k0 .. k0+ks) reduced over the down-projection's slabs
    reduce_parts4(p.part1 + (size_t)t0 * N1 + k0, (size_t)T * N1, MLA_PL(s1), nt * ks / 4, ks / 4, N1, xs, scratch, sy);
    if (tile == 0) {
      const int tt = threadIdx.x >> 5, rp = threadIdx.x & 31;
      float s = 0.f;
      if (tt < nt)
        for (int r = rp; r < ks; r += 32) s = fmaf(xs[tt * ks + r], xs[tt * ks + r], s);
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
      if (tt < nt && rp == 0) sy.st(p.ssq + (size_t)slab * T + t0 + tt, s);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = threadIdx.x + k * kBlock;
      if (r < ks)
        for (int tt = 0; tt < nt; ++tt) xs[tt * ks + r] *= gq[k];
    }
    for (int r = threadIdx.x + 2 * kBlock; r < ks; r += kBlock) {
      const float g = p.g_q[k0 + r];
      for (int tt = 0; tt < nt; ++tt) xs[tt * ks + r] *= g;
    }
    __syncthreads();
    gemv_tile<NTT, gemv_unroll(NTT)>(p.wq_b, MLA_D(N2), k0, ks, c0, nc, xs, ks, nt, p.part2 + ((size_t)slab * T + t0) * MLA_D(N2), MLA_D(N2), red, v, sy);
  }
}

// Per-token scalars beta = alpha * inv_q (the scale of the wq_b output) from
// the partial sums of squares: pairs q < nt*(s1 + s2), the down-projection's
// slabs of sum(x^2) first, then the up-projection's slabs of sum(acc_a^2).
// tscale_load issues this thread's pairs q = tid + k*kBlock; a workgroup
// calls it before its weight loads, so the answers are not queued behind the
// weight stream (loads return in order).  tscale_finish stages the pairs in
// `scr` (nt*(s1 + s2) floats of LDS) and adds each token's slabs in order.
constexpr int kTsPre = 2;

template <class Sy>
__device__ __forceinline__ float tscale_at(const StepParams& p, int t0, int nt, int q, const Sy& sy) {
  const int n1 = nt * MLA_PL(s1);
  if (q < n1) return sy.ld(p.ssx + (size_t)(q / nt) * MLA_PL(T) + t0 + q % nt);
  q -= n1;
  return sy.ld(p.ssq + (size_t)(q / nt) * MLA_PL(T) + t0 + q % nt);
}

template <class Sy>
__device__ __forceinline__ void tscale_load(const StepParams& p, int t0, int nt, float (&v)[kTsPre], const Sy& sy) {
  const int nq = nt * (MLA_PL(s1) + MLA_PL(s2));
#pragma unroll
  for (int k = 0; k < kTsPre; ++k) {
    const int q = threadIdx.x + k * kBlock;
    v[k] = q < nq ? tscale_at(p, t0, nt, q, sy) : 0.f;
  }
}

template <class Sy>
__device__ __forceinline__ void tscale_finish(const StepParams& p, int t0, int nt, const float (&v)[kTsPre],
                                              float* beta, float* scr, const Sy& sy) {
  const Plan& pl = p.pl;
  const int nq = nt * (MLA_PL(s1) + MLA_PL(s2));
#pragma unroll
  for (int k = 0; k < kTsPre; ++k) {
    const int q = threadIdx.x + k * kBlock;
    if (q < nq) scr[q] = v[k];
  }
  for (int q = threadIdx.x + kTsPre * kBlock; q < nq; q += kBlock) scr[q] = tscale_at(p, t0, nt, q, sy);
  __syncthreads();
  if ((int)threadIdx.x < nt) {
    const int tt = threadIdx.x;
    float sx = 0.f, sq = 0.f;
    for (int sl = 0; sl < MLA_PL(s1); ++sl) sx += scr[sl * nt + tt];
    for (int sl = 0; sl < MLA_PL(s2); ++sl) sq += scr[(MLA_PL(s1) + sl) * nt + tt];
    const float a = inv_rms(sx, MLA_D(H), p.eps);
    const float iq = 1.f / sqrtf(a * a * sq / (float)MLA_D(Q) + p.eps);
    beta[tt] = a * iq;
  }
  __syncthreads();
}

// q_nope slab terms per thread loaded ahead of the token scales (one token per
// pass leaves one or two terms per thread)
__host__ __device__ constexpr int abs_pre(int ntt) { return ntt == 1 ? 2 : 8; }

// ---------------------------------------------------------------------------
// k_absorb: q = beta * (sum of wq_b partials); q_lat[t,h,:] = q_nope[t,h,:] @
// q_absorb_w[h] for a 64-column chunk; the chunk-0 workgroup also ropes q_pe.
// Output: bf16 Qcat[t][h] = [q_lat | q_pe] * softmax_scale * log2(e), laid out
// like a cache row (the core's scores come out in the log2 domain).  Extra
// workgroups (one per token) finish the kv branch: kv-latent RMSNorm,
// interleaved RoPE of the rotary part, bf16 write of the row at slot_mapping[t].
// ---------------------------------------------------------------------------
static_assert(kTT * 32 <= kBlock, "one RoPE pair per thread for every token of a pass (qk_rope_head_dim <= 64)");

template <int NTT, class Sy = HandoffNone>
__device__ __attribute__((always_inline)) void phase_absorb(const StepParams& p, int b, float* lds, const Sy& sy = Sy()) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T);
  float* xs = lds + GemvLds<NTT>::xs;
  float* red = lds + GemvLds<NTT>::red;
  float* scratch = lds + GemvLds<NTT>::scratch;
  const int n_abs = MLA_D(NH) * MLA_PL(ncc3);
  if (b >= n_abs) {
    const int t = b - n_abs;
    const float* kv = p.kvr + (size_t)t * MLA_D(KVR);
    // inputs first: g_kv of columns tid + 256k (kv_lora_rank <= 512) and
    // the RoPE table of pair tid (qk_rope_head_dim <= 64)
    const int half = MLA_D(DR) / 2;
    float gk[2], rc = 0.f, rs = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = threadIdx.x + k * kBlock;
      gk[k] = c < MLA_D(R) ? p.g_kv[c] : 0.f;
    }
    if ((int)threadIdx.x < half) {
      rc = p.cos_t[(size_t)t * half + threadIdx.x];
      rs = p.sin_t[(size_t)t * half + threadIdx.x];
    }
    sy.wait();
    float ss = 0.f;
    for (int i = threadIdx.x; i < MLA_PL(nkv); i += kBlock) ss += sy.ld(p.kvss + (size_t)t * MLA_PL(nkv) + i);
    ss = block_sum(ss, scratch);
    const float inv = inv_rms(ss, MLA_D(R), p.eps);
    if (!slot_ok(p, t)) return;
    bf16_t* row = p.cache + (size_t)p.slot[t] * MLA_D(KVR);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = threadIdx.x + k * kBlock;
      if (c < MLA_D(R)) sy.st(row + c, f32_to_bf16(sy.ld(kv + c) * inv * gk[k]));
    }
    if ((int)threadIdx.x < half) {
      const int i = threadIdx.x;
      const float x0 = sy.ld(kv + MLA_D(R) + 2 * i), x1 = sy.ld(kv + MLA_D(R) + 2 * i + 1);
      sy.st(row + MLA_D(R) + 2 * i, f32_to_bf16(x0 * rc - x1 * rs));
      sy.st(row + MLA_D(R) + 2 * i + 1, f32_to_bf16(x0 * rs + x1 * rc));
    }
    return;
  }
  const int h = b / MLA_PL(ncc3), cc = b % MLA_PL(ncc3);
  const int c0 = cc * 64;
  float* beta = lds + GemvLds<NTT>::aux;
  float* qo = lds + GemvLds<NTT>::aux + 512;  // [NTT][64]
  const bf16_t* W = p.w_qabs + (size_t)h * MLA_D(DN) * MLA_D(R);
  for (int t0 = 0; t0 < T; t0 += NTT) {
    const int nt = min(NTT, T - t0);
    // the small loads go out before the weight stream (in one launch with
    // the producers: after it, since they wait for the producers): the
    // token-scale partials, then q_nope summed over the wq_b slabs: this
    // thread's item (token, 4 columns) and slab part sp (s = sp, sp + nsp,
    // ...), its first kAbsPre terms
    u32x4 v[gemv_unroll(NTT)];
    if constexpr (Sy::kWeightsFirst) gemv_first<gemv_unroll(NTT)>(W, MLA_D(R), 0, MLA_D(DN), c0, 64, v);
    // the chunk-0 workgroup's RoPE tables: pair idx = tid of token idx / half
    // (nt * half <= kTT * 32 <= kBlock), inputs, so before any wait
    const int half = MLA_D(DR) / 2;
    float rc = 0.f, rs = 0.f;
    if (cc == 0 && (int)threadIdx.x < nt * half) {
      const int t = t0 + (int)threadIdx.x / half, i = (int)threadIdx.x % half;
      rc = p.cos_t[(size_t)t * half + i];
      rs = p.sin_t[(size_t)t * half + i];
    }
    if constexpr (Sy::kWeightsFirst) sy.wait();
    float tsv[kTsPre];
    tscale_load(p, t0, nt, tsv, sy);
    const int n4 = nt * MLA_D(DN) / 4, w4 = MLA_D(DN) / 4;
    const int nsp = max(1, min(16, kBlock / n4));
    const bool one_item = n4 * nsp <= kBlock;
    const int item = threadIdx.x % n4, sp = threadIdx.x / n4;
    const bool has_item = one_item && (int)threadIdx.x < n4 * nsp;
    const float* src = p.part2 + (size_t)(t0 + item / w4) * MLA_D(N2) + (size_t)h * MLA_D(QKH) + 4 * (item % w4);
    const size_t sstride = (size_t)T * MLA_D(N2);
    constexpr int kAbsPre = abs_pre(NTT);
    float4 xpre[kAbsPre];
#pragma unroll
    for (int k = 0; k < kAbsPre; ++k) {
      const int sl = sp + k * nsp;
      xpre[k] = (has_item && sl < MLA_PL(s2)) ? sy.ld4(src + (size_t)sl * sstride) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the chunk-0 workgroup's q_pe partials: (slab, item) pairs q = s*nr + i,
    // staged in the reduction area after the GEMV and added in slab order
    // (when they fit it)
    constexpr int kRopePre = 4;
    const int nr = nt * MLA_D(DR), nrs = nr * MLA_PL(s2);
    const bool rope_lds = cc == 0 && nrs <= 3 * NTT * kTile;
    const float* rsrc = p.part2 + (size_t)t0 * MLA_D(N2) + (size_t)h * MLA_D(QKH) + MLA_D(DN);
    auto rope_at = [&](int q) {
      const int sl = q / nr, i = q % nr;
      return sy.ld(rsrc + ((size_t)sl * T + i / MLA_D(DR)) * MLA_D(N2) + i % MLA_D(DR));
    };
    float rp[kRopePre];
#pragma unroll
    for (int k = 0; k < kRopePre; ++k) {
      const int q = threadIdx.x + k * kBlock;
      rp[k] = (rope_lds && q < nrs) ? rope_at(q) : 0.f;
    }
    if constexpr (!Sy::kWeightsFirst) gemv_first<gemv_unroll(NTT)>(W, MLA_D(R), 0, MLA_D(DN), c0, 64, v);
    tscale_finish(p, t0, nt, tsv, beta, red, sy);  // `red` is free until the GEMV
    if (one_item) {
      float4* out = reinterpret_cast<float4*>(nsp == 1 ? xs : scratch);
      if (has_item) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < kAbsPre; ++k) {
          a.x += xpre[k].x; a.y += xpre[k].y; a.z += xpre[k].z; a.w += xpre[k].w;  // zeros past the last slab
        }
        for (int sl = sp + kAbsPre * nsp; sl < MLA_PL(s2); sl += nsp) {
          const float4 x = sy.ld4(src + (size_t)sl * sstride);
          a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
        }
        out[sp * n4 + item] = a;
      }
      __syncthreads();
      if (nsp > 1) {
        for (int i = threadIdx.x; i < n4; i += kBlock) {
          float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int q = 0; q < nsp; ++q) {
            const float4 x = reinterpret_cast<const float4*>(scratch)[q * n4 + i];
            a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
          }
          reinterpret_cast<float4*>(xs)[i] = a;
        }
        __syncthreads();
      }
    } else {
      reduce_parts4(p.part2 + (size_t)t0 * MLA_D(N2) + (size_t)h * MLA_D(QKH), (size_t)T * MLA_D(N2), MLA_PL(s2), nt * MLA_D(DN) / 4,
                    MLA_D(DN) / 4, MLA_D(N2), xs, scratch, sy);
    }
    for (int idx = threadIdx.x; idx < nt * MLA_D(DN); idx += kBlock) xs[idx] *= beta[idx / MLA_D(DN)];
    __syncthreads();
    gemv_tile<NTT, gemv_unroll(NTT)>(W, MLA_D(R), 0, MLA_D(DN), c0, 64, xs, MLA_D(DN), nt, qo - c0, 64, red, v);
    for (int idx = threadIdx.x; idx < nt * 64; idx += kBlock) {
      const int tt = idx / 64, c = idx % 64;
      sy.st(p.qcat + ((size_t)(t0 + tt) * MLA_D(NH) + h) * MLA_D(KVR) + c0 + c, f32_to_bf16(qo[tt * 64 + c] * p.scale_log2));
    }
    if (cc == 0) {
      if (rope_lds) {
#pragma unroll
        for (int k = 0; k < kRopePre; ++k) {
          const int q = threadIdx.x + k * kBlock;
          if (q < nrs) red[q] = rp[k];
        }
        for (int q = threadIdx.x + kRopePre * kBlock; q < nrs; q += kBlock) red[q] = rope_at(q);
        __syncthreads();
        for (int i = threadIdx.x; i < nr; i += kBlock) {
          float a = 0.f;
          for (int sl = 0; sl < MLA_PL(s2); ++sl) a += red[sl * nr + i];
          xs[i] = a;
        }
        __syncthreads();
      } else {
        reduce_parts(p.part2 + (size_t)t0 * MLA_D(N2) + (size_t)h * MLA_D(QKH) + MLA_D(DN), (size_t)T * MLA_D(N2), MLA_PL(s2), nt * MLA_D(DR),
                     MLA_D(DR), MLA_D(N2), xs, scratch, sy);
      }
      if ((int)threadIdx.x < nt * half) {
        const int tt = threadIdx.x / half, i = threadIdx.x % half, t = t0 + tt;
        // the query tile is stored pre-scaled by softmax_scale * log2(e)
        const float bq = beta[tt] * p.scale_log2;
        const float x0 = bq * xs[tt * MLA_D(DR) + 2 * i], x1 = bq * xs[tt * MLA_D(DR) + 2 * i + 1];
        bf16_t* q = p.qcat + ((size_t)t * MLA_D(NH) + h) * MLA_D(KVR) + MLA_D(R);
        sy.st(q + 2 * i, f32_to_bf16(x0 * rc - x1 * rs));
        sy.st(q + 2 * i + 1, f32_to_bf16(x0 * rs + x1 * rc));
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// k_absorb_core (fused variant, <= 16 heads): workgroups [0, T) finish the kv
// rows, [T, T + NH*ncc3) run the absorption tiles, the rest run the core.  A
// core workgroup waits for every kv row before it reads the cache (a token may
// select its own position), issues its first row loads, then waits for its
// heads' query tiles.  The producers work in the same LDS array.
// ---------------------------------------------------------------------------
template <int NT, int HG, int CS>
struct CoreWaitFused {
  static constexpr bool kEarlyQ = false;  // the query tiles are produced in the same launch
  const StepParams& p;
  // one wave polls, fences (invalidating the CU's L1 and stale L2 lines for
  // every wave of the workgroup), then releases the others at the barrier
  __device__ void before_rows(int) const {
    if (threadIdx.x == 0) {
      wait_count(p.sync, (unsigned)MLA_PL(T), p.sync + kSyncStride);
      __threadfence();
    }
    __syncthreads();
  }
  __device__ void before_q(int h0) const {
    const int i = threadIdx.x;
    if (i < 64) {
      if (i < 16 * HG && h0 + i < MLA_D(NH))
        wait_count(p.sync + (2 + h0 + i) * kSyncStride, (unsigned)MLA_PL(ncc3), p.sync + kSyncStride);
      __threadfence();  // after every polling lane of the wave is done
    }
    __syncthreads();
  }
  // results are read by the next kernel
  __device__ __forceinline__ void st(float* q, float v) const { *q = v; }
};

template <int NT, int HG, int CS>
__device__ void phase_absorb_core(const StepParams& p, int b, char* lds) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T), n_abs = MLA_D(NH) * MLA_PL(ncc3);
  if (b < T) {  // kv row of token b
    phase_absorb<kTT>(p, n_abs + b, reinterpret_cast<float*>(lds));
    count_done(p.sync);
    return;
  }
  if (b < T + n_abs) {
    phase_absorb<kTT>(p, b - T, reinterpret_cast<float*>(lds));
    count_done(p.sync + (2 + (b - T) / MLA_PL(ncc3)) * kSyncStride);
    return;
  }
  core_phase<NT, HG, CS>(p, b - T - n_abs, lds, CoreWaitFused<NT, HG, CS>{p});
}

// ---------------------------------------------------------------------------
// k_oabsorb: workgroup (head h, 64-column chunk j of kv_lora_rank, token
// chunk).  It combines the core's split partials of its columns into o_lat
// (softmax normalisation; a token with no valid entry gets zeros) and forms
// the chunk's share of o_v for every row d:
//   ovp[j][t][h*DV + d] = out_absorb_w[h, d, 64j : 64j+64] . o_lat[t, h, 64j : 64j+64]
// k_oproj adds the chunks' shares in chunk order.  Splitting by latent column
// keeps each split partial read once, however many splits the core made.
// The first weight pieces are loaded before the combine.
// ---------------------------------------------------------------------------
constexpr int kOabsCols = 64;    // latent columns per workgroup
constexpr int kOabsPieces = 4;   // 16-byte weight pieces per lane per pass: 128 rows x 8 pieces
constexpr int kMaxOabsChunks = 8;  // kv_lora_rank <= 512
constexpr int kOabsPre = 8;  // split partials per thread loaded ahead of the split weights

template <class Sy = HandoffNone>
__device__ __attribute__((always_inline)) void phase_oabsorb(const StepParams& p, int b, float* lds, const Sy& sy = Sy()) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T), NSP = MLA_PL(nsplit), R = MLA_D(R), DV = MLA_D(DV);
  const int per_h = pl.nc5 * MLA_PL(nt5c);
  const int h = b / per_h, rem = b % per_h;
  const int j = rem / MLA_PL(nt5c), tch = rem % MLA_PL(nt5c);
  const int t0 = tch * MLA_PL(tc5), nt = min(MLA_PL(tc5), T - t0);
  const int c0 = j * kOabsCols;
  const int tid = threadIdx.x;
  // piece q = i*256 + tid of a 128-row pass: row q / 8, columns c0 + 8*(q % 8) .. +8
  const bf16_t* W = p.w_oabs + (size_t)h * DV * R + c0;
  auto load_pass = [&](int d0, u32x4 (&wr)[kOabsPieces]) {
#pragma unroll
    for (int i = 0; i < kOabsPieces; ++i) {
      const int q = i * kBlock + tid, d = d0 + (q >> 3);
      wr[i] = u32x4{0u, 0u, 0u, 0u};
      if (d < DV) wr[i] = ld_stream(W + (size_t)d * R + 8 * (q & 7));
    }
  };
  u32x4 wr[kOabsPieces];
  load_pass(0, wr);
  sy.wait();
  float* pmL = lds;                  // [tc5][NSP]: split weights
  float* linv = pmL + MLA_PL(tc5) * NSP;  // [tc5]
  float* ol = lds + kOabsOl;            // [tc5][64]
  float* scratch = lds + kOabsScratch;  // 256 float4
  // this thread's combine item (token, 4 columns) and part sp of the splits
  // (s = sp, sp + nsp, ...): its first kOabsPre split partials are loaded
  // before the split weights are known, so the two loads overlap
  constexpr int C4 = kOabsCols / 4;
  const int n4 = nt * C4;
  const int nsp = max(1, min(16, kBlock / n4));
  const bool has_item = tid < n4 * nsp;
  const int item = tid % n4, sp = tid / n4;
  const int tti = item / C4, c4i = item % C4;
  const float* src = p.po + ((size_t)(t0 + tti) * NSP * MLA_D(NH) + h) * R + c0 + 4 * c4i;
  const size_t sstride = (size_t)MLA_D(NH) * R;
  float4 xpre[kOabsPre];
#pragma unroll
  for (int k = 0; k < kOabsPre; ++k) {
    const int s = sp + k * nsp;
    xpre[k] = (has_item && s < NSP) ? *reinterpret_cast<const float4*>(src + (size_t)s * sstride)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // split weights w_s = 2^(m_s - M) and 1/L, L = sum_s w_s * l_s: a wave per
  // token, a lane per split (at most 64 splits on this path); the butterfly
  // sums leave the same value in every lane
  {
    const int lane = tid & 63, wv = tid >> 6;
    for (int tt = wv; tt < nt; tt += kBlock / kWave) {
      const size_t q = ((size_t)(t0 + tt) * NSP + lane) * MLA_D(NH) + h;
      const float m = lane < NSP ? p.pm[q] : -INFINITY;
      const float l = lane < NSP ? p.pden[q] : 0.f;
      const float M = wave_max_dpp(m);
      const float w = (M == -INFINITY || lane >= NSP) ? 0.f : exp2f(m - M);
      const float L = wave_sum_dpp(l * w);
      if (lane < NSP) pmL[tt * NSP + lane] = w;
      if (lane == 0) linv[tt] = (L > 0.f) ? 1.f / L : 0.f;
    }
  }
  __syncthreads();
  // o_lat[tt][c] = linv * sum_s w_s * po[t][s][h][c0 + c], each part in split order
  {
    float4* out = reinterpret_cast<float4*>(nsp == 1 ? ol : scratch);
    if (has_item) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kOabsPre; ++k) {
        const int s = sp + k * nsp;
        if (s < NSP) {
          const float w = pmL[tti * NSP + s];
          a.x = fmaf(w, xpre[k].x, a.x);
          a.y = fmaf(w, xpre[k].y, a.y);
          a.z = fmaf(w, xpre[k].z, a.z);
          a.w = fmaf(w, xpre[k].w, a.w);
        }
      }
      for (int s = sp + kOabsPre * nsp; s < NSP; s += nsp) {  // more splits than prefetched
        const float w = pmL[tti * NSP + s];
        const float4 x = *reinterpret_cast<const float4*>(src + (size_t)s * sstride);
        a.x = fmaf(w, x.x, a.x);
        a.y = fmaf(w, x.y, a.y);
        a.z = fmaf(w, x.z, a.z);
        a.w = fmaf(w, x.w, a.w);
      }
      out[sp * n4 + item] = a;
    }
    __syncthreads();
    if (nsp > 1) {
      const float4* sc = reinterpret_cast<const float4*>(scratch);
      for (int i = tid; i < n4; i += kBlock) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q = 0; q < nsp; ++q) {
          const float4 x = sc[q * n4 + i];
          a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
        }
        reinterpret_cast<float4*>(ol)[i] = a;
      }
      __syncthreads();
    }
    for (int i = tid; i < nt * kOabsCols; i += kBlock) ol[i] *= linv[i / kOabsCols];
    __syncthreads();
  }
  // the eight lanes of a row hold its eight pieces: dot products, then a
  // fixed-order reduction over the eight lanes
  float* ovp = p.ov + (size_t)j * T * MLA_D(NH) * DV;
  for (int d0 = 0; d0 < DV; d0 += kBlock * kOabsPieces / 8) {
    if (d0 > 0) load_pass(d0, wr);
#pragma unroll
    for (int i = 0; i < kOabsPieces; ++i) {
      const int q = i * kBlock + tid, d = d0 + (q >> 3), pc = q & 7;
      float w[8];
      unpack8v(wr[i], w);
      for (int tt = 0; tt < nt; ++tt) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(w[e], ol[tt * kOabsCols + 8 * pc + e], a);
        a += __shfl_xor(a, 1, kWave);
        a += __shfl_xor(a, 2, kWave);
        a += __shfl_xor(a, 4, kWave);
        if (pc == 0 && d < DV) sy.st(ovp + (size_t)(t0 + tt) * MLA_D(NH) * DV + (size_t)h * DV + d, a);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_oproj: o_v @ o_proj_w split-K partials (this rank's partial output)
// ---------------------------------------------------------------------------
template <int NTT, class Sy = HandoffNone>
__device__ __attribute__((always_inline)) void phase_oproj(const StepParams& p, int b, float* lds, const Sy& sy = Sy()) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T);
  const int K = MLA_D(NH) * MLA_D(DV);
  const int slab = b / pl.nt6, tile = b % pl.nt6;
  const int c0 = tile * MLA_PL(tw6), nc = min(MLA_PL(tw6), MLA_D(H) - c0);
  const int k0 = slab * MLA_PL(ks6), ks = min(MLA_PL(ks6), K - k0);
  float* xs = lds + GemvLds<NTT>::xs;
  float* red = lds + GemvLds<NTT>::red;
  for (int t0 = 0; t0 < T; t0 += NTT) {
    const int nt = min(NTT, T - t0);
    u32x4 v[gemv_unroll(NTT)];
    gemv_first<gemv_unroll(NTT)>(p.w_o, MLA_D(H), k0, ks, c0, nc, v);
    sy.wait();
    // o_v = the output absorption's column-chunk shares, added in chunk order
    for (int idx = threadIdx.x; idx < nt * ks; idx += kBlock) {
      const int tt = idx / ks, r = idx % ks;
      const float* src = p.ov + (size_t)(t0 + tt) * K + k0 + r;
      float v[kMaxOabsChunks];
#pragma unroll
      for (int c = 0; c < kMaxOabsChunks; ++c) v[c] = c < pl.nc5 ? sy.ld(src + (size_t)c * T * K) : 0.f;
      float a = v[0];
#pragma unroll
      for (int c = 1; c < kMaxOabsChunks; ++c)
        if (c < pl.nc5) a += v[c];
      xs[tt * kTile + r] = a;
    }
    __syncthreads();
    gemv_tile<NTT, gemv_unroll(NTT)>(p.w_o, MLA_D(H), k0, ks, c0, nc, xs, kTile, nt, p.part6 + ((size_t)slab * T + t0) * MLA_D(H), MLA_D(H), red, v, sy);
  }
}

// ---------------------------------------------------------------------------
// k_out: out[t][c] = bf16(sum over the o-projection's slabs).  A workgroup
// covers 256 columns of one token: four lanes per 4-column group each add
// every fourth slab (in order), then the four partials are added in a fixed
// order, so the result is reproducible.
// ---------------------------------------------------------------------------
constexpr int kOutCols = kBlock;  // columns per k_out workgroup: kBlock/4 groups of four columns

template <class Sy = HandoffNone>
__device__ __attribute__((always_inline)) void phase_out(const StepParams& p, int b, float*, const Sy& sy = Sy()) {
  const Plan& pl = p.pl;
  sy.wait();
  const int ncg = (MLA_D(H) + kOutCols - 1) / kOutCols;
  const int t = b / ncg;
  const int part = threadIdx.x & 3;
  const int c = (b % ncg) * kOutCols + 4 * (threadIdx.x >> 2);
  const bool ok = c < MLA_D(H);  // H % 8 == 0: a group of four is wholly inside or outside
  const size_t stride = (size_t)MLA_PL(T) * MLA_D(H);
  const float* src = p.part6 + (size_t)t * MLA_D(H) + (ok ? c : 0);
  // this lane's slabs s = part, part + 4, ..., eight loads at a time; a lane
  // loads only slabs that exist (with eight or nine slabs a lane needs two or
  // three, and an unconditional reload of the last would triple the loads)
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  const int S = MLA_PL(s6);
  for (int s = part; s < S; s += 32) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = s + 4 * u < S ? sy.ld4(src + (size_t)(s + 4 * u) * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a.x += v[u].x; a.y += v[u].y; a.z += v[u].z; a.w += v[u].w;
    }
  }
  // partials of lanes 4i .. 4i+3: ((p0 + p1) + (p2 + p3))
  float r[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] += __shfl_xor(r[i], 1, kWave);
    r[i] += __shfl_xor(r[i], 2, kWave);
  }
  if (ok && part == 0) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
    *reinterpret_cast<uint2*>(p.out + (size_t)t * MLA_D(H) + c) = o;
  }
}

// ---------------------------------------------------------------------------
// GEMV path: the output sum folded into the o-projection.  Each o-projection
// workgroup (column tile `tile`, one slab) has stored its partials with
// device scope; once they are complete it counts itself in the tile's
// arrival counter, and the last of the tile's s6 slabs to arrive adds the
// tile's slabs, in slab order whichever arrives last (so the result is
// reproducible), and writes the bf16 output of the tile's columns.  Returns
// whether this workgroup was the last.  The counters start each step at zero
// (the step's first kernel or item clears them).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool oproj_fold_out(const StepParams& p, int tile, float* lds) {
  const Plan& pl = p.pl;
  const int T = MLA_PL(T), S = MLA_PL(s6);
  const int c0 = tile * MLA_PL(tw6), nc = min(MLA_PL(tw6), MLA_D(H) - c0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  unsigned* arrived = reinterpret_cast<unsigned*>(lds);
  if (threadIdx.x == 0)
    arrived[0] = __hip_atomic_fetch_add(p.tcnt + tile * kSyncStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (arrived[0] != (unsigned)S - 1u) return false;
  const int n4 = nc / 4;  // H % 8 == 0 and tw6 % 8 == 0
  const size_t sstride = (size_t)T * MLA_D(H);
  for (int it = threadIdx.x; it < T * n4; it += kBlock) {
    const int tt = it / n4, c = c0 + 4 * (it % n4);
    const float* src = p.part6 + (size_t)tt * MLA_D(H) + c;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < S; s += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = s + u < S ? ld_dev4(src + (size_t)(s + u) * sstride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a.x += v[u].x; a.y += v[u].y; a.z += v[u].z; a.w += v[u].w;
      }
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    o.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    *reinterpret_cast<uint2*>(p.out + (size_t)tt * MLA_D(H) + c) = o;
  }
  return true;
}

}  // namespace MLA_PHASE_NS
