// Projections on the matrix cores, for steps with more than a few tokens.
//
//   out[t, c] = sum_k A[t, k] * W[k, c]
//
// W is a bf16 [K, N] weight, row-major (columns contiguous); A is an fp32
// activation.  Rounding A to bf16 would cost 8 bits on every product, so each
// activation is split into hi = bf16(a) and lo = bf16(a - hi) and both halves
// meet the weight (two MFMAs per fragment): about 16 significant bits.  Up to
// 32 tokens the projections stay bound by the weight stream even with the
// matrix work doubled.  A GEMM can also read the hi halves alone (AH = 1),
// which the o-projection of 32- to 128-token blocks does (phases_mfma.h).
//
// Tiles: 16 tokens (an m-tile) x NC columns (64 to 256) x 32 k (a k-step).  A
// workgroup owns one NC-column tile, one K slab and a block of MTB m-tiles;
// four waves split the block 2 x 2 (1 x 4 for a single m-tile), eight waves
// (128-token blocks) 2 x 4.
//
// Both operands are loaded into registers several k-steps ahead of use (16-byte
// global loads, non-temporal for the weight) and written to one of two LDS
// stage buffers while the previous step's MFMAs run; the two small stages
// leave room for several workgroups per CU.
//   A comes from the previous kernel already in fragment order: for every
//     (k-step, m-tile, half) a 1 KB block with lane l's eight bf16 at 16*l.
//   B is the 32 x NC weight tile; row r keeps its 16-byte pieces XOR-swizzled
//     (low three bits) by r mod 8.  Transposing LDS reads (ds_read_b64_tr_b16) hand each lane
//     four consecutive k of one column, twice per fragment.
// Contraction order inside a k-step: lane group g (= lane / 16) carries
// k = 4g..4g+3 and 16+4g..16+4g+3, the order the transposing read delivers;
// the A fragments are written in that order (afrag_pi).  Where B comes
// straight from a k-contiguous weight, the plain order (afrag_std) is used.
#pragma once

#include "device_util.h"
#include "mfma_util.h"

namespace mla {

constexpr int kMgK = 32;          // k per step
constexpr int kAFragElems = 512;  // bf16 per (k-step, m-tile, half) block

// Offset of A[m][kk] (m < 16, kk < 32) in a 512-element fragment block.
__host__ __device__ __forceinline__ int afrag_pi(int m, int kk) {
  const int g = (kk & 15) >> 2, j = ((kk & 16) >> 2) | (kk & 3);
  return (g * 16 + m) * 8 + j;
}
__host__ __device__ __forceinline__ int afrag_std(int m, int kk) { return ((kk >> 3) * 16 + m) * 8 + (kk & 7); }

// Global A buffer in fragment order: [k-step][m-tile < mt_pad][half][512].
__device__ __forceinline__ size_t abuf_index(int t, int k, int mt_pad) {
  return ((size_t)((k >> 5) * mt_pad + (t >> 4)) * 2) * kAFragElems + afrag_pi(t & 15, k & 31);
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16_t a, bf16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

// hi/lo halves of four activations, packed as two 8-byte runs.
__device__ __forceinline__ void split4(const float* a, uint2& hi, uint2& lo) {
  bf16_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f32_to_bf16(a[i]);
    l[i] = f32_to_bf16(a[i] - bf16_to_f32(h[i]));
  }
  hi = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
  lo = make_uint2(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]));
}

// A[t][k..k+3] (k % 4 == 0) into a global fragment-order buffer.  In both
// orders four consecutive k of one token are one 8-byte run of each half.
// Without `lo` the lo half is left unwritten (its consumer reads hi alone).
__device__ __forceinline__ void put_a4(bf16_t* buf, int mt_pad, int t, int k, const float* a, bool lo_too = true) {
  uint2 hi, lo;
  split4(a, hi, lo);
  const size_t i = abuf_index(t, k, mt_pad);
  *reinterpret_cast<uint2*>(buf + i) = hi;
  if (lo_too) *reinterpret_cast<uint2*>(buf + i + kAFragElems) = lo;
}

// The same into an LDS block array [k-step][m-tile < mtb][half][512], either order.
template <bool PI>
__device__ __forceinline__ void put_a4_lds(char* ares, int mtb, int tt, int k, const float* a) {
  uint2 hi, lo;
  split4(a, hi, lo);
  const int e = PI ? afrag_pi(tt & 15, k & 31) : afrag_std(tt & 15, k & 31);
  char* blk = ares + ((size_t)((k >> 5) * mtb + (tt >> 4)) * 2) * (kAFragElems * 2);
  *reinterpret_cast<uint2*>(blk + e * 2) = hi;
  *reinterpret_cast<uint2*>(blk + kAFragElems * 2 + e * 2) = lo;
}

// Columns per GEMM tile: 128 for blocks of up to 32 tokens (twice the
// workgroups), 256 for 64 and 128 tokens, where a wider tile streams fewer
// activation bytes per weight byte (the activation, hi and lo, is as large per
// k as a 128-column weight row at 64 tokens).
__host__ __device__ constexpr int mg_cols(int mtb) { return mtb >= 4 ? 256 : 128; }
// Waves per GEMM workgroup: eight for blocks of 64 and 128 tokens (two per
// SIMD, so one wave's loads, stores and barrier waits overlap the other's
// products; with four waves a 128-token block held 368 registers a wave and
// ran one wave per SIMD), four for smaller blocks.
__host__ __device__ constexpr int mg_waves(int mtb) { return mtb >= 4 ? 8 : 4; }

// Activation halves a GEMM reads: 2 (hi and lo) or 1 (hi alone, a plain bf16
// activation).
template <int MTB, int NC = mg_cols(MTB), int NW = mg_waves(MTB), int AH = 2>
struct Mg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int WM = MTB >= 2 ? 2 : 1;  // waves along tokens
  static constexpr int WN = NW / WM;           // waves along columns
  static constexpr int MTW = MTB / WM;         // m-tiles per wave
  static constexpr int NTW = NC / 16 / WN;     // 16-column n-tiles per wave
  static constexpr int kABytes = MTB * AH * kAFragElems * 2;
  static constexpr int kBBytes = kMgK * NC * 2;
  static constexpr int kStep = kABytes + kBBytes;
  static constexpr int kAPieces = (MTB * 64 * AH + kThreads - 1) / kThreads;  // A pieces per lane per step
  static constexpr int kBPieces = NC * 4 / kThreads;                       // B pieces per lane per step
  static constexpr int kPieces = kAPieces + kBPieces;
  static constexpr int kAhead = NC >= 256 ? 3 : 6;           // k-steps loaded ahead into registers
  static constexpr int kStage = 2 * kStep;                   // two LDS stage buffers
};

// Workgroup b -> (unit u, token block tb).  The token blocks of one unit sit
// 8 workgroup indices apart, so they run on one XCD and share its L2 copy of
// the unit's weight tile.
__device__ __forceinline__ bool mg_unit(int b, int nunits, int ntb, int& u, int& tb) {
  const int grp = b / (8 * ntb), rem = b % (8 * ntb);
  tb = rem >> 3;
  u = grp * 8 + (rem & 7);
  return u < nunits;
}

// Swizzled 16-byte slot of piece pc in row r of a weight tile: the low three
// bits are XORed with r mod 8 (transposing reads of four rows hit distinct banks).
__device__ __forceinline__ int bswz(int pc, int r) { return (pc & ~7) | ((pc & 7) ^ (r & 7)); }

// Sixteen-byte operand pieces of one k-step held in registers.
template <int NV>
struct Pieces {
  u32x4_t v[NV];
};

__device__ __forceinline__ u32x4_t load16(const bf16_t* src) { return *reinterpret_cast<const u32x4_t*>(src); }
// Weights are read once per step: non-temporal loads, which stream from HBM at
// more than twice the rate of cached ones on this chip.
__device__ __forceinline__ u32x4_t load16_nt(const bf16_t* src) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
}
__device__ __forceinline__ void store16(char* dst, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(dst) = v; }

// This lane's pieces of a 32 x NC weight tile at k-step 0.  Piece i is LDS
// slot q = NTHR i + tid: row r = q / (NC/8), swizzled 16-byte column piece.
template <int NC, int NTHR = kBlock>
struct BTileSrc {
  const bf16_t* p[NC * 4 / NTHR];  // nullptr: the piece's columns lie past N
  int row[NC * 4 / NTHR];          // the piece's row at k-step 0; rows >= K read as zeros
  size_t step;                     // elements per k-step
  int K;
};

template <int NC, int NTHR = kBlock>
__device__ __forceinline__ BTileSrc<NC, NTHR> btile_src(const bf16_t* W, int K, int N, int k0, int c0) {
  BTileSrc<NC, NTHR> s;
#pragma unroll
  for (int i = 0; i < NC * 4 / NTHR; ++i) {
    const int q = i * NTHR + threadIdx.x;
    const int r = q / (NC / 8), pc = bswz(q % (NC / 8), r);
    const int col = c0 + 8 * pc;
    s.p[i] = (col < N) ? W + (size_t)(k0 + r) * N + col : nullptr;
    s.row[i] = k0 + r;
  }
  s.step = (size_t)kMgK * N;
  s.K = K;
  return s;
}

// One k-step: B fragments by transposing reads, A fragments (hi, and lo when
// AH == 2; the stage holds AH blocks per m-tile), MFMAs.
template <int MTB, int NC, int NW = mg_waves(MTB), int AH = 2>
__device__ __forceinline__ void mg_step(const char* bufA, const char* bufB,
                                        f32x4_t (&acc)[Mg<MTB, NC, NW>::MTW][Mg<MTB, NC, NW>::NTW]) {
  using S = Mg<MTB, NC, NW, AH>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int g = lane >> 4, l16 = lane & 15;
  const int r1 = 4 * g + (l16 >> 2);
  const int within = 8 * (l16 & 1);
  bf16x8_t bfr[S::NTW];
#pragma unroll
  for (int nt = 0; nt < S::NTW; ++nt) {
    const int pc = 2 * (wn * S::NTW + nt) + ((l16 & 3) >> 1);
    const char* a1 = bufB + r1 * (2 * NC) + (bswz(pc, r1) << 4) + within;  // rows r1 and r1+16 share r mod 8
    const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a1);
    const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a1 + 16 * (2 * NC)));
    bfr[nt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt) {
    const int m = wm * S::MTW + mt;
    const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t*>(bufA + ((m * AH) * 64 + lane) * 16);
    bf16x8_t alo = ahi;
    if constexpr (AH == 2) alo = *reinterpret_cast<const bf16x8_t*>(bufA + ((m * 2 + 1) * 64 + lane) * 16);
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt) {
      // transposed product (weight fragment as the A operand): lane (g, l16)
      // gets columns 4g..4g+3 of token l16, stored four at a time
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nt], ahi, acc[mt][nt], 0, 0, 0);
      if constexpr (AH == 2) acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nt], alo, acc[mt][nt], 0, 0, 0);
    }
  }
}

// Pipelined loop over nsteps k-steps.  load(st) returns this lane's pieces of
// step st (zeros once st >= nsteps; it must issue the same loads on every call,
// reading a zero buffer where there is no data, or the compiler's waits for
// the oldest loads degrade to waits for all of them); store(pieces,
// buf) writes them to an LDS stage buffer; step(st, buf) consumes a stage.
// Steps are loaded P ahead; stage st % 2 is written during step st - 1 and
// read after the barrier that ends it.  Returns with both stages free.
// The prologue (the first P loads) may be issued early, before work the loop
// does not depend on.
template <int NV, int P, class Load>
__device__ __forceinline__ void mg_pipe_prologue(Pieces<NV> (&q)[P], Load&& load) {
#pragma unroll
  for (int j = 0; j < P; ++j) q[j] = load(j);
}

template <int NV, int P, class Load, class Store, class Step>
__device__ __forceinline__ void mg_pipe_loop(Pieces<NV> (&q)[P], int nsteps, char* stage, int step_bytes,
                                             Load&& load, Store&& store, Step&& step) {
  store(q[0], stage);
  q[0] = load(P);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int s = s0 + j;
      if (s >= nsteps) break;
      step(s, stage + (s & 1) * step_bytes);
      // unconditional, also past the last step: stage (s+1) % 2 was last read
      // by step s-1, which every wave finished before the previous barrier
      store(q[(j + 1) % P], stage + ((s + 1) & 1) * step_bytes);
      q[(j + 1) % P] = load(s + 1 + P);
      __syncthreads();
    }
  }
}

template <int NV, int P, class Load, class Store, class Step>
__device__ __forceinline__ void mg_pipe(int nsteps, char* stage, int step_bytes, Load&& load, Store&& store,
                                        Step&& step) {
  Pieces<NV> q[P];
  mg_pipe_prologue(q, load);
  mg_pipe_loop(q, nsteps, stage, step_bytes, load, store, step);
}

// acc = A[token block] @ W[k0 : k0 + 32*nks, c0 : c0 + NC] with A from a
// global fragment-order buffer (its m-tiles mt0 .. mt0+MTB-1); with AH == 1
// only the hi blocks are read, so A enters as plain bf16.
template <int MTB, int NC = mg_cols(MTB), int NW = mg_waves(MTB), int AH = 2>
__device__ __forceinline__ void mgemm(const bf16_t* A, int mt_pad, int mt0, const bf16_t* W, int K, int N, int k0,
                                      int nks, int c0, const bf16_t* zero16, char* stage,
                                      f32x4_t (&acc)[Mg<MTB, NC, NW>::MTW][Mg<MTB, NC, NW>::NTW]) {
  using S = Mg<MTB, NC, NW, AH>;
  constexpr int NTHR = S::kThreads;
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const BTileSrc<NC, NTHR> bs = btile_src<NC, NTHR>(W, K, N, k0, c0);
  const int ks0 = k0 / kMgK;
  const int tid = threadIdx.x;
  const bf16_t* Ab = A + ((size_t)ks0 * mt_pad + mt0) * (2 * kAFragElems);
  const size_t astep = (size_t)mt_pad * 2 * kAFragElems;
  mg_pipe<S::kPieces, S::kAhead>(
      nks, stage, S::kStep,
      [&](int st) {
        // every piece is loaded (zeros from zero16 where there is no data), so
        // the loads stay unconditional and the compiler's vmcnt waits exact
        Pieces<S::kPieces> r;
        const bool live = st < nks;
#pragma unroll
        for (int i = 0; i < S::kAPieces; ++i) {
          // piece q: block q / 64 of the stage (m-tile, half), lane q % 64;
          // with AH == 1 block m is the hi block of m-tile m in global memory
          const int q = i * NTHR + tid;
          const bf16_t* src = zero16;
          if (live && q < MTB * 64 * AH)
            src = Ab + astep * st + (AH == 2 ? (size_t)q * 8 : (size_t)(q >> 6) * 2 * kAFragElems + (q & 63) * 8);
          r.v[i] = load16(src);
        }
#pragma unroll
        for (int i = 0; i < S::kBPieces; ++i) {
          const bf16_t* src = zero16;
          if (live && bs.p[i] && bs.row[i] + kMgK * st < bs.K) src = bs.p[i] + bs.step * st;
          r.v[S::kAPieces + i] = load16_nt(src);
        }
        return r;
      },
      [&](const Pieces<S::kPieces>& r, char* buf) {
#pragma unroll
        for (int i = 0; i < S::kAPieces; ++i)
          if (i * NTHR + tid < MTB * 64 * AH) store16(buf + (i * NTHR + tid) * 16, r.v[i]);
#pragma unroll
        for (int i = 0; i < S::kBPieces; ++i) store16(buf + S::kABytes + (i * NTHR + tid) * 16, r.v[S::kAPieces + i]);
      },
      [&](int, const char* buf) { mg_step<MTB, NC, NW, AH>(buf, buf + S::kABytes, acc); });
}

// Lane (g, l16) of a wave holds out[token l16][columns 4g .. 4g+3] of each
// 16x16 output tile (the products are taken transposed).  Visits (token,
// first column, four values) of the wave's tiles for a block starting at token t0.
template <int MTB, int NC = mg_cols(MTB), int NW = mg_waves(MTB), class F>
__device__ __forceinline__ void mg_for_outputs4(const f32x4_t (&acc)[Mg<MTB, NC, NW>::MTW][Mg<MTB, NC, NW>::NTW],
                                                int t0, int c0, F&& f) {
  using S = Mg<MTB, NC, NW>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt)
      f(t0 + 16 * (wm * S::MTW + mt) + l16, c0 + 16 * (wn * S::NTW + nt) + 4 * g, acc[mt][nt]);
}

// Four consecutive fp32 outputs out[c .. c+3] (c % 4 == 0), columns from n on dropped.
__device__ __forceinline__ void store_f32x4(float* out, int c, int n, const f32x4_t& v) {
  if (c + 4 <= n) {
    *reinterpret_cast<f32x4_t*>(out + c) = v;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c + i < n) out[c + i] = v[i];
  }
}

}  // namespace mla
