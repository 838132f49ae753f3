// Projections on the matrix cores, for steps with more than a few tokens.
//
//   out[t, c] = sum_k A[t, k] * W[k, c]
//
// W is a bf16 [K, N] weight, row-major (columns contiguous); A is an fp32
// activation.  Rounding A to bf16 would cost 8 bits on every product, so each
// activation is split into hi = bf16(a) and lo = bf16(a - hi) and both halves
// meet the weight (two MFMAs per fragment): about 16 significant bits.  The
// projections stay bound by the weight stream even with the matrix work doubled.
//
// Tiles: 16 tokens (an m-tile) x NC columns (64 or 128) x 32 k (a k-step).  A
// workgroup of four waves owns one NC-column tile, one K slab and a block of
// MTB m-tiles; the waves split the block 2 x 2 (1 x 4 for a single m-tile).
//
// Both operands reach LDS through direct global->LDS loads into a ring of
// kMgDepth k-steps, so the main loop holds no compiler-visible global load and
// its only waits are the ring's explicit vmcnt waits.
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

constexpr int kMgCols = 64;       // output columns per tile
constexpr int kMgK = 32;          // k per step
constexpr int kMgDepth = 8;       // ring depth in k-steps
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
__device__ __forceinline__ void put_a4(bf16_t* buf, int mt_pad, int t, int k, const float* a) {
  uint2 hi, lo;
  split4(a, hi, lo);
  const size_t i = abuf_index(t, k, mt_pad);
  *reinterpret_cast<uint2*>(buf + i) = hi;
  *reinterpret_cast<uint2*>(buf + i + kAFragElems) = lo;
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

// Columns per GEMM tile: 64 for one m-tile, 128 for larger token blocks (the
// wider tile halves the activation bytes streamed per weight byte).
__host__ __device__ constexpr int mg_cols(int mtb) { return mtb >= 2 ? 128 : 64; }

template <int MTB, int NC = mg_cols(MTB)>
struct Mg {
  static constexpr int WM = MTB >= 2 ? 2 : 1;  // waves along tokens
  static constexpr int WN = 4 / WM;            // waves along columns
  static constexpr int MTW = MTB / WM;         // m-tiles per wave
  static constexpr int NTW = NC / 16 / WN;     // 16-column n-tiles per wave
  static constexpr int kABytes = MTB * 2 * kAFragElems * 2;
  static constexpr int kBBytes = kMgK * NC * 2;
  static constexpr int kStep = kABytes + kBBytes;
  static constexpr int kADma = (MTB * 128 + 255) / 256;  // A pieces per lane per step
  static constexpr int kBDma = NC / 64;                  // B pieces per lane per step
  static constexpr int kRing = kMgDepth * kStep;
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

// Sources of this lane's pieces of a 32 x NC weight tile at k-step 0.
template <int NC>
struct BTileSrc {
  const bf16_t* p[NC / 64];  // nullptr: the piece's columns lie past N
  int row[NC / 64];          // the piece's row at k-step 0; rows >= K read zeros
  size_t step;               // elements per k-step
  int K;
};

template <int NC>
__device__ __forceinline__ BTileSrc<NC> btile_src(const bf16_t* W, int K, int N, int k0, int c0) {
  BTileSrc<NC> s;
#pragma unroll
  for (int i = 0; i < NC / 64; ++i) {
    const int q = i * 256 + threadIdx.x;  // LDS slot of this piece
    const int r = q / (NC / 8), pc = bswz(q % (NC / 8), r);
    const int col = c0 + 8 * pc;
    s.p[i] = (col < N) ? W + (size_t)(k0 + r) * N + col : nullptr;
    s.row[i] = k0 + r;
  }
  s.step = (size_t)kMgK * N;
  s.K = K;
  return s;
}

// NC/64 direct loads per lane: k-step st of the weight tile into bufB.
template <int NC>
__device__ __forceinline__ void issue_btile(const BTileSrc<NC>& s, int st, bool live, char* bufB,
                                            const void* zero16) {
#pragma unroll
  for (int i = 0; i < NC / 64; ++i) {
    const void* src = zero16;
    if (live && s.p[i] && s.row[i] + kMgK * st < s.K) src = s.p[i] + s.step * st;
    dma16(src, bufB + (i * 256 + (threadIdx.x & ~63)) * 16);
  }
}

// kADma direct loads per lane: the MTB m-tiles of k-step ks (both halves, contiguous) into bufA.
template <int MTB>
__device__ __forceinline__ void issue_atile(const bf16_t* A, int mt_pad, int mt0, int ks, bool live, char* bufA,
                                            char* sink, const void* zero16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < Mg<MTB>::kADma; ++i) {
    const int q0 = i * 256 + wave * 64;  // first piece of this wave's load
    const bool in = q0 < MTB * 128;
    const void* src = zero16;
    if (in && live) src = A + ((size_t)ks * mt_pad + mt0) * (2 * kAFragElems) + (size_t)(q0 + lane) * 8;
    dma16(src, in ? bufA + q0 * 16 : sink);
  }
}

// One k-step: B fragments by transposing reads, A fragments (hi, lo), MFMAs.
template <int MTB, int NC>
__device__ __forceinline__ void mg_step(const char* bufA, const char* bufB,
                                        f32x4_t (&acc)[Mg<MTB, NC>::MTW][Mg<MTB, NC>::NTW]) {
  using S = Mg<MTB, NC>;
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
    const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t*>(bufA + ((m * 2) * 64 + lane) * 16);
    const bf16x8_t alo = *reinterpret_cast<const bf16x8_t*>(bufA + ((m * 2 + 1) * 64 + lane) * 16);
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt) {
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfr[nt], acc[mt][nt], 0, 0, 0);
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfr[nt], acc[mt][nt], 0, 0, 0);
    }
  }
}

// Pipelined loop over nsteps k-steps.  issue(st, buf) issues exactly NDMA
// direct loads per lane for step st (loads of zeros once st >= nsteps);
// step(st, buf) consumes a landed step.  Returns with every load landed and
// the ring free.
// The ring's first DEPTH-1 steps; issue them as early as possible (before
// work the loop does not depend on), then run mg_ring_loop.
template <int DEPTH = kMgDepth, class Issue>
__device__ __forceinline__ void mg_ring_prologue(char* ring, int step_bytes, Issue&& issue) {
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s) issue(s, ring + s * step_bytes);
}

template <int NDMA, int DEPTH = kMgDepth, class Issue, class Step>
__device__ __forceinline__ void mg_ring_loop(int nsteps, char* ring, int step_bytes, Issue&& issue, Step&& step) {
  static_assert(NDMA * (DEPTH - 2) < 64, "vmcnt range");
  for (int s = 0; s < nsteps; ++s) {
    wait_vmcnt<NDMA * (DEPTH - 2)>();  // step s landed (this wave's oldest loads)
    __syncthreads();                   // ... for every wave; buffer of step s-1 consumed
    const int sn = s + DEPTH - 1;
    issue(sn, ring + (sn % DEPTH) * step_bytes);
    step(s, ring + (s % DEPTH) * step_bytes);
  }
  wait_vmcnt<0>();
  __syncthreads();
}

template <int NDMA, int DEPTH = kMgDepth, class Issue, class Step>
__device__ __forceinline__ void mg_ring(int nsteps, char* ring, int step_bytes, Issue&& issue, Step&& step) {
  mg_ring_prologue<DEPTH>(ring, step_bytes, issue);
  mg_ring_loop<NDMA, DEPTH>(nsteps, ring, step_bytes, issue, step);
}

// acc = A[token block] @ W[k0 : k0 + 32*nks, c0 : c0 + NC] with A from a
// global fragment-order buffer (its m-tiles mt0 .. mt0+MTB-1).
template <int MTB, int NC = mg_cols(MTB)>
__device__ __forceinline__ void mgemm(const bf16_t* A, int mt_pad, int mt0, const bf16_t* W, int K, int N, int k0,
                                      int nks, int c0, const void* zero16, char* ring, char* sink,
                                      f32x4_t (&acc)[Mg<MTB, NC>::MTW][Mg<MTB, NC>::NTW]) {
  using S = Mg<MTB, NC>;
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const BTileSrc<NC> bs = btile_src<NC>(W, K, N, k0, c0);
  const int ks0 = k0 / kMgK;
  mg_ring<S::kADma + S::kBDma>(
      nks, ring, S::kStep,
      [&](int st, char* buf) {
        const bool live = st < nks;
        issue_atile<MTB>(A, mt_pad, mt0, ks0 + st, live, buf, sink, zero16);
        issue_btile<NC>(bs, st, live, buf + S::kABytes, zero16);
      },
      [&](int, const char* buf) { mg_step<MTB, NC>(buf, buf + S::kABytes, acc); });
}

// Lane (g, l16) of a wave holds D[4g+i][l16] of each 16x16 output tile.
// Visits (token, column, value) of the wave's tiles for a block starting at token t0.
template <int MTB, int NC = mg_cols(MTB), class F>
__device__ __forceinline__ void mg_for_outputs(const f32x4_t (&acc)[Mg<MTB, NC>::MTW][Mg<MTB, NC>::NTW], int t0,
                                               int c0, F&& f) {
  using S = Mg<MTB, NC>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < S::MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < S::NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f(t0 + 16 * (wm * S::MTW + mt) + 4 * g + i, c0 + 16 * (wn * S::NTW + nt) + l16, acc[mt][nt][i]);
}

}  // namespace mla
