// Gather-attention core on the matrix cores (gfx950, wave64).
//
// For one token, every head attends over the cache rows its selected
// positions resolve to.  Scores and the latent output are two dense
// contractions over the gathered rows, shared by all heads (MLA keeps one
// latent KV head):
//   S^T[row, head] = sum_k K[row, k] * Qcat[head, k]    (k over kv_row = latent | rope)
//   O[head, c]    += sum_row P[head, row] * K[row, c]     (c over the latent width)
// A wave owns 16 heads ("head group") and a slice of the latent columns.  Each
// step takes a chunk of 32 gathered rows: two 16x16x32 bf16 score tiles (rows
// 0-15 and 16-31), an online-softmax update, and one 16x16x32 bf16 PV product
// per 16 output columns.  The score tiles' output layout (lane l holds rows
// 4*(l/16)+i and 16+4*(l/16)+i of head l%16) is used directly as the PV
// A operand; the value operand takes the same rows with two transposing LDS
// reads (each hands lane l four consecutive rows of one column), so the
// contraction index matches on both sides.
//
// Rows reach LDS through a ring of three 32-row buffers filled by direct
// global-to-LDS loads two chunks ahead (no staging registers); the chunk's
// flat row ids are read from LDS, staged once per workgroup.  A buffer row
// spans an odd number of 16-byte pieces (whole k-steps, zero past kv_row, then
// one pad piece), so 16 rows read at one column fall on distinct LDS banks and
// every fragment address is a per-lane base plus a compile-time offset.
// Masked rows load zeros and get a -inf score bias, written once per chunk.
// Query tiles arrive pre-scaled by softmax_scale * log2(e), so scores are in
// the log2 domain as they leave the matrix cores.
#pragma once

#include "device_util.h"
#include "mfma_util.h"
#include "step_params.h"

namespace MLA_PHASE_NS {
using namespace ::mla;

constexpr int kCoreChunk = 32;  // gathered rows per step
constexpr int kCoreRing = 3;    // chunk buffers in flight

constexpr int kMaxSplitRows = 4096;  // row ids staged in LDS per core workgroup

// 16-byte pieces per LDS row for a latent width of 16*nt: whole 32-wide
// k-steps over kv_row <= 16*nt + 64, made odd.  A buffer is rounded up to
// whole 1 KB (64 slots), so the last wave load of a chunk, which may run past
// the chunk's slots, stays inside its buffer.
__host__ __device__ constexpr int core_row_pieces(int nt) { return (2 * nt + 8) | 1; }
__host__ __device__ constexpr int core_buf_bytes(int nt) { return (kCoreChunk * core_row_pieces(nt) * 16 + 1023) / 1024 * 1024; }

// LDS of a core workgroup, carved from one array: ring (`ring` chunk buffers)
// | row ids (`maxr`) | sink | partial score tiles (HG*CS*128 x 16 B) | score
// bias (ring x 32 floats).
__host__ __device__ constexpr int core_ofs_ids(int nt, int ring = kCoreRing) { return ring * core_buf_bytes(nt); }
__host__ __device__ constexpr int core_ofs_sink(int nt, int ring = kCoreRing, int maxr = kMaxSplitRows) {
  return core_ofs_ids(nt, ring) + maxr * 4;
}
__host__ __device__ constexpr int core_ofs_sx(int nt, int ring = kCoreRing, int maxr = kMaxSplitRows) {
  return core_ofs_sink(nt, ring, maxr) + 1024;
}
__host__ __device__ constexpr int core_ofs_bias(int nt, int hg, int cs, int ring = kCoreRing, int maxr = kMaxSplitRows) {
  return core_ofs_sx(nt, ring, maxr) + hg * cs * 128 * 16;
}
__host__ __device__ constexpr int core_lds_bytes(int nt, int hg, int cs, int ring = kCoreRing, int maxr = kMaxSplitRows) {
  return core_ofs_bias(nt, hg, cs, ring, maxr) + ring * kCoreChunk * 4;
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four row groups of an
// MFMA output tile) with the lane-swap instructions: after a swap every lane
// of a pair holds (lower lane's value, upper lane's value), so both lanes form
// the same result in the same order, with no LDS round trip.  The operands
// and both results pass through empty asm statements: the optimiser would
// otherwise take the two results of swapping equal values as equal and fold
// the pair reduction away.
template <bool K32>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  const unsigned a = __builtin_bit_cast(unsigned, v);
  unsigned b = a;
  asm volatile("" : "+v"(b));
  const auto r = K32 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                     : __builtin_amdgcn_permlane16_swap(a, b, false, false);
  unsigned r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max4groups(float v) {
  float lo, hi;
  lane_pair<false>(v, lo, hi);
  lane_pair<true>(fmaxf(lo, hi), lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum4groups(float v) {
  float lo, hi;
  lane_pair<false>(v, lo, hi);
  lane_pair<true>(lo + hi, lo, hi);
  return lo + hi;
}

// Reductions over all 64 lanes with no LDS round trip: within each row of 16
// lanes by DPP moves (the two quad swaps, then the half-row and row mirrors;
// after each step every lane of the group holds the same partial, formed in
// the same order), then over the four rows with the lane swaps above.  Every
// lane returns the same value.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  return max4groups(v);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<kDppQuadXor1>(v);
  v += dpp_mov<kDppQuadXor2>(v);
  v += dpp_mov<kDppRowHalfMirror>(v);
  v += dpp_mov<kDppRowMirror>(v);
  return sum4groups(v);
}

// Hooks of the separately launched core: every input is complete at kernel
// start, and the results are read by a later kernel.
struct CoreNoWait {
  static constexpr bool kEarlyQ = true;  // the query tiles may load before the row ids
  __device__ void before_rows(int) const {}
  __device__ void before_q(int) const {}
  __device__ __forceinline__ void st(float* p, float v) const { *p = v; }
};

// Hooks: before_rows(token) runs before the first read of the row ids or the
// cache; before_q(first head) after the first row loads are issued and before
// the query tiles are read (kEarlyQ: the tiles are complete at kernel start, so
// they load first, before the row ids).  Every thread of the workgroup calls
// both.
// st(p, v) stores one of the split's results (m, l, o).
// RING chunk buffers are in flight (1: each chunk is loaded after the previous
// one is consumed); MAXR is the most rows a split may hold.
// NT: latent width / 16.  HG: head groups of 16 per workgroup.  CS: column
// splits.  The CS waves of a head group each own NT/CS output tiles; they
// split the score's k-steps between them and add their partial score tiles
// through LDS (`sx`), so every wave of the group holds the same scores and
// the same softmax state.  The workgroup has HG*CS waves.  `lds` holds
// core_lds_bytes(NT, HG, CS) bytes, 16-byte aligned.
template <int NT, int HG, int CS, class Hooks = CoreNoWait, int RING = kCoreRing, int MAXR = kMaxSplitRows>
__device__ __attribute__((always_inline)) void core_phase(const StepParams& p, int b, char* lds,
                                                          const Hooks& hooks = Hooks()) {
  static_assert(RING >= 1 && RING <= 3, "ring depth");
  char* ring = lds;
  int* ids = reinterpret_cast<int*>(lds + core_ofs_ids(NT, RING));
  char* sink = lds + core_ofs_sink(NT, RING, MAXR);
  f32x4_t* sx = reinterpret_cast<f32x4_t*>(lds + core_ofs_sx(NT, RING, MAXR));
  float* bias = reinterpret_cast<float*>(lds + core_ofs_bias(NT, HG, CS, RING, MAXR));
  constexpr int NW = HG * CS;
  constexpr int NTW = NT / CS;       // output tiles (16 columns) per wave
  constexpr int KSMAX = NT / 2 + 2;  // 32-wide k-steps over kv_row = 16*NT + DR, DR <= 64
  constexpr int KSW = (KSMAX + CS - 1) / CS;  // score k-steps per wave
  constexpr int NPMAX = core_row_pieces(NT);
  constexpr int NI = (kCoreChunk * NPMAX + 64 * NW - 1) / (64 * NW);  // loads per wave per chunk
  constexpr int BUF = core_buf_bytes(NT);
  const Plan& pl = p.pl;
  const int KVR = MLA_D(KVR);
  const int ks = (KVR + 31) >> 5;    // score k-steps
  const int npieces = KVR >> 3;      // 16-byte pieces of a cache row
  const int npad = (4 * ks) | 1;     // LDS row stride in pieces (odd, <= NPMAX)
  const int rstride = npad * 16;
  const int slots = kCoreChunk * npad;

  // Workgroups of the same (token, split) but different head blocks sit 8
  // block indices apart, so they land on the same XCD and share the gathered
  // rows through its L2.
  const int nhb = pl.core_nhb;
  const int pair = (b / (8 * nhb)) * 8 + (b % 8);
  const int hb = (b / 8) % nhb;
  if (pair >= MLA_PL(T) * MLA_PL(nsplit)) return;  // padding workgroup (whole group exits before any barrier)
  const int t = pair / MLA_PL(nsplit), split = pair % MLA_PL(nsplit);
  const int j0 = split * pl.ps, j1 = min(p.P, j0 + pl.ps);
  const int nrows = j1 - j0;
  const int nchunks = (nrows + kCoreChunk - 1) / kCoreChunk;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave / CS, cs = wave % CS;
  const int g = lane >> 4, l16 = lane & 15;
  const int hbase = (hb * HG + hg) * 16;
  const int head = hbase + l16;  // this lane's head for Q fragments and softmax state

  // this wave's k-steps: kk = kb + j for j < nj (nj may be smaller than KSW,
  // or not positive for the last waves of a short row)
  const int kb = cs * KSW;
  const int nj = min(KSW, ks - kb);
  const int nlive = (ks + KSW - 1) / KSW;  // waves holding score k-steps
  // Q fragments: lane l holds Qcat[head][32*kk + 8*g .. +8] (B operand of the score product)
  bf16x8_t qf[KSW];
  auto load_q = [&]() {
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const int k = 32 * (kb + j) + 8 * g;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (j < nj && head < MLA_D(NH) && k < KVR)
        v = *reinterpret_cast<const u32x4_t*>(p.qcat + ((size_t)t * MLA_D(NH) + head) * KVR + k);
      qf[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  if constexpr (Hooks::kEarlyQ) load_q();  // its round trip overlaps the row ids'

  hooks.before_rows(t);
  // this split's flat row ids (-1: causally masked, or past the split)
  for (int i = tid; i < nchunks * kCoreChunk; i += NW * 64)
    ids[i] = (i < nrows) ? p.rows[(size_t)t * p.P + j0 + i] : -1;
  __syncthreads();  // row ids visible

  // Direct global->LDS loads of chunk c into ring buffer c % RING.  Every
  // wave issues exactly NI loads per chunk (slots past the buffer go to the
  // sink) so that the vmcnt arithmetic below is static.  Chunks past the
  // split's last are not loaded (each DMA instruction holds the issuing wave
  // for about as long whatever it reads); the waits below count only the
  // chunks that were.  Per-lane geometry,
  // the same for every chunk: the row inside the chunk of the piece this lane
  // loads (-1: zeros) and its byte offset in the cache row.
  int lrow[NI], lofs[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int s = (i * NW + wave) * 64 + lane;
    lrow[i] = -1;
    lofs[i] = 0;
    if (s < slots) {
      const int r = s / npad, pc = s % npad;
      if (pc < npieces) {
        lrow[i] = r;
        lofs[i] = pc * 16;
      }
    }
  }
  const unsigned row_bytes = (unsigned)KVR * 2u;
  auto issue_chunk = [&](int c) {
    const int bsel = c % RING;
    char* buf = ring + bsel * BUF;
    const bool live = c < nchunks;
    const int* cid = ids + min(c, nchunks - 1) * kCoreChunk;
    if (wave == 0 && lane < kCoreChunk) bias[bsel * kCoreChunk + lane] = (live && cid[lane] >= 0) ? 0.f : -INFINITY;
    int rid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) rid[i] = cid[max(lrow[i], 0)];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s0 = (i * NW + wave) * 64;  // first slot of this load (wave-uniform)
      const char* src = reinterpret_cast<const char*>(p.zero16);
      if (live && lrow[i] >= 0 && rid[i] >= 0)
        src = reinterpret_cast<const char*>(p.cache) + (size_t)(unsigned)rid[i] * row_bytes + lofs[i];
      dma16(src, (s0 < slots) ? buf + s0 * 16 : sink);  // lanes past `slots` stay inside the 1 KB-rounded buffer
    }
  };

  f32x4_t o[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

#pragma unroll
  for (int c = 0; c < (RING > 1 ? RING - 1 : 1); ++c)
    if (c < nchunks) issue_chunk(c);

  hooks.before_q(hb * HG * 16);
  if constexpr (!Hooks::kEarlyQ) load_q();
  // nothing but ring loads is outstanding below
  wait_vmcnt<0>();

  // LDS-space views (addresses fold into the instructions' offset fields)
  const lds_char_t* lring = (const lds_char_t*)ring;
  const lds_char_t* lbias = (const lds_char_t*)bias;
  // per-lane LDS offsets: score fragments (rows l16 and 16+l16, pieces 4*kk+g)
  // and value fragments (rows r1 and r1+16, this wave's output columns)
  const int sofs = l16 * rstride + 16 * g + 64 * kb;
  const int r1 = 4 * g + (l16 >> 2);
  const int vofs = r1 * rstride + 8 * (l16 & 3) + 32 * (cs * NTW);
  const int rs16 = 16 * rstride;

  for (int c = 0; c < nchunks; ++c) {
    if constexpr (RING > 1) {
      // chunk c's loads are this wave's oldest; the younger chunk, if it was
      // loaded, may stay in flight
      if (c + RING - 2 < nchunks)
        wait_vmcnt<NI * (RING - 2)>();
      else
        wait_vmcnt<0>();
      __syncthreads();  // chunk c visible to every wave; buffer (c-1) % ring consumed
      if (c + RING - 1 < nchunks) issue_chunk(c + RING - 1);
    } else {
      if (c > 0) {  // chunk 0 was issued before the query tiles were read
        __syncthreads();  // every wave is done with chunk c-1's buffer and bias
        issue_chunk(c);
        wait_vmcnt<0>();
      }
      __syncthreads();  // chunk c visible to every wave
    }
    const int bsel = c % RING;
    const lds_char_t* buf = lring + bsel * BUF;
    // scores: tile A rows 0-15, tile B rows 16-31, fragments loaded two steps ahead
    f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const lds_char_t* pa = buf + sofs;
      const lds_char_t* pb = pa + rs16;
      auto ld = [&](const lds_char_t* q, int j) { return *(const lds_bf16x8_t*)(q + 64 * j); };
      if (nj == KSW) {  // every k-step of this wave is live (uniform branch)
        bf16x8_t fa0 = ld(pa, 0), fb0 = ld(pb, 0), fa1 = fa0, fb1 = fb0;
        if (KSW > 1) {
          fa1 = ld(pa, 1);
          fb1 = ld(pb, 1);
        }
#pragma unroll
        for (int j = 0; j < KSW; ++j) {
          bf16x8_t fa2 = fa1, fb2 = fb1;
          if (j + 2 < KSW) {
            fa2 = ld(pa, j + 2);
            fb2 = ld(pb, j + 2);
          }
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, qf[j], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0, qf[j], sb, 0, 0, 0);
          fa0 = fa1; fb0 = fb1;
          fa1 = fa2; fb1 = fb2;
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {  // the last column splits of a short row: fewer live k-steps
        // (fragments past the last live one reload it: every read stays in
        // the buffer, and only live k-steps reach the matrix cores)
        const int jl = max(nj - 1, 0);
        bf16x8_t fa0 = ld(pa, 0), fb0 = ld(pb, 0), fa1 = fa0, fb1 = fb0;
        if (KSW > 1) {
          fa1 = ld(pa, min(1, jl));
          fb1 = ld(pb, min(1, jl));
        }
#pragma unroll
        for (int j = 0; j < KSW; ++j) {
          bf16x8_t fa2 = fa1, fb2 = fb1;
          if (j + 2 < KSW) {
            fa2 = ld(pa, min(j + 2, jl));
            fb2 = ld(pb, min(j + 2, jl));
          }
          if (j < nj) {
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, qf[j], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0, qf[j], sb, 0, 0, 0);
          }
          fa0 = fa1; fb0 = fb1;
          fa1 = fa2; fb1 = fb2;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (CS > 1) {
      // add the group's partial score tiles, in wave order (identical in every
      // wave); waves past the last k-step hold none
      f32x4_t* mine = sx + ((hg * CS + cs) * 2) * 64;
      if (cs < nlive) {
        mine[lane] = sa;
        mine[64 + lane] = sb;
      }
      __syncthreads();
      const f32x4_t* grp = sx + (hg * CS * 2) * 64;
      sa = grp[lane];
      sb = grp[64 + lane];
#pragma unroll
      for (int w = 1; w < CS; ++w) {
        if (w < nlive) {
          sa += grp[w * 128 + lane];
          sb += grp[w * 128 + 64 + lane];
        }
      }
    }
    // rows 4g+i (tile A) and 16+4g+i (tile B): masked rows carry -inf
    const f32x4_t ba = *(const lds_f32x4_t*)(lbias + 4 * (bsel * kCoreChunk + 4 * g));
    const f32x4_t bb = *(const lds_f32x4_t*)(lbias + 4 * (bsel * kCoreChunk + 16 + 4 * g));
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = sa[i] + ba[i];
      s[4 + i] = sb[i] + bb[i];
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = max4groups(mx);
    // Lazy rescaling: the reference maximum m_run (log2 domain) moves only when
    // a chunk's maximum exceeds it by more than 8, so probabilities stay below
    // 2^8 and most chunks leave the accumulators alone.  The result is exact:
    // (m, l, o) are kept consistent with whatever reference is in use.
    float alpha = 1.f;
    if (mx > m_run + 8.f) {  // also the first valid chunk (m_run = -inf)
      alpha = __builtin_amdgcn_exp2f(m_run - mx);  // m_run = -inf gives 0
      m_run = mx;
    }
    float pr[8];
    if (m_run != -INFINITY) {  // the same in every lane: all heads see the same valid rows
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(s[i] - m_run);  // masked: exp2(-inf) = 0
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = 0.f;
    }
    float ps = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    ps = sum4groups(ps);
    l_run = l_run * alpha + ps;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // wave-uniform
      // rescale: lane l holds heads 4g+i of each output tile
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
      for (int n = 0; n < NTW; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= ai[i];
    }
    // PV: A slots 0-3 = rows 4g+i, slots 4-7 = rows 16+4g+i; B takes the same rows
    bf16x8_t pab;
#pragma unroll
    for (int i = 0; i < 8; ++i) pab[i] = (__bf16)pr[i];
    // 32-bit LDS addresses of this lane's value fragments (tile n adds 32*n bytes)
    const unsigned av = (unsigned)(uintptr_t)(buf + vofs), av2 = av + (unsigned)rs16;
    auto vfrag = [&](int n) {
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(av + 32u * n));
      const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(av2 + 32u * n));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t vf = vfrag(0);
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      bf16x8_t vn = vf;
      if (n + 1 < NTW) vn = vfrag(n + 1);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pab, vf, o[n], 0, 0, 0);
      vf = vn;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // every chunk loaded was waited for; kept as a guard

  // this split's partial result; waves of one head group hold identical (m, l)
  const size_t pb = ((size_t)t * MLA_PL(nsplit) + split) * MLA_D(NH);
  if (cs == 0 && g == 0 && head < MLA_D(NH)) {
    hooks.st(p.pm + pb + head, m_run);
    hooks.st(p.pden + pb + head, l_run);
  }
  constexpr int R = 16 * NT;
  if (pl.po16) {
    // o / l in fp16 (the matrix-core path, whose hooks store plainly): lane
    // (g, l16) holds heads hbase + 4g + i, whose l lane 4g + i holds
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l_run, 4 * g + i, 64);
      inv[i] = li > 0.f ? 1.f / li : 0.f;
    }
    _Float16* po16 = reinterpret_cast<_Float16*>(p.po);
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hbase + 4 * g + i;
        if (h < MLA_D(NH)) po16[(pb + h) * R + 16 * (cs * NTW + n) + l16] = (_Float16)(o[n][i] * inv[i]);
      }
  } else {
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hbase + 4 * g + i;
        if (h < MLA_D(NH)) hooks.st(p.po + (pb + h) * R + 16 * (cs * NTW + n) + l16, o[n][i]);
      }
  }
}

// ---------------------------------------------------------------------------
// Many heads: 64 heads per workgroup of eight waves, row-split scores.
//
// Wave w owns head tile ht = w/2 (16 heads) and row half rh = w%2 of each
// 32-row chunk for the scores: S^T[16 rows x 16 heads] over the whole kv_row,
// so no partial score tiles are exchanged.  The two waves of a head tile swap
// their chunk maxima through LDS and so keep identical softmax references;
// each keeps the row sum of its own rows (added at the end).  Each wave then
// writes its probabilities into the PV operand of its head tile in LDS (rows
// 4g+i of the half in slots 4*rh .. 4*rh+3, the order the transposing value
// reads deliver) and, for the PV product, takes NT/8 output tiles (16 latent
// columns each) for all 64 heads: every value fragment read from LDS serves
// four MFMAs, and each gathered row is read from LDS once for the values.
// LDS: ring | row ids | sink | chunk maxima [2][4][16] | P [4][64 lanes][16 B]
//      | rescale factors [4][16] | row sums [4][16].  The validity of each
// lane's score rows stays in registers from the chunk's issue to its use.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int core_rs_ofs_max(int nt) { return core_ofs_sink(nt) + 1024; }
__host__ __device__ constexpr int core_rs_ofs_p(int nt) { return core_rs_ofs_max(nt) + 2 * 4 * 16 * 4; }
__host__ __device__ constexpr int core_rs_ofs_alpha(int nt) { return core_rs_ofs_p(nt) + 4 * 64 * 16; }
__host__ __device__ constexpr int core_rs_ofs_l(int nt) { return core_rs_ofs_alpha(nt) + 4 * 16 * 4; }
__host__ __device__ constexpr int core_rs_lds_bytes(int nt) { return core_rs_ofs_l(nt) + 4 * 16 * 4; }

template <int NT>
__device__ __attribute__((always_inline)) void core_phase_rs(const StepParams& p, int b, char* lds) {
  static_assert(NT % 8 == 0, "eight waves split the output tiles");
  constexpr int NW = 8;
  constexpr int NTW = NT / 8;        // output tiles per wave in the PV product
  constexpr int KSMAX = NT / 2 + 2;  // 32-wide k-steps over kv_row = 16*NT + DR, DR <= 64
  constexpr int NPMAX = core_row_pieces(NT);
  constexpr int NI = (kCoreChunk * NPMAX + 64 * NW - 1) / (64 * NW);  // loads per wave per chunk
  constexpr int BUF = core_buf_bytes(NT);
  char* ring = lds;
  int* ids = reinterpret_cast<int*>(lds + core_ofs_ids(NT));
  char* sink = lds + core_ofs_sink(NT);
  float* cmax = reinterpret_cast<float*>(lds + core_rs_ofs_max(NT));     // [rh][ht][16]
  char* pbuf = lds + core_rs_ofs_p(NT);                                  // [ht][lane][16 B]
  float* alph = reinterpret_cast<float*>(lds + core_rs_ofs_alpha(NT));  // [ht][16]
  float* lsum = reinterpret_cast<float*>(lds + core_rs_ofs_l(NT));      // [ht][16]
  const Plan& pl = p.pl;
  const int KVR = MLA_D(KVR);
  const int ks = (KVR + 31) >> 5;  // score k-steps
  const int npieces = KVR >> 3;    // 16-byte pieces of a cache row
  const int npad = (4 * ks) | 1;   // LDS row stride in pieces (odd, <= NPMAX)
  const int rstride = npad * 16;
  const int slots = kCoreChunk * npad;

  // workgroups of the same (token, split) but different head blocks sit 8
  // block indices apart: same XCD, shared gathered rows in its L2
  const int nhb = pl.core_nhb;
  const int pair = (b / (8 * nhb)) * 8 + (b % 8);
  const int hb = (b / 8) % nhb;
  if (pair >= MLA_PL(T) * MLA_PL(nsplit)) return;  // padding workgroup (whole group exits before any barrier)
  const int t = pair / MLA_PL(nsplit), split = pair % MLA_PL(nsplit);
  const int j0 = split * pl.ps, j1 = min(p.P, j0 + pl.ps);
  const int nrows = j1 - j0;
  const int nchunks = (nrows + kCoreChunk - 1) / kCoreChunk;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ht = wave >> 1, rh = wave & 1;
  const int g = lane >> 4, l16 = lane & 15;
  const int hblk = hb * 64;                   // first head of the workgroup
  const int head = hblk + 16 * ht + l16;      // this lane's head in the score product

  for (int i = tid; i < nchunks * kCoreChunk; i += NW * 64)
    ids[i] = (i < nrows) ? p.rows[(size_t)t * p.P + j0 + i] : -1;
  __syncthreads();

  int lrow[NI], lofs[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int s = (i * NW + wave) * 64 + lane;
    lrow[i] = -1;
    lofs[i] = 0;
    if (s < slots) {
      const int r = s / npad, pc = s % npad;
      if (pc < npieces) {
        lrow[i] = r;
        lofs[i] = pc * 16;
      }
    }
  }
  const unsigned row_bytes = (unsigned)KVR * 2u;
  // issues chunk c's row loads; returns the validity of this lane's score
  // rows 16*rh + 4g + i (bit i), kept in registers until the chunk is used
  auto issue_chunk = [&](int c) -> unsigned {
    const int bsel = c % kCoreRing;
    char* buf = ring + bsel * BUF;
    const bool live = c < nchunks;
    const int* cid = ids + min(c, nchunks - 1) * kCoreChunk;
    const int4 mine = *reinterpret_cast<const int4*>(cid + 16 * rh + 4 * g);
    const unsigned valid = live ? ((mine.x >= 0 ? 1u : 0u) | (mine.y >= 0 ? 2u : 0u) | (mine.z >= 0 ? 4u : 0u) |
                                   (mine.w >= 0 ? 8u : 0u))
                                : 0u;
    int rid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) rid[i] = cid[max(lrow[i], 0)];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s0 = (i * NW + wave) * 64;
      const char* src = reinterpret_cast<const char*>(p.zero16);
      if (live && lrow[i] >= 0 && rid[i] >= 0)
        src = reinterpret_cast<const char*>(p.cache) + (size_t)(unsigned)rid[i] * row_bytes + lofs[i];
      dma16(src, (s0 < slots) ? buf + s0 * 16 : sink);
    }
    return valid;
  };

  f32x4_t o[4][NTW];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int n = 0; n < NTW; ++n) o[q][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // per head l16 of head tile ht; l over this wave's rows

  static_assert(kCoreRing == 3, "the validity masks rotate through three registers");
  unsigned vm0 = issue_chunk(0), vm1 = issue_chunk(1);

  // Q fragments of the whole kv_row: lane l holds Qcat[head][32*kk + 8*g .. +8]
  bf16x8_t qf[KSMAX];
#pragma unroll
  for (int kk = 0; kk < KSMAX; ++kk) {
    const int k = 32 * kk + 8 * g;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (kk < ks && head < MLA_D(NH) && k < KVR)
      v = *reinterpret_cast<const u32x4_t*>(p.qcat + ((size_t)t * MLA_D(NH) + head) * KVR + k);
    qf[kk] = __builtin_bit_cast(bf16x8_t, v);
  }
  wait_vmcnt<0>();

  const lds_char_t* lring = (const lds_char_t*)ring;
  // score fragments: row 16*rh + l16, pieces 4*kk + g
  const int sofs = (16 * rh + l16) * rstride + 16 * g;
  // value fragments: rows r1 and r1 + 16, this wave's output columns
  const int r1 = 4 * g + (l16 >> 2);
  const int vofs = r1 * rstride + 8 * (l16 & 3) + 32 * (wave * NTW);
  const int rs16 = 16 * rstride;

  for (int c = 0; c < nchunks; ++c) {
    wait_vmcnt<NI * (kCoreRing - 2)>();
    __syncthreads();  // chunk c visible; the previous chunk's LDS buffers consumed
    const int bsel = c % kCoreRing;
    const lds_char_t* buf = lring + bsel * BUF;
    // scores of this wave's 16 rows: two accumulators (even / odd k-steps),
    // key fragments loaded two steps ahead
    f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const lds_char_t* pa = buf + sofs;
      auto ld = [&](int kk) { return *(const lds_bf16x8_t*)(pa + 64 * kk); };
      if (ks == KSMAX) {  // kv_row fills every k-step (uniform branch)
        bf16x8_t f0 = ld(0), f1 = ld(1);
#pragma unroll
        for (int kk = 0; kk < KSMAX; ++kk) {
          bf16x8_t f2 = f1;
          if (kk + 2 < KSMAX) f2 = ld(kk + 2);
          if (kk & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, qf[kk], sb, 0, 0, 0);
          else sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, qf[kk], sa, 0, 0, 0);
          f0 = f1;
          f1 = f2;
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KSMAX; ++kk) {
          if (kk < ks) {
            if (kk & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld(kk), qf[kk], sb, 0, 0, 0);
            else sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld(kk), qf[kk], sa, 0, 0, 0);
          }
        }
      }
    }
    // the loads of chunk c+2 go out after this chunk's score reads; its ring
    // buffer was last read by chunk c-1, finished by every wave before the barrier
    const unsigned vm2 = issue_chunk(c + kCoreRing - 1);
    // rows 16*rh + 4g + i: masked rows carry -inf
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = ((vm0 >> i) & 1u) ? sa[i] + sb[i] : -INFINITY;
    vm0 = vm1;
    vm1 = vm2;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = max4groups(mx);
    if (g == 0) cmax[(rh * 4 + ht) * 16 + l16] = mx;
    __syncthreads();  // chunk maxima of both halves visible
    mx = fmaxf(mx, cmax[((1 - rh) * 4 + ht) * 16 + l16]);  // the same value in both waves of the tile
    // lazy rescaling as in core_phase: the reference moves only when the chunk
    // maximum exceeds it by more than 8 (both waves decide alike)
    float alpha = 1.f;
    if (mx > m_run + 8.f) {
      alpha = __builtin_amdgcn_exp2f(m_run - mx);  // m_run = -inf gives 0
      m_run = mx;
    }
    float pr[4];
    if (m_run != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(s[i] - m_run);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = 0.f;
    }
    float ps = (pr[0] + pr[1]) + (pr[2] + pr[3]);
    ps = sum4groups(ps);
    l_run = l_run * alpha + ps;
    // this half's probabilities into slots 4*rh .. 4*rh+3 of the head tile's PV operand
    {
      bf16_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = f32_to_bf16(pr[i]);
      uint2 w;
      w.x = (uint32_t)pb[0] | ((uint32_t)pb[1] << 16);
      w.y = (uint32_t)pb[2] | ((uint32_t)pb[3] << 16);
      *reinterpret_cast<uint2*>(pbuf + (ht * 64 + lane) * 16 + 8 * rh) = w;
    }
    if (rh == 0 && g == 0) alph[ht * 16 + l16] = alpha;
    __syncthreads();  // probabilities and rescale factors of all head tiles visible
    // PV: this wave's output tiles for all four head tiles
    bf16x8_t pab[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pab[q] = *reinterpret_cast<const bf16x8_t*>(pbuf + (q * 64 + lane) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // lane (g, l16) holds heads 4g+i of each output tile
      const f32x4_t ai = *reinterpret_cast<const f32x4_t*>(alph + q * 16 + 4 * g);
      const bool any = (ai[0] != 1.f) || (ai[1] != 1.f) || (ai[2] != 1.f) || (ai[3] != 1.f);
      if (__builtin_amdgcn_ballot_w64(any) != 0) {  // wave-uniform
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[q][n][i] *= ai[i];
      }
    }
    const unsigned av = (unsigned)(uintptr_t)(buf + vofs), av2 = av + (unsigned)rs16;
    auto vfrag = [&](int n) {
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(av + 32u * n));
      const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(av2 + 32u * n));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t vf = vfrag(0);
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      bf16x8_t vn = vf;
      if (n + 1 < NTW) vn = vfrag(n + 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pab[q], vf, o[q][n], 0, 0, 0);
      vf = vn;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // the trailing loads (zero rows into unused buffers or the sink)

  // (m, l): the waves of a head tile hold the same m; l adds the two halves
  if (rh == 1 && g == 0) lsum[ht * 16 + l16] = l_run;
  __syncthreads();
  const size_t pb = ((size_t)t * MLA_PL(nsplit) + split) * MLA_D(NH);
  if (rh == 0 && g == 0 && head < MLA_D(NH)) {
    p.pm[pb + head] = m_run;
    p.pden[pb + head] = l_run + lsum[ht * 16 + l16];
  }
  constexpr int R = 16 * NT;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hblk + 16 * q + 4 * g + i;
        if (h < MLA_D(NH)) p.po[(pb + h) * R + 16 * (wave * NTW + n) + l16] = o[q][n][i];
      }
}


// ---------------------------------------------------------------------------
// Many heads, one head tile per wave: 128 heads per workgroup of eight waves.
//
// Wave w owns heads 16w .. 16w+15 of the workgroup's block for the whole
// chunk: both score tiles (rows 0-15 and 16-31) over the whole kv_row, the
// softmax of its heads, and the PV product over every latent column.  No wave
// reads another wave's results, so the ring's barrier is the only one per
// chunk, and every gathered row is loaded once for all 128 heads.  The PV
// product is taken transposed, O^T[c, head] += sum_row V^T[c, row] P^T[row, head]:
// the value fragments are the A operand and the probabilities, which stay in
// the lanes the score tiles left them in, the B operand.  Lane l's
// accumulators then all belong to head l%16, so a rescale is a per-lane
// multiply with no cross-lane moves.
// A buffer row spans 4*ks + 2 16-byte pieces: at that stride (2 mod 4) the
// score fragments' 16-byte reads ran 16 % faster than at the odd stride of
// the other shapes, and the transposing value reads 3 % slower.
// LDS: ring | row ids | sink | score bias (ring x 32 floats).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int core_wide_row_pieces(int nt) { return 2 * nt + 10; }
__host__ __device__ constexpr int core_wide_buf_bytes(int nt) {
  return (kCoreChunk * core_wide_row_pieces(nt) * 16 + 1023) / 1024 * 1024;
}
// Four chunk buffers keep three chunks' loads in flight (3 % faster than
// three buffers at large128); the row ids of a split then get the 10 KB left.
constexpr int kWideRing = 4;
constexpr int kWideMaxSplitRows = 2560;  // row ids staged per workgroup
__host__ __device__ constexpr int core_wide_ofs_ids(int nt) { return kWideRing * core_wide_buf_bytes(nt); }
__host__ __device__ constexpr int core_wide_ofs_sink(int nt) { return core_wide_ofs_ids(nt) + kWideMaxSplitRows * 4; }
__host__ __device__ constexpr int core_wide_ofs_bias(int nt) { return core_wide_ofs_sink(nt) + 1024; }
__host__ __device__ constexpr int core_wide_lds_bytes(int nt) {
  return core_wide_ofs_bias(nt) + kWideRing * kCoreChunk * 4;
}
static_assert(core_wide_lds_bytes(32) <= 160 * 1024, "one workgroup's LDS");

template <int NT>
__device__ __attribute__((always_inline)) void core_phase_wide(const StepParams& p, int b, char* lds) {
  constexpr int NW = 8;
  constexpr int KD = 2;                 // key-fragment k-steps in flight
  constexpr int VD = NT >= 4 ? 4 : NT;  // value-fragment tiles in flight
  constexpr int KSMAX = NT / 2 + 2;  // 32-wide k-steps over kv_row = 16*NT + DR, DR <= 64
  constexpr int NPMAX = core_wide_row_pieces(NT);
  constexpr int NI = (kCoreChunk * NPMAX + 64 * NW - 1) / (64 * NW);  // loads per wave per chunk
  constexpr int BUF = core_wide_buf_bytes(NT);
  char* ring = lds;
  int* ids = reinterpret_cast<int*>(lds + core_wide_ofs_ids(NT));
  char* sink = lds + core_wide_ofs_sink(NT);
  float* bias = reinterpret_cast<float*>(lds + core_wide_ofs_bias(NT));
  const Plan& pl = p.pl;
  const int KVR = MLA_D(KVR);
  const int ks = (KVR + 31) >> 5;  // score k-steps
  const int npieces = KVR >> 3;    // 16-byte pieces of a cache row
  const int npad = 4 * ks + 2;     // LDS row stride in pieces (<= NPMAX)
  const int rstride = npad * 16;
  const int slots = kCoreChunk * npad;

  // workgroups of the same (token, split) but different head blocks sit 8
  // block indices apart: same XCD, shared gathered rows in its L2
  const int nhb = pl.core_nhb;
  const int pair = (b / (8 * nhb)) * 8 + (b % 8);
  const int hb = (b / 8) % nhb;
  if (pair >= MLA_PL(T) * MLA_PL(nsplit)) return;  // padding workgroup (whole group exits before any barrier)
  const int t = pair / MLA_PL(nsplit), split = pair % MLA_PL(nsplit);
  const int j0 = split * pl.ps, j1 = min(p.P, j0 + pl.ps);
  const int nrows = j1 - j0;
  const int nchunks = (nrows + kCoreChunk - 1) / kCoreChunk;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar arithmetic below
  const int g = lane >> 4, l16 = lane & 15;
  const int head = hb * (16 * NW) + 16 * wave + l16;  // this lane's head (scores, softmax, output)

  for (int i = tid; i < nchunks * kCoreChunk; i += NW * 64)
    ids[i] = (i < nrows) ? p.rows[(size_t)t * p.P + j0 + i] : -1;
  __syncthreads();

  // Per-lane geometry of the ring loads, the same for every chunk: load i of
  // this wave fills slots (i*NW + wave)*64 + lane; geo[i] = (row in the chunk
  // << 16) | byte offset in the cache row, or -1 for a padding piece (zeros).
  int geo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int s = (i * NW + wave) * 64 + lane;
    const int r = s / npad, pc = s % npad;
    geo[i] = (s < slots && pc < npieces) ? ((r << 16) | (pc * 16)) : -1;
  }
  const unsigned row_bytes = (unsigned)KVR * 2u;
  const char* cache = reinterpret_cast<const char*>(p.cache);
  const char* zsrc = reinterpret_cast<const char*>(p.zero16);
  auto issue_chunk = [&](int c) {
    const int bsel = c % kWideRing;
    char* buf = ring + bsel * BUF;
    const bool live = c < nchunks;  // wave-uniform
    const int* cid = ids + min(c, nchunks - 1) * kCoreChunk;
    if (wave == 0 && lane < kCoreChunk) bias[bsel * kCoreChunk + lane] = (live && cid[lane] >= 0) ? 0.f : -INFINITY;
    int rid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) rid[i] = cid[max(geo[i] >> 16, 0)];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s0 = (i * NW + wave) * 64;  // first slot of this load (scalar)
      int gi = geo[i];
      asm volatile("" : "+v"(gi));  // keep the row offset 32-bit; no hoisted 64-bit bases
      const char* src = zsrc;
      if (live && gi >= 0 && rid[i] >= 0)
        src = cache + ((uint64_t)(unsigned)rid[i] * row_bytes + (unsigned)(gi & 0xffff));
      dma16(src, (s0 < slots) ? buf + s0 * 16 : sink);  // lanes past `slots` stay inside the 1 KB-rounded buffer
    }
  };

  f32x4_t o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // head l16; l over this lane's rows (groups added at the end)

  // chunks past the split's last are not loaded (a DMA instruction holds its
  // wave about as long whatever it reads); the waits count only those that were
#pragma unroll
  for (int c = 0; c + 1 < kWideRing; ++c)
    if (c < nchunks) issue_chunk(c);

  // Q fragments of the whole kv_row: lane l holds Qcat[head][32*kk + 8*g .. +8]
  // (loaded from a clamped address and zeroed past the heads or the row)
  bf16x8_t qf[KSMAX];
  {
    const bool hl = head < MLA_D(NH);
    const uint16_t* qrow = p.qcat + ((size_t)t * MLA_D(NH) + (hl ? head : 0)) * KVR;
#pragma unroll
    for (int kk = 0; kk < KSMAX; ++kk) {
      const int k = 32 * kk + 8 * g;
      const bool ok = hl && kk < ks && k < KVR;
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + (ok ? k : 0));
      if (!ok) v = u32x4_t{0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  wait_vmcnt<0>();

  const lds_char_t* lring = (const lds_char_t*)ring;
  const lds_char_t* lbias = (const lds_char_t*)bias;
  // score fragments: rows l16 and 16+l16, pieces 4*kk+g
  const int sofs = l16 * rstride + 16 * g;
  // value fragments: rows r1 and r1+16, columns 16n + 4*(l16&3) .. +3 of each tile
  const int r1 = 4 * g + (l16 >> 2);
  const int vofs = r1 * rstride + 8 * (l16 & 3);
  const int rs16 = 16 * rstride;

  const bool late_issue = wave >= NW / 2;  // the second wave of each SIMD (scalar)
  for (int c = 0; c < nchunks; ++c) {
    // chunk c's loads are this wave's oldest; those of c+1 and c+2, if loaded, may stay in flight
    static_assert(kWideRing == 4, "the waits below count three chunks in flight");
    if (c + 2 < nchunks)
      wait_vmcnt<2 * NI>();
    else if (c + 1 < nchunks)
      wait_vmcnt<NI>();
    else
      wait_vmcnt<0>();
    __syncthreads();   // chunk c visible to every wave; buffer (c-1) % ring consumed
    // The loads of chunk c+3 stall the issuing wave until the memory system
    // takes them (they go out at the gather's rate), so the two waves of a
    // SIMD issue them at different points: waves 0-3 first, waves 4-7 after
    // their softmax.  Each wave's stall then overlaps the other's products.
    const bool more = c + kWideRing - 1 < nchunks;  // uniform
    if (!late_issue && more) issue_chunk(c + kWideRing - 1);
    const int bsel = c % kWideRing;
    const lds_char_t* buf = lring + bsel * BUF;
    // scores: tile A rows 0-15, tile B rows 16-31, key fragments KD k-steps ahead
    f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const lds_char_t* pa = buf + sofs;
      const lds_char_t* pb = pa + rs16;
      auto ld = [&](const lds_char_t* q, int kk) { return *(const lds_bf16x8_t*)(q + 64 * kk); };
      if (ks == KSMAX) {  // kv_row fills every k-step (uniform branch)
        bf16x8_t fa[KD], fb[KD];
#pragma unroll
        for (int j = 0; j < KD; ++j) {
          fa[j] = ld(pa, j);
          fb[j] = ld(pb, j);
        }
#pragma unroll
        for (int kk = 0; kk < KSMAX; ++kk) {
          const bf16x8_t ca = fa[kk % KD], cb = fb[kk % KD];
          if (kk + KD < KSMAX) {
            fa[kk % KD] = ld(pa, kk + KD);
            fb[kk % KD] = ld(pb, kk + KD);
          }
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca, qf[kk], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cb, qf[kk], sb, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KSMAX; ++kk) {
          if (kk < ks) {
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld(pa, kk), qf[kk], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld(pb, kk), qf[kk], sb, 0, 0, 0);
          }
        }
      }
    }
    // rows 4g+i (tile A) and 16+4g+i (tile B): masked rows carry -inf
    const f32x4_t ba = *(const lds_f32x4_t*)(lbias + 4 * (bsel * kCoreChunk + 4 * g));
    const f32x4_t bb = *(const lds_f32x4_t*)(lbias + 4 * (bsel * kCoreChunk + 16 + 4 * g));
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = sa[i] + ba[i];
      s[4 + i] = sb[i] + bb[i];
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = max4groups(mx);  // the chunk maximum of head l16, the same in its four lanes
    // lazy rescaling, per head: the reference moves only when the chunk
    // maximum exceeds it by more than 8 (log2 units)
    float alpha = 1.f;
    if (mx > m_run + 8.f) {
      alpha = __builtin_amdgcn_exp2f(m_run - mx);  // m_run = -inf gives 0
      m_run = mx;
    }
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = (m_run != -INFINITY) ? __builtin_amdgcn_exp2f(s[i] - m_run) : 0.f;
    l_run = l_run * alpha + (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7])));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // wave-uniform
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] *= alpha;
    }
    if (late_issue && more) issue_chunk(c + kWideRing - 1);
    // B operand of the PV product: k-slots 0-3 = rows 4g+i, 4-7 = rows 16+4g+i
    bf16x8_t pab;
#pragma unroll
    for (int i = 0; i < 8; ++i) pab[i] = (__bf16)pr[i];
    const unsigned av = (unsigned)(uintptr_t)(buf + vofs), av2 = av + (unsigned)rs16;
    auto vfrag = [&](int n) {
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(av + 32u * n));
      const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(av2 + 32u * n));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // value fragments VD tiles ahead
    bf16x8_t vq[VD];
#pragma unroll
    for (int j = 0; j < VD; ++j) vq[j] = vfrag(j);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8_t cv = vq[n % VD];
      if (n + VD < NT) vq[n % VD] = vfrag(n + VD);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv, pab, o[n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // every chunk loaded was waited for; kept as a guard

  const float l_tot = sum4groups(l_run);
  const size_t pb = ((size_t)t * MLA_PL(nsplit) + split) * MLA_D(NH);
  if (head < MLA_D(NH)) {
    if (g == 0) {
      p.pm[pb + head] = m_run;
      p.pden[pb + head] = l_tot;
    }
    constexpr int R = 16 * NT;
    // lane (g, l16) holds columns 16n + 4g + i of head l16
    if (pl.po16) {  // o / l in fp16, four columns in one 8-byte store
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      _Float16* po16 = reinterpret_cast<_Float16*>(p.po) + (pb + head) * R + 4 * g;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const f16x4_t v = f16x4_t{(_Float16)(o[n][0] * inv), (_Float16)(o[n][1] * inv), (_Float16)(o[n][2] * inv),
                                  (_Float16)(o[n][3] * inv)};
        *reinterpret_cast<f16x4_t*>(po16 + 16 * n) = v;
      }
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4_t*>(p.po + (pb + head) * R + 16 * n + 4 * g) = o[n];
    }
  }
}

}  // namespace MLA_PHASE_NS
