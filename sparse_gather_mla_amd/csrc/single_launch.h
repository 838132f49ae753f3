// Single-launch step: every phase of a few-token step as workgroups of one
// kernel, in the order of the MLA attention block gather decode API page's
// description -- the index build first (its inputs are tiny and every gather
// depends on them), then the down-projections, the query up-projection, the
// absorption with the kv-row write, the gather core, the output absorption
// and the o-projection, whose last-arriving slab of each column tile writes
// the output (oproj_fold_out).
//
// Workgroup b runs item b of that list.  An item waits only for the items of
// earlier phases whose results it reads (HandoffFlags, handoff.h): a
// q up-projection slab for the down-projection tiles over its rows, an
// absorption tile for its head's up-projection tiles, an o-projection slab
// for the output absorption of its heads.  The hardware dispatches workgroups in
// index order, so the lowest unfinished phase always runs: no wait can
// deadlock.  Each GEMV item issues its first weight loads before it waits, so
// a phase's weight stream overlaps the tail of the phase before it, and a
// consumer starts as soon as its own producers are done.
//
// Occupancy: two workgroups per CU (at most 256 registers a lane, LDS below
// 80 KB), so the core keeps one chunk buffer instead of three and stages at
// most kSingleMaxRows row ids.
#pragma once

#include "phases.h"

namespace mla {

constexpr int kSingleRing = 1;
constexpr int kSingleMaxRows = 2048;
// the flag region: [0] epoch, [16] completed o-projection column tiles, flags from word 64
constexpr int kFlagHeaderWords = 64;
constexpr int kFlagRegionWords = 16384;
constexpr int kSingleMaxItems = kFlagRegionWords - kFlagHeaderWords;

template <int NTT, int NT>
constexpr int single_lds_bytes() {
  constexpr int g = GemvLds<NTT>::floats * 4;
  constexpr int o = (kOabsScratch + 1024) * 4;  // output absorption: weights, o_lat, scratch
  constexpr int c = core_lds_bytes(NT, 1, 4, kSingleRing, kSingleMaxRows);
  return g > o ? (g > c ? g : c) : (o > c ? o : c);
}

// Core hooks: the row ids and every token's cache row before the first row
// id is read (a token may select a row another token of the step writes);
// the query tiles of the workgroup's heads after the first chunk's row loads
// are out.  All of them are read with ordinary loads: each wait covers every
// producer of the lines read.
struct CoreWaitSingle {
  static constexpr bool kEarlyQ = false;  // the query tiles are produced in the same launch
  const StepParams& p;
  unsigned e;
  __device__ void before_rows(int) const {
    const Plan& pl = p.pl;
    const int n_tiles = p.NH * pl.ncc3;
    wait_flags(p.flags, FlagSet().add(0, pl.i_down).add(pl.i_abs + n_tiles, pl.i_core - pl.i_abs - n_tiles), e, p.err);
  }
  __device__ void before_q(int h0) const {
    const Plan& pl = p.pl;
    const int h1 = min(p.NH, h0 + 16);
    wait_flags(p.flags, FlagSet().add(pl.i_abs + h0 * pl.ncc3, (h1 - h0) * pl.ncc3), e, p.err);
  }
  __device__ __forceinline__ void st(float* q, float v) const { st_dev(q, v); }
};

// Items of the split-K GEMVs are numbered tile-major (item = tile * slabs +
// slab), so the slabs of one column tile, which a consumer waits for, have
// adjacent flags; the phase functions take b = slab * tiles + tile.
__device__ __forceinline__ int slab_major(int item, int slabs, int tiles) {
  return (item % slabs) * tiles + item / slabs;
}

template <int NTT, int NT>
__device__ __attribute__((always_inline)) void step_single(const StepParams& p, int b, char* lds) {
  const Plan& pl = p.pl;
  float* fl = reinterpret_cast<float*>(lds);
  // this step's epoch: one past the last completed step's (never 0, the
  // value of a zeroed workspace)
  unsigned e = *p.epoch + 1u;
  if (e == 0u) e = 1u;
  const int T = pl.T;
  auto sync = [&](const FlagSet& fs) { return HandoffFlags{p.flags, p.err, e, fs}; };
  if (b < pl.i_down) {
    if (b == 0) {  // the zero region and the o-projection tiles' arrival counters
      if (threadIdx.x < 64) st_dev(const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(p.zero16)) + threadIdx.x, 0u);
      for (int i = threadIdx.x; i < pl.nt6; i += kBlock) st_dev(p.tcnt + i * kSyncStride, 0u);
    }
    index_build(p, b * kBlock + threadIdx.x, sync(FlagSet()));
  } else if (b < pl.i_qup) {
    phase_down<NTT>(p, slab_major(b - pl.i_down, pl.s1, pl.nt1), fl, sync(FlagSet()));
  } else if (b < pl.i_abs) {
    const int i = b - pl.i_qup, n_gemv = pl.nt2 * pl.s2;
    FlagSet fs;
    int bq = i;
    if (i < n_gemv) {
      // acc_a columns [k0, k0 + ks): the down-projection's q tiles over them
      const int slab = i % pl.s2, k0 = slab * pl.ks2, ks = min(pl.ks2, p.Q - k0);
      const int ta = k0 / pl.tw1, tb = (k0 + ks - 1) / pl.tw1;
      fs.add(pl.i_down + ta * pl.s1, (tb - ta + 1) * pl.s1);
      bq = slab_major(i, pl.s2, pl.nt2);
    } else {
      // kv-row columns [c0, c0 + nc): the kv tiles over them, and tile 0 (sums of x^2)
      const int c0 = ((i - n_gemv) % pl.nkv) * kKvSlice, nc = min(kKvSlice, p.KVR - c0);
      const int ta = pl.nt_q + c0 / pl.tw1, tb = pl.nt_q + (c0 + nc - 1) / pl.tw1;
      fs.add(pl.i_down + ta * pl.s1, (tb - ta + 1) * pl.s1).add(pl.i_down, pl.s1);
    }
    phase_qup<NTT>(p, bq, fl, sync(fs));
  } else if (b < pl.i_core) {
    const int i = b - pl.i_abs, n_tiles = p.NH * pl.ncc3, n_gemv = pl.nt2 * pl.s2;
    FlagSet fs;
    if (i < n_tiles) {
      // head h's wq_b columns, the up-projection's tile 0 (sums of acc_a^2) and
      // the down-projection's tile 0 (sums of x^2)
      const int h = i / pl.ncc3;
      const int ta = h * p.QKH / pl.tw2, tb = (h * p.QKH + p.QKH - 1) / pl.tw2;
      fs.add(pl.i_qup + ta * pl.s2, (tb - ta + 1) * pl.s2).add(pl.i_qup, pl.s2).add(pl.i_down, pl.s1);
    } else {
      fs.add(pl.i_qup + n_gemv + (i - n_tiles) * pl.nkv, pl.nkv);  // token t's kv-row slices
    }
    phase_absorb<NTT>(p, i, fl, sync(fs));
  } else if (b < pl.i_oabs) {
    core_phase<NT, 1, 4, CoreWaitSingle, kSingleRing, kSingleMaxRows>(p, b - pl.i_core, lds, CoreWaitSingle{p, e});
  } else if (b < pl.i_oproj) {
    // every split of the token chunk's tokens (one head block at <= 16 heads);
    // the last chunk also covers the core's padding items, so that every item
    // of the launch is waited for before the step ends
    const int tch = (b - pl.i_oabs) % pl.nt5c, t0 = tch * pl.tc5, nt = min(pl.tc5, T - t0);
    const int lo = pl.i_core + t0 * pl.nsplit, hi = tch == pl.nt5c - 1 ? pl.i_oabs : lo + nt * pl.nsplit;
    phase_oabsorb(p, b - pl.i_oabs, fl, sync(FlagSet().add(lo, hi - lo)));
  } else {
    // o_v rows [k0, k0 + ks): the output absorption of their heads
    const int i = b - pl.i_oproj, slab = i % pl.s6, tile = i / pl.s6;
    const int k0 = slab * pl.ks6, ks = min(pl.ks6, p.NH * p.DV - k0);
    const int ha = k0 / p.DV, hb = (k0 + ks - 1) / p.DV, per_h = pl.nc5 * pl.nt5c;
    phase_oproj<NTT>(p, slab * pl.nt6 + tile, fl, sync(FlagSet().add(pl.i_oabs + ha * per_h, (hb - ha + 1) * per_h)));
    // The last slab of each tile writes the tile's output; the last tile to
    // be written ends the step.  Every other item has finished reading the
    // epoch by then (each item's results are waited for, directly or through
    // its consumers, by some o-projection slab, and every slab is counted),
    // so that one advances it.
    if (oproj_fold_out(p, tile, fl)) {
      __syncthreads();
      if (threadIdx.x == 0) {
        unsigned* done = p.epoch + 16;
        const unsigned old = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (unsigned)pl.nt6 - 1u) {
          st_dev(done, 0u);
          st_dev(p.epoch, e);
        }
      }
    }
    return;
  }
  publish_flag(p.flags + b, e);
}

}  // namespace mla
