// MLA gather-decode step for MI355X (gfx950): kernels and the C ABI declared
// in include/mla_gather_decode.h.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mla_gather_decode.h"
#include "fixed_shape.h"
#include "phases.h"
#include "phases_mfma.h"
#include "single_launch.h"

using namespace mla;

// ---------------------------------------------------------------------------
// kernels: one phase each, launched in order on the caller's stream
// ---------------------------------------------------------------------------

template <int NTT>
__global__ __launch_bounds__(kBlock) void k_down(StepParams p) {
  extern __shared__ float lds[];
  // the fused variant's counters and the o-projection tiles' arrival counters
  // start each step at zero (this step's later kernels run after this one;
  // the previous step's have finished)
  if (blockIdx.x == 0) {
    if (p.pl.fused && (int)threadIdx.x < p.NH + 2) p.sync[threadIdx.x * kSyncStride] = 0u;
    for (int i = threadIdx.x; i < p.pl.nt6; i += kBlock) p.tcnt[i * kSyncStride] = 0u;
  }
  clear_zero_region(p, blockIdx.x);
  phase_down<NTT>(p, blockIdx.x, lds);
}

template <int NTT>
__global__ __launch_bounds__(kBlock) void k_qup(StepParams p) {
  extern __shared__ float lds[];
  phase_qup<NTT>(p, blockIdx.x, lds);
}

template <int NTT>
__global__ __launch_bounds__(kBlock) void k_absorb(StepParams p) {
  extern __shared__ float lds[];
  phase_absorb<NTT>(p, blockIdx.x, lds);
}

template <int NT, int HG, int CS>
__global__ __launch_bounds__(HG * CS * 64) void k_core(StepParams p) {
  __shared__ __attribute__((aligned(16))) char lds[core_lds_bytes(NT, HG, CS)];
  core_phase<NT, HG, CS>(p, blockIdx.x, lds);
}

// many heads (64 per workgroup, eight waves): row-split scores (core_mfma.h)
template <int NT>
__global__ __launch_bounds__(512) void k_core_rs(StepParams p) {
  __shared__ __attribute__((aligned(16))) char lds[core_rs_lds_bytes(NT)];
  core_phase_rs<NT>(p, blockIdx.x, lds);
}

// more heads (128 per workgroup, eight waves): one head tile per wave (core_mfma.h)
template <int NT>
__global__ __launch_bounds__(512) void k_core_wide(StepParams p) {
  __shared__ __attribute__((aligned(16))) char lds[core_wide_lds_bytes(NT)];
  core_phase_wide<NT>(p, blockIdx.x, lds);
}

// single-launch variant: the whole step as one launch (single_launch.h)
template <int NTT, int NT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_step(StepParams p) {
  __shared__ __attribute__((aligned(16))) char lds[single_lds_bytes<NTT, NT>()];
  step_single<NTT, NT>(p, blockIdx.x, lds);
}

// fused variant: kv rows, absorption and core in one launch (phase_absorb_core);
// the producers reuse the core's LDS
template <int NT>
__global__ __launch_bounds__(kBlock) void k_absorb_core(StepParams p) {
  constexpr int kBytes = core_lds_bytes(NT, 1, 4) > kGemvLdsFloats * (int)sizeof(float)
                             ? core_lds_bytes(NT, 1, 4)
                             : kGemvLdsFloats * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) char lds[kBytes];
  phase_absorb_core<NT, 1, 4>(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(kBlock) void k_oabsorb(StepParams p) {
  extern __shared__ float lds[];
  phase_oabsorb(p, blockIdx.x, lds);
}

// o-projection slabs; the last slab of each column tile to arrive writes the
// tile's output (oproj_fold_out)
template <int NTT>
__global__ __launch_bounds__(kBlock) void k_oproj(StepParams p) {
  extern __shared__ float lds[];
  phase_oproj<NTT>(p, blockIdx.x, lds, HandoffDevStores());
  oproj_fold_out(p, blockIdx.x % p.pl.nt6, lds);
}

__global__ __launch_bounds__(kBlock) void k_out(StepParams p) {
  extern __shared__ float lds[];
  phase_out(p, blockIdx.x, lds);
}

// matrix-core path (phases_mfma.h)

__global__ __launch_bounds__(kBlock) void k_prep(StepParams p) {
  extern __shared__ float lds[];
  phase_prep(p, blockIdx.x, lds);
}

template <int MTB>
__global__ __launch_bounds__(64 * mg_waves(MTB)) void k_down_m(StepParams p) {
  __shared__ __attribute__((aligned(16))) char stage[Mg<MTB>::kStage];
  phase_down_m<MTB>(p, blockIdx.x, stage);
}

__global__ __launch_bounds__(kBlock) void k_qa(StepParams p) {
  extern __shared__ float lds[];
  phase_qa(p, blockIdx.x, lds);
}

template <int MTB>
__global__ __launch_bounds__(64 * mg_waves(MTB)) void k_qup_m(StepParams p) {
  __shared__ __attribute__((aligned(16))) char stage[Mg<MTB>::kStage];
  phase_qup_m<MTB>(p, blockIdx.x, stage);
}

template <int MTB, int NCA>
__global__ __launch_bounds__(kBlock) void k_absorb_m(StepParams p) {
  extern __shared__ float lds[];
  phase_absorb_m<MTB, NCA>(p, blockIdx.x, reinterpret_cast<char*>(lds));
}


template <int MTB, int Q5, bool PO16>
__global__ __launch_bounds__(kBlock) void k_oabsorb_m(StepParams p) {
  extern __shared__ float lds[];
  phase_oabsorb_m<MTB, Q5, PO16>(p, blockIdx.x, reinterpret_cast<char*>(lds));
}

template <int MTB>
__global__ __launch_bounds__(64 * mg_waves(MTB)) void k_oproj_m(StepParams p) {
  __shared__ __attribute__((aligned(16))) char stage[Mg<MTB, mg_cols(MTB), mg_waves(MTB), oproj_ah(MTB)>::kStage];
  phase_oproj_m<MTB>(p, blockIdx.x, stage);
}

__global__ __launch_bounds__(kBlock) void k_zero_u32(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (size_t)gridDim.x * kBlock) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct mla_gd_handle {
  mla_gd_dims d;
  int device;
  int last_hip_error;
  bool lds_ready;  // dynamic-LDS limits of the kernels raised on this device
  // With MLA_GD_FLAG_GRAPH: the step's launches captured once into a HIP graph
  // on a private stream (default priority) and replayed on the caller's
  // stream; captured again whenever any kernel argument differs.
  hipStream_t cap_stream;
  hipGraph_t graph;
  hipGraphExec_t exec;
  bool graph_broken;        // a graph call failed once: launch directly from then on
  unsigned char key[sizeof(mla::StepParams)];  // the captured kernel arguments
  // workspace_size: ws_most[t] = the largest plan total over steps of 1..t
  // tokens, filled on first use
  std::vector<size_t> ws_most;
  // MLA_GD_LOG set at create: each step size's plan is printed to stderr once
  bool log_plans;
  std::vector<bool> logged;
};

namespace {

inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

constexpr int kTargetWG = 384;  // workgroups per GEMV phase (1.5 per CU)

// split-K: about kTargetWG workgroups over `ntiles` column tiles, slabs of at
// most 512 rows (the LDS activation slab) and at least 16.
void choose_split(int K, int ntiles, int* s_out, int* ks_out) {
  int s = cdiv(kTargetWG, ntiles);
  s = clampi(s, cdiv(K, kTile), std::max(1, K / 16));
  int ks = cdiv(K, s);
  ks = std::min(kTile, (ks + 3) / 4 * 4);
  *ks_out = ks;
  *s_out = cdiv(K, ks);
}

struct CoreShape {
  int hg, cs;
};

// <= 16 heads: one head group, eight waves (four below a 512-wide latent)
// splitting the latent columns and the score k-steps; 17-64 heads: four head
// groups per workgroup, two waves per group; more: eight head groups, one
// wave each.  Eight waves against four for 16 heads at the 512-wide latent
// (cold kernel time): 7.3 against 8.4 us at one token, 23.0 against 23.4 at
// 32 tokens.
CoreShape core_shape(int n_heads, int R) {
  return n_heads <= 16 ? CoreShape{1, R >= 512 ? 8 : 4} : (n_heads <= 64 ? CoreShape{4, 2} : CoreShape{8, 1});
}

int core_grid(const Plan& pl) { return cdiv(pl.T * pl.nsplit, 8) * 8 * pl.core_nhb; }

// More tokens: projections on the matrix cores.  Cold steps of the
// DeepSeek-V3.2 dims (16 heads, n_prior 2048) took, GEMV path against
// matrix-core path: 2 tokens 65 / 83 us, 3 tokens 79 / 83, 4 tokens 89 / 84,
// 8 tokens 136 / 86.
constexpr int kGemvMaxTokens = 3;
static_assert(kGemvMaxTokens <= kTT, "one GEMV pass per step");

// Matrix-core split-K: about `target` workgroups over `units` (tile, token
// block) pairs, slabs of at least 8 k-steps.
void split_m(int kt, int units, int target, int* s_out, int* ks_out) {
  // at most `target` workgroups: one more would start a second round on some CU
  int s = target / units;
  s = clampi(s, 1, std::max(1, kt / 8));
  const int ks = cdiv(kt, s);
  *ks_out = ks;
  *s_out = cdiv(kt, ks);
}

int mg_grid(int nunits, int ntb) { return cdiv(nunits, 8) * 8 * ntb; }

size_t absorb_lds_bytes(const Plan& pl, int DN) {
  return (size_t)2 * kMgK * pl.nca3 * 2 + kAbsorbBetaBytes + (size_t)cdiv(DN, kMgK) * pl.mtb3 * 2 * kAFragElems * 2;
}

size_t oabsorb_lds_bytes(const Plan& pl, int R) {
  return oabsorb_hdr_bytes(pl.mtb5, pl.nsplit) + (size_t)(R / kMgK) * pl.mtb5 * 2 * kAFragElems * 2;
}

// Plan of the matrix-core path; `pl` already holds T, the index build and the core's split.
Plan make_plan_mfma(const mla_gd_dims& d, Plan pl) {
  const int H = d.hidden, Q = d.q_lora_rank, R = d.kv_lora_rank, DR = d.qk_rope_head_dim;
  const int KVR = R + DR, QKH = d.qk_nope_head_dim + DR, N2 = d.n_heads * QKH, NH = d.n_heads;
  const int P = d.n_prior, DV = d.v_head_dim, DN = d.qk_nope_head_dim;
  const int T = pl.T;
  pl.mfma = 1;
  pl.po16 = pl.core_rs ? 0 : 1;  // every core shape but the row-split one (17-64 heads)
  pl.mtb = T <= 16 ? 1 : (T <= 32 ? 2 : (T <= 64 ? 4 : 8));
  pl.ntb = cdiv(T, 16 * pl.mtb);
  pl.mt_pad = pl.ntb * pl.mtb;
  // about one workgroup per CU, for the 128-column tiles too: at 32 tokens
  // (cold steps) 256 workgroups against 512 took the down-projection from
  // 12.3 to 11.3 us, the q-latent reduction (half the slabs) from 7.4 to 6.4
  // and the o-projection from 11.7 to 10.7; 192 and 128 were slower again
  const int nc = mg_cols(pl.mtb);
  const int target = 256;
  pl.kt1 = cdiv(H, kMgK);
  pl.ntq1m = cdiv(Q, nc);
  pl.nt1m = pl.ntq1m + cdiv(KVR, nc);
  split_m(pl.kt1, pl.nt1m * pl.ntb, target, &pl.s1, &pl.ks1m);
  pl.kt2 = cdiv(Q, kMgK);
  pl.nt2m = cdiv(N2, nc);
  split_m(pl.kt2, pl.nt2m * pl.ntb, target, &pl.s2, &pl.ks2m);
  pl.mtb3 = std::min(pl.mtb, 4);  // 128-token blocks measured slower here
  while (pl.mtb3 > 1 && (size_t)cdiv(DN, kMgK) * pl.mtb3 * 2048 > 96 * 1024) pl.mtb3 /= 2;
  pl.ntb3 = cdiv(T, 16 * pl.mtb3);
  // 128-column absorption tiles (256-byte weight row segments) where the latent
  // width allows and the tiles still give two workgroups per CU; 64 otherwise
  pl.nca3 = (R % 128 == 0 && NH * pl.ntb3 * (R / 128) >= 256) ? 128 : 64;
  pl.nct3 = R / pl.nca3;
  // as many tiles per workgroup as keep at least 128 workgroups busy
  pl.tpw3 = pl.nct3;
  while (pl.tpw3 > 1 && NH * pl.ntb3 * (pl.nct3 / pl.tpw3) < 128) pl.tpw3 /= 2;
  // Many heads at a 512-wide latent: one tile of every column, so each weight
  // row is read whole (1 KB) instead of in 256-byte pieces, with the largest
  // token block that still gives one workgroup per CU.
  if (R == 512 && (size_t)cdiv(DN, kMgK) * 2048 <= 48 * 1024) {
    int m = std::min(pl.mtb, 4);
    while (m > 1 && NH * cdiv(T, 16 * m) < 256) m /= 2;
    if (NH * cdiv(T, 16 * m) >= 256 && (size_t)cdiv(DN, kMgK) * m * 2048 <= 48 * 1024) {
      pl.mtb3 = m;
      pl.ntb3 = cdiv(T, 16 * m);
      pl.nca3 = 512;
      pl.nct3 = 1;
      pl.tpw3 = 1;
    }
  }
  // two m-tiles per workgroup when many heads give enough workgroups: half the
  // weight re-reads across token blocks
  pl.mtb5 = (NH >= 64 && T > 64) ? 2 : 1;
  pl.ntb5 = cdiv(T, 16 * pl.mtb5);
  // few (head, token block) pairs: split each pair's output tiles over
  // workgroups of four tiles (one per wave), each combining the splits itself
  {
    const int ndt = cdiv(DV, 16);
    pl.nq5 = (NH * pl.ntb5 < 128 && ndt > 4) ? cdiv(ndt, 4) : 1;
    pl.q5 = pl.nq5 > 1 ? 1 : 2;
  }
  pl.nxc = cdiv(pl.kt1 * kMgK, kPrepChunk);
  pl.nqc = cdiv(Q, kQaChunk);
  pl.kt6 = cdiv(NH * DV, kMgK);
  pl.nt6m = cdiv(H, nc);
  split_m(pl.kt6, pl.nt6m * pl.ntb, target, &pl.s6, &pl.ks6m);
  pl.n7 = T * cdiv(H, kOutCols);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t f = sizeof(float);
  const size_t frag = 2 * kAFragElems * sizeof(uint16_t);  // one (k-step, m-tile): both halves
  pl.off_zero = take(256);
  pl.off_err = take(256);  // debug error word: the same offset for every n_tokens
  pl.off_flags = take((size_t)kFlagRegionWords * 4);  // the same offset and size in every plan
  pl.off_sync = take((size_t)(NH + 2) * 64);
  pl.off_rows = take((size_t)T * P * sizeof(int32_t));
  pl.off_a1 = take((size_t)pl.kt1 * pl.mt_pad * frag);
  pl.off_ssx = take((size_t)pl.nxc * T * f);
  pl.off_part1 = take((size_t)pl.s1 * T * (Q + KVR) * f);
  pl.off_ssq = take((size_t)pl.nqc * T * f);
  pl.off_a2 = take((size_t)pl.kt2 * pl.mt_pad * frag);
  pl.off_part2 = take((size_t)pl.s2 * T * N2 * f);
  pl.off_qcat = take((size_t)T * NH * KVR * sizeof(uint16_t));
  pl.off_pm = take((size_t)T * pl.nsplit * NH * f);
  pl.off_pl = take((size_t)T * pl.nsplit * NH * f);
  pl.off_po = take((size_t)T * pl.nsplit * NH * R * f);
  pl.off_a5 = take((size_t)pl.kt6 * pl.mt_pad * frag);
  pl.off_part6 = take((size_t)pl.s6 * T * H * f);
  pl.total = off;
  return pl;
}

// Rows of one batch of weight loads of a GEMV tile nc columns wide (the lane
// geometry of gemv_geom): a slab no longer than this streams in one round trip.
int gemv_batch_rows(int nc, int ntt) {
  int lpr = 64;
  while (lpr > 8 && (lpr >> 1) >= nc / 8) lpr >>= 1;
  return (kBlock / 64) * (64 / lpr) * gemv_unroll(ntt);
}

Plan make_plan(const mla_gd_dims& d, int T) {
  Plan pl;
  memset(&pl, 0, sizeof(pl));
  const int H = d.hidden, Q = d.q_lora_rank, R = d.kv_lora_rank, DR = d.qk_rope_head_dim;
  const int KVR = R + DR, QKH = d.qk_nope_head_dim + DR, N2 = d.n_heads * QKH, NH = d.n_heads;
  const int P = d.n_prior, DV = d.v_head_dim;
  pl.T = T;
  pl.tw1 = 128;
  pl.tw2 = 64;
  pl.tw6 = T == 1 ? 128 : 64;  // one token: 256-byte row segments of o_proj_w
  pl.nt_q = cdiv(Q, pl.tw1);
  pl.nt_kv = cdiv(KVR, pl.tw1);
  pl.nt1 = pl.nt_q + pl.nt_kv;
  choose_split(H, pl.nt1, &pl.s1, &pl.ks1);
  // one token: slabs of the down-projection no longer than one batch of loads
  // (a second batch would wait for the first one's products)
  if (T == 1 && pl.ks1 > gemv_batch_rows(pl.tw1, 1)) {
    pl.ks1 = gemv_batch_rows(pl.tw1, 1);
    pl.s1 = cdiv(H, pl.ks1);
  }
  pl.n_idx_wg = cdiv(T * P, kBlock);

  pl.nt2 = cdiv(N2, pl.tw2);
  choose_split(Q, pl.nt2, &pl.s2, &pl.ks2);
  pl.nkv = cdiv(KVR, 64);
  pl.ncc3 = R / 64;
  const CoreShape cs = core_shape(NH, R);
  pl.core_hg = cs.hg;
  pl.core_cs = cs.cs;
  pl.core_nhb = cdiv(NH, 16 * cs.hg);
  // more than 16 heads and a latent width of 128 or more: the row-split core
  // (the same 64 heads per workgroup in eight waves)
  pl.core_rs = (cs.hg == 4 && cs.cs == 2 && R % 128 == 0) ? 1 : 0;
  {
    // about one workgroup per CU.  The matrix-core path's combine kernel reads
    // every split for every column, so it keeps at most 16; the GEMV path's
    // output absorption reads each split once per column chunk.
    int ns = cdiv(256, T * pl.core_nhb);
    ns = std::min(ns, T > kGemvMaxTokens ? 16 : 64);
    ns = clampi(ns, cdiv(P, cs.hg == 8 ? kWideMaxSplitRows : kMaxSplitRows), cdiv(P, kCoreChunk));
    pl.ps = cdiv(cdiv(P, ns), kCoreChunk) * kCoreChunk;
    pl.nsplit = cdiv(P, pl.ps);
  }
  if (T > kGemvMaxTokens) return make_plan_mfma(d, pl);
  pl.fused = (d.flags & MLA_GD_FLAG_FUSED) && pl.core_hg == 1;
  pl.single = (d.flags & MLA_GD_FLAG_SINGLE_LAUNCH) && pl.core_hg == 1;
  if (pl.fused || pl.single) pl.core_cs = 4;  // their core runs in 256-thread workgroups
  if (pl.single) {
    // splits of at most kSingleMaxRows rows (the single launch's core stages fewer row ids)
    const int ns = std::max(pl.nsplit, cdiv(P, kSingleMaxRows));
    if (ns > 64) {
      pl.single = 0;
    } else {
      pl.ps = cdiv(cdiv(P, ns), kCoreChunk) * kCoreChunk;
      pl.nsplit = cdiv(P, pl.ps);
    }
  }
  pl.nc5 = R / kOabsCols;
  pl.tc5 = std::min(T, kTT);
  pl.nt5c = cdiv(T, pl.tc5);
  pl.nt6 = cdiv(H, pl.tw6);
  choose_split(NH * DV, pl.nt6, &pl.s6, &pl.ks6);
  if (T == 1 && pl.ks6 > gemv_batch_rows(pl.tw6, 1)) {  // as for the down-projection
    pl.ks6 = gemv_batch_rows(pl.tw6, 1);
    pl.s6 = cdiv(NH * DV, pl.ks6);
  }
  pl.n7 = 0;  // the output sum runs in the o-projection's last-arriving slabs
  pl.fold_out = 1;
  if (pl.single) {
    pl.i_down = pl.n_idx_wg;
    pl.i_qup = pl.i_down + pl.nt1 * pl.s1;
    pl.i_abs = pl.i_qup + pl.nt2 * pl.s2 + T * pl.nkv;
    pl.i_core = pl.i_abs + NH * pl.ncc3 + T;
    pl.i_oabs = pl.i_core + core_grid(pl);
    pl.i_oproj = pl.i_oabs + NH * pl.nc5 * pl.nt5c;
    pl.i_out = pl.i_oproj + pl.nt6 * pl.s6;
    pl.n_items = pl.i_out;
    if (pl.n_items > kSingleMaxItems) pl.single = 0;  // then the separate kernels (same split)
  }

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t f = sizeof(float);
  pl.off_zero = take(256);
  pl.off_err = take(256);  // debug error word: the same offset for every n_tokens
  pl.off_flags = take((size_t)kFlagRegionWords * 4);  // the same offset and size in every plan
  pl.off_sync = take((size_t)(NH + 2) * 64);
  pl.off_rows = take((size_t)T * P * sizeof(int32_t));
  pl.off_part1 = take((size_t)pl.s1 * T * (Q + KVR) * f);
  pl.off_ssx = take((size_t)pl.s1 * T * f);
  pl.off_part2 = take((size_t)pl.s2 * T * N2 * f);
  pl.off_ssq = take((size_t)pl.s2 * T * f);
  pl.off_kvr = take((size_t)T * KVR * f);
  pl.off_kvss = take((size_t)T * pl.nkv * f);
  pl.off_qcat = take((size_t)T * NH * KVR * sizeof(uint16_t));
  pl.off_pm = take((size_t)T * pl.nsplit * NH * f);
  pl.off_pl = take((size_t)T * pl.nsplit * NH * f);
  pl.off_po = take((size_t)T * pl.nsplit * NH * R * f);
  pl.off_ov = take((size_t)pl.nc5 * T * NH * DV * f);
  pl.off_part6 = take((size_t)pl.s6 * T * H * f);
  pl.off_tcnt = take((size_t)pl.nt6 * kSyncStride * 4);
  pl.total = off;
  return pl;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int validate_dims(const mla_gd_dims& d) {
  if (d.hidden <= 0 || d.q_lora_rank <= 0 || d.kv_lora_rank <= 0 || d.qk_nope_head_dim <= 0 ||
      d.qk_rope_head_dim <= 0 || d.v_head_dim <= 0 || d.n_heads <= 0 || d.block_size <= 0 ||
      d.max_blocks_per_seq <= 0 || d.n_blocks <= 0 || d.n_prior <= 0 || d.max_tokens <= 0)
    return MLA_GD_E_INVAL;
  if (d.qk_rope_head_dim % 2 != 0) return MLA_GD_E_INVAL;
  if ((d.flags & ~(MLA_GD_FLAG_FUSED | MLA_GD_FLAG_GRAPH | MLA_GD_FLAG_DEBUG_CHECKS | MLA_GD_FLAG_SINGLE_LAUNCH)) != 0u)
    return MLA_GD_E_INVAL;
  if ((d.flags & MLA_GD_FLAG_FUSED) && (d.flags & MLA_GD_FLAG_SINGLE_LAUNCH)) return MLA_GD_E_INVAL;
  if (!isfinite(d.softmax_scale) || !isfinite(d.norm_eps) || d.norm_eps < 0.f) return MLA_GD_E_INVAL;
  const long long KVR = (long long)d.kv_lora_rank + d.qk_rope_head_dim;
  const long long N2 = (long long)d.n_heads * (d.qk_nope_head_dim + d.qk_rope_head_dim);
  if (d.hidden % 8 || d.q_lora_rank % 8 || KVR % 8 || N2 % 8 || d.qk_nope_head_dim % 8) return MLA_GD_E_UNSUPPORTED;
  if ((d.qk_nope_head_dim + d.qk_rope_head_dim) % 4) return MLA_GD_E_UNSUPPORTED;
  const int r = d.kv_lora_rank;
  if (r != 64 && r != 128 && r != 256 && r != 512) return MLA_GD_E_UNSUPPORTED;
  if (d.qk_rope_head_dim > 64 || d.qk_nope_head_dim > 512 || d.v_head_dim > 4096) return MLA_GD_E_UNSUPPORTED;
  if (d.max_tokens > 4096) return MLA_GD_E_UNSUPPORTED;
  // one token's down-projection row is reduced in LDS; the core's split partials fit its combine
  if ((long long)d.q_lora_rank + KVR > 16384) return MLA_GD_E_UNSUPPORTED;
  if (d.n_prior > 64 * kMaxSplitRows) return MLA_GD_E_UNSUPPORTED;
  // more than 64 heads: the core stages fewer row ids per split (at most 64 splits)
  if (d.n_heads > 64 && d.n_prior > 64 * kWideMaxSplitRows) return MLA_GD_E_UNSUPPORTED;
  // flat cache rows and element offsets must fit the kernels' index arithmetic
  if ((long long)d.n_blocks * d.block_size > (1LL << 31) - 1) return MLA_GD_E_UNSUPPORTED;
  if ((long long)d.max_tokens * d.n_prior > (1LL << 31) - 1) return MLA_GD_E_UNSUPPORTED;
  return MLA_GD_OK;
}

typedef void (*core_kernel_t)(StepParams);

template <int HG, int CS>
core_kernel_t pick_core_nt(int nt) {
  switch (nt) {
    case 4: return k_core<4, HG, CS>;
    case 8: return k_core<8, HG, CS>;
    case 16: return k_core<16, HG, CS>;
    default: return k_core<32, HG, CS>;
  }
}

core_kernel_t pick_fused(int R) {
  switch (R / 16) {
    case 4: return k_absorb_core<4>;
    case 8: return k_absorb_core<8>;
    case 16: return k_absorb_core<16>;
    default: return k_absorb_core<32>;
  }
}

template <int NTT>
core_kernel_t pick_step_nt(int R) {
  switch (R / 16) {
    case 4: return k_step<NTT, 4>;
    case 8: return k_step<NTT, 8>;
    case 16: return k_step<NTT, 16>;
    default: return k_step<NTT, 32>;
  }
}

core_kernel_t pick_step(int ntt, int R) {
  switch (ntt) {
    case 1: return pick_step_nt<1>(R);
    case 2: return pick_step_nt<2>(R);
    default: return pick_step_nt<4>(R);
  }
}

core_kernel_t pick_core(const Plan& pl, int R) {
  if (pl.core_hg == 8) {
    switch (R / 16) {
      case 4: return k_core_wide<4>;
      case 8: return k_core_wide<8>;
      case 16: return k_core_wide<16>;
      default: return k_core_wide<32>;
    }
  }
  if (pl.core_rs) {
    switch (R / 16) {
      case 8: return k_core_rs<8>;
      case 16: return k_core_rs<16>;
      default: return k_core_rs<32>;
    }
  }
  if (pl.core_hg == 1) return pl.core_cs == 8 ? k_core<32, 1, 8> : pick_core_nt<1, 4>(R / 16);
  return pick_core_nt<4, 2>(R / 16);
}

// Kernels of a step, in launch order: the GEMV path (few tokens) and the matrix-core path.
const char* const kKernelNamesGemv[] = {"k_down", "k_qup", "k_absorb", "k_core", "k_oabsorb", "k_oproj"};
const char* const kKernelNamesFused[] = {"k_down", "k_qup", "k_absorb_core", "k_oabsorb", "k_oproj"};
const char* const kKernelNamesMfma[] = {"k_prep", "k_down",    "k_qa",    "k_qup", "k_absorb",
                                        "k_core", "k_oabsorb", "k_oproj", "k_out"};
constexpr int kNumKernelsGemv = 6;
constexpr int kNumKernelsMfma = 9;
constexpr size_t kGemvLdsBytes = kGemvLdsFloats * sizeof(float);
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr size_t kErrOffset = 256;  // Plan::off_err in every plan (right after the zero bytes)
constexpr size_t kFlagsOffset = 512;  // Plan::off_flags in every plan (right after the error word)

int num_kernels(const Plan& pl) {
  if (pl.single) return 1;
  if (pl.fused) return kNumKernelsGemv - 1;
  if (!pl.mfma) return kNumKernelsGemv;
  return kNumKernelsMfma;
}

const char* kernel_name(const Plan& pl, int i) {
  if (pl.single) return "k_step";
  if (pl.fused) return kKernelNamesFused[i];
  if (!pl.mfma) return kKernelNamesGemv[i];
  return kKernelNamesMfma[i];
}

hipError_t set_lds_limits(const mla_gd_dims& d) {
  hipError_t e = hipSuccess;
  const void* gemv[] = {(const void*)k_down<4>, (const void*)k_qup<4>,
                        (const void*)k_absorb<4>, (const void*)k_oproj<4>, (const void*)k_oabsorb,
                        (const void*)k_out, (const void*)k_prep, (const void*)k_qa};
  for (const void* k : gemv)
    if (e == hipSuccess) e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemvLdsBytes);
  const void* big[] = {(const void*)k_absorb_m<1, 64>, (const void*)k_absorb_m<2, 64>, (const void*)k_absorb_m<4, 64>,
                       (const void*)k_absorb_m<1, 128>, (const void*)k_absorb_m<2, 128>, (const void*)k_absorb_m<4, 128>,
                       (const void*)k_absorb_m<1, 512>, (const void*)k_absorb_m<2, 512>, (const void*)k_absorb_m<4, 512>,
                       (const void*)k_oabsorb_m<1, 1, false>, (const void*)k_oabsorb_m<2, 1, false>,
                       (const void*)k_oabsorb_m<1, 2, false>, (const void*)k_oabsorb_m<2, 2, false>,
                       (const void*)k_oabsorb_m<1, 1, true>, (const void*)k_oabsorb_m<2, 1, true>,
                       (const void*)k_oabsorb_m<1, 2, true>, (const void*)k_oabsorb_m<2, 2, true>};
  for (const void* k : big)
    if (e == hipSuccess) e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
  if (e == hipSuccess) e = fixed_shape_init();
  return e;
}

typedef void (*step_kernel_t)(StepParams);

// GEMV-path kernels for NTT tokens per pass, and their dynamic LDS
#define MLA_GD_NTT_PICK(fn, K) \
  step_kernel_t fn(int ntt) { return ntt == 1 ? K<1> : (ntt == 2 ? K<2> : K<4>); }
MLA_GD_NTT_PICK(pick_down, k_down)
MLA_GD_NTT_PICK(pick_qup, k_qup)
MLA_GD_NTT_PICK(pick_absorb, k_absorb)
MLA_GD_NTT_PICK(pick_oproj, k_oproj)
#undef MLA_GD_NTT_PICK

size_t gemv_lds_bytes(int ntt) {
  switch (ntt) {
    case 1: return GemvLds<1>::floats * sizeof(float);
    case 2: return GemvLds<2>::floats * sizeof(float);
    default: return GemvLds<4>::floats * sizeof(float);
  }
}

int gemv_ntt(int T) { return T <= 1 ? 1 : (T <= 2 ? 2 : 4); }

step_kernel_t pick_down_m(int mtb) {
  return mtb == 1 ? k_down_m<1> : (mtb == 2 ? k_down_m<2> : (mtb == 4 ? k_down_m<4> : k_down_m<8>));
}
step_kernel_t pick_qup_m(int mtb) {
  return mtb == 1 ? k_qup_m<1> : (mtb == 2 ? k_qup_m<2> : (mtb == 4 ? k_qup_m<4> : k_qup_m<8>));
}
step_kernel_t pick_oproj_m(int mtb) {
  return mtb == 1 ? k_oproj_m<1> : (mtb == 2 ? k_oproj_m<2> : (mtb == 4 ? k_oproj_m<4> : k_oproj_m<8>));
}
step_kernel_t pick_absorb_m(int mtb, int nca) {
  if (nca == 512) return mtb == 1 ? k_absorb_m<1, 512> : (mtb == 2 ? k_absorb_m<2, 512> : k_absorb_m<4, 512>);
  if (nca == 128) return mtb == 1 ? k_absorb_m<1, 128> : (mtb == 2 ? k_absorb_m<2, 128> : k_absorb_m<4, 128>);
  return mtb == 1 ? k_absorb_m<1, 64> : (mtb == 2 ? k_absorb_m<2, 64> : k_absorb_m<4, 64>);
}
template <bool PO16>
step_kernel_t pick_oabsorb_m_t(int mtb, int q5) {
  if (q5 == 1) return mtb == 2 ? k_oabsorb_m<2, 1, PO16> : k_oabsorb_m<1, 1, PO16>;
  return mtb == 2 ? k_oabsorb_m<2, 2, PO16> : k_oabsorb_m<1, 2, PO16>;
}

step_kernel_t pick_oabsorb_m(const Plan& pl) {
  return pl.po16 ? pick_oabsorb_m_t<true>(pl.mtb5, pl.q5) : pick_oabsorb_m_t<false>(pl.mtb5, pl.q5);
}

}  // namespace

extern "C" {

int mla_gather_decode_abi_version(void) { return MLA_GD_ABI_VERSION; }

const char* mla_gather_decode_strerror(int code) {
  switch (code) {
    case MLA_GD_OK: return "ok";
    case MLA_GD_E_INVAL: return "invalid argument";
    case MLA_GD_E_ALIGN: return "misaligned pointer";
    case MLA_GD_E_WORKSPACE: return "workspace too small";
    case MLA_GD_E_UNSUPPORTED: return "unsupported dimensions";
    case MLA_GD_E_HIP: return "HIP runtime error";
    case MLA_GD_E_DEVICE_CHECK: return "device check failed (invalid index data in an earlier step)";
    default: return "unknown error";
  }
}

int mla_gather_decode_create(const mla_gd_dims* dims, int device, mla_gd_handle** out_handle) {
  if (!dims || !out_handle) return MLA_GD_E_INVAL;
  *out_handle = nullptr;
  const int rc = validate_dims(*dims);
  if (rc != MLA_GD_OK) return rc;
  if (device < 0) return MLA_GD_E_INVAL;
  mla_gd_handle* h = new (std::nothrow) mla_gd_handle;
  if (!h) return MLA_GD_E_INVAL;
  h->d = *dims;
  h->device = device;
  h->last_hip_error = 0;
  h->lds_ready = false;
  h->cap_stream = nullptr;
  h->graph = nullptr;
  h->exec = nullptr;
  h->graph_broken = false;
  memset(h->key, 0, sizeof(h->key));
  const char* lg = getenv("MLA_GD_LOG");
  h->log_plans = lg && *lg && strcmp(lg, "0") != 0;
  *out_handle = h;
  return MLA_GD_OK;
}

void mla_gather_decode_destroy(mla_gd_handle* handle) {
  if (!handle) return;
  if (handle->exec || handle->graph || handle->cap_stream) {
    int cur = -1;
    const bool restore = hipGetDevice(&cur) == hipSuccess && cur != handle->device;
    if (hipSetDevice(handle->device) == hipSuccess) {
      if (handle->exec) (void)hipGraphExecDestroy(handle->exec);
      if (handle->graph) (void)hipGraphDestroy(handle->graph);
      if (handle->cap_stream) (void)hipStreamDestroy(handle->cap_stream);
    }
    if (restore) (void)hipSetDevice(cur);
  }
  delete handle;
}

int mla_gather_decode_last_hip_error(const mla_gd_handle* handle) { return handle ? handle->last_hip_error : 0; }

size_t mla_gather_decode_workspace_size(const mla_gd_handle* handle, int32_t n_tokens) {
  if (!handle || n_tokens < 1 || n_tokens > handle->d.max_tokens) return 0;
  mla_gd_handle* h = const_cast<mla_gd_handle*>(handle);
  if (h->ws_most.empty()) {  // one plan per step size, once per handle
    std::vector<size_t> most((size_t)h->d.max_tokens + 1, 0);
    for (int t = 1; t <= h->d.max_tokens; ++t) most[t] = std::max(most[t - 1], make_plan(h->d, t).total);
    h->ws_most.swap(most);
  }
  return h->ws_most[n_tokens];
}

int mla_gather_decode_workspace_init(const mla_gd_handle* handle, void* workspace, size_t bytes, void* stream) {
  if (!handle || !workspace) return MLA_GD_E_INVAL;
  if (!aligned(workspace, 16) || bytes % 4) return MLA_GD_E_ALIGN;
  mla_gd_handle* h = const_cast<mla_gd_handle*>(handle);
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) { h->last_hip_error = (int)e; return MLA_GD_E_HIP; }
  const size_t n = bytes / 4;
  if (n == 0) return MLA_GD_OK;
  const int grid = (int)std::min<size_t>(2048, (n + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(k_zero_u32, dim3(grid), dim3(kBlock), 0, (hipStream_t)stream, (uint32_t*)workspace, n);
  e = hipGetLastError();
  if (e != hipSuccess) { h->last_hip_error = (int)e; return MLA_GD_E_HIP; }
  return MLA_GD_OK;
}

}  // extern "C"

namespace {

// Enqueue the step's kernels on stream s; with `events`, record events[i]
// before kernel i and after the last one.
// Launches the kernels of a step one by one.  A profiled step either records
// events[i] before kernel i and events[count] after the last (bracket false),
// or hands events[2i] and events[2i+1] to kernel i's launch, which stamps the
// kernel's own start and end (bracket true: the intervals exclude the
// dispatch gaps between kernels).
struct Launcher {
  const StepParams* p;
  hipStream_t s;
  void* const* events;
  bool bracket;
  hipError_t e = hipSuccess;
  int i = 0;
  void operator()(step_kernel_t k, dim3 grid, dim3 block, size_t lds) {
    if (e != hipSuccess) return;
    void* args[] = {const_cast<StepParams*>(p)};
    if (events && bracket) {
      e = hipExtLaunchKernel((const void*)k, grid, block, args, lds, s, (hipEvent_t)events[2 * i],
                             (hipEvent_t)events[2 * i + 1], 0);
    } else {
      if (events) e = hipEventRecord((hipEvent_t)events[i], s);
      if (e == hipSuccess) e = hipLaunchKernel((const void*)k, grid, block, args, lds, s);
    }
    ++i;
  }
  hipError_t finish() {
    if (e == hipSuccess && events && !bracket) e = hipEventRecord((hipEvent_t)events[i], s);
    return e;
  }
};

hipError_t launch_kernels(const StepParams& p, hipStream_t s, void* const* events, bool bracket = false) {
  const Plan& pl = p.pl;
  const int T = pl.T;
  Launcher L{&p, s, events, bracket};
  const size_t gl = kGemvLdsBytes;
  const int ntt = gemv_ntt(T);
  const size_t gll = gemv_lds_bytes(ntt);  // GEMV phases passing over ntt tokens
  const dim3 blk(kBlock);
  const dim3 core_blk(64 * pl.core_hg * pl.core_cs);
  if (pl.single) {
    L(pick_step(ntt, p.R), dim3(pl.n_items), blk, 0);
  } else if (pl.fused) {
    L(pick_down(ntt), dim3(pl.nt1 * pl.s1 + pl.n_idx_wg), blk, gll);
    L(pick_qup(ntt), dim3(pl.nt2 * pl.s2 + T * pl.nkv), blk, gll);
    L(pick_fused(p.R), dim3(T + p.NH * pl.ncc3 + core_grid(pl)), blk, 0);
    L(k_oabsorb, dim3(p.NH * pl.nc5 * pl.nt5c), blk, gl);
    L(pick_oproj(ntt), dim3(pl.nt6 * pl.s6), blk, gll);
  } else if (!pl.mfma) {
    // the DeepSeek-V3.2 one-token shape runs the same phases compiled with
    // its sizes as constants (fixed_shape.h), the same grids and LDS
    const bool fx = fixed_shape_applies(p);
    const FixedShapeKernels& F = fixed_shape_kernels();
    L(fx ? F.down : pick_down(ntt), dim3(pl.nt1 * pl.s1 + pl.n_idx_wg), blk, gll);
    L(fx ? F.qup : pick_qup(ntt), dim3(pl.nt2 * pl.s2 + T * pl.nkv), blk, gll);
    L(fx ? F.absorb : pick_absorb(ntt), dim3(p.NH * pl.ncc3 + T), blk, gll);
    L(fx ? F.core : pick_core(pl, p.R), dim3(core_grid(pl)), core_blk, 0);
    L(fx ? F.oabsorb : k_oabsorb, dim3(p.NH * pl.nc5 * pl.nt5c), blk, gl);
    L(fx ? F.oproj : pick_oproj(ntt), dim3(pl.nt6 * pl.s6), blk, gll);
  } else {
    L(k_prep, dim3(pl.n_idx_wg + T * pl.nxc), blk, 1024);
    const dim3 gblk(64 * mg_waves(pl.mtb));  // GEMM workgroups: eight waves for 128-token blocks
    L(pick_down_m(pl.mtb), dim3(mg_grid(pl.nt1m * pl.s1, pl.ntb)), gblk, 0);
    L(k_qa, dim3(T * (pl.nqc + 1)), blk, gl);
    L(pick_qup_m(pl.mtb), dim3(mg_grid(pl.nt2m * pl.s2, pl.ntb)), gblk, 0);
    L(pick_absorb_m(pl.mtb3, pl.nca3), dim3(mg_grid(p.NH * (pl.nct3 / pl.tpw3), pl.ntb3)), blk, absorb_lds_bytes(pl, p.DN));
    L(pick_core(pl, p.R), dim3(core_grid(pl)), core_blk, 0);
    L(pick_oabsorb_m(pl), dim3(mg_grid(p.NH * pl.nq5, pl.ntb5)), blk, oabsorb_lds_bytes(pl, p.R));
    L(pick_oproj_m(pl.mtb), dim3(mg_grid(pl.nt6m * pl.s6, pl.ntb)), gblk, 0);
    L(k_out, dim3(pl.n7), blk, gl);
  }
  hipError_t e = L.finish();
  if (e == hipSuccess) e = hipGetLastError();
  return e;
}

// Replay the captured graph of these kernel arguments on stream s, capturing
// it first when the arguments differ from the last capture.
hipError_t launch_graph(mla_gd_handle* h, const StepParams& p, hipStream_t s) {
  static_assert(sizeof(h->key) == sizeof(StepParams), "graph key");
  if (!h->exec || memcmp(h->key, &p, sizeof(p)) != 0) {
    hipError_t e = hipSuccess;
    if (!h->cap_stream) e = hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking);
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (e == hipSuccess) e = hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeRelaxed);
    if (e == hipSuccess) {
      const hipError_t el = launch_kernels(p, h->cap_stream, nullptr);
      e = hipStreamEndCapture(h->cap_stream, &graph);
      if (e == hipSuccess) e = el;
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      (void)hipGetLastError();
      return e;
    }
    if (h->exec) (void)hipGraphExecDestroy(h->exec);
    if (h->graph) (void)hipGraphDestroy(h->graph);
    h->exec = exec;
    h->graph = graph;
    memcpy(h->key, &p, sizeof(p));
  }
  return hipGraphLaunch(h->exec, s);
}

// Debug checks: wait for the work on `stream`, read the workspace's error
// word into *bits and clear it (with a fill kernel, so the call stays free of
// memset nodes).
int read_clear_err(mla_gd_handle* h, void* workspace, hipStream_t s, uint32_t* bits) {
  unsigned* err = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + kErrOffset);
  uint32_t w = 0;
  hipError_t e = hipSetDevice(h->device);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (e == hipSuccess) e = hipStreamIsCapturing(s, &cap);
  if (e == hipSuccess && cap != hipStreamCaptureStatusNone) return MLA_GD_E_INVAL;  // a read-back cannot be captured
  if (e == hipSuccess) e = hipMemcpyAsync(&w, err, sizeof(w), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && w != 0u) {
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(kBlock), 0, s, err, (size_t)1);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    h->last_hip_error = (int)e;
    return MLA_GD_E_HIP;
  }
  *bits = w;
  return w ? MLA_GD_E_DEVICE_CHECK : MLA_GD_OK;
}

// MLA_GD_LOG: the work decomposition of a step size, once per handle and size.
void log_plan(mla_gd_handle* h, const Plan& pl) {
  if (h->logged.size() != (size_t)h->d.max_tokens + 1) h->logged.assign((size_t)h->d.max_tokens + 1, false);
  if (h->logged[pl.T]) return;
  h->logged[pl.T] = true;
  const char* core = pl.core_hg == 8 ? "one 16-head tile per wave, 128 heads per workgroup"
                                     : (pl.core_rs ? "row-split, 64 heads per workgroup"
                                                   : (pl.core_hg == 1 ? "16 heads, 4 waves" : "64 heads, 8 waves"));
  fprintf(stderr, "[mla_gd] T=%d: %s path%s%s; core: %s, %d split(s) of %d rows x %d head block(s) = %d workgroups, "
                  "%s split partials; workspace %zu bytes\n",
          pl.T, pl.mfma ? "matrix-core" : "GEMV", pl.single ? ", single launch" : "", pl.fused ? ", fused" : "", core,
          pl.nsplit, pl.ps, pl.core_nhb, core_grid(pl), pl.po16 ? "fp16 o/l" : "fp32", pl.total);
  if (pl.mfma)
    fprintf(stderr, "[mla_gd]   token blocks of %d x 16 (%d); down %d slabs x %d k-steps; up %d slabs x %d; "
                    "absorption %d-column tiles, %d per workgroup, blocks of %d x 16; output absorption blocks of %d x 16, "
                    "%d part(s); o-projection %d slabs x %d\n",
            pl.mtb, pl.ntb, pl.s1, pl.ks1m, pl.s2, pl.ks2m, pl.nca3, pl.tpw3, pl.mtb3, pl.mtb5, pl.nq5, pl.s6, pl.ks6m);
  else
    fprintf(stderr, "[mla_gd]   down %d tiles x %d slabs of %d rows; up %d tiles x %d slabs of %d rows; "
                    "o-projection %d tiles x %d slabs of %d rows\n",
            pl.nt1, pl.s1, pl.ks1, pl.nt2, pl.s2, pl.ks2, pl.nt6, pl.s6, pl.ks6);
}

int run_step(mla_gd_handle* h, const mla_gd_tensors* tn, int32_t n_tokens, void* workspace,
             size_t workspace_bytes, void* stream, void* const* events, int n_events, bool force_direct = false) {
  if (!h || !tn || !workspace) return MLA_GD_E_INVAL;
  const mla_gd_dims& d = h->d;
  if (n_tokens < 1 || n_tokens > d.max_tokens) return MLA_GD_E_INVAL;
  const Plan pl = make_plan(d, n_tokens);
  const int nk = num_kernels(pl);
  if (events && n_events < nk + 1) return MLA_GD_E_INVAL;
  const bool bracket = events && n_events >= 2 * nk;  // a start and an end event per kernel
  if (events)
    for (int i = 0; i < (bracket ? 2 * nk : nk + 1); ++i)
      if (!events[i]) return MLA_GD_E_INVAL;
  const void* bf[] = {tn->hidden_states, tn->wq_a, tn->wq_b, tn->wkv_a, tn->q_absorb_w, tn->out_absorb_w,
                      tn->o_proj_w, tn->kv_cache, tn->out};
  const void* w4[] = {tn->input_norm_w, tn->q_norm_w, tn->kv_norm_w, tn->cos_table, tn->sin_table,
                      tn->slot_mapping, tn->block_table, tn->positions, tn->gather_indices};
  for (const void* q : bf) if (!q) return MLA_GD_E_INVAL;
  for (const void* q : w4) if (!q) return MLA_GD_E_INVAL;
  for (const void* q : bf) if (!aligned(q, 16)) return MLA_GD_E_ALIGN;
  for (const void* q : w4) if (!aligned(q, 4)) return MLA_GD_E_ALIGN;
  if (tn->gather_rows_out && !aligned(tn->gather_rows_out, 4)) return MLA_GD_E_ALIGN;
  if (tn->token_seq && !aligned(tn->token_seq, 4)) return MLA_GD_E_ALIGN;
  if (!aligned(workspace, 256)) return MLA_GD_E_ALIGN;

  if (h->log_plans) log_plan(h, pl);
  if (pl.off_err != kErrOffset || pl.off_flags != kFlagsOffset) return MLA_GD_E_INVAL;  // layout invariant
  if (workspace_bytes < pl.total) return MLA_GD_E_WORKSPACE;
  if (d.flags & MLA_GD_FLAG_DEBUG_CHECKS) {
    uint32_t bits = 0;
    const int rc = read_clear_err(h, workspace, (hipStream_t)stream, &bits);
    if (rc != MLA_GD_OK) return rc;
  }

  StepParams p;
  memset(&p, 0, sizeof(p));
  p.H = d.hidden; p.Q = d.q_lora_rank; p.R = d.kv_lora_rank; p.DN = d.qk_nope_head_dim;
  p.DR = d.qk_rope_head_dim; p.DV = d.v_head_dim; p.NH = d.n_heads; p.BS = d.block_size;
  p.MB = d.max_blocks_per_seq; p.P = d.n_prior; p.KVR = p.R + p.DR; p.QKH = p.DN + p.DR;
  p.N2 = p.NH * p.QKH;
  p.NBLK = d.n_blocks;
  p.dbg = (d.flags & MLA_GD_FLAG_DEBUG_CHECKS) ? 1 : 0;
  p.scale_log2 = d.softmax_scale * 1.4426950408889634f;
  p.eps = d.norm_eps;
  p.x = (const uint16_t*)tn->hidden_states; p.g_in = tn->input_norm_w; p.wq_a = (const uint16_t*)tn->wq_a;
  p.g_q = tn->q_norm_w; p.wq_b = (const uint16_t*)tn->wq_b; p.wkv_a = (const uint16_t*)tn->wkv_a;
  p.g_kv = tn->kv_norm_w; p.w_qabs = (const uint16_t*)tn->q_absorb_w; p.w_oabs = (const uint16_t*)tn->out_absorb_w;
  p.w_o = (const uint16_t*)tn->o_proj_w; p.cos_t = tn->cos_table; p.sin_t = tn->sin_table;
  p.cache = (uint16_t*)tn->kv_cache; p.slot = tn->slot_mapping; p.btab = tn->block_table; p.pos = tn->positions;
  p.gidx = tn->gather_indices; p.out = (uint16_t*)tn->out; p.rows_out = tn->gather_rows_out;
  p.tseq = tn->token_seq;
  char* ws = (char*)workspace;
  p.zero16 = (const uint16_t*)(ws + pl.off_zero);
  p.rows = (int32_t*)(ws + pl.off_rows);
  p.part1 = (float*)(ws + pl.off_part1); p.ssx = (float*)(ws + pl.off_ssx);
  p.part2 = (float*)(ws + pl.off_part2); p.ssq = (float*)(ws + pl.off_ssq);
  p.kvr = (float*)(ws + pl.off_kvr); p.kvss = (float*)(ws + pl.off_kvss);
  p.qcat = (uint16_t*)(ws + pl.off_qcat);
  p.pm = (float*)(ws + pl.off_pm); p.pden = (float*)(ws + pl.off_pl); p.po = (float*)(ws + pl.off_po);
  p.ov = (float*)(ws + pl.off_ov); p.part6 = (float*)(ws + pl.off_part6);
  if (pl.mfma) {
    p.kvr = nullptr; p.kvss = nullptr; p.ov = nullptr;
    p.a1 = (uint16_t*)(ws + pl.off_a1); p.a2 = (uint16_t*)(ws + pl.off_a2); p.a5 = (uint16_t*)(ws + pl.off_a5);
    p.ssq = (float*)(ws + pl.off_ssq);
  }
  p.sync = (unsigned*)(ws + pl.off_sync);
  p.err = (unsigned*)(ws + pl.off_err);
  p.epoch = (unsigned*)(ws + pl.off_flags);
  p.flags = p.epoch + kFlagHeaderWords;
  p.tcnt = pl.fold_out ? (unsigned*)(ws + pl.off_tcnt) : nullptr;
  p.pl = pl;

  hipError_t e = hipSetDevice(h->device);
  if (e == hipSuccess && !h->lds_ready) {
    e = set_lds_limits(d);
    h->lds_ready = (e == hipSuccess);
  }
  if (e != hipSuccess) { h->last_hip_error = (int)e; return MLA_GD_E_HIP; }
  hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (e == hipSuccess) e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) { h->last_hip_error = (int)e; return MLA_GD_E_HIP; }
  // replay the captured graph only when asked for, and never for the
  // profiled step or inside the caller's own capture
  const bool direct = force_direct || events || cap != hipStreamCaptureStatusNone ||
                      !(d.flags & MLA_GD_FLAG_GRAPH) || h->graph_broken;
  if (!direct) {
    e = launch_graph(h, p, s);
    if (e != hipSuccess) {
      h->graph_broken = true;  // fall back to direct launches for this handle
      h->last_hip_error = (int)e;
      e = launch_kernels(p, s, nullptr);
    }
  } else {
    e = launch_kernels(p, s, events, bracket);
  }
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) { h->last_hip_error = (int)e; return MLA_GD_E_HIP; }
  return MLA_GD_OK;
}

}  // namespace

extern "C" {

int mla_gather_decode_step(mla_gd_handle* h, const mla_gd_tensors* tn, int32_t n_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run_step(h, tn, n_tokens, workspace, workspace_bytes, stream, nullptr, 0);
}

int mla_gather_decode_debug_status(const mla_gd_handle* handle, void* workspace, uint32_t* bits, void* stream) {
  if (!handle || !workspace || !bits || !(handle->d.flags & MLA_GD_FLAG_DEBUG_CHECKS)) return MLA_GD_E_INVAL;
  return read_clear_err(const_cast<mla_gd_handle*>(handle), workspace, (hipStream_t)stream, bits);
}

int mla_gather_decode_step_profiled(mla_gd_handle* h, const mla_gd_tensors* tn, int32_t n_tokens,
                                    void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                                    int n_events) {
  if (!events) return MLA_GD_E_INVAL;
  return run_step(h, tn, n_tokens, workspace, workspace_bytes, stream, events, n_events);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free entry point's workspace: one static device array.  Host
// code never uses the array's name as an address (on the host it names a
// stand-in, not device memory); each device's copy is looked up once with
// hipGetSymbolAddress and that pointer is what the kernels get.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MLA_GD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// This device's copy of `scratch` (the device must be current).  At the first
// lookup on a device, the array's fixed head (zero bytes, error word and the
// single-launch epoch and flags, the same bytes in every plan) is cleared on
// `stream` with a fill kernel, as a fresh workspace would be.
hipError_t scratch_on_device(int device, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    const size_t words = (kFlagsOffset + (size_t)kFlagRegionWords * 4) / 4;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((words + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream,
                       (uint32_t*)ptr, words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace

extern "C" {

int mla_gather_decode_step_noalloc(mla_gd_handle* h, const mla_gd_tensors* tn, int32_t n_tokens, void* stream) {
  if (!h || !tn) return MLA_GD_E_INVAL;
  if (h->d.flags & MLA_GD_FLAG_DEBUG_CHECKS) return MLA_GD_E_INVAL;
  if (n_tokens < 1 || n_tokens > h->d.max_tokens) return MLA_GD_E_INVAL;
  if (h->device >= kMaxScratchDevices) return MLA_GD_E_INVAL;
  if (make_plan(h->d, n_tokens).total > (size_t)MLA_GD_STATIC_SCRATCH_BYTES) return MLA_GD_E_WORKSPACE;
  hipError_t e = hipSetDevice(h->device);
  void* ws = nullptr;
  if (e == hipSuccess) e = scratch_on_device(h->device, (hipStream_t)stream, &ws);
  if (e != hipSuccess) {
    h->last_hip_error = (int)e;
    return MLA_GD_E_HIP;
  }
  return run_step(h, tn, n_tokens, ws, MLA_GD_STATIC_SCRATCH_BYTES, stream, nullptr, 0, /*direct=*/true);
}

int mla_gather_decode_kernel_count(const mla_gd_handle* h, int32_t n_tokens) {
  if (!h || n_tokens < 1 || n_tokens > h->d.max_tokens) return 0;
  return num_kernels(make_plan(h->d, n_tokens));
}

const char* mla_gather_decode_kernel_name(const mla_gd_handle* h, int32_t n_tokens, int i) {
  const int n = mla_gather_decode_kernel_count(h, n_tokens);
  if (i < 0 || i >= n) return "";
  return kernel_name(make_plan(h->d, n_tokens), i);
}

}  // extern "C"
