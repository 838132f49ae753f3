// Kernel-argument block and launch plan of one MLA gather-decode step.
#pragma once

#include <stddef.h>
#include <stdint.h>

// The phase code (phases.h, core_mfma.h) reads the step's dimensions and the
// plan values of the one-token GEMV path through these two macros.  Normally
// they read the kernel argument `p`; a translation unit that defines
// MLA_FIXED_SHAPE (and the struct MlaFixedShape with the values, plus its own
// MLA_PHASE_NS) compiles the same code with them as constants, so the index
// arithmetic folds (fixed_shape.hip).
#ifdef MLA_FIXED_SHAPE
#define MLA_D(x) (MlaFixedShape::x)
#define MLA_PL(x) (MlaFixedShape::pl_##x)
#else
#define MLA_D(x) (p.x)
#define MLA_PL(x) (p.pl.x)
#endif
#ifndef MLA_PHASE_NS
#define MLA_PHASE_NS mla
#endif

namespace mla {

// Work decomposition of one step.  Computed on the host from the dimensions
// and n_tokens; every kernel reads the same copy.
struct Plan {
  int T;  // tokens in this step
  // GEMV-path tile widths (columns, <= 512) of the three split-K GEMVs: narrower
  // tiles give as many workgroups with fewer slabs for the consumers to reduce
  int tw1, tw2, tw6;
  // k_down: index build + [wq_a | wkv_a] split-K GEMV (tw1-column tiles x slabs of hidden)
  int nt_q, nt_kv, nt1, s1, ks1, n_idx_wg;
  // k_qup: wq_b split-K GEMV (tw2-column tiles x slabs of q_lora_rank) + kv-row reduction (token x 64-column slice)
  int nt2, s2, ks2, nkv;
  // k_absorb: heads x 64-column chunks of kv_lora_rank, + one kv-finalise workgroup per token
  int ncc3;
  // k_core: (token, split, head block); hg head groups of 16 x cs column splits per workgroup
  int core_hg, core_cs, core_nhb, nsplit, ps;
  int core_rs;  // many heads: the row-split core (core_phase_rs)
  // k_oabsorb: heads x 64-column chunks of kv_lora_rank x token chunks of tc5
  int nc5, tc5, nt5c;
  // k_oproj: tw6-column tiles over hidden x slabs of n_heads*v_head_dim
  int nt6, s6, ks6;
  // k_out: 64-column groups x token chunks
  int n7;
  // GEMV path: the output sum is folded into the o-projection (no k_out); the
  // last slab of each column tile to arrive adds the tile's slabs
  int fold_out;
  // matrix-core path, every core shape but the row-split one: the core stores
  // each split's latent output normalised by its own denominator (o / l) in
  // fp16, half the bytes of the fp32 partials it otherwise writes
  int po16;
  // fused variant: one launch for the kv-row write, the absorption and the core
  int fused;
  // single-launch variant: the whole step as one launch; item (workgroup)
  // ranges of its phases: index build [0, i_down), down-projections [i_down,
  // i_qup), up-projection [i_qup, i_abs), absorption [i_abs, i_core), core
  // [i_core, i_oabs), output absorption [i_oabs, i_oproj), o-projection
  // [i_oproj, i_out), output sum [i_out, n_items)
  int single;
  int i_down, i_qup, i_abs, i_core, i_oabs, i_oproj, i_out, n_items;
  // Matrix-core path (more than a few tokens).  Token blocks of mtb m-tiles
  // (16 tokens each), ntb blocks, m-tiles padded to mt_pad = ntb*mtb.  For each
  // projection: kt* k-steps of 32 in all, ks* per slab, column tiles of
  // mg_cols(mtb) weight columns (128 for up to two m-tiles, 256 otherwise).
  int mfma;
  int mtb, ntb, mt_pad;
  int kt1, ks1m, nt1m, ntq1m;  // [wq_a | wkv_a]: slabs in s1
  int kt2, ks2m, nt2m;         // wq_b: slabs in s2
  int mtb3, ntb3, nca3, nct3, tpw3;  // absorption: token blocks, nca3-column tiles of kv_lora_rank (nct3), tiles per workgroup
  int mtb5, ntb5, nq5, q5;     // output absorption: token blocks, parts per (head, block), tiles per wave
  int nxc, nqc;                // k_prep chunks of hidden; k_qa chunks of q_lora_rank (per token)
  int kt6, ks6m, nt6m;         // o_proj: slabs in s6
  // workspace layout (byte offsets)
  size_t off_zero, off_err, off_rows, off_part1, off_ssx, off_part2, off_ssq, off_kvr, off_kvss, off_qcat;
  size_t off_pm, off_pl, off_po, off_ov, off_part6;
  size_t off_a1, off_a2, off_a5;
  size_t off_sync;  // fused variant's counters (same offset for every n_tokens)
  size_t off_flags;  // single-launch epoch and arrival flags (the same offset and size in every plan)
  size_t off_tcnt;   // GEMV path: per o-projection column tile arrival counters (kSyncStride words apart)
  size_t total;
};

struct StepParams {
  // dimensions
  int H, Q, R, DN, DR, DV, NH, BS, MB, P, KVR, QKH, N2;
  int NBLK;  // n_blocks (pool blocks)
  int dbg;   // debug checks of the index data (MLA_GD_FLAG_DEBUG_CHECKS)
  float scale_log2;  // softmax_scale * log2(e): scores live in the log2 domain
  float eps;
  // inputs (device pointers)
  const uint16_t* x;
  const float* g_in;
  const uint16_t* wq_a;
  const float* g_q;
  const uint16_t* wq_b;
  const uint16_t* wkv_a;
  const float* g_kv;
  const uint16_t* w_qabs;
  const uint16_t* w_oabs;
  const uint16_t* w_o;
  const float* cos_t;
  const float* sin_t;
  uint16_t* cache;
  const int32_t* slot;
  const int32_t* btab;
  const int32_t* pos;
  const int32_t* gidx;
  uint16_t* out;
  int32_t* rows_out;  // optional
  const int32_t* tseq;  // optional [T]: block-table row of each token (NULL: row t)
  // workspace views
  const uint16_t* zero16;  // 256 zero bytes (source of padding loads)
  int32_t* rows;    // [T][P] flat cache row or -1
  float* part1;     // [s1][T][Q+KVR] split-K partials of (x*gamma) @ [wq_a | wkv_a]
  float* ssx;       // [s1][T] partial sums of x^2 (matrix-core path: [nxc][T])
  float* part2;     // [s2][T][N2] split-K partials of (acc_q*gamma_q) @ wq_b
  float* ssq;       // [s2][T] partial sums of acc_q^2 (matrix-core path: [nqc][T])
  float* kvr;       // [T][KVR] alpha * (x * g_in) @ wkv_a: the kv row before its own norm
  float* kvss;      // [T][nkv] partial sums of squares of the kv row's latent part
  uint16_t* qcat;   // [T][NH][KVR] bf16: per head [q_lat | roped q_pe]
  float* pm;        // [T][nsplit][NH] running max (log2 domain) per split
  float* pden;      // [T][nsplit][NH] softmax denominators per split
  float* po;        // [T][nsplit][NH][R] unnormalised latent outputs per split (fp32), or
                    // with pl.po16 normalised ones (fp16, o / l; zeros where l = 0)
  float* ov;        // [T][NH*DV] output-absorbed values
  float* part6;     // [s6][T][H] split-K partials of the o-projection
  // matrix-core path: activations in fragment order (hi/lo bf16), per-token scales
  uint16_t* a1;     // x * g_in               [kt1][mt_pad][2][512]
  uint16_t* a2;     // acc_q * g_q            [kt2][mt_pad][2][512]
  uint16_t* a5;     // o_v                    [kt6][mt_pad][2][512]
  // fused variant: counters kSyncStride words apart -- [0] kv rows written,
  // [1] error flag (a wait timed out), [2 + h] absorption tiles of head h done
  unsigned* sync;
  unsigned* err;  // debug error word (MLA_GD_CHECK_* bits)
  // single-launch variant: epoch[0] = the last completed step's number,
  // epoch[16] = output workgroups done in this step; flags[item] = the step
  // number that item last completed
  unsigned* epoch;
  unsigned* flags;
  unsigned* tcnt;  // GEMV path: o-projection column tiles' arrival counters
  Plan pl;
};

}  // namespace mla
