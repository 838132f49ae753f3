// Kernel-argument block and launch plan of one MLA gather-decode step.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mla {

// Work decomposition of one step.  Computed on the host from the dimensions
// and n_tokens; every kernel reads the same copy.
struct Plan {
  int T;             // tokens in this step
  // down-projection [wq_a | wkv_a]: 512-column tiles x K-slabs over hidden
  int nt_q, nt_kv, nt1, s1, ks1, n_idx_wg;
  // up-projection wq_b: tiles x slabs over q_lora_rank
  int nt2, s2, ks2;
  // q absorption: heads x 512-column tiles over kv_lora_rank
  int nt_r;
  // attention core: head groups of 16 x splits of n_prior
  int nhg, nsplit, ps;
  // output absorption: rows (h, d) of out_absorb_w, 4 per workgroup
  int n_oabs_wg;
  // o-projection: tiles over hidden x slabs over n_heads*v_head_dim
  int nt5, s5, ks5;
  // workspace layout (byte offsets)
  size_t off_rows, off_part1, off_ss1, off_qa, off_kv, off_part2, off_ss2, off_q;
  size_t off_qlat, off_qpe, off_cm, off_cl, off_co, off_olat, off_ov, off_part5, off_cnt;
  size_t n_cnt, total;
  // counter bases (in counters)
  int cnt1, cnt2, cnt3, cnt5;
};

struct StepParams {
  // dimensions
  int H, Q, R, DN, DR, DV, NH, BS, MB, P, KVR, QKH, N2, NBLK;
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
  // workspace views
  int32_t* rows;
  float *part1, *ss1, *qa, *kvb, *part2, *ss2, *q, *qlat, *qpe, *cm, *cl, *co, *olat, *ov, *part5;
  unsigned* cnt;
  Plan pl;
};

}  // namespace mla
