// MLA gather-decode step for MI355X (gfx950): kernels and the C ABI declared
// in include/mla_gather_decode.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "../../include/mla_gather_decode.h"
#include "phases.h"

using namespace mla;

// ---------------------------------------------------------------------------
// kernels: one phase each (separately launched variant)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void k_down(StepParams p) {
  __shared__ float lds[4 * kGemvTT * kTile];
  __shared__ int flag;
  phase_down(p, blockIdx.x, lds, &flag);
}

__global__ __launch_bounds__(kBlock) void k_qup(StepParams p) {
  __shared__ float lds[4 * kGemvTT * kTile];
  __shared__ int flag;
  phase_qup(p, blockIdx.x, lds, &flag);
}

__global__ __launch_bounds__(kBlock) void k_absorb(StepParams p) {
  __shared__ float lds[4 * kGemvTT * kTile];
  phase_absorb(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(kBlock) void k_core(StepParams p) {
  __shared__ float lds[kCoreLds];
  __shared__ int flag;
  phase_core(p, blockIdx.x, lds, &flag);
}

__global__ __launch_bounds__(kBlock) void k_oabsorb(StepParams p) { phase_oabsorb(p, blockIdx.x); }

__global__ __launch_bounds__(kBlock) void k_oproj(StepParams p) {
  __shared__ float lds[4 * kGemvTT * kTile];
  __shared__ int flag;
  phase_oproj(p, blockIdx.x, lds, &flag);
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
};

namespace {

inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// split-K factor: about `target` workgroups in total, at least `min_rows` rows
// per slab, and partial sums no larger than a quarter of the weight bytes.
void choose_split(int K, int ntiles, int T, int min_rows, int* s_out, int* ks_out) {
  const int target = 512;
  int s = std::max(1, cdiv(target, ntiles));
  s = std::min(s, std::max(1, K / min_rows));
  s = std::min(s, std::max(1, K / (4 * T)));
  int ks = cdiv(K, s);
  ks = (ks + 3) / 4 * 4;
  s = cdiv(K, ks);
  *s_out = s;
  *ks_out = ks;
}

Plan make_plan(const mla_gd_dims& d, int T) {
  Plan pl;
  memset(&pl, 0, sizeof(pl));
  const int H = d.hidden, Q = d.q_lora_rank, R = d.kv_lora_rank, DR = d.qk_rope_head_dim;
  const int KVR = R + DR, QKH = d.qk_nope_head_dim + DR, N2 = d.n_heads * QKH, NH = d.n_heads;
  const int P = d.n_prior;
  pl.T = T;
  pl.nt_q = cdiv(Q, kTile);
  pl.nt_kv = cdiv(KVR, kTile);
  pl.nt1 = pl.nt_q + pl.nt_kv;
  choose_split(H, pl.nt1, T, 16, &pl.s1, &pl.ks1);
  pl.n_idx_wg = cdiv(T * P, kBlock);
  pl.nt2 = cdiv(N2, kTile);
  choose_split(Q, pl.nt2, T, 16, &pl.s2, &pl.ks2);
  pl.nt_r = cdiv(R, kTile);
  pl.nhg = cdiv(NH, kHeadGroup);
  {
    int ns = std::max(1, cdiv(512, T * pl.nhg));
    ns = std::min(ns, cdiv(P, kChunk));
    pl.ps = cdiv(cdiv(P, ns), kChunk) * kChunk;
    pl.nsplit = cdiv(P, pl.ps);
  }
  pl.n_oabs_wg = cdiv(NH * d.v_head_dim, 4);
  pl.nt5 = cdiv(H, kTile);
  choose_split(NH * d.v_head_dim, pl.nt5, T, 16, &pl.s5, &pl.ks5);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  // Arrival counters first, at a fixed offset and sized for max_tokens, so a
  // step with fewer tokens finds them where the previous step left them (zero).
  pl.cnt1 = 0;
  pl.cnt2 = pl.cnt1 + pl.nt1;
  pl.cnt3 = pl.cnt2 + pl.nt2;
  pl.cnt5 = pl.cnt3 + T * pl.nhg;
  pl.n_cnt = (size_t)pl.cnt5 + pl.nt5;
  const size_t max_cnt = (size_t)pl.nt1 + pl.nt2 + (size_t)d.max_tokens * pl.nhg + pl.nt5;
  pl.off_cnt = take(max_cnt * sizeof(unsigned));
  const size_t f = sizeof(float);
  pl.off_rows = take((size_t)T * P * sizeof(int32_t));
  pl.off_part1 = take((size_t)pl.s1 * T * (Q + KVR) * f);
  pl.off_ss1 = take((size_t)pl.nt1 * pl.s1 * T * f);
  pl.off_qa = take((size_t)T * Q * f);
  pl.off_kv = take((size_t)T * KVR * f);
  pl.off_part2 = take((size_t)pl.s2 * T * N2 * f);
  pl.off_ss2 = take((size_t)pl.nt2 * pl.s2 * T * f);
  pl.off_q = take((size_t)T * N2 * f);
  pl.off_qlat = take((size_t)T * NH * R * f);
  pl.off_qpe = take((size_t)T * NH * DR * f);
  pl.off_cm = take((size_t)T * pl.nsplit * NH * f);
  pl.off_cl = take((size_t)T * pl.nsplit * NH * f);
  pl.off_co = take((size_t)T * pl.nsplit * NH * R * f);
  pl.off_olat = take((size_t)T * NH * R * f);
  pl.off_ov = take((size_t)T * NH * d.v_head_dim * f);
  pl.off_part5 = take((size_t)pl.s5 * T * H * f);
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
  if ((d.flags & ~MLA_GD_FLAG_FUSED) != 0u) return MLA_GD_E_INVAL;
  if (!isfinite(d.softmax_scale) || !isfinite(d.norm_eps) || d.norm_eps < 0.f) return MLA_GD_E_INVAL;
  const long long KVR = (long long)d.kv_lora_rank + d.qk_rope_head_dim;
  const long long N2 = (long long)d.n_heads * (d.qk_nope_head_dim + d.qk_rope_head_dim);
  if (d.hidden % 8 || d.q_lora_rank % 8 || KVR % 8 || N2 % 8 || d.kv_lora_rank % 16) return MLA_GD_E_UNSUPPORTED;
  if (d.kv_lora_rank > 512 || d.qk_rope_head_dim > 128) return MLA_GD_E_UNSUPPORTED;
  if (d.max_tokens > 4096) return MLA_GD_E_UNSUPPORTED;
  // flat cache rows and element offsets must fit the kernels' index arithmetic
  if ((long long)d.n_blocks * d.block_size > (1LL << 31) - 1) return MLA_GD_E_UNSUPPORTED;
  if ((long long)d.max_tokens * d.n_prior > (1LL << 31) - 1) return MLA_GD_E_UNSUPPORTED;
  return MLA_GD_OK;
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
  *out_handle = h;
  return MLA_GD_OK;
}

void mla_gather_decode_destroy(mla_gd_handle* handle) { delete handle; }

int mla_gather_decode_last_hip_error(const mla_gd_handle* handle) { return handle ? handle->last_hip_error : 0; }

size_t mla_gather_decode_workspace_size(const mla_gd_handle* handle, int32_t n_tokens) {
  if (!handle || n_tokens < 1 || n_tokens > handle->d.max_tokens) return 0;
  size_t most = 0;
  for (int t = 1; t <= n_tokens; ++t) most = std::max(most, make_plan(handle->d, t).total);
  return most;
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

const char* const kKernelNames[] = {"k_down", "k_qup", "k_absorb", "k_core", "k_oabsorb", "k_oproj"};
constexpr int kNumKernels = 6;

int run_step(mla_gd_handle* h, const mla_gd_tensors* tn, int32_t n_tokens, void* workspace,
             size_t workspace_bytes, void* stream, void* const* events, int n_events) {
  if (!h || !tn || !workspace) return MLA_GD_E_INVAL;
  if (events && n_events < kNumKernels + 1) return MLA_GD_E_INVAL;
  if (events)
    for (int i = 0; i <= kNumKernels; ++i)
      if (!events[i]) return MLA_GD_E_INVAL;
  const mla_gd_dims& d = h->d;
  if (n_tokens < 1 || n_tokens > d.max_tokens) return MLA_GD_E_INVAL;
  const void* bf[] = {tn->hidden_states, tn->wq_a, tn->wq_b, tn->wkv_a, tn->q_absorb_w, tn->out_absorb_w,
                      tn->o_proj_w, tn->kv_cache, tn->out};
  const void* w4[] = {tn->input_norm_w, tn->q_norm_w, tn->kv_norm_w, tn->cos_table, tn->sin_table,
                      tn->slot_mapping, tn->block_table, tn->positions, tn->gather_indices};
  for (const void* q : bf) if (!q) return MLA_GD_E_INVAL;
  for (const void* q : w4) if (!q) return MLA_GD_E_INVAL;
  for (const void* q : bf) if (!aligned(q, 16)) return MLA_GD_E_ALIGN;
  for (const void* q : w4) if (!aligned(q, 4)) return MLA_GD_E_ALIGN;
  if (tn->gather_rows_out && !aligned(tn->gather_rows_out, 4)) return MLA_GD_E_ALIGN;
  if (!aligned(workspace, 256)) return MLA_GD_E_ALIGN;

  const Plan pl = make_plan(d, n_tokens);
  if (workspace_bytes < pl.total) return MLA_GD_E_WORKSPACE;

  StepParams p;
  memset(&p, 0, sizeof(p));
  p.H = d.hidden; p.Q = d.q_lora_rank; p.R = d.kv_lora_rank; p.DN = d.qk_nope_head_dim;
  p.DR = d.qk_rope_head_dim; p.DV = d.v_head_dim; p.NH = d.n_heads; p.BS = d.block_size;
  p.MB = d.max_blocks_per_seq; p.P = d.n_prior; p.KVR = p.R + p.DR; p.QKH = p.DN + p.DR;
  p.N2 = p.NH * p.QKH; p.NBLK = d.n_blocks;
  p.scale_log2 = d.softmax_scale * kLog2e;
  p.eps = d.norm_eps;
  p.x = (const uint16_t*)tn->hidden_states; p.g_in = tn->input_norm_w; p.wq_a = (const uint16_t*)tn->wq_a;
  p.g_q = tn->q_norm_w; p.wq_b = (const uint16_t*)tn->wq_b; p.wkv_a = (const uint16_t*)tn->wkv_a;
  p.g_kv = tn->kv_norm_w; p.w_qabs = (const uint16_t*)tn->q_absorb_w; p.w_oabs = (const uint16_t*)tn->out_absorb_w;
  p.w_o = (const uint16_t*)tn->o_proj_w; p.cos_t = tn->cos_table; p.sin_t = tn->sin_table;
  p.cache = (uint16_t*)tn->kv_cache; p.slot = tn->slot_mapping; p.btab = tn->block_table; p.pos = tn->positions;
  p.gidx = tn->gather_indices; p.out = (uint16_t*)tn->out; p.rows_out = tn->gather_rows_out;
  char* ws = (char*)workspace;
  p.rows = (int32_t*)(ws + pl.off_rows);
  p.part1 = (float*)(ws + pl.off_part1); p.ss1 = (float*)(ws + pl.off_ss1); p.qa = (float*)(ws + pl.off_qa);
  p.kvb = (float*)(ws + pl.off_kv); p.part2 = (float*)(ws + pl.off_part2); p.ss2 = (float*)(ws + pl.off_ss2);
  p.q = (float*)(ws + pl.off_q); p.qlat = (float*)(ws + pl.off_qlat); p.qpe = (float*)(ws + pl.off_qpe);
  p.cm = (float*)(ws + pl.off_cm); p.cl = (float*)(ws + pl.off_cl); p.co = (float*)(ws + pl.off_co);
  p.olat = (float*)(ws + pl.off_olat); p.ov = (float*)(ws + pl.off_ov); p.part5 = (float*)(ws + pl.off_part5);
  p.cnt = (unsigned*)(ws + pl.off_cnt);
  p.pl = pl;

  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) { h->last_hip_error = (int)e; return MLA_GD_E_HIP; }
  hipStream_t s = (hipStream_t)stream;
  const int T = n_tokens;
  auto mark = [&](int i) {
    if (events && e == hipSuccess) e = hipEventRecord((hipEvent_t)events[i], s);
  };
  mark(0);
  hipLaunchKernelGGL(k_down, dim3(pl.nt1 * pl.s1 + pl.n_idx_wg), dim3(kBlock), 0, s, p);
  mark(1);
  hipLaunchKernelGGL(k_qup, dim3(pl.nt2 * pl.s2 + T), dim3(kBlock), 0, s, p);
  mark(2);
  hipLaunchKernelGGL(k_absorb, dim3(p.NH * pl.nt_r), dim3(kBlock), 0, s, p);
  mark(3);
  hipLaunchKernelGGL(k_core, dim3(T * pl.nhg * pl.nsplit), dim3(kBlock), 0, s, p);
  mark(4);
  hipLaunchKernelGGL(k_oabsorb, dim3(pl.n_oabs_wg), dim3(kBlock), 0, s, p);
  mark(5);
  hipLaunchKernelGGL(k_oproj, dim3(pl.nt5 * pl.s5), dim3(kBlock), 0, s, p);
  mark(6);
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

int mla_gather_decode_step_profiled(mla_gd_handle* h, const mla_gd_tensors* tn, int32_t n_tokens,
                                    void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                                    int n_events) {
  if (!events) return MLA_GD_E_INVAL;
  return run_step(h, tn, n_tokens, workspace, workspace_bytes, stream, events, n_events);
}

int mla_gather_decode_kernel_count(const mla_gd_handle* h) { return h ? kNumKernels : 0; }

const char* mla_gather_decode_kernel_name(const mla_gd_handle* h, int i) {
  if (!h || i < 0 || i >= kNumKernels) return "";
  return kKernelNames[i];
}

}  // extern "C"
