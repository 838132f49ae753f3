// The one-token GEMV path of the MLA gather-decode step, compiled for one fixed
// shape (fixed_shape.h says which and why).  Same phase code as the generic
// kernels in mla_gather_decode.hip; MLA_D / MLA_PL read the constants below.
#define MLA_FIXED_SHAPE 1
#define MLA_PHASE_NS mla_fx

#include <hip/hip_runtime.h>

// The compiled shape: dimensions and the plan make_plan derives for one token.
struct MlaFixedShape {
  static constexpr int H = 7168, Q = 1536, R = 512, DN = 128, DR = 64, DV = 128, NH = 16;
  static constexpr int KVR = R + DR, QKH = DN + DR, N2 = NH * QKH;
  static constexpr int pl_T = 1;
  static constexpr int pl_tw1 = 128, pl_s1 = 28, pl_ks1 = 256;  // down-projection: 128-column tiles, 28 slabs
  static constexpr int pl_tw2 = 64, pl_s2 = 8, pl_ks2 = 192;    // q up-projection
  static constexpr int pl_ncc3 = 8, pl_nkv = 9;                 // absorption chunks, kv-row slices
  static constexpr int pl_tw6 = 128, pl_s6 = 8, pl_ks6 = 256;   // o-projection
  static constexpr int pl_nsplit = 64;                          // core row splits
  static constexpr int pl_tc5 = 1, pl_nt5c = 1;                 // output absorption token chunks
};

#include "fixed_shape.h"
#include "phases.h"

using mla::StepParams;

__global__ __launch_bounds__(mla::kBlock) void k_down_fx(StepParams p) {
  extern __shared__ float lds[];
  // as k_down: the fused variant never runs here; the o-projection tiles'
  // arrival counters start each step at zero
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < p.pl.nt6; i += mla::kBlock) p.tcnt[i * mla_fx::kSyncStride] = 0u;
  mla_fx::clear_zero_region(p, blockIdx.x);
  mla_fx::phase_down<1>(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(mla::kBlock) void k_qup_fx(StepParams p) {
  extern __shared__ float lds[];
  mla_fx::phase_qup<1>(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(mla::kBlock) void k_absorb_fx(StepParams p) {
  extern __shared__ float lds[];
  mla_fx::phase_absorb<1>(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(8 * 64) void k_core_fx(StepParams p) {
  __shared__ __attribute__((aligned(16))) char lds[mla_fx::core_lds_bytes(32, 1, 8)];
  mla_fx::core_phase<32, 1, 8>(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(mla::kBlock) void k_oabsorb_fx(StepParams p) {
  extern __shared__ float lds[];
  mla_fx::phase_oabsorb(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(mla::kBlock) void k_oproj_fx(StepParams p) {
  extern __shared__ float lds[];
  mla_fx::phase_oproj<1>(p, blockIdx.x, lds, mla::HandoffDevStores());
  mla_fx::oproj_fold_out(p, blockIdx.x % p.pl.nt6, lds);
}

namespace mla {

bool fixed_shape_applies(const StepParams& p) {
  using F = MlaFixedShape;
  const Plan& pl = p.pl;
  return p.H == F::H && p.Q == F::Q && p.R == F::R && p.DN == F::DN && p.DR == F::DR && p.DV == F::DV &&
         p.NH == F::NH && p.KVR == F::KVR && p.QKH == F::QKH && p.N2 == F::N2 && pl.T == F::pl_T && !pl.mfma &&
         !pl.fused && !pl.single && pl.tw1 == F::pl_tw1 && pl.s1 == F::pl_s1 && pl.ks1 == F::pl_ks1 &&
         pl.tw2 == F::pl_tw2 && pl.s2 == F::pl_s2 && pl.ks2 == F::pl_ks2 && pl.ncc3 == F::pl_ncc3 &&
         pl.nkv == F::pl_nkv && pl.tw6 == F::pl_tw6 && pl.s6 == F::pl_s6 && pl.ks6 == F::pl_ks6 &&
         pl.nsplit == F::pl_nsplit && pl.tc5 == F::pl_tc5 && pl.nt5c == F::pl_nt5c && pl.core_hg == 1 &&
         pl.core_cs == 8 && pl.fold_out == 1;
}

const FixedShapeKernels& fixed_shape_kernels() {
  static const FixedShapeKernels k = {k_down_fx, k_qup_fx, k_absorb_fx, k_core_fx, k_oabsorb_fx, k_oproj_fx};
  return k;
}

hipError_t fixed_shape_init() {
  hipError_t e = hipSuccess;
  const size_t gl = mla_fx::kGemvLdsFloats * sizeof(float);
  const void* ks[] = {(const void*)k_down_fx, (const void*)k_qup_fx, (const void*)k_absorb_fx,
                      (const void*)k_oabsorb_fx, (const void*)k_oproj_fx};
  for (const void* k : ks)
    if (e == hipSuccess) e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)gl);
  return e;
}

}  // namespace mla
