// One-token GEMV-path kernels compiled for one fixed shape (fixed_shape.hip).
//
// The phase code reads the step's dimensions and plan values through MLA_D /
// MLA_PL (step_params.h).  fixed_shape.hip compiles the six kernels of the
// one-token GEMV path once more with those values as compile-time constants:
// the DeepSeek-V3.2 attention dimensions (hidden 7168, q_lora_rank 1536,
// kv_lora_rank 512, qk_nope_head_dim 128, qk_rope_head_dim 64, v_head_dim
// 128) with 16 heads (one tensor-parallel rank's share of 128), one token.
// Their index arithmetic then folds; the results are the generic kernels'
// bit for bit (same plan, same reduction orders).  A step uses them only when
// its dimensions and its whole plan equal the compiled ones.
#pragma once

#include <hip/hip_runtime.h>

#include "step_params.h"

namespace mla {

typedef void (*fixed_kernel_t)(StepParams);

struct FixedShapeKernels {
  fixed_kernel_t down, qup, absorb, core, oabsorb, oproj;
};

// Whether step `p` (dimensions and plan) is the compiled shape.
bool fixed_shape_applies(const StepParams& p);
const FixedShapeKernels& fixed_shape_kernels();
// Raises the dynamic-LDS limits of the kernels that need it (once per device).
hipError_t fixed_shape_init();

}  // namespace mla
