/*
 * rmsnorm_router_topk.h -- C ABI of the fused RMSNorm + MoE router top-K on an
 * MI355X (gfx950), the single-device part of the "RMSNorm Router Top-K A2AV
 * Kernel API Reference" page (awsdocs-neuron, nkilib experimental moe_block):
 * its "API Reference" parameter and return list and its "Notes" (the ACT2
 * pipeline: top-K on the raw logits, the activation on the selected experts
 * only).  The all-to-all dispatch and the two-core duplication of the page are
 * not part of it.
 *
 * For T tokens of width H and E experts:
 *   x_hat[t]       = hidden[t] / sqrt(mean(hidden[t]^2) + eps) * gamma
 *   logits[t]      = x_hat[t] @ router_weights (+ router_bias)
 *   indices[t]     = the top_k experts by logit, descending (ties: lower index first)
 *   affinities[t]  = zero except at indices[t]: sigmoid(logit), or the softmax
 *                    over the top_k selected logits
 * The logits are accumulated in fp32 from the bf16 (or fp16) inputs; x_hat is
 * stored in the input type but the router consumes it unrounded.  From 9
 * tokens on with bf16 inputs the products run on the matrix cores, with
 * hidden * gamma carried as two bf16 halves (about 16 significant bits, a
 * relative error near 2^-17 per product) against the bf16 weight.  A single
 * token runs as one launch: the last workgroup to finish its share of the
 * logits (an arrival counter in the workspace) selects the experts.
 *
 * Conventions: every tensor pointer is a device pointer on the current HIP
 * device, row-major; bf16 tensors and the workspace are 16-byte aligned, fp32
 * and int32 ones 4-byte.  The caller owns every buffer; the call allocates
 * nothing, only enqueues work on `stream` (hipStream_t; NULL = default stream)
 * and never synchronises the host.  Calls return 0 or a positive error code.
 */
#ifndef RMSNORM_ROUTER_TOPK_H
#define RMSNORM_ROUTER_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RT_OK 0
#define RT_E_INVAL 1        /* NULL pointer, size out of range, unknown activation */
#define RT_E_ALIGN 2        /* a pointer misaligned for its type */
#define RT_E_WORKSPACE 3    /* workspace smaller than rmsnorm_router_topk_workspace_size() */
#define RT_E_UNSUPPORTED 4  /* shape outside the limits below */
#define RT_E_HIP 5          /* a kernel launch failed */

#define RT_ACT_SIGMOID 0
#define RT_ACT_SOFTMAX 1
#define RT_DTYPE_BF16 0 /* hidden_states, gamma, router_weights and normed_out in bf16 */
#define RT_DTYPE_FP16 1 /* ... in fp16 (the page's second input type) */

/*
 * Device workspace bytes for (n_tokens, hidden, n_experts), 0 if the shape is
 * unsupported.  Limits: 1 <= n_tokens <= 128 (the page's single-tile bound),
 * hidden a multiple of 128 (the page's) up to 65536, n_experts a multiple of 8
 * up to 1024.  The workspace holds an arrival counter and the split-K
 * partial logits.  It must be zero-filled before its first call; every call
 * leaves the counter at zero again.  Calls that may overlap in time need
 * separate workspaces.
 */
size_t rmsnorm_router_topk_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_experts);

/*
 * One call of the page's function.
 *   hidden_states  [n_tokens, hidden] bf16       (the page's [B, S, H], B*S = n_tokens)
 *   gamma          [hidden] bf16                  RMSNorm scale
 *   router_weights [hidden, n_experts] bf16
 *   router_bias    [n_experts] fp32, or NULL      added to the raw logits
 *   eps >= 0, 1 <= top_k <= min(n_experts, 32), act RT_ACT_SIGMOID or RT_ACT_SOFTMAX
 * Outputs (written): normed_out [n_tokens, hidden] bf16, topk_indices
 * [n_tokens, top_k] int32, affinities [n_tokens, n_experts] bf16.
 */
int rmsnorm_router_topk(const void* hidden_states, const void* gamma, const void* router_weights,
                        const float* router_bias, int32_t n_tokens, int32_t hidden, int32_t n_experts,
                        int32_t top_k, float eps, int32_t act, void* normed_out, int32_t* topk_indices,
                        void* affinities, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same call with the input type chosen: dtype RT_DTYPE_BF16 (as
 * rmsnorm_router_topk) or RT_DTYPE_FP16, which the page allows for
 * hidden_states, gamma and router_weights ("API Reference": bf16/fp16).  The
 * three inputs share the type, normed_out has it too (rounded to nearest
 * even), and affinities stay bf16 as the page returns them.  RT_E_INVAL for
 * another dtype.
 */
int rmsnorm_router_topk_typed(int32_t dtype, const void* hidden_states, const void* gamma, const void* router_weights,
                              const float* router_bias, int32_t n_tokens, int32_t hidden, int32_t n_experts,
                              int32_t top_k, float eps, int32_t act, void* normed_out, int32_t* topk_indices,
                              void* affinities, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif
