/*
 * mla_gather_decode.h -- C ABI of one MLA gather-decode step on an MI355X (gfx950).
 *
 * The step is the operation of the "MLA Attention Block Gather Decode Kernel
 * API Reference" page (awsdocs-neuron, nkilib experimental deepseek_v32).  For
 * each decode token it applies the input norm and the low-rank query and
 * key/value projections, writes the token's row into the paged latent cache,
 * attends over the earlier positions listed for that token, and projects the
 * result back to the hidden width (this rank's heads only; no residual add).
 * Tensor names, shapes and meanings follow the page ("API Reference"
 * parameter list; "Notes"; "Dimensions").
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer on the handle's device, in
 *     row-major layout with the shape given below.  bf16 tensors are raw
 *     16-bit bfloat16 words.  The caller owns every buffer; the library never
 *     allocates, frees or keeps a pointer after a call returns.
 *   - bf16 tensor pointers and the workspace must be 16-byte aligned (the
 *     kernels use 16-byte vector loads); fp32 and int32 pointers 4-byte.
 *   - Calls return 0 (MLA_GD_OK) or a positive error code; nothing is thrown
 *     across the ABI.  mla_gather_decode_strerror() names a code.
 *   - mla_gather_decode_step() only enqueues work on the given HIP stream and
 *     never synchronises the host; errors inside kernels are not reported
 *     (device data validity -- slot and block ids in range, distinct slots --
 *     is the caller's contract, as on the page).  A handle created with
 *     MLA_GD_FLAG_DEBUG_CHECKS is the exception: its steps check that data
 *     on the device and wait for the stream once per step (see the flag).
 *   - Calls that touch the device make the handle's device current on the
 *     calling thread.
 *   - A handle may be used from one thread at a time.  Two steps that overlap
 *     in time must use different workspaces.
 *   - Arithmetic: bf16 operands, fp32 accumulation.  Projections of steps
 *     with more than 3 tokens carry each fp32 activation as two bf16 halves
 *     (about 16 significant bits), except the o-projection of steps with more
 *     than 16 tokens, which takes its input as plain bf16.  In steps of more
 *     than 3 tokens the attention core hands its per-split latent outputs,
 *     each a weighted mean of cache rows, to the output absorption in fp16
 *     (except with 17 to 64 heads at kv_lora_rank >= 128): latent cache values
 *     must then stay below 65504 in magnitude (the rows are RMS-normalised, so
 *     any realistic cache does).
 */
#ifndef MLA_GATHER_DECODE_H
#define MLA_GATHER_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_GD_ABI_VERSION 4

/* error codes */
#define MLA_GD_OK 0
#define MLA_GD_E_INVAL 1        /* null pointer, non-positive or inconsistent dimension, bad flag */
#define MLA_GD_E_ALIGN 2        /* a pointer is not aligned as required above */
#define MLA_GD_E_WORKSPACE 3    /* workspace smaller than mla_gather_decode_workspace_size() */
#define MLA_GD_E_UNSUPPORTED 4  /* dimensions outside what the kernels handle (see create) */
#define MLA_GD_E_HIP 5          /* a HIP runtime call or kernel launch failed */
#define MLA_GD_E_DEVICE_CHECK 6 /* with MLA_GD_FLAG_DEBUG_CHECKS: an earlier step found invalid index data */

/* flags (mla_gd_dims.flags) */
/* Fused variant (ablation): the kv-row write, the absorption and the gather
 * core run as one launch whose core workgroups wait on device-scope counters
 * in the workspace instead of a kernel boundary.  Applies to steps of at most
 * 3 tokens (the GEMV path) with at most 16 heads; other steps run the
 * separate kernels. */
#define MLA_GD_FLAG_FUSED 1u
/* Capture the step's launches once into a HIP graph (on a private stream of
 * default priority, owned by the handle) and replay it on the caller's stream;
 * the step is captured again whenever a tensor pointer, the workspace or
 * n_tokens changes.  Profiled steps and steps enqueued on a stream that the
 * caller is capturing launch directly.  Without the flag every step launches
 * its kernels one by one (measured faster on MI355X for this step). */
#define MLA_GD_FLAG_GRAPH 2u
/* Device-side checks of the caller's index data, which the page leaves to the
 * caller: slot_mapping[t] inside the pool and distinct across the step's
 * tokens, and for every selected position that passes the causal mask a
 * block-table column inside max_blocks_per_seq and a block id inside
 * n_blocks.  A failing token row is not written and a failing gathered entry
 * is treated as masked (no out-of-range access either way); the kernels set
 * bits of an error word in the workspace (MLA_GD_CHECK_*).  With the flag,
 * mla_gather_decode_step() first waits for the steps enqueued before it on
 * `stream`, reads and clears that word, and returns MLA_GD_E_DEVICE_CHECK
 * without launching anything if it was set; mla_gather_decode_debug_status()
 * reads and clears it on demand.  Off by default: the checks cost a
 * synchronisation per step, and a step with them cannot be enqueued on a
 * stream under capture (MLA_GD_E_INVAL). */
#define MLA_GD_FLAG_DEBUG_CHECKS 4u
/* Single-launch step (ablation): every phase of the step -- the index build
 * first, then the down-projections, the query up-projection, the absorption
 * with the kv-row write, the gather core, the output absorption, the
 * o-projection and the output sum -- runs as workgroups of ONE kernel launch,
 * in that order of workgroup index.  A workgroup issues its first weight
 * loads, then waits on device-scope arrival flags in the workspace for the
 * workgroups whose results it reads (never for a later one, so in-order
 * dispatch always makes progress); results pass through device-scope
 * (write-through) stores.  Applies to steps of at most 3 tokens with at most
 * 16 heads and n_prior <= 131072; other steps run the separate kernels.
 * Cannot be combined with MLA_GD_FLAG_FUSED (MLA_GD_E_INVAL).  Needs a
 * workspace zeroed by mla_gather_decode_workspace_init (as every workspace
 * does); if a wait ever times out (MLA_GD_CHECK_WAIT_TIMEOUT), zero the
 * workspace again before the next step. */
#define MLA_GD_FLAG_SINGLE_LAUNCH 8u

/* bits of the debug error word */
#define MLA_GD_CHECK_SLOT_RANGE 1u     /* slot_mapping[t] outside [0, n_blocks * block_size): row not written */
#define MLA_GD_CHECK_BLOCK_RANGE 2u    /* a block_table entry outside [0, n_blocks): entry masked */
#define MLA_GD_CHECK_TABLE_COLUMN 4u   /* position / block_size >= max_blocks_per_seq: entry masked */
#define MLA_GD_CHECK_SLOT_SHARED 8u    /* two tokens share a slot: both write it, one value survives */
#define MLA_GD_CHECK_SEQ_RANGE 16u     /* token_seq[t] outside [0, n_tokens): the token's entries masked */
#define MLA_GD_CHECK_WAIT_TIMEOUT 32u  /* fused or single-launch variant: a wait for another workgroup's
                                          results gave up (set whether or not the debug checks are on) */

/*
 * Dimensions of the step, fixed when the handle is created.  The page passes
 * n_heads, qk_nope_head_dim, qk_rope_head_dim, kv_lora_rank, softmax_scale
 * and norm_eps as arguments and reads every other size off tensor shapes; a C
 * ABI has no shapes, so they are all explicit here.
 *   hidden              width of the residual stream (hidden_states [T, hidden])
 *   q_lora_rank         query latent width (wq_a [hidden, q_lora_rank])
 *   kv_lora_rank        latent width of a cache row
 *   qk_nope_head_dim    per-head query/key width RoPE does not rotate
 *   qk_rope_head_dim    per-head query/key width RoPE rotates (even)
 *   v_head_dim          per-head value width (out_absorb_w [n_heads, v_head_dim, kv_lora_rank])
 *   n_heads             attention heads on this rank
 *   block_size          rows per cache block
 *   max_blocks_per_seq  columns of block_table
 *   n_blocks            blocks in the cache pool
 *   n_prior             selected prior positions per token (width of gather_indices)
 *   max_tokens          largest n_tokens a step may be called with
 *   softmax_scale       score scale (conventionally 1/sqrt(qk_nope_head_dim + qk_rope_head_dim))
 *   norm_eps            epsilon of every RMSNorm (the page's default is 1e-6)
 * A cache row is kv_lora_rank + qk_rope_head_dim wide: [normalised latent | rotated key].
 */
typedef struct mla_gd_dims {
  int32_t hidden;
  int32_t q_lora_rank;
  int32_t kv_lora_rank;
  int32_t qk_nope_head_dim;
  int32_t qk_rope_head_dim;
  int32_t v_head_dim;
  int32_t n_heads;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t n_blocks;
  int32_t n_prior;
  int32_t max_tokens;
  float softmax_scale;
  float norm_eps;
  uint32_t flags;
} mla_gd_dims;

/*
 * The tensors of one step (T = n_tokens; nh, dn, dr, dv, r as in mla_gd_dims;
 * kv_row = r + dr).  Shapes and meanings are the page's parameter list.
 */
typedef struct mla_gd_tensors {
  const void* hidden_states;   /* [T, hidden] bf16: this step's residual-stream hidden states */
  const float* input_norm_w;   /* [hidden] fp32: RMSNorm gamma of the layer input */
  const void* wq_a;            /* [hidden, q_lora_rank] bf16: query down-projection */
  const float* q_norm_w;       /* [q_lora_rank] fp32: RMSNorm gamma of the query latent */
  const void* wq_b;            /* [q_lora_rank, nh*(dn+dr)] bf16: query up-projection, per head [q_nope | q_pe] */
  const void* wkv_a;           /* [hidden, kv_row] bf16: KV down-projection, one cache row per token */
  const float* kv_norm_w;      /* [r] fp32: RMSNorm gamma of the KV latent */
  const void* q_absorb_w;      /* [nh, dn, r] bf16: nope half of wkv_b (nope query -> latent) */
  const void* out_absorb_w;    /* [nh, dv, r] bf16: value half of wkv_b (latent output -> value width) */
  const void* o_proj_w;        /* [nh*dv, hidden] bf16: o-projection rows of this rank's heads */
  const float* cos_table;      /* [T, dr/2] fp32: cosine table of interleaved RoPE */
  const float* sin_table;      /* [T, dr/2] fp32: sine table of interleaved RoPE */
  void* kv_cache;              /* [n_blocks, 1, block_size, kv_row] bf16, MUTATED IN PLACE:
                                  row slot_mapping[t] is overwritten with token t's row */
  const int32_t* slot_mapping; /* [T] int32: flat cache row that receives token t's new row */
  const int32_t* block_table;  /* [n_seqs, max_blocks_per_seq] int32: per sequence, logical block ->
                                  physical block; n_seqs = T without token_seq */
  const int32_t* positions;    /* [T] int32: absolute position of each token in its sequence */
  const int32_t* gather_indices; /* [T, n_prior] int32: selected absolute prior positions, unsorted */
  void* out;                   /* [T, hidden] bf16, written: this rank's attention-block output
                                  (partial o-projection; no residual add, no cross-rank reduction) */
  int32_t* gather_rows_out;    /* optional (may be NULL) [T, n_prior] int32, written: the flat cache
                                  row each selected position resolved to, or -1 where the causal
                                  mask removed it */
  const int32_t* token_seq;    /* optional (may be NULL) [T] int32: the block_table row (sequence) of
                                  token t, in [0, n_tokens).  NULL: row t, one sequence per token.
                                  Several tokens of one sequence (multi-token or speculative decode)
                                  share a row; see mla_gather_decode_step() for what they see. */
} mla_gd_tensors;

typedef struct mla_gd_handle mla_gd_handle;

/*
 * Validate dims and create a handle for HIP device `device`.  The handle holds
 * host-side configuration only.  Returns MLA_GD_E_INVAL for inconsistent dims
 * and MLA_GD_E_UNSUPPORTED for shapes the kernels do not handle: hidden,
 * q_lora_rank, qk_nope_head_dim, kv_lora_rank + qk_rope_head_dim and
 * n_heads*(dn+dr) must be multiples of 8; kv_lora_rank one of 64, 128, 256,
 * 512; qk_rope_head_dim even and at most 64; qk_nope_head_dim at most 512;
 * qk_nope_head_dim + qk_rope_head_dim a multiple of 4; q_lora_rank +
 * kv_lora_rank + qk_rope_head_dim at most 16384; n_prior at most 262144
 * (163840 with more than 64 heads); max_tokens at most 4096.
 * If the environment variable MLA_GD_LOG is set (and not "0") at creation,
 * the first step of each size prints its work decomposition (kernel path,
 * core shape and splits, GEMM slabs, workspace bytes) to stderr.
 */
int mla_gather_decode_create(const mla_gd_dims* dims, int device, mla_gd_handle** out_handle);

/* Release a handle (NULL is accepted). */
void mla_gather_decode_destroy(mla_gd_handle* handle);

/*
 * Bytes of device workspace that serves every step of up to n_tokens tokens
 * (0 if the handle is NULL or n_tokens is out of range).  The workspace holds split-K
 * partial sums, the query tiles, attention partials and arrival counters.
 */
size_t mla_gather_decode_workspace_size(const mla_gd_handle* handle, int32_t n_tokens);

/*
 * Zero a workspace of `bytes` bytes on `stream` (hipStream_t; NULL = default
 * stream).  A workspace must be zeroed once before its first step; every step
 * leaves it ready for the next one.
 */
int mla_gather_decode_workspace_init(const mla_gd_handle* handle, void* workspace, size_t bytes,
                                     void* stream);

/*
 * Enqueue one decode step for n_tokens tokens (1 <= n_tokens <= max_tokens) on
 * `stream` (hipStream_t; NULL = default stream).  Reads every input tensor,
 * writes `out`, row slot_mapping[t] of kv_cache for every token, the optional
 * gather_rows_out, and the workspace.  Every token's row is written before
 * any token gathers, so the row a token writes is visible to the gather of
 * every token in the same step: a token that selects its own position reads
 * this step's row, and with token_seq a token that selects the position of
 * an earlier token of its sequence reads the row that token wrote in this
 * step (later tokens' positions are causally masked).  The result equals
 * running the tokens of each sequence as successive single-token steps in
 * position order.  The tokens of one step must have distinct slots.
 */
int mla_gather_decode_step(mla_gd_handle* handle, const mla_gd_tensors* tensors, int32_t n_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing.  A step of n_tokens tokens runs as
 * mla_gather_decode_kernel_count(handle, n_tokens) kernel launches (steps of
 * more than 3 tokens run the projections on the matrix cores, with two more
 * kernels; 0 for an invalid handle or n_tokens).
 * mla_gather_decode_step_profiled() is mla_gather_decode_step() with timing
 * events (created hipEvent_t handles owned by the caller), in one of two forms:
 *   n_events >= 2*count: kernel i is launched with events[2i] and events[2i+1]
 *     as its start and stop events (hipExtLaunchKernel), which stamp the
 *     kernel's own execution, without the dispatch gaps between kernels;
 *   count + 1 <= n_events < 2*count: hipEventRecord(events[i], stream) before
 *     kernel i and events[count] after the last one.
 * Fewer events, or a null handle among those used, give MLA_GD_E_INVAL.
 * Kernel names are static strings ("" for an index out of range).
 */
int mla_gather_decode_kernel_count(const mla_gd_handle* handle, int32_t n_tokens);
const char* mla_gather_decode_kernel_name(const mla_gd_handle* handle, int32_t n_tokens, int index);
int mla_gather_decode_step_profiled(mla_gd_handle* handle, const mla_gd_tensors* tensors, int32_t n_tokens,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* const* events, int n_events);

/*
 * Allocation-free step, for callers that cannot allocate device memory or
 * create runtime objects: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same step as
 * mla_gather_decode_step(), with the workspace taken from a static device
 * array of MLA_GD_STATIC_SCRATCH_BYTES bytes inside the library (one copy per
 * GPU, held from the first such call on that GPU until the process ends).
 * The caller passes the tensors and `out` as usual.
 *   - Returns MLA_GD_E_WORKSPACE, without launching anything, when a step of
 *     n_tokens tokens needs more workspace than that (16 heads of the
 *     DeepSeek-V3.2 dims fit up to 32 tokens; 128 heads do not fit).
 *   - Calls no hipMalloc/hipFree and creates no stream, event or graph: the
 *     kernels are launched one by one on `stream` (MLA_GD_FLAG_GRAPH is
 *     ignored).  Handles created with MLA_GD_FLAG_DEBUG_CHECKS get
 *     MLA_GD_E_INVAL (their read-back is a synchronising copy).
 *   - The first call on a GPU looks up that GPU's copy of the array
 *     (hipGetSymbolAddress) with the handle's device current, and clears the
 *     array's first 64 KB + 512 bytes (as mla_gather_decode_workspace_init
 *     would) with a fill kernel on `stream`; MLA_GD_E_HIP if either fails.
 *   - Every call on one GPU, from every handle, shares that GPU's array, and
 *     the array keeps the last step's contents (each step rewrites what it
 *     reads, clears at its start what must start at zero, and leaves the
 *     single-launch flags ready for the next step of any handle).  Two
 *     steps that may overlap in time on one GPU (different streams, threads
 *     or handles) race on it: serialise them, or give them
 *     mla_gather_decode_step() with separate workspaces.
 */
#define MLA_GD_STATIC_SCRATCH_BYTES (32u << 20)
int mla_gather_decode_step_noalloc(mla_gd_handle* handle, const mla_gd_tensors* tensors, int32_t n_tokens,
                                   void* stream);

/*
 * Debug checks (MLA_GD_FLAG_DEBUG_CHECKS): wait for the work enqueued on
 * `stream`, store the workspace's error word (MLA_GD_CHECK_* bits) in *bits
 * and clear it.  Returns MLA_GD_E_DEVICE_CHECK if any bit was set,
 * MLA_GD_E_INVAL for a NULL handle, workspace or bits pointer or a handle
 * created without the flag.  Not for use while `stream` is being captured.
 */
int mla_gather_decode_debug_status(const mla_gd_handle* handle, void* workspace, uint32_t* bits, void* stream);

/* Human-readable name of an error code (never NULL). */
const char* mla_gather_decode_strerror(int code);

/* hipError_t of the last failed HIP call made through this handle (0 if none). */
int mla_gather_decode_last_hip_error(const mla_gd_handle* handle);

/* MLA_GD_ABI_VERSION of the built library. */
int mla_gather_decode_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_GATHER_DECODE_H */
