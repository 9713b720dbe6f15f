/*
 * moe.h — C-ABI of a top-K routed mixture-of-experts FFN layer (forward pass)
 * for the AMD MI355X (gfx950).
 *
 * The layer (Lensa ML explainer "Mixture of Experts", Steps 2-4; maptheai.com
 * "Mixture of Experts", section "The mechanism"; Curionode "Mixture of
 * Experts." Plate VII.4, introduction):
 *   logits = h . W_r (+ b_r)         a linear router, kept in float32
 *   p      = softmax over the E experts
 *   choose the K experts with the largest logits
 *   gates  = softmax over the K chosen logits (renormalised, Mixtral form)
 *            or p_i itself (Switch top-1 form)
 *   y      = sum over the chosen experts of gate * Expert_e(h)
 *   aux    = E * sum_e f_e * P_e     (f_e = share of the T*K routing slots on e,
 *                                     P_e = mean of p over tokens; Step 4)
 * Only the chosen experts run, each on the rows routed to it.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every pointer argument is a DEVICE pointer (memory owned by the caller,
 *    e.g. a torch tensor), except `desc`, which is a host pointer read during
 *    the call only. All tensors are contiguous, row-major, 16-byte aligned.
 *  - The library never allocates device memory and never synchronises the
 *    host. Scratch comes from the caller's workspace `ws` (`ws_bytes` long,
 *    256-byte aligned), sized by moe_workspace_size(), or for
 *    moe_forward_noalloc from a static device array. All work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and is complete once the
 *    stream is; outputs are not valid before that.
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    error nothing is enqueued, no output is touched, and a nonzero moe_status
 *    is returned. Nothing aborts, throws or prints.
 *  - Results are bitwise identical from run to run on the same device (no
 *    floating-point atomics anywhere).
 *  - T = 0 is valid: routing outputs become zeros, aux becomes 0.
 *  - Inputs must be finite; behaviour on NaN/Inf is unspecified.
 *  - Calls keep no state between them (apart from the trace switch below) and
 *    may run concurrently on different streams with disjoint buffers.
 *
 * Tensor layouts (S = T*K routing slots, bpe = 4 for MOE_F32, 2 for MOE_BF16)
 *  h        [T][d]          dtype    token representations
 *  W_r      [d][E]          float32  router weight (always float32)
 *  b_r      [E]             float32  optional router bias (see moe_bias_mode)
 *  W1, W3   [E][width][d]   dtype    row n of expert e = column n of the d x width
 *                                    matrix of the math (output-major: the reduction
 *                                    dimension d is contiguous). The input-major
 *                                    layout [E][d][width] is not accepted: a caller
 *                                    holding it transposes once per weight load.
 *  b1       [E][width]      dtype    GELU experts only (optional)
 *  W2       [E][d][width]   dtype    row j of expert e = column j of the width x d matrix
 *  b2       [E][d]          dtype    GELU experts only (optional)
 *  topk_idx [T][K]          int32    chosen experts, largest logit first; equal
 *                                    logits: lower expert index first
 *  topk_gate[T][K]          float32  gate of each choice
 *  expert_counts [E]        int32    routing slots per expert (sum = S)
 *  expert_offsets[E+1]      int32    exclusive prefix sum of the counts
 *  slot_token [S]           int32    token held by grouped row s
 *  token_slot [T][K]        int32    grouped row of the j-th choice of token t
 *  h_perm   [S][d]          dtype    h grouped by expert: rows of expert e are
 *                                    offsets[e] .. offsets[e+1]-1, tokens ascending
 *  o_perm   [S][d]          float32  ungated expert output of each grouped row
 *  y        [T][d]          dtype    layer output
 *
 * Expert MLPs (Lensa ML Step 1: each expert is a full FFN):
 *  MOE_ACT_GELU:   o = GELU(x W1 + b1) W2 + b2   (exact erf GELU; biases optional)
 *  MOE_ACT_SWIGLU: o = (SiLU(x W1) * (x W3)) W2  (no biases; W3 required)
 *
 * Numerics: router logits are float32 in one fixed order, so expert selection
 * depends on no implementation choice: k is cut into groups of four
 * consecutive values, group g = k / 4 feeds chain g mod 4, each of the four
 * chains is a fused-multiply-add chain from +0 over its k in ascending order,
 * logit = (c0 + c1) + (c2 + c3), and the bias is added afterwards. Softmax,
 * gates and aux are float32. Expert GEMMs
 * accumulate in float32 (bf16 inputs use bf16 MFMA); the hidden activation
 * is stored in the input dtype; o_perm is float32; y is rounded once.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,        /* T < 0, d or width < 1, E < 1, K < 1 or K > E */
  MOE_ERR_UNSUPPORTED = 3,  /* E > 64, K > 8, d or width not a multiple of 8,
                               d or width above 2^20, T*K above 2^31 - 1, an operand
                               matrix (S x d, S x width or d x width) of more than
                               2^31 - 2^22 elements, an unknown act/gate/dtype, a
                               misaligned pointer, an unknown bias_mode, or W3
                               missing for SwiGLU */
  MOE_ERR_WORKSPACE = 4,    /* ws_bytes smaller than moe_workspace_size(), or ws misaligned */
  MOE_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum moe_act { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;
typedef enum moe_gate { MOE_GATE_RENORM = 0, MOE_GATE_RAW = 1 } moe_gate;
typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
/* What the router bias b_r acts on. MOE_BIAS_LOGITS: it is part of the logits
 * (choice, softmax, gates, P). MOE_BIAS_SELECT: it steers only which experts
 * are chosen (Lensa ML explainer, Step 4: DeepSeek-V3 keeps the load even with
 * a per-expert routing bias instead of the aux loss); the softmax, the gates
 * and P use the unbiased logits h . W_r. Without b_r both are the same. */
typedef enum moe_bias_mode { MOE_BIAS_LOGITS = 0, MOE_BIAS_SELECT = 1 } moe_bias_mode;

/* Shape of one layer, in the pages' terms: T tokens of width d, E experts of
 * width `width`, K chosen per token (Lensa ML Steps 1 and 3). */
typedef struct moe_desc {
  int64_t T;
  int64_t d;
  int64_t E;
  int64_t K;
  int64_t width;
  int32_t act;    /* moe_act */
  int32_t gate;   /* moe_gate */
  int32_t dtype;  /* moe_dtype: h, W1, W3, W2, b1, b2, h_perm, y */
  int32_t capacity; /* slots per expert (Lensa ML Step 5, "Capacity & Dropped
                       Tokens"); 0 = dropless (every slot is processed). With
                       C > 0 each expert processes its first C slots in token
                       order and drops the rest: a dropped slot adds nothing
                       to y and its token_slot entry is -1; a token with no
                       kept slot gets y = 0 (the layer adds nothing to its
                       residual). Counts, offsets and the aux loss describe
                       the router's choices before any drop. Negative values
                       are MOE_ERR_SHAPE. moe_capacity_slots() gives C for a
                       capacity factor. */
  int32_t bias_mode; /* moe_bias_mode; any other value is MOE_ERR_UNSUPPORTED */
} moe_desc;

/* Human-readable name of a moe_status value (static string, never NULL). */
const char* moe_status_string(int status);

/* Slots per expert for a capacity factor (Lensa ML Step 5): C = factor * T * K / E,
 * rounded up when fractional (the product is taken in double precision; a
 * value within 1e-9 relative of an integer counts as that integer). Host-only.
 * Writes *slots; returns MOE_ERR_NULL for a NULL `slots`, MOE_ERR_SHAPE for
 * factor < 0, T < 0, K < 1 or E < 1 (or a non-finite factor), and
 * MOE_ERR_UNSUPPORTED if C would exceed 2^31 - 1. */
int moe_capacity_slots(double factor, int64_t T, int64_t K, int64_t E, int32_t* slots);

/* Bytes of workspace that any entry point below needs for this layer shape.
 * Host-only; enqueues nothing. */
int moe_workspace_size(const moe_desc* desc, size_t* bytes);

/* Router (Lensa ML Step 2: a linear layer and a softmax; Step 3: top-k and
 * gates; Step 4: slot counts and the load-balance loss).
 * In:  h, W_r, b_r (nullable), noise [T][E] float32 (nullable): values added
 *      to the logits after the bias, one float32 add each, which enter the
 *      choice, the gates and P (noisy top-k routing, arjunjaggi.com "Load
 *      Balancing": the caller draws and scales the noise).
 * Out: topk_idx, topk_gate, expert_counts, prob_mean [E] (P_e, nullable),
 *      aux_loss [1] (nullable), logits [T][E] float32 (nullable): the scores
 *      the choice is made on, h . W_r + b_r (+ noise) (with either bias_mode),
 *      z_loss [1] (nullable): the router z-loss (arjunjaggi.com "Mixtral and
 *      the Open MoE Era": ST-MoE's penalty on large router logits), the mean
 *      over tokens of the squared log-sum-exp of the logits the softmax sees.
 * A NaN score never wins the choice: a token with fewer than K scores that
 * are not NaN gets id 0x7fffffff in its remaining slots, which are not
 * counted and get no grouped row (moe_permute skips them; moe_forward's y then
 * has nothing from them: 0 for a token with none left when K > 1 or with a
 * capacity, unwritten for K = 1 without one); P, aux and the z-loss come out
 * NaN. Memory-safe: no access depends on a score's value.
 * Returns a moe_status. */
int moe_route(const moe_desc* desc, const void* h, const float* W_r, const float* b_r,
              int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
              float* prob_mean, float* aux_loss, float* logits, const float* noise,
              float* z_loss, void* ws, size_t ws_bytes, void* stream);

/* Grouping of the routing slots by expert (Lensa ML Step 5: experts take any
 * number of tokens). Stable: inside each expert's group tokens keep their order.
 * In:  topk_idx, h. The K ids of a token must be distinct (as moe_route
 *      writes them); an id outside [0, E) is skipped: it gets token_slot -1 and
 *      no grouped row, and it is not counted in expert_offsets.
 * Out: expert_offsets, slot_token, token_slot, h_perm (gathered rows of h).
 * With desc->capacity = C > 0, token_slot is -1 for every slot at rank C or
 * more in its expert's group (dropped); the groups themselves keep every slot.
 * Returns a moe_status. */
int moe_permute(const moe_desc* desc, const int32_t* topk_idx, const void* h,
                int32_t* expert_offsets, int32_t* slot_token, int32_t* token_slot,
                void* h_perm, void* ws, size_t ws_bytes, void* stream);

/* Each expert's FFN on its own grouped rows only (maptheai.com "The mechanism":
 * only the chosen experts run; Lensa ML Step 1: each expert is a full FFN).
 * In:  h_perm, expert_offsets, W1, b1 (nullable), W3 (SwiGLU), W2, b2 (nullable).
 * Out: o_perm (ungated float32 expert outputs, one row per grouped slot).
 * With desc->capacity = C > 0 only the first C rows of each group are
 * computed; the o_perm rows of dropped slots are left as they were.
 * expert_offsets must be non-decreasing from 0 to S = T*K (as moe_permute
 * writes them); otherwise the outputs are unspecified, but every expert's row
 * range is clamped into [0, S), so no access leaves the buffers.
 * ws is scratch: the hidden activations and, for bfloat16 layers on large
 * groups, float32 partial rows of the experts' short last row tiles, whose
 * reduction is split in parts and summed in a fixed order (same bits every
 * call). Returns a moe_status. */
int moe_expert_ffn(const moe_desc* desc, const void* h_perm, const int32_t* expert_offsets,
                   const void* W1, const void* b1, const void* W3, const void* W2,
                   const void* b2, float* o_perm, void* ws, size_t ws_bytes, void* stream);

/* Gated combine y[t] = sum_j gate[t][j] * o_perm[token_slot[t][j]] (Lensa ML
 * Step 3; maptheai.com "The mechanism"), accumulated in float32 in ascending j
 * and rounded once to dtype. A gather: each y row is written by one owner.
 * Entries of token_slot that are negative (slots dropped at capacity) are
 * skipped; entries of S = T*K or more give unspecified values in y but are
 * clamped, so no access leaves o_perm. Needs no workspace. Returns a moe_status. */
int moe_combine(const moe_desc* desc, const float* o_perm, const int32_t* token_slot,
                const float* topk_gate, void* y, void* stream);

/* The whole layer: route -> group -> experts -> combine, plus the aux loss.
 * In:  h, W_r, b_r (nullable), W1, b1 (nullable), W3 (SwiGLU), W2, b2 (nullable),
 *      noise [T][E] (nullable, as in moe_route).
 * Out: y, aux_loss [1] (nullable), expert_counts [E] (nullable), z_loss [1]
 *      (nullable, as in moe_route).
 * For K = 1 and no capacity the second expert GEMM writes gate * o straight
 * into y; with a capacity (desc->capacity > 0) dropped slots add nothing.
 * Returns a moe_status. */
int moe_forward(const moe_desc* desc, const void* h, const float* W_r, const float* b_r,
                const void* W1, const void* b1, const void* W3, const void* W2,
                const void* b2, void* y, float* aux_loss, int32_t* expert_counts,
                const float* noise, float* z_loss, void* ws, size_t ws_bytes, void* stream);

/* Size in bytes of the static device scratch of moe_forward_noalloc (one
 * array per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): it calls no allocating routine. Its scratch is a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES that each GPU holds from the
 * library's first call on it until the process ends; make that first call
 * outside stream capture (it looks up the array's device address once per
 * device). Layers whose moe_workspace_size() exceeds MOE_NOALLOC_SCRATCH_BYTES
 * (the Mixtral-shaped prefill layer needs about 0.43 GB; decode batches and the
 * Switch-style layer fit) return MOE_ERR_WORKSPACE with nothing enqueued.
 * All calls on one GPU share the array and it keeps the last call's contents:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give unspecified results; calls ordered on one stream are safe. The
 * kernels write every scratch byte before they read it, so nothing needs
 * clearing between calls. Arguments, outputs and numerics as moe_forward
 * (bitwise the same results). Returns a moe_status. */
int moe_forward_noalloc(const moe_desc* desc, const void* h, const float* W_r, const float* b_r,
                        const void* W1, const void* b1, const void* W3, const void* W2,
                        const void* b2, void* y, float* aux_loss, int32_t* expert_counts,
                        const float* noise, float* z_loss, void* stream);

/* Bytes of workspace moe_backward needs for this layer shape. Host-only;
 * enqueues nothing. */
int moe_backward_workspace_size(const moe_desc* desc, size_t* bytes);

/* Backward pass of the layer: gradients of loss = sum(dy * y) + daux * aux
 * + dz * z_loss with respect to every input, for bfloat16 and float32 layers
 * (bfloat16 layers round the recomputed pre-activations, the hidden
 * activation and the intermediate gradients to bfloat16; float32 layers keep
 * everything in float32). The gradient reaches the
 * router only through the gate weights of the chosen experts (maptheai.com
 * "Mixture of Experts", "The difficulties": the top-k choice is not
 * differentiable), through p_i for raw gates (Lensa ML Step 3), and through
 * P of the aux loss, whose f is a count (Step 4: only P_i is
 * differentiable); the choice and the capacity drops are held fixed, and a
 * selection-only bias gets a zero gradient. The routing (bit for bit the
 * same), the grouping and the first expert GEMM are recomputed from the
 * inputs; the caller keeps no activations.
 * In:  the forward's inputs (h, W_r, b_r, W1, b1, W3, W2, b2, noise
 *      (nullable; held fixed: an input, not differentiated)), dy [T][d] dtype,
 *      daux and dz (finite; the weights of aux and of z_loss in the loss).
 * Out: dh [T][d] dtype; dW_r [d][E], db_r [E] (nullable), dW1 [E][width][d],
 *      db1 [E][width] (nullable, GELU only), dW3 [E][width][d] (SwiGLU),
 *      dW2 [E][d][width], db2 [E][d] (nullable, GELU only), all float32.
 *      With T = 0 every gradient is zero.
 * Sums over tokens and slots run in a fixed order: results are bitwise
 * reproducible. Returns a moe_status (MOE_ERR_UNSUPPORTED for bias gradients
 * of SwiGLU layers, or transposed operands past the 32-bit offset range;
 * MOE_ERR_SHAPE for a non-finite daux or dz). */
int moe_backward(const moe_desc* desc, const void* h, const float* W_r, const float* b_r,
                 const void* W1, const void* b1, const void* W3, const void* W2, const void* b2,
                 const void* dy, float daux, const float* noise, float dz, void* dh, float* dW_r,
                 float* db_r, float* dW1, float* db1, float* dW3, float* dW2, float* db2, void* ws,
                 size_t ws_bytes, void* stream);

/* Instrumentation (not part of the layer). While enabled, every kernel the
 * library launches is bracketed by two hipEvents recorded on its launch
 * stream, for up to `capacity` launches (later launches are not traced).
 * moe_trace_enable creates the events (host-side HIP calls); moe_trace_read
 * waits for the recorded events, writes up to `max` entries of kernel id
 * (moe_kernel_id) and duration in milliseconds, sets *n, and rewinds the
 * buffer; moe_trace_disable frees the events. Not thread-safe. */
typedef enum moe_kernel_id {
  MOE_K_ROUTE = 0, MOE_K_FINALIZE = 1, MOE_K_HIST = 2,
  MOE_K_PERMUTE = 3,  /* grouping; in moe_forward for T <= 256 also the finalize statistics (one launch) */
  MOE_K_GEMM1 = 4, MOE_K_GEMM2 = 5, MOE_K_COMBINE = 6, MOE_K_ZERO = 7,
  MOE_K_BWD = 8,   /* backward pass: elementwise, transpose and reduction kernels */
  MOE_K_WGRAD = 9  /* backward pass: weight-gradient GEMMs */
} moe_kernel_id;
int moe_trace_enable(int capacity);
int moe_trace_read(int32_t* kernel_id, float* ms, int max, int* n);
int moe_trace_disable(void);

/* Name of a kernel id for reports (static string, never NULL). */
const char* moe_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
