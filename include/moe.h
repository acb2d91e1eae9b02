/*
 * moe.h -- C ABI of libmoe: the forward pass of a sparse Mixture-of-Experts
 * FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer follows the page "Mixture of experts" (rayaq.ca,
 * ml-models/mixture-of-experts), section Mechanics:
 *   h = W_r x,  p = softmax(h),  y = sum_{i in TopK(h)} g_i(x) E_i(x)
 * ("Replacing the feed-forward block"), with the gate conventions of
 * "Top-k gating", the statistics of "The load-balancing loss" and the
 * capacity rule of "Capacity and dropped tokens"; the expert is the
 * bias-free SwiGLU (or a ReLU/GELU FFN) of the Implementation section,
 * whose loop over experts is replaced here by a sort of tokens by expert
 * and a grouped matrix multiply, as that section describes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers to row-major arrays, owned by
 *    the caller, aligned to 16 bytes.  The library never allocates or frees
 *    device memory and keeps no per-call state.
 *  - "act dtype" below means fp32 when desc->dtype == MOE_DTYPE_F32 and
 *    bf16 (uint16 bit patterns) when desc->dtype == MOE_DTYPE_BF16.  The
 *    router (W_r, bias, noise, logits) is always fp32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and runs asynchronously; no call synchronises with the host.  Results
 *    are valid once the caller has synchronised the stream.  Calls on
 *    distinct streams with distinct buffers may run concurrently.
 *  - Every argument is validated before anything is enqueued: a call that
 *    returns an error has launched nothing.  Errors are returned as status
 *    codes (below); nothing is thrown across the ABI.  A fault inside a
 *    kernel (e.g. a pointer to too small a buffer) cannot be detected by
 *    the call and surfaces at the caller's next synchronisation.
 *  - `ws` is a device workspace of at least moe_workspace_size() bytes,
 *    `ws_bytes` its size.  Its contents on entry do not matter.
 *  - Given the same inputs, every output is bitwise reproducible: no
 *    floating-point atomics are used, and every sum runs in a fixed order.
 *
 * Shapes (T tokens, d model width, d_ff expert hidden width, E experts,
 * k experts per token):
 *   x            [T][d]        act dtype    tokens, batch and sequence flattened
 *   W_r          [E][d]        fp32         router rows
 *   bias         [E]           fp32         optional router bias (NULL = none)
 *   noise        [T][E]        fp32         optional logit noise (NULL = none)
 *   W1, W3       [E][d_ff][d]  act dtype    up projections (W3 only for SwiGLU)
 *   W2           [E][d][d_ff]  act dtype    down projection
 *   topk_idx     [T][k]        int32        chosen experts, largest logit first
 *   gates        [T][k]        fp32         gate of each chosen expert
 *   routed_counts[E]           int32        assignments per expert before drops
 *   kept_counts  [E]           int32        min(routed, C)
 *   offsets      [E+1]         int32        exclusive prefix sum of kept_counts
 *   row_of_slot  [T][k]        int32        permuted row of (t, s), -1 if dropped
 *   token_of_row [T*k]         int32        token of each permuted row; entries
 *                                           at and after offsets[E] are -1
 *   dropped      [T][k]        uint8        1 if (t, s) was dropped by capacity
 *   x_perm       [T*k][d]      act dtype    x rows in expert order (first
 *                                           offsets[E] rows written)
 *   y_perm       [T*k][d]      fp32         expert outputs in the same order
 *   y            [T][d]        act dtype    layer output
 *   stats        [2E+2]        fp32         f[E], P[E], aux, z (see moe_route)
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* bad size, null required pointer, bad enum */
#define MOE_ERR_UNSUPPORTED (-2) /* valid but outside what the kernels handle */
#define MOE_ERR_HIP (-3)         /* the HIP runtime reported an error        */
#define MOE_ERR_WORKSPACE (-4)   /* ws_bytes below moe_workspace_size()       */
#define MOE_ERR_SCRATCH (-5)     /* moe_forward_noalloc: needs more than the
                                    static scratch (MOE_NOALLOC_SCRATCH_BYTES) */

/* ---- gate conventions ("Top-k gating") ---------------------------------- */
/* Renormalised top-k (Mixtral): softmax over the k selected logits. */
#define MOE_GATE_RENORM 0
/* Switch: the full-softmax probability p of each selected expert (k = 1 is
 * the Switch Transformer gate; k > 1 keeps p for every selected expert). */
#define MOE_GATE_SWITCH 1

/* ---- expert activation --------------------------------------------------- */
#define MOE_ACT_RELU 0   /* W2 relu(W1 x)                                   */
#define MOE_ACT_GELU 1   /* W2 gelu(W1 x), exact erf form                   */
#define MOE_ACT_SWIGLU 2 /* W2 (silu(W1 x) * W3 x)  ("Implementation")      */

/* ---- storage type of x, expert weights, x_perm and y --------------------- */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* Router logits of one token live in registers: E is at most this. */
#define MOE_MAX_EXPERTS 128

/* Number of kernel stages of moe_forward, for the optional stage events. */
#define MOE_FORWARD_STAGES 7

/*
 * Problem description: the page's MoE(d, d_ff, num_experts, k, capacity)
 * plus the batch size T, the gate convention, the activation and the
 * storage type.
 *
 * capacity_factor: 0 means no capacity limit (dropless).  Otherwise the
 * capacity of every expert is C = ceil(capacity_factor * T * k / E),
 * evaluated in double precision in exactly that order ("Capacity and
 * dropped tokens": tokens per batch over experts, times the factor; with k
 * slots per token the batch holds T*k assignments).  Each expert keeps its
 * first C assignments in token order and drops the rest.
 *
 * stage_events / n_stage_events: optional profiling hook.  When non-NULL,
 * stage_events points to n_stage_events hipEvent_t handles; moe_forward
 * records event j after its j-th kernel stage (event 0 before the first),
 * for j < n_stage_events, on `stream`; MOE_FORWARD_STAGES + 1 events
 * bracket every stage, and a NULL entry is skipped (each recorded event
 * separates the kernels around it by a few microseconds, so record only
 * the ones needed).  The two events around expert-up, which is one kernel,
 * are instead timestamped by that kernel's launch (its start and end): they
 * add no gap; in moe_forward the same holds for the two around the combine
 * (so the expert-down stage then ends at the combine's start).  NULL disables the hook.  The stages, in order: route,
 * route-finalize, dispatch, gather, expert-up, expert-down, combine; in
 * moe_forward the gather is folded into expert-up (its rows of x are read
 * through token_of_row), so that stage is empty, and the statistics are
 * finished by extra blocks of the dispatch launch, so route-finalize is
 * empty as well.  moe_dispatch takes events 0 and 1, when given, as the
 * start and end timestamps of its gather launch.
 * The other entry points ignore it.
 */
typedef struct moe_desc {
    int32_t T, d, d_ff, E, k;
    int32_t gate;  /* MOE_GATE_*  */
    int32_t act;   /* MOE_ACT_*   */
    int32_t dtype; /* MOE_DTYPE_* */
    double capacity_factor;
    void *const *stage_events;
    int32_t n_stage_events;
} moe_desc;

/*
 * Workspace bytes needed by any entry point for this description.
 * Returns MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED (the same
 * validation as the compute calls).  Host only; enqueues nothing.
 */
int moe_workspace_size(const moe_desc *desc, size_t *bytes);

/*
 * The capacity C for this description, or -1 when there is no limit.
 * Host only.
 */
int moe_capacity(const moe_desc *desc, int64_t *capacity);

/*
 * Router, gate and load-balancing statistics ("Replacing the feed-forward
 * block", "Top-k gating", "The load-balancing loss").
 *   h[t][i]  = sum_j x[t][j] W_r[i][j] + bias[i] + noise[t][i]   (fp32)
 *   p[t]     = softmax(h[t]),  lse[t] = log sum_i exp h[t][i]
 *   topk_idx = the k largest logits, largest first, ties to the lower index
 *   gates    = RENORM: softmax over the k selected logits
 *              SWITCH: p of each selected expert
 *   stats    = f[E]  : share of tokens whose top choice (slot 0) is i,
 *                      counted before any capacity drop
 *              P[E]  : mean over tokens of p[t][i]
 *              aux   : E * sum_i f[i] P[i]   (unweighted; 1 when balanced)
 *              z     : mean over tokens of lse[t]^2   (unweighted)
 * Inputs x, W_r, bias?, noise?; outputs topk_idx, gates, stats.
 */
int moe_route(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
              const float *noise, int32_t *topk_idx, float *gates, float *stats, void *ws,
              size_t ws_bytes, void *stream);

/*
 * Capacity and dispatch ("Capacity and dropped tokens"; the
 * Implementation section's sort of tokens by expert).  For each expert,
 * its assignments (t, s) are ranked in token order; the first C are kept
 * and laid out expert after expert (expert e owns rows
 * [offsets[e], offsets[e+1]) in token order), the rest are dropped.
 * Then x_perm[r] = x[token_of_row[r]] for r < offsets[E].
 * Input x, topk_idx; outputs routed_counts, kept_counts, offsets,
 * row_of_slot, token_of_row, dropped, x_perm.
 * topk_idx must hold, for every token, k distinct experts in [0, E) (as
 * moe_route returns them).  An entry outside [0, E), or one repeating an
 * expert of an earlier slot of the same token, is not a valid choice: it is
 * treated as dropped (dropped = 1, row_of_slot = -1) and counted nowhere,
 * so no expert gets more rows than tokens.
 */
int moe_dispatch(const moe_desc *desc, const void *x, const int32_t *topk_idx,
                 int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                 int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, void *x_perm,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Expert FFNs as a grouped matrix multiply over the ragged per-expert row
 * blocks given by offsets (read on the device; the host never learns the
 * counts).  For every row r of expert e (offsets[e] <= r < offsets[e+1]):
 *   H      = act(x_perm[r] W1_e^T) [* (x_perm[r] W3_e^T) for SwiGLU]
 *   y_perm[r] = H W2_e^T
 * H is kept in the workspace in the act dtype; accumulation is fp32.  When
 * the down projection has too few output tiles to fill the GPU (bf16, long
 * d_ff) it sums K in two halves; the second half's fp32 partial rows are
 * kept in the workspace and added into y_perm before the call returns (in
 * moe_forward the combine adds them), so the result does not depend on
 * which entry point ran.
 * Experts with no rows read none of their weights.  W3 must be NULL
 * unless act is SwiGLU (then it is required).
 */
int moe_expert_ffn(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                   const void *W1, const void *W3, const void *W2, float *y_perm, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * Gate-weighted combine (the equation for y): for every token t,
 *   y[t] = sum_{s = 0..k-1, row_of_slot[t][s] >= 0} gates[t][s] * y_perm[row_of_slot[t][s]]
 * summed in fp32 in slot order and stored in the act dtype.  A token whose
 * every slot was dropped gets 0 (the residual outside the layer carries
 * it).  Gates are not renormalised after drops.
 */
int moe_combine(const moe_desc *desc, const float *y_perm, const int32_t *row_of_slot,
                const float *gates, void *y, void *stream);

/*
 * The whole layer: moe_route, moe_dispatch, moe_expert_ffn and moe_combine
 * in sequence on `stream`, with x_perm and y_perm held in the workspace.
 * Required: x, W_r, W1, W2 (W3 for SwiGLU), y, ws.  Every other output
 * pointer may be NULL, in which case that tensor lives in the workspace
 * and is not returned.
 */
int moe_forward(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                const float *noise, const void *W1, const void *W3, const void *W2, void *y,
                int32_t *topk_idx, float *gates, int32_t *routed_counts, int32_t *kept_counts,
                int32_t *offsets, int32_t *row_of_slot, int32_t *token_of_row,
                uint8_t *dropped, float *stats, void *ws, size_t ws_bytes, void *stream);

/* ---- shared experts and the block residual --------------------------------
 *
 * Section "Total versus active parameters" of the page names DeepSeek-V3's
 * layer: many small routed experts beside shared experts that every token
 * visits.  The Implementation section's block adds the layer output to its
 * hidden state (h + moe_out).  Here a shared expert has the routed experts'
 * shape and activation, no gate (weight 1), and runs on every token,
 * including tokens that capacity dropped from every routed expert ("Capacity
 * and dropped tokens": such a token keeps its residual; no routing decision
 * touches a shared expert).  The layer output becomes
 *   y[t] = residual[t] + ( sum over kept slots, in slot order, of
 *                          gates[t][s] * y_perm[row_of_slot[t][s]]
 *                        + y_shared[t] )
 *   y_shared[t] = sum over j = 0..S-1 of E^shared_j(x[t])
 * summed in fp32 in that order (routed slots, shared experts, residual) and
 * stored once in the act dtype.
 *
 * All S shared experts see every token, so they run as one dense layer:
 * the up projection against their W1 (and W3) read as [S*d_ff][d], and the
 * down projection with K = S*d_ff, whose fp32 accumulation sums the S
 * experts (in expert order within each K block).  y_shared is that sum;
 * each expert's own output is not formed.
 *
 * Shapes (S shared experts):
 *   W1, W3      [S][d_ff][d]  act dtype   up projections (W3 only for SwiGLU)
 *   W2          [S][d][d_ff]  act dtype   down projection
 *   residual    [T][d]        act dtype   optional (NULL = none)
 *   y_shared    [T][d]        fp32        summed output of the shared experts
 */

/* Shared experts per layer: at most this many. */
#define MOE_MAX_SHARED 16

/* Kernel stages of moe_forward_shared: those of moe_forward with "shared"
 * (the shared experts' two matrix multiplies) between expert-down and
 * combine. */
#define MOE_FORWARD_SHARED_STAGES 8

typedef struct moe_shared {
    int32_t n_shared;     /* S, 0 <= S <= MOE_MAX_SHARED                    */
    const void *W1;       /* [S][d_ff][d]; required when S > 0              */
    const void *W3;       /* [S][d_ff][d]; SwiGLU only (then required)      */
    const void *W2;       /* [S][d][d_ff]; required when S > 0              */
    const void *residual; /* [T][d] or NULL                                 */
} moe_shared;

/*
 * Workspace bytes for the entry points below with this description and
 * S = shared->n_shared shared experts (at least moe_workspace_size(); for
 * S > 1 it holds a copy of the shared W2 laid out [d][S*d_ff]).  Same
 * validation and return codes as moe_workspace_size; an S outside
 * [0, MOE_MAX_SHARED] is MOE_ERR_INVALID_ARG, S*d_ff >= 2^31
 * MOE_ERR_UNSUPPORTED.  Only n_shared is read.  Host only.
 */
int moe_workspace_size_shared(const moe_desc *desc, const moe_shared *shared, size_t *bytes);

/*
 * The shared experts on every token: y_shared[t] = sum over j of
 * E^shared_j(x[t]), E^shared_j being the expert of moe_expert_ffn on
 * shared->W1/W3/W2[j] (H in the act dtype in the workspace, fp32
 * accumulation; a K split of the down projection is added back before the
 * call returns).  shared->residual is ignored.  S = 0 enqueues nothing.
 * ws: moe_workspace_size_shared() bytes.
 */
int moe_shared_ffn(const moe_desc *desc, const moe_shared *shared, const void *x,
                   float *y_shared, void *ws, size_t ws_bytes, void *stream);

/*
 * The combine of moe_combine plus the shared experts' summed output and
 * the residual, fused in one pass (the equation above).  y_shared and
 * residual may each be NULL (that term is absent); with both NULL the
 * result equals moe_combine's bit for bit.
 */
int moe_combine_shared(const moe_desc *desc, const float *y_perm, const int32_t *row_of_slot,
                       const float *gates, const float *y_shared, const void *residual, void *y,
                       void *stream);

/*
 * The whole layer with shared experts and the residual: moe_forward's
 * stages, then the shared experts on every token (moe_shared_ffn, with
 * y_shared in the workspace), then the fused combine (moe_combine_shared).
 * Arguments as moe_forward, plus `shared` (required; S = 0 and no residual
 * give moe_forward's results bit for bit).  ws: moe_workspace_size_shared()
 * bytes.  Stage events, when given, follow MOE_FORWARD_SHARED_STAGES.
 */
int moe_forward_shared(const moe_desc *desc, const moe_shared *shared, const void *x,
                       const float *W_r, const float *bias, const float *noise, const void *W1,
                       const void *W3, const void *W2, void *y, int32_t *topk_idx, float *gates,
                       int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                       int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped,
                       float *stats, void *ws, size_t ws_bytes, void *stream);

/* ---- expert weights in 8-bit floating point (E4M3) ----------------------------
 *
 * Page "Mixture of experts", Mechanics, "Total versus active parameters":
 * decoding at small batch sizes is limited by reading expert weights;
 * "Tradeoffs": quantisation helps serving.  The glossary page "Mixture of
 * Experts (MoE)" (inferensys.com, inference optimization), entry on model
 * quantization: post-training quantisation of a trained model's weights.
 * Here every weight row i (a row of W1[e], W3[e] or W2[e]) is stored as
 * E4M3 codes (the Open Compute Project 8-bit floating point format: bias
 * 7, 3 mantissa bits, largest value 448, 0x7F/0xFF NaN) and one fp32
 * scale: row i = s[i] * value(q[i][:]).  Activations stay bf16; the codes
 * are widened to bf16 exactly inside the kernels, and each row's
 * accumulated product is multiplied by its scale in fp32.
 *
 * Shapes:
 *   W1, W3   [E][d_ff][d]  uint8  e4m3 codes (W3 only for SwiGLU)
 *   W2       [E][d][d_ff]  uint8  e4m3 codes
 *   s1, s3   [E][d_ff]     fp32   scales of the rows of W1, W3
 *   s2       [E][d]        fp32   scales of the rows of W2
 */
typedef struct moe_fp8_experts {
    const uint8_t *W1, *W3, *W2;
    const float *s1, *s3, *s2;
} moe_fp8_experts;

/*
 * Row-wise post-training quantisation of a [rows][cols] matrix (fp32 when
 * dtype is MOE_DTYPE_F32, bf16 when MOE_DTYPE_BF16) to E4M3 codes q
 * [rows][cols] and scales [rows]:
 *   amax = max_j |W[i][j]|,  scales[i] = fl32(amax / 448)  (1 when that is 0)
 *   q[i][j] = e4m3(clamp(fl32(W[i][j] / scales[i]), -448, 448))
 * with correctly rounded fp32 divisions and the conversion rounding to the
 * nearest e4m3 value, ties to the even code; the largest magnitude of each
 * row becomes +-448.  Finite inputs only (a NaN in a row makes that row
 * unspecified).  Applied to an expert weight tensor viewed as
 * [E * rows_per_expert][cols] it gives the codes and scales above.
 * rows = 0 enqueues nothing.  Errors: MOE_ERR_INVALID_ARG (bad dtype,
 * rows < 0, cols < 1, null pointer with rows > 0).
 */
int moe_quantize_e4m3(int32_t dtype, const void *W, int64_t rows, int64_t cols, uint8_t *q,
                      float *scales, void *stream);

/*
 * moe_expert_ffn with E4M3 expert weights.  Supported for decode-sized
 * batches, where reading the weights is the bound: desc->dtype bf16, at
 * most 48 rows per expert (T, or the capacity C when smaller, <= 48), and
 * d, d_ff multiples of 128; otherwise MOE_ERR_UNSUPPORTED.  w->W3 and
 * w->s3 are required for SwiGLU and must be NULL otherwise.
 */
int moe_expert_ffn_fp8(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                       const moe_fp8_experts *w, float *y_perm, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * moe_forward with E4M3 expert weights (w in place of W1, W3, W2); the
 * same shapes are supported as for moe_expert_ffn_fp8.  Routing, dispatch,
 * statistics and the combine are those of moe_forward.  ws:
 * moe_workspace_size() bytes.  Stage events as moe_forward.
 */
int moe_forward_fp8(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                    const float *noise, const moe_fp8_experts *w, void *y, int32_t *topk_idx,
                    float *gates, int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                    int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, float *stats,
                    void *ws, size_t ws_bytes, void *stream);

/* ---- expert weights in the streaming tile layout ------------------------------
 *
 * Page "Mixture of experts", Mechanics, "Total versus active parameters":
 * at small batch sizes a step is limited by reading the expert weights.
 * For such batches (the shapes moe_expert_ffn_fp8 accepts: bf16
 * activations, at most 48 rows per expert, d and d_ff multiples of 128) the
 * expert GEMMs stream every touched weight row once, 16 rows at a time per
 * wavefront.  In row-major storage each of their 16-byte load instructions
 * touches 16 rows; in the streaming tile layout the same values are ordered
 * so that each instruction reads 1 KB of contiguous memory, which the
 * memory system serves faster.  The values, the products and their order
 * are unchanged, so the results equal those of moe_forward (bf16 weights)
 * or moe_forward_fp8 (e4m3 codes) bit for bit.  Packing is a one-time
 * re-ordering of the weights, done when they are loaded.
 *
 * Streaming tile layout of a [rows][cols] matrix of elem_bytes-byte
 * elements (2: bf16, 1: e4m3 codes), rows % 16 == 0, cols % 128 == 0, in
 * units of 16 bytes (16 / elem_bytes elements):
 *   - blocks of 16 rows x 128 columns; block (rb, cb) (rows 16 rb ..,
 *     columns 128 cb ..) is the (rb * cols / 128 + cb)-th block of
 *     128 * elem_bytes units;
 *   - in row n (0..15) of a block, unit u covers columns
 *     u * 16 / elem_bytes .. +16 / elem_bytes of the block; with
 *     V = 2 * elem_bytes units per 32 columns, unit u = V * g + r
 *     (g = 0..3, r = 0..V-1) is stored at unit position r * 64 + 16 * g + n
 *     of the block.
 * An expert weight tensor [E][rows_per_expert][cols] is packed as one
 * [E * rows_per_expert][cols] matrix (rows_per_expert % 16 == 0 keeps every
 * block inside one expert).  Row scales of e4m3 weights stay as
 * moe_quantize_e4m3 writes them.
 */
#define MOE_WEIGHTS_BF16 1 /* bf16 values (the value of MOE_DTYPE_BF16) */
#define MOE_WEIGHTS_E4M3 2 /* e4m3 codes with fp32 row scales           */

typedef struct moe_packed_experts {
    int32_t format;            /* MOE_WEIGHTS_BF16 or MOE_WEIGHTS_E4M3 */
    const void *W1, *W3, *W2;  /* packed [E*d_ff][d], [E*d_ff][d] (SwiGLU only), [E*d][d_ff] */
    const float *s1, *s3, *s2; /* E4M3: scales [E][d_ff], [E][d_ff] (SwiGLU only), [E][d];
                                  BF16: all NULL */
} moe_packed_experts;

/*
 * Writes W [rows][cols] (elem_bytes 2 or 1) to W_packed (rows * cols *
 * elem_bytes bytes, not overlapping W) in the streaming tile layout.
 * rows = 0 enqueues nothing.  Errors: MOE_ERR_INVALID_ARG (elem_bytes not
 * 1 or 2, rows < 0, rows % 16 != 0, cols < 128, cols % 128 != 0, null
 * pointer with rows > 0).
 */
int moe_pack_stream(int32_t elem_bytes, const void *W, int64_t rows, int64_t cols, void *W_packed,
                    void *stream);

/*
 * moe_expert_ffn with packed expert weights.  Supported shapes are those of
 * moe_expert_ffn_fp8 (otherwise MOE_ERR_UNSUPPORTED).  MOE_ERR_INVALID_ARG
 * for an unknown format, a missing W1/W2 (or, for e4m3, s1/s2), or W3 (s3)
 * given without SwiGLU or missing with it; scales given for bf16 weights.
 */
int moe_expert_ffn_packed(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                          const moe_packed_experts *w, float *y_perm, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * moe_forward with packed expert weights (w in place of W1, W3, W2), for the
 * shapes of moe_expert_ffn_packed.  Routing, dispatch, statistics and the
 * combine are those of moe_forward; ws: moe_workspace_size() bytes; stage
 * events as moe_forward.
 */
int moe_forward_packed(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                       const float *noise, const moe_packed_experts *w, void *y, int32_t *topk_idx,
                       float *gates, int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                       int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, float *stats,
                       void *ws, size_t ws_bytes, void *stream);

/* ---- backward (training gradients) -------------------------------------------
 *
 * Page "Mixture of experts", Mechanics: the top-k choice is discrete, but
 * the gate values are differentiable, which is how the router learns
 * ("Replacing the feed-forward block"); "The load-balancing loss": with f_i
 * a count, d aux / d P_i = E f_i; the z statistic is mean_t lse_t^2.
 * moe_backward gives the gradients of
 *     L = sum_t <dy_t, y_t> + alpha_aux * aux + alpha_z * z
 * with respect to x, W_r, the router bias and the expert weights, for the
 * routing moe_forward took (held fixed: pass its topk_idx, gates, offsets,
 * row_of_slot, token_of_row and stats, with the same x, weights, bias and
 * noise).  The expert activations are recomputed (nothing else of the
 * forward is needed).  bf16 layers: at most about 4.19 million kept rows
 * (65535 * 64 once each expert's count is rounded up to 64),
 * MOE_ERR_UNSUPPORTED otherwise, before any launch.  fp32 layers: any shape
 * the forward takes.
 *   dy     [T][d]          the layer's dtype (bf16 or fp32): gradient of
 *                          the layer output
 *   dx     [T][d]          fp32
 *   dW_r   [E][d]          fp32
 *   dbias  [E]             fp32   optional (requires bias)
 *   dW1, dW3 [E][d_ff][d]  fp32   (dW3 exactly for SwiGLU)
 *   dW2    [E][d][d_ff]    fp32
 * Every gradient is written in full (an expert without rows gets zeros);
 * sums run in a fixed order, so results are reproducible.  Internally the
 * weights are transposed into the workspace once per call and the expert
 * GEMMs use the forward's grouped GEMM kernels.  bf16 layers: the weight
 * gradients are a GEMM over each expert's row block (activations transposed
 * into a layout whose experts start on multiples of 64 rows, zero-padded)
 * and intermediate activations are rounded to bf16; fp32 layers keep every
 * intermediate in fp32 and sum each weight gradient over the expert's rows
 * in row order.  ws: moe_backward_workspace_size() (it differs by dtype).
 */
int moe_backward_workspace_size(const moe_desc *desc, size_t *bytes);

int moe_backward(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                 const float *noise, const void *W1, const void *W3, const void *W2,
                 const int32_t *topk_idx, const float *gates, const int32_t *offsets,
                 const int32_t *row_of_slot, const int32_t *token_of_row, const float *stats,
                 const void *dy, float alpha_aux, float alpha_z, float *dx, float *dW_r,
                 float *dbias, float *dW1, float *dW3, float *dW2, void *ws, size_t ws_bytes,
                 void *stream);

/* ---- a forward pass that allocates nothing ----------------------------------
 *
 * For callers that cannot call hipMalloc or take a workspace argument:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  moe_forward_noalloc is moe_forward (same arguments minus ws
 * and ws_bytes, same kernels, same results bit for bit) whose workspace is a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES inside the library: each
 * device the library runs on holds its own copy of that array from its first
 * use until the process ends.  The call allocates nothing and calls no
 * allocating routine; its first call on a device looks up that device's
 * copy (hipGetSymbolAddress) with the device current.
 *
 * Limit: the description's moe_workspace_size() must be at most
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. a decode batch of the
 * Mixtral-shape layer, or T = 4096 on the Switch-shape layer); larger
 * problems return MOE_ERR_SCRATCH before anything is enqueued.
 * Every call on one device shares that device's array, which keeps the
 * last call's contents: calls that overlap on one device (concurrent
 * streams, or host threads) race and must be serialised by the caller
 * (successive calls on one stream are ordered and safe).  Nothing in the
 * array needs to start at zero: the kernels initialise what they read.
 * Other errors as moe_forward; a failed device lookup returns MOE_ERR_HIP.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int moe_forward_noalloc(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                        const float *noise, const void *W1, const void *W3, const void *W2,
                        void *y, int32_t *topk_idx, float *gates, int32_t *routed_counts,
                        int32_t *kept_counts, int32_t *offsets, int32_t *row_of_slot,
                        int32_t *token_of_row, uint8_t *dropped, float *stats, void *stream);

/* A static, human-readable name for a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
