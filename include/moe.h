/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN layer, forward and backward.
 *
 * The layer (Zero to Frontier §13.1 "Why MoE", section "The MoE layer"; the routing
 * paragraph of the kevinluzbetak.com "Mixture-Of-Experts" page): for each token row x,
 *   r = x W_r (+ b)                       one fp32 logit per expert
 *   p = softmax(r)                        over all E experts, fp32
 *   K = the k experts with largest r      lower expert index wins a tie
 *   g_j = p_{K_j} / sum_{i in K} p_i      (renormalize = 1)   or   g_j = p_{K_j} (renormalize = 0)
 *   y = sum_{j : kept} g_j (SiLU(x W_g^{K_j}) * x W_u^{K_j}) W_d^{K_j}   (+ shared SwiGLU(x))
 * with an optional per-expert capacity (AI Engineering Illustrated, "The safety valve is a
 * capacity limit"): each expert keeps its first `capacity` assignments in arrival order
 * t*k + j; dropped assignments contribute nothing, so a token whose every assignment is
 * dropped gets y = 0 and the caller's residual carries it through.
 *
 * Conventions for every call below
 *   - Row-major arrays.  Weights are stored [out, in] (nn.Linear), so every product
 *     reads both operands along the contraction dimension.
 *   - Element type of x and of every weight: shape->dtype (MOE_F32 or MOE_BF16; bf16 is
 *     stored as raw 16-bit patterns).  Router bias, gates, f, P, aux, o and y are fp32.
 *     Indices and counts are int32.
 *   - Every pointer argument is DEVICE memory owned by the caller, except `shape`
 *     (host).  The library allocates nothing and keeps no state between calls; scratch
 *     comes from the caller's workspace `ws` of at least moe_workspace_bytes() bytes.
 *     Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream); no call
 *     synchronises the host.
 *   - Arguments are checked on the host before any HIP call; the first failure is
 *     returned and nothing is launched.  A failed launch returns MOE_ERR_HIP.  Kernels do
 *     not report data errors: NaN or Inf inputs, or indices outside [0, E) passed to
 *     moe_permute, are outside the contract.
 *   - Results are deterministic: the same inputs give bit-identical outputs (no float
 *     atomics; integer work is order-free or ordered).
 *
 * Supported shapes (else MOE_ERR_UNSUPPORTED or MOE_ERR_SHAPE):
 *   T >= 0; 1 <= E <= 1024; 1 <= k <= min(E, 16); d, d_e, d_e_shared multiples of 128;
 *   d_e_shared >= 0 (0 = no shared expert); T*k < 2^31; dtype in {MOE_F32, MOE_BF16};
 *   scoring in {MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID}; 1 <= n_group <= 64 dividing E;
 *   1 <= topk_group <= n_group; k <= topk_group * E / n_group; T*d*elem_size < 2^32 for
 *   moe_forward (its gather uses 32-bit byte offsets); wfmt in {MOE_W_NATIVE, MOE_W_FP8_E4M3,
 *   MOE_W_MXFP4}, quantised weights only with dtype MOE_BF16; afmt in {MOE_A_NATIVE,
 *   MOE_A_MXFP8}, MOE_A_MXFP8 only with quantised weights.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is negative or inconsistent (k > E, k < 1, ...) */
  MOE_ERR_UNSUPPORTED = 3, /* valid but outside the supported set above */
  MOE_ERR_WORKSPACE = 4,   /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 5          /* a HIP launch or runtime call failed */
} moe_status;

typedef struct {
  int32_t T;           /* tokens (rows of x) */
  int32_t d;           /* model width */
  int32_t d_e;         /* routed expert hidden width */
  int32_t E;           /* routed experts */
  int32_t k;           /* experts per token */
  int32_t capacity;    /* per-expert kept-assignment limit; < 0 = unlimited */
  int32_t renormalize; /* 1: gates renormalised over the k chosen; 0: raw softmax p */
  int32_t d_e_shared;  /* hidden width of the always-on shared expert; 0 = none */
  int32_t dtype;       /* moe_dtype of x and all weights */
  int32_t scoring;     /* moe_scoring: how router logits become scores (see below) */
  int32_t n_group;     /* expert groups (consecutive blocks of E / n_group); 1 = no group limit */
  int32_t topk_group;  /* groups a token may use (1 <= topk_group <= n_group; 1 when n_group = 1) */
  int32_t wfmt;        /* moe_wfmt of the expert weights (router weight: always dtype) */
  int32_t afmt;        /* moe_afmt of the activations entering the expert products */
} moe_shape;

/* Storage of the expert weights (routed and shared).
 * MOE_W_NATIVE:   weights in the shape's dtype.
 * MOE_W_FP8_E4M3: one byte per weight, OCP FP8 E4M3 (bias 7, subnormals, no infinities,
 *   S.1111.111 = NaN; largest finite 448), plus one fp32 scale per output row: the
 *   weight is scale[row] * e4m3(code).  The pages keep expert weights in one byte per
 *   parameter (jacopoparretti.dev, "Memory") because small batches are bound by reading
 *   them (AI Engineering Illustrated, "Trade-offs to weigh").  Products run in bf16 on the
 *   decoded codes (exact in bf16) with fp32 accumulation; the row scale multiplies each
 *   output before SiLU (gate/up) or before it is written (down).
 * MOE_W_MXFP4: OCP MX FP4 (AI Engineering Illustrated, "Total parameters and active parameters
 *   are different budgets": MoE weights kept in MXFP4).  Elements are E2M1 (bias 1; magnitudes
 *   0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte, element 2j of a row in the low nibble of byte j;
 *   every 32 consecutive elements of a row share one E8M0 scale byte (2^(s-127); 255 = NaN).
 *   Weights [G, rows, K/2] bytes; scales [G, K/32, rows] bytes (block-major).  Decoded values
 *   (element x scale, exact in bf16) feed bf16 products with fp32 accumulation. */
typedef enum { MOE_W_NATIVE = 0, MOE_W_FP8_E4M3 = 1, MOE_W_MXFP4 = 2 } moe_wfmt;

/* Activations entering the expert products (the router always sees x in dtype).
 * MOE_A_NATIVE: x and h in dtype (bf16 with quantised weights: the decoded weights meet bf16
 *   activations in bf16 products).
 * MOE_A_MXFP8: both products run on gfx950's scaled FP8 MFMA.  x (per token row) and h (per
 *   row) are OCP MXFP8: every 32 consecutive elements along the contraction share an E8M0 scale
 *   2^X, X = floor(log2 of the block's largest magnitude) - 8, and each element is the nearest
 *   E4M3 value of v / 2^X (ties to even, saturating at 448); h is rounded from its fp32 value.
 *   The weights' own scales apply as in MOE_A_NATIVE (FP8: fp32 row scales; MXFP4: E8M0 block
 *   scales, applied by the MFMA).  Requires wfmt MOE_W_FP8_E4M3 or MOE_W_MXFP4 (dtype bf16).
 *   The pages store weights in 8 or 4 bits (jacopoparretti.dev, "Memory"; AI Engineering
 *   Illustrated, "Total parameters and active parameters are different budgets") and leave the
 *   activations' format open; MXFP8 is the form the scaled MFMA consumes.  Forward only. */
typedef enum { MOE_A_NATIVE = 0, MOE_A_MXFP8 = 1 } moe_afmt;

/* Scales of quantised expert weights (device pointers; G = E for routed experts, 1 for the
 * shared expert).  K is the contraction width of the matrix: d for W_g and W_u, d_e for W_d.
 *   MOE_W_FP8_E4M3: fp32, one per row    gate, up [G, d_e];      down [G, d]
 *   MOE_W_MXFP4:    E8M0 bytes per block  gate, up [G, d/32, d_e]; down [G, d_e/32, d] */
typedef struct {
  const void *gate;    /* scales of W_g */
  const void *up;      /* scales of W_u */
  const void *down;    /* scales of W_d */
} moe_wscales;

/* Router scoring.
 * MOE_SCORE_SOFTMAX: p = softmax(r + b) over all E; the k largest p are chosen; gates are p
 *   renormalised over the k (or raw p).  b, if given, is part of the logits.
 * MOE_SCORE_SIGMOID: the DeepSeek-V3 rule (AI Engineering Illustrated, "The router is small but
 *   it decides everything" and "Fix 2 nudges a bias instead"; jacopoparretti.dev, "Experts and a
 *   router" and "A bias"): an independent affinity s = sigmoid(r) per expert; b is added to s
 *   only to choose the k experts; gates are the chosen s renormalised over the k (or raw s).
 *   P averages s.
 * Group limit (both scorings; jacopoparretti.dev, "Smaller experts, more of them"): with
 * n_group > 1 a token may only use experts of its topk_group best groups, a group's score being
 * its best member's selection score; ties go to the lower group index. */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_scoring;

/* ---------------------------------------------------------------- host-only helpers
 * No device access; usable on a machine without a GPU. */

/* Per-expert capacity floor(C * T * k / E) (the kevinluzbetak.com capacity worked
 * example counts top-k slots; at k = 1 it is AI Engineering Illustrated's
 * tokens / experts * factor).  Errors: cap NULL -> MOE_ERR_NULL; T < 0, k < 1, E < 1,
 * C < 0 or not finite, or a result >= 2^31 -> MOE_ERR_SHAPE. */
moe_status moe_capacity(int32_t T, int32_t k, int32_t E, double C, int32_t *cap);

/* Workspace bytes needed by moe_forward for this shape; the same figure covers each of
 * the split calls (moe_route, moe_permute, moe_expert_ffn).  Validates the shape. */
moe_status moe_workspace_bytes(const moe_shape *shape, size_t *bytes);

/* Static string naming a status code. */
const char *moe_status_str(moe_status status);

/* ---------------------------------------------------------------- device calls */

/* Router: logits, scores (softmax or sigmoid, see moe_scoring), top-k (group-limited when
 * n_group > 1), gates and the Switch load-balance statistics (kevinluzbetak.com page,
 * load-balancing fixes and the layer's auxiliary-loss code).
 *   x      [T, d]        dtype     token rows
 *   w_r    [E, d]        dtype     router weight
 *   b_r    [E]           fp32      per-expert bias (logit bias for softmax, selection-only bias
 *                                  for sigmoid), or NULL
 *   idx    [T, k]        int32     out: chosen experts, descending gate; idx[:,0] = top-1
 *   gate   [T, k]        fp32      out: gates
 *   counts [E]           int32     out: assignments per expert over all k choices, before capacity
 *   f      [E]           fp32      out: counts / (T*k)      (0 when T = 0)
 *   P      [E]           fp32      out: mean over tokens of p (softmax) or s (sigmoid); 0 if T = 0
 *   aux    [1]           fp32      out: E * sum_e f_e P_e (no loss weight applied)
 * Logits, softmax and selection are fp32; bf16 inputs are multiplied exactly and summed
 * in fp32. */
moe_status moe_route(const moe_shape *shape, const void *x, const void *w_r, const float *b_r,
                     int32_t *idx, float *gate, int32_t *counts, float *f, float *P, float *aux,
                     void *ws, size_t ws_bytes, void *stream);

/* Dispatch: counting sort of the T*k assignments by expert, stable in arrival order
 * t*k + j, truncated at shape->capacity, then a gather of token rows into
 * expert-contiguous order (the per-expert token lists of the PyTorch layer on the
 * kevinluzbetak.com page, laid out as one list: tokens sorted by expert).
 *   x         [T, d]      dtype     token rows
 *   idx       [T, k]      int32     expert of each assignment (each in [0, E))
 *   kept      [E]         int32     out: min(count_e, capacity)
 *   offsets   [E+1]       int32     out: exclusive scan of kept; offsets[E] = kept rows R
 *   row_token [T*k]       int32     out: token of expert-ordered row r < R (rest untouched)
 *   row_of    [T, k]      int32     out: row of assignment (t, j), or -1 if dropped
 *   x_perm    [T*k, d]    dtype     out: x_perm[r] = x[row_token[r]] for r < R */
moe_status moe_permute(const moe_shape *shape, const void *x, const int32_t *idx, int32_t *kept,
                       int32_t *offsets, int32_t *row_token, int32_t *row_of, void *x_perm,
                       void *ws, size_t ws_bytes, void *stream);

/* Grouped SwiGLU experts over expert-contiguous rows (Zero to Frontier §13.1, "The MoE
 * layer": FFN_i(x) = (SiLU(x W_g) * x W_u) W_d).  Rows offsets[e] .. offsets[e+1]-1 of
 * x_perm go through expert e; offsets[E] <= T*k.
 *   x_perm  [T*k, d]          dtype
 *   offsets [E+1]             int32
 *   w_gate  [E, d_e, d]       dtype; uint8 E4M3 codes (MOE_W_FP8_E4M3); [E, d_e, d/2] packed
 *                             E2M1 codes (MOE_W_MXFP4)
 *   w_up    [E, d_e, d]       same
 *   w_down  [E, d, d_e]       same ([E, d, d_e/2] for MOE_W_MXFP4)
 *   scales  scales of the three (required iff wfmt != MOE_W_NATIVE, else ignored)
 *   o       [T*k, d]          fp32      out: rows < offsets[E]; the rest untouched
 * The hidden activation is rounded to dtype between the two products (bf16 RNE for
 * MOE_BF16).  The shared expert is this call with E = 1, k = 1, d_e = d_e_shared and
 * offsets = {0, T}. */
moe_status moe_expert_ffn(const moe_shape *shape, const void *x_perm, const int32_t *offsets,
                          const void *w_gate, const void *w_up, const void *w_down,
                          const moe_wscales *scales, float *o, void *ws, size_t ws_bytes, void *stream);

/* Gate-weighted combine back to token order (the layer's weighted sum,
 * Zero to Frontier "The MoE layer" equation):
 *   y[t] = shared_out[t] (or 0) + sum_{j = 0..k-1, row_of[t,j] >= 0} gate[t,j] * o[row_of[t,j]]
 * summed in that fixed order.
 *   o [T*k, d] fp32; row_of [T, k] int32; gate [T, k] fp32; shared_out [T, d] fp32 or NULL;
 *   y [T, d] fp32 out. */
moe_status moe_combine(const moe_shape *shape, const float *o, const int32_t *row_of,
                       const float *gate, const float *shared_out, float *y, void *stream);

/* The whole layer: route -> dispatch -> grouped experts (+ shared expert) -> combine.
 * Arguments as in the split calls; ws_gate/ws_up ([d_e_shared, d]) and ws_down
 * ([d, d_e_shared]) are the shared expert's weights, required iff d_e_shared > 0.
 * scales / shared_scales: scales of the routed / shared expert weights, required
 * (shared_scales iff d_e_shared > 0) when wfmt != MOE_W_NATIVE, else ignored.
 * offsets [E+1], row_token [T*k] and row_of [T, k] are optional outputs (NULL: kept in the
 * workspace).
 * stage_events: NULL, or a host array of MOE_NUM_STAGES + 1 hipEvent_t (created by the
 * caller) that the call records on `stream` at the stage boundaries, in the order of
 * moe_stage, then once after the last stage; elapsed time between events i and i+1 is
 * stage i.  NULL entries are skipped (record only the boundaries you need: each record
 * costs a few microseconds of stream time).  Stages that do not run for this shape (the
 * shared expert when d_e_shared = 0) are recorded as empty.  For timing only; results do
 * not depend on it. */
typedef enum {
  MOE_STAGE_ROUTER = 0,      /* logits, softmax, top-k, gates, partial statistics */
  MOE_STAGE_SCAN = 1,        /* counts, capacity, offsets, f, P, aux */
  MOE_STAGE_PERMUTE = 2,     /* stable ranks, row_of / row_token, gather into x_perm */
  MOE_STAGE_GATE_UP = 3,     /* grouped SiLU(x W_g) * (x W_u) */
  MOE_STAGE_DOWN = 4,        /* grouped h W_d */
  MOE_STAGE_SHARED_GATE_UP = 5,
  MOE_STAGE_SHARED_DOWN = 6,
  MOE_STAGE_COMBINE = 7,     /* gate-weighted sum back to token order */
  MOE_NUM_STAGES = 8
} moe_stage;

moe_status moe_forward(const moe_shape *shape, const void *x, const void *w_r, const float *b_r,
                       const void *w_gate, const void *w_up, const void *w_down,
                       const void *ws_gate, const void *ws_up, const void *ws_down,
                       const moe_wscales *scales, const moe_wscales *shared_scales,
                       float *y, int32_t *idx, float *gate, int32_t *counts, int32_t *kept,
                       float *f, float *P, float *aux,
                       int32_t *offsets, int32_t *row_token, int32_t *row_of,
                       void *ws, size_t ws_bytes, void *stream, void *const *stage_events);

/* moe_forward for callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc.  The same layer, the same
 * kernels and bit-identical outputs as moe_forward; instead of a caller workspace it uses a
 * scratch array of MOE_STATIC_SCRATCH_BYTES (64 MiB) compiled into the library, one per GPU,
 * held by each GPU the library runs on until the process ends.  It allocates nothing (no
 * hipMalloc, hipFree or allocating library call); the device address of the current device's
 * scratch is looked up (hipGetSymbolAddress) on that device's first call.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (two streams,
 * two host threads, or a call enqueued while another is still running) race and give wrong
 * results.  Calls ordered on one stream are safe.  No part of the scratch needs clearing
 * between calls (every byte a call reads is written earlier in the same call).
 * Errors: as moe_forward, checked on the host before any HIP call; a shape whose workspace
 * (moe_workspace_bytes) exceeds MOE_STATIC_SCRATCH_BYTES -> MOE_ERR_WORKSPACE (e.g. more than
 * about 600 tokens at the Mixtral 8x7B layer shape, or 160 at the DeepSeek-V3 shape with its
 * shared expert); more than 64 GPUs, or a failed lookup -> MOE_ERR_HIP. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_shape *shape, const void *x, const void *w_r, const float *b_r,
                               const void *w_gate, const void *w_up, const void *w_down,
                               const void *ws_gate, const void *ws_up, const void *ws_down,
                               const moe_wscales *scales, const moe_wscales *shared_scales,
                               float *y, int32_t *idx, float *gate, int32_t *counts, int32_t *kept,
                               float *f, float *P, float *aux,
                               int32_t *offsets, int32_t *row_token, int32_t *row_of,
                               void *stream, void *const *stage_events);

/* MXFP8 rows (the MOE_A_MXFP8 activation format) of x [rows, K] (bf16, 16-byte aligned; device):
 * codes [rows, K] E4M3 bytes and scales [rows, K/32] E8M0 bytes (device, caller-owned).  The
 * same rounding the layer applies to its activations.  Errors: rows < 0 or K not a positive
 * multiple of 32 -> MOE_ERR_SHAPE; a NULL pointer with rows > 0 -> MOE_ERR_NULL; a failed
 * launch -> MOE_ERR_HIP. */
moe_status moe_mxfp8_quantize(int32_t rows, int32_t K, const void *x, uint8_t *codes, uint8_t *scales,
                              void *stream);

/* ---------------------------------------------------------------- backward pass */

/* Workspace bytes needed by moe_backward for this shape (validates it; native weights only). */
moe_status moe_backward_workspace_bytes(const moe_shape *shape, size_t *bytes);

/* Gradients of L = sum(dy * y) + d_aux * aux for the layer of moe_forward, with that forward's
 * routing held fixed.  The choice of experts is a hard selection and carries no gradient: the
 * router learns only through the weights of the experts it chose (Moatlab AI-064,
 * "Inside the Router"); aux = E * sum_e f_e P_e adds d_aux * E * f_e / T to dL/dp[t, e] (f_e
 * are counts).  Capacity drops are part of the routing: a dropped assignment passes no
 * gradient, and a kept gate is not renormalised over the survivors.
 *   x, w_r, b_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down   as given to moe_forward
 *   idx, gate, counts, offsets, row_token, row_of                moe_forward's outputs for them
 *   dy      [T, d]        fp32   dL/dy
 *   d_aux                 host   dL/daux (e.g. the auxiliary-loss weight)
 * Outputs (fp32, overwritten; layouts of the corresponding inputs):
 *   dx [T, d]; dw_r [E, d]; db_r [E] or NULL (the logit bias under softmax scoring gets
 *   sum_t dL/dr_t; under sigmoid scoring the bias only picks experts and gets 0);
 *   dw_gate, dw_up [E, d_e, d]; dw_down [E, d, d_e] (an expert with no rows gets zeros);
 *   dws_gate, dws_up [d_e_shared, d], dws_down [d, d_e_shared] (required iff d_e_shared > 0);
 *   dgate [T, k] or NULL: dL/dg per slot (0 for a dropped slot).
 * Precision: the gate/up products are recomputed (bit-identical to the forward's); every
 * product takes dtype operands with fp32 accumulation, so with MOE_BF16 dy, g * dy, dA and dB
 * are rounded to bf16 before the products that consume them (as h is in the forward); router
 * gradients, dW_r and the sums into dx are fp32.  Deterministic (fixed summation orders).
 * Only wfmt = MOE_W_NATIVE (else MOE_ERR_UNSUPPORTED).
 * stage_events: NULL or a host array of MOE_NUM_BSTAGES + 1 hipEvent_t, recorded as for
 * moe_forward at the boundaries of the stages of moe_bstage.  For timing only. */
typedef enum {
  MOE_BSTAGE_PREP = 0,           /* padded layouts, transposed weights, dy to dtype */
  MOE_BSTAGE_RECOMPUTE = 1,      /* gate/up products again: a, b, and h transposed */
  MOE_BSTAGE_DOWN_BWD = 2,       /* u = dy W_d, dA, dB, dL/dg partial dots */
  MOE_BSTAGE_ROUTER_BWD = 3,     /* dL/dg, dL/dr */
  MOE_BSTAGE_DX_EXPERT = 4,      /* dX = dA W_g + dB W_u per row */
  MOE_BSTAGE_WGRAD_DOWN = 5,     /* dW_d = (g dy)^T h per expert */
  MOE_BSTAGE_WGRAD_GATE_UP = 6,  /* dW_g = dA^T x, dW_u = dB^T x per expert */
  MOE_BSTAGE_SHARED = 7,         /* the shared expert's backward */
  MOE_BSTAGE_DX = 8,             /* dx = dr W_r + sum of rows + shared; dW_r, db_r */
  MOE_NUM_BSTAGES = 9
} moe_bstage;

moe_status moe_backward(const moe_shape *shape, const void *x, const void *w_r, const float *b_r,
                        const void *w_gate, const void *w_up, const void *w_down,
                        const void *ws_gate, const void *ws_up, const void *ws_down,
                        const int32_t *idx, const float *gate, const int32_t *counts,
                        const int32_t *offsets, const int32_t *row_token, const int32_t *row_of,
                        const float *dy, float d_aux,
                        float *dx, float *dw_r, float *db_r, float *dw_gate, float *dw_up, float *dw_down,
                        float *dws_gate, float *dws_up, float *dws_down, float *dgate,
                        void *ws, size_t ws_bytes, void *stream, void *const *stage_events);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
