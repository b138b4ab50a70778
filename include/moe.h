/*
 * moe.h -- C ABI of the sparse Mixture-of-Experts layer forward pass on one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer maps token representations x [T, d_model] to y [T, d_model]:
 *   1. router   : logits h(x) = W_r . x, gates p = softmax(h), top-k experts
 *                 (Switch Transformers notes, section 2.1, Eq. 1; top-1 Switch
 *                 routing; top-2 X-MoE routing from the TorchScale review), or a
 *                 weightless uniform pick inside the token's expert group
 *                 (PanGu-Sigma review, Random Routed Experts);
 *   2. dispatch : capacity-limited slot assignment (Switch notes, section 2.2,
 *                 Eq. 3 and the token-dropping rule);
 *   3. gather   : rows of x copied into an expert-major buffer;
 *   4. experts  : y_e = act(x_e W1_e) W2_e per expert;
 *   5. combine  : y = sum over the token's served choices of p_i(x) E_i(x)
 *                 (Switch notes, section 2.1, Eq. 2).
 *
 * Conventions shared by every entry point
 *   - Pointers named x, w_r, bias, group_id, w1, w2, y, expert_idx, gate, slot,
 *     expert_count, slot_token, x_e, y_e and ws are DEVICE pointers owned by the
 *     caller.  The library allocates nothing and keeps no state between calls
 *     (moe_forward_noalloc's static scratch aside, see there).
 *     `cfg` is a HOST pointer, read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All GPU work is enqueued on it; no call synchronises the host.  Results
 *     are valid once the caller has synchronised the stream.
 *   - Return value: MOE_OK, or a negative status.  On MOE_ERR_ARG and
 *     MOE_ERR_UNSUPPORTED nothing was launched and no output was touched;
 *     moe_last_error() returns a message (thread-local, valid until the next
 *     call on the same thread).  MOE_ERR_HIP means a HIP launch failed;
 *     outputs are then undefined.  Faults inside kernels surface at the
 *     caller's next synchronisation, as for any HIP work.
 *   - All buffers must be 16-byte aligned (torch allocations are 256-byte).
 *   - Shapes are row-major, last index contiguous.  "dtype" below means
 *     cfg->dtype: MOE_DTYPE_BF16 (raw bfloat16) or MOE_DTYPE_F32.
 *   - Supported sizes: T >= 0; 1 <= E <= 512; 1 <= k <= min(E, 8);
 *     d_model and d_ff positive multiples of 64; capacity_factor finite > 0;
 *     RRE needs k == 1, n_groups >= 1 and E % n_groups == 0.
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by events).
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;
/* Expert activation.  RELU / GELU: the plain FFN act(x W1) W2 (GELU in its erf
 * form, x * (1 + erf(x / sqrt 2)) / 2, with erf evaluated within 4.3e-7).  REGLU / GEGLU: the gated-linear-unit FFN of the MosaicBERT review
 * (methodology: gated linear units in the feed-forward layer),
 * (act(x W) * (x V)) W2 with act ReLU / GELU, the product elementwise; W and V
 * are stored stacked in w1 (see moe_expert_ffn), so w1 has 2 * d_ff rows. */
typedef enum { MOE_ACT_RELU = 0, MOE_ACT_GELU = 1, MOE_ACT_REGLU = 2, MOE_ACT_GEGLU = 3 } moe_act;
typedef enum { MOE_ROUTE_TOPK = 0, MOE_ROUTE_RRE = 1 } moe_route;

enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,          /* a null pointer, a bad enum or an inconsistent size */
  MOE_ERR_UNSUPPORTED = -2,  /* valid configuration outside the supported sizes */
  MOE_ERR_HIP = -3           /* a HIP runtime call or kernel launch failed */
};

typedef struct moe_config {
  int64_t T;               /* tokens in the call (all sequences flattened)          */
  int64_t d_model;         /* token width                                            */
  int64_t d_ff;            /* expert hidden width                                    */
  int32_t E;               /* experts                                                */
  int32_t k;               /* expert choices per token                               */
  double capacity_factor;  /* Switch notes 2.2, Eq. 3                                */
  int32_t route;           /* moe_route                                              */
  int32_t n_groups;        /* RRE: expert groups (experts g*E/n_groups ... next)     */
  uint64_t rre_seed;       /* RRE: SplitMix64 seed                                   */
  int32_t act;             /* moe_act: ReLU, GELU (erf form), or their GLU forms    */
  int32_t dtype;           /* moe_dtype of x, w1, w2, x_e, y_e, y                    */
} moe_config;

/* Expert capacity C = ceil(k * T * capacity_factor / E), evaluated exactly on
 * the binary value of capacity_factor (Switch notes 2.2, Eq. 3; each token
 * takes k slots, and the fraction rounds up).  Returns C >= 0, or a negative
 * status for an invalid configuration. */
int64_t moe_capacity(const moe_config* cfg);

/* Bytes of device workspace every entry point below needs (`ws`).  It holds
 * the step-wise scratch (router histograms, slot offsets, the split router
 * weight, the expert hidden activations) and, for moe_forward, every
 * intermediate result at the offsets of moe_workspace_offset.  Negative status
 * on an invalid configuration. */
int64_t moe_workspace_bytes(const moe_config* cfg);

/* Regions of the workspace that moe_forward fills, for inspection after the call.
 * One exception: on bfloat16 layers with capacity <= 64, d_model <= 768 and
 * E <= 512, and on bfloat16 layers with capacity > 160 and d_model < 2048, the
 * up-projection inside moe_forward reads each slot's token row from x itself
 * (through slot_token), and moe_forward leaves MOE_WS_X_E unwritten there
 * (moe_dispatch always writes its x_e; moe_backward gathers the rows again). */
typedef enum {
  MOE_WS_EXPERT_IDX = 0,   /* int32 [T, k]                                   */
  MOE_WS_GATE = 1,         /* float [T, k]                                   */
  MOE_WS_SLOT = 2,         /* int32 [T, k]                                   */
  MOE_WS_EXPERT_COUNT = 3, /* int32 [E]                                      */
  MOE_WS_SLOT_TOKEN = 4,   /* int32 [E, C]                                   */
  MOE_WS_X_E = 5,          /* dtype [E, C, d_model]                          */
  MOE_WS_HIDDEN = 6,       /* dtype [E, C, d_ff]  hidden activations H       */
  MOE_WS_Y_E = 7,          /* dtype [E, C, d_model]                          */
  MOE_WS_N_REGIONS = 8
} moe_ws_region;

/* Byte offset of a region inside the workspace (256-byte aligned), or a
 * negative status. */
int64_t moe_workspace_offset(const moe_config* cfg, int32_t region);

/* Step 1, router.  Switch notes 2.1 (logits h = W_r . x, Eq. 1 softmax gate,
 * top-k set) and 2.4 (router arithmetic in float32); TorchScale review (X-MoE
 * top-1/top-2); PanGu-Sigma review (RRE).
 *   x          [T, d_model] dtype
 *   w_r        [E, d_model] float32 (learned routing; ignored for RRE)
 *   bias       [E] float32 or NULL: added to each logit after the dot product,
 *              with one float32 rounding
 *   group_id   [T] int32 (RRE only; NULL for learned routing)
 *   expert_idx [T, k] int32 out: column c is the (c+1)-th choice; larger logit
 *              first, equal logits to the lower expert index.  RRE: expert
 *              g*(E/n_groups) + (SplitMix64 output t for rre_seed) mod
 *              (E/n_groups); a group id outside [0, n_groups) gives -1.
 *   gate       [T, k] float32 out: raw softmax probability of the chosen
 *              expert over all E (no renormalisation); RRE: 1 (0 for -1).
 *   ws         workspace of moe_workspace_bytes(cfg) bytes (scratch).
 * The logits are computed in float32 arithmetic (bf16 x is widened exactly;
 * the float32 w_r is split into three bfloat16 terms when it is not already
 * bfloat16-exact, so each product is exact). */
int moe_router(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
               const int32_t* group_id, int32_t* expert_idx, float* gate, void* ws,
               void* stream);

/* Step 1 plus the load-balancing auxiliary loss of Switch notes 2.2 (Eq. 4-6),
 * learned routing only (RRE has no router probabilities: MOE_ERR_UNSUPPORTED).
 * Arguments and results of moe_router, and
 *   alpha  the loss coefficient (Switch uses 1e-2)
 *   aux    [1 + 2E] float32 out: aux[0] = alpha * E * sum_i f_i * P_i,
 *          aux[1 + i] = f_i, the fraction of the T tokens whose first choice
 *          (the argmax of the router probability, equal logits to the lower
 *          index) is expert i, before any capacity drop (Eq. 5);
 *          aux[1 + E + i] = P_i, the mean over the T tokens of the router
 *          probability of expert i (Eq. 6).
 * P_i sums float32 probabilities per router block in a fixed order and the
 * blocks in float64, so repeated calls give identical bits.  T must be >= 1. */
int moe_router_aux(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                   int32_t* expert_idx, float* gate, double alpha, float* aux, void* ws,
                   void* stream);

/* Steps 2 and 3, capacity-limited dispatch and gather.  Switch notes 2.2
 * (Eq. 3 capacity; an assignment to a full expert is dropped).
 * Assignments are placed choice by choice and, inside a choice, in token
 * order: every first choice takes its slot before any second choice.
 *   x            [T, d_model] dtype
 *   expert_idx   [T, k] int32; entries outside [0, E) are not routed
 *   slot         [T, k] int32 out: slot in the expert's buffer, -1 if dropped
 *   expert_count [E] int32 out: filled slots per expert (<= C)
 *   slot_token   [E, C] int32 out: token of each slot, -1 where empty
 *   x_e          [E, C, d_model] dtype out: x_e[e, s] = x[slot_token[e, s]] for
 *                s < expert_count[e]; rows past the count are not written.
 *   ws           workspace (scratch). */
int moe_dispatch(const moe_config* cfg, const void* x, const int32_t* expert_idx, int32_t* slot,
                 int32_t* expert_count, int32_t* slot_token, void* x_e, void* ws, void* stream);

/* Step 4, expert FFN.  Switch notes 2.1 (one FFN E_i per expert):
 * y_e[e, s] = H[e, s] W2_e for s < expert_count[e], W2_e = w2[e]^T, with the
 * hidden activations H[e, s] = act(x_e[e, s] W1_e), W1_e = w1[e]^T, or, for the
 * GLU activations (MosaicBERT review, methodology), H[e, s] = act(x_e[e, s] W_e)
 * * (x_e[e, s] V_e) with W_e^T = w1[e][0 : d_ff] and V_e^T = w1[e][d_ff : 2 d_ff].
 *   x_e          [E, C, d_model] dtype (rows past the count are never read)
 *   expert_count [E] int32 (values above C are treated as C)
 *   w1           [E, d_ff, d_model] dtype (stored output x input);
 *                GLU: [E, 2 * d_ff, d_model], the W rows then the V rows
 *   w2           [E, d_model, d_ff] dtype (stored output x input)
 *   y_e          [E, C, d_model] dtype out (rows past the count are not written)
 *   ws           workspace: the hidden activations H in dtype.
 * bf16: matrix products on bf16 MFMA with float32 accumulation; H and y_e are
 * rounded to bf16 (GLU: the gate product is formed in float32 from the two
 * float32 accumulators, then rounded once).  f32: float32 throughout. */
int moe_expert_ffn(const moe_config* cfg, const void* x_e, const int32_t* expert_count,
                   const void* w1, const void* w2, void* y_e, void* ws, void* stream);

/* Step 4 in one launch, without the hidden activations in memory (bf16 only;
 * capacity 1..64, d_model a multiple of 384, d_ff a multiple of 128, ReLU or
 * GELU; otherwise MOE_ERR_UNSUPPORTED).  Same arguments and results as moe_expert_ffn, bit for
 * bit (each hidden and output element is accumulated from the same bf16
 * products in the same order), and no workspace: per expert, d_ff is walked in
 * chunks of 128 whose activated hidden tile stays in on-chip memory and is
 * multiplied into register accumulators of y_e at once.  It moves no hidden
 * bytes but streams w1 once per 384-column group of y_e; moe_expert_ffn is the
 * faster choice on the Switch-Base shape (E=128, d_model=768, C=64). */
int moe_expert_ffn_fused(const moe_config* cfg, const void* x_e, const int32_t* expert_count,
                         const void* w1, const void* w2, void* y_e, void* stream);

/* The two halves of step 4, for callers that keep the hidden activations:
 *   moe_expert_up:   hidden[e, s] = H[e, s] as in moe_expert_ffn (one grouped GEMM
 *                    launch; GLU: the gate product in its epilogue)
 *   moe_expert_down: y_e[e, s]    = hidden[e, s] W2_e     (one grouped GEMM launch)
 * for s < expert_count[e]; hidden is [E, C, d_ff] in dtype (caller-owned device
 * memory; rows past the count are not written / not read).  moe_expert_ffn is
 * moe_expert_up followed by moe_expert_down through the workspace. */
int moe_expert_up(const moe_config* cfg, const void* x_e, const int32_t* expert_count,
                  const void* w1, void* hidden, void* stream);
int moe_expert_down(const moe_config* cfg, const void* hidden, const int32_t* expert_count,
                    const void* w2, void* y_e, void* stream);

/* Step 5, combine.  Switch notes 2.1, Eq. 2: y[t] = sum over c with
 * slot[t, c] >= 0 of gate[t, c] * y_e[expert_idx[t, c], slot[t, c]],
 * accumulated in float32 in choice order; a token with no served choice gets
 * y[t] = 0 (Switch notes 2.2: it continues through the residual, which is the
 * caller's).
 *   y_e [E, C, d_model] dtype; expert_idx, slot [T, k] int32; gate [T, k] float;
 *   y   [T, d_model] dtype out. */
int moe_combine(const moe_config* cfg, const void* y_e, const int32_t* expert_idx,
                const int32_t* slot, const float* gate, void* y, void* stream);

/* The whole layer, steps 1-5, on one stream.  Same arguments and results as
 * the step-wise calls, bit for bit; every intermediate is left in `ws` at the
 * offsets of moe_workspace_offset (x_e: see moe_ws_region).  Capacity comes
 * from the configuration alone, so no device-to-host copy happens anywhere. */
int moe_forward(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                const int32_t* group_id, const void* w1, const void* w2, void* y, void* ws,
                void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as moe_forward minus `ws`:
 * the intermediates go to a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * (80 MiB, enough for a Switch-Base-sized layer: E = 128, capacity 64,
 * d_model 768, d_ff 3072 needs 73.2 MiB) that each GPU the library runs on holds
 * from the first call on it until the process ends.  Nothing in the call
 * allocates.  Nothing in the scratch needs to start at zero: every kernel writes
 * what it later reads.  Every call on one GPU shares that GPU's array and leaves
 * its intermediates there, laid out as moe_workspace_offset describes, until the
 * next call; calls that overlap on one GPU (other streams, other threads) race
 * on it and must be serialised by the caller.
 * MOE_ERR_UNSUPPORTED (nothing launched) when moe_workspace_bytes(cfg) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES; MOE_ERR_HIP if the array's device address cannot be
 * obtained on the current device. */
#define MOE_NOALLOC_SCRATCH_BYTES (80LL << 20)
int moe_forward_noalloc(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                        const int32_t* group_id, const void* w1, const void* w2, void* y,
                        void* stream);

/* Bytes of the second device workspace moe_backward needs (`bws`: its scratch;
 * the forward workspace `ws` keeps the forward's results).  Negative status on an
 * invalid configuration. */
int64_t moe_backward_workspace_bytes(const moe_config* cfg);

/* Backward pass of the whole layer (training): gradients of a loss L through
 * y = sum over served choices c of p_{i_c}(x) E_{i_c}(x) (Switch notes 2.1,
 * Eq. 2; the gate keeps the router differentiable), E_i = act(x W1_i) W2_i and
 * p = softmax(W_r x + bias) (Eq. 1); for the GLU activations
 * E_i = (act(x W_i) * (x V_i)) W2_i.  The chosen experts and the capacity drop
 * (2.2) are piecewise constant: no gradient flows through them and a dropped
 * choice contributes nothing.  Random routed experts have constant gates 1, so
 * the router gets no gradient (w_r, bias, dw_r, dbias are ignored).
 * Precondition: `ws` holds the results of moe_forward on the same cfg, x, w_r,
 * bias, w1 and w2 (routing, slots, x_e, hidden activations and y_e); the
 * router is run again here and rewrites identical values into `ws`, and where
 * moe_forward left x_e unwritten (see moe_ws_region) it is gathered here from
 * x and slot_token.
 *   dy    [T, d_model] dtype: dL/dy
 *   dx    [T, d_model] dtype out: dL/dx (expert path plus router path)
 *   dw_r  [E, d_model] float32 out (learned routing): dL/dW_r
 *   dbias [E] float32 out or NULL: dL/dbias (the sum of dL/dh over tokens)
 *   dw1   [E, d_ff, d_model] (GLU: [E, 2 * d_ff, d_model]), dw2 [E, d_model, d_ff]
 *         dtype out: dL/dw1, dL/dw2
 *         (every element written; zero for experts that served no token)
 *   bws   workspace of moe_backward_workspace_bytes(cfg) bytes.
 * bf16: products on bf16 MFMA with float32 accumulation; dy_e = gate * dy, dZ,
 * dx_e and the outputs are rounded to bf16; the pre-activation (GELU, and both
 * halves for GLU) is recomputed in bf16.  The router gradient is float32 (float32 MFMA); its token
 * contraction is split into at most 64 ranges (a function of E and d_model)
 * added in order, so repeated calls give identical bits. */
int moe_backward(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                 const void* w1, const void* w2, const void* dy, void* dx, float* dw_r,
                 float* dbias, void* dw1, void* dw2, void* ws, void* bws, void* stream);

/* SparseClip (TorchScale review, methodology): gradient clipping for sparse MoE
 * models whose norm re-weights the MoE gradients by kappa = 1/sqrt(E) against the
 * dense ones, norm = ||(g_dense, kappa g_moe)||_2.  Here the dense gradients are
 * the router's (dw_r, dbias: each may be NULL) and the MoE gradients the
 * experts' (dw1, dw2, dtype, as moe_backward writes them).  Every gradient is
 * multiplied in place by coef = min(1, max_norm / (norm + 1e-6)) (float32
 * product, rounded to the gradient's dtype).
 *   norm_coef  [2] float32 out (device): norm, coef
 *   bws        the backward workspace (moe_backward_workspace_bytes).
 * Sums of squares run in float64 in a fixed order (identical bits on repeat). */
int moe_sparse_clip(const moe_config* cfg, float* dw_r, float* dbias, void* dw1, void* dw2,
                    double max_norm, float* norm_coef, void* bws, void* stream);

/* Message of the last non-OK status on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
