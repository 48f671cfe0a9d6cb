/*
 * moe.h -- C ABI of the MI355X (gfx950) top-k token-choice MoE-layer forward.
 *
 * The layer (as defined on "Lab: build a tiny MoE in PyTorch", sections
 * "The contract" and "Full implementation", and "2.9 Mixture-of-Experts (MoE)
 * Architectures", section "A Toy MoE Layer From Scratch"):
 *
 *   h      = x W_r^T (+ logit_bias)                               router
 *   score  = softmax(h) over experts, or sigmoid(h)               fp32
 *   sel    = score (+ select_bias), optionally group-limited      selection
 *   ids    = top-k(sel), descending, ties to the lower index
 *   w      = route_scale * score[ids] / sum(score[ids])  (renormalize)
 *          | route_scale * score[ids]                    (otherwise)
 *   keep   = first-come per expert in token order, at most C (capacity)
 *   out[t] = sum_{kept s} w[t,s] * FFN_{ids[t,s]}(x[t])  (+ FFN_shared(x[t]))
 *   FFN(z) = W_down (silu(W_gate z) * (W_up z))
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *    and contiguous.  The library never allocates or frees memory; scratch
 *    comes from the caller's workspace of moe_workspace_bytes(cfg) bytes
 *    (256-byte aligned).
 *  - Tokens are flattened: t = b*S + s for an input of shape (B, S, D).
 *    Assignment index a = t*top_k + slot.
 *  - Weights use the nn.Linear layout per expert: w_gate, w_up [E, H, D];
 *    w_down [E, D, H]; router [E, D]; shared expert [Hs, D], [Hs, D], [D, Hs].
 *  - Calls are asynchronous on `stream`: the host validates arguments,
 *    enqueues kernels and returns; it never waits for or reads device data.
 *    Outputs are undefined if a call returns an error.  Arguments are checked
 *    before anything is enqueued, so an error status means nothing ran.
 *  - Calls on different streams with different workspaces may run
 *    concurrently; two calls sharing one workspace must be stream-ordered.
 *  - gfx950 only.  bf16 paths need D and H to be multiples of 64.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a size or switch outside its documented range   */
  MOE_ERR_NULL_PTR = 2,    /* a required pointer is NULL                      */
  MOE_ERR_UNSUPPORTED = 3, /* valid in principle, not implemented (dtype/size) */
  MOE_ERR_WORKSPACE = 4,   /* workspace NULL, misaligned or too small         */
  MOE_ERR_DEVICE = 5,      /* a pointer is not device memory of this device   */
  MOE_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed      */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
/* Router scores (NeMo Gate score_func): softmax over the experts, sigmoid,
 * or sqrt(softplus(h)); the last two are normalised over the selected
 * experts when renormalize is set.  A select_bias turns softmax and sigmoid
 * into the "_with_bias" forms (bias used for selection only). */
typedef enum {
  MOE_SCORE_SOFTMAX = 0,
  MOE_SCORE_SIGMOID = 1,
  MOE_SCORE_SQRTSOFTPLUS = 2
} moe_score;
/* Group score for group-limited routing: sum of the two largest selection
 * scores of the group, or the largest one. */
typedef enum { MOE_GROUP_TOP2SUM = 0, MOE_GROUP_MAX = 1 } moe_group_rule;

typedef struct moe_config {
  int32_t T;            /* tokens (B*S), >= 1                                  */
  int32_t D;            /* d_model                                             */
  int32_t H;            /* d_hidden of each routed expert                      */
  int32_t E;            /* routed experts, 1..256                              */
  int32_t top_k;        /* 1 <= top_k <= E, and <= 32                          */
  int32_t H_shared;     /* d_hidden of the always-on shared expert; 0 = none   */
  int32_t act_dtype;    /* moe_dtype of x, expert weights and the output       */
  int32_t router_dtype; /* moe_dtype of W_r (fp32 allowed with bf16 x)         */
  int32_t score_func;   /* moe_score                                           */
  int32_t renormalize;  /* 1: divide by the sum of the k selected scores       */
  float route_scale;    /* multiplies the final weights (1.0 if unused)        */
  int32_t n_groups;     /* contiguous expert groups (1 = no group limit)       */
  int32_t topk_groups;  /* groups each token may use, 1..n_groups              */
  int32_t group_rule;   /* moe_group_rule                                      */
  double capacity_factor; /* <= 0: dropless; else C = max(1, ceil(cf*T*k/E))   */
  float swiglu_limit;   /* > 0: gate and up projections clamped to [-L, L]
                           before silu(g)*u (NeMo MLP swiglu_limit); 0 = off   */
  int32_t pre_norm;     /* 1: moe_forward RMS-normalises x first (moe_rmsnorm)
                           and the whole layer takes the normalised rows; the
                           workspace then also holds them.  0 = off           */
  float norm_eps;       /* eps of moe_rmsnorm, finite and >= 0                */
} moe_config;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Validate the configuration alone (no pointers).  Mirrors the layer's
 * constructor checks: top_k must lie in [1, E] ("Lab: build a tiny MoE in
 * PyTorch", "Full implementation"); group settings must divide E. */
moe_status moe_check_config(const moe_config* cfg);

/* Capacity per expert for this configuration: max(1, ceil(cf*T*k/E)) in
 * double precision ("Add a capacity limit" on the lab page; "A Toy MoE Layer
 * From Scratch" on the book page), or T*k when dropless.  Returns -1 if the
 * configuration is invalid. */
int32_t moe_capacity(const moe_config* cfg);

/* Upper bound on expert-major rows: min(T*k, E*C) (T*k when dropless). */
int32_t moe_max_rows(const moe_config* cfg);

/* Workspace bytes that suffice for every entry point below with this
 * configuration (0 if the configuration is invalid). */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Routing ("Full implementation" on the lab page: router, fp32 softmax,
 * top-k, renormalised weights, bincount, balance and z losses; "The Router"
 * on the book page for the selection-only bias; NeMo Gate attributes
 * score_func / n_groups / topk_groups / route_scale).
 *   x            [T, D]   act_dtype
 *   w_router     [E, D]   router_dtype
 *   logit_bias   [E] f32 or NULL: added to the logits (softmax input, z-loss)
 *   select_bias  [E] f32 or NULL: added to the scores for selection only
 *   token_mask   [T] uint8 or NULL (all valid): 0 marks a padding token
 *                (NeMo Gate.forward token_mask); such a token is not routed:
 *                its IDs are -1 and weights 0, it adds nothing to counts, and
 *                the means in P_e and z run over the unmasked tokens only
 *   expert_ids   [T, k] int32 out: slot j = j-th largest selection score
 *   gate_w       [T, k] f32 out
 *   counts       [E] int32 out: assignments per expert before any drop
 *   aux          [2] f32 out or NULL: {balance = E*sum f_e P_e, z = mean lse^2}
 *   mean_prob    [E] f32 out or NULL: P_e = mean_t p_te (sigmoid: s_te/sum s)
 * Deterministic: repeated calls give identical bits. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* select_bias,
                     const uint8_t* token_mask, int32_t* expert_ids, float* gate_w,
                     int32_t* counts, float* aux, float* mean_prob, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Dispatch bookkeeping ("Add a capacity limit" on the lab page: keep the
 * first C assignments of each expert in token order; the sorted expert-major
 * token list of "MoE in Practice" on the book page).
 *   expert_ids     [T, k] int32 in, values in [0, E) and a token's k IDs
 *                  distinct; other values (-1 for a masked token) mean
 *                  "not routed": the slot is neither counted nor kept
 *   capacity       > 0: per-expert limit; <= 0: dropless
 *   expert_offsets [E+1] int32 out: kept rows of expert e are
 *                  [offsets[e], offsets[e+1])
 *   row_to_assign  [max_rows] int32 out: assignment a of each row, rows sorted
 *                  by (expert, token); entries past n_kept are unspecified
 *   assign_to_row  [T*k] int32 out: row of assignment a, -1 if dropped
 *   n_kept         [1] int32 out (device)
 * Integer-only and bit-exact. */
moe_status moe_permute(const moe_config* cfg, const int32_t* expert_ids,
                       int32_t capacity, int32_t* expert_offsets,
                       int32_t* row_to_assign, int32_t* assign_to_row,
                       int32_t* n_kept, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Grouped SwiGLU experts ("Full implementation" on the lab page,
 * SwiGLUExpert, and its per-expert gather / run / scale loop):
 *   y_rows[r] = g(r) * W_down,e (silu(W_gate,e x_t) * (W_up,e x_t))
 * for every row r of group e, t = row_to_assign[r] / top_k and
 * g(r) = gate_w[row_to_assign[r]] (1 if gate_w is NULL).
 *   n_experts, hidden  groups in this call and their d_hidden
 *   row_to_assign      [max_rows] int32, or NULL for the identity map
 *                      (row r = token r, one group of T rows: shared expert)
 *   expert_offsets     [n_experts+1] int32 (device), NULL with identity
 *   max_rows           host bound on the rows (grid size); rows beyond
 *                      offsets[n_experts] are neither read nor written
 *   w_gate, w_up       [n_experts, hidden, D]; w_down [n_experts, D, hidden]
 *   y_rows             [max_rows, D] act_dtype out
 *   workspace          at least max_rows*hidden act_dtype elements (the
 *                      silu(g)*u rows); a workspace of moe_workspace_bytes(cfg)
 *                      also holds the fp32 partial tiles with which the bf16
 *                      large-tile kernels split their last round along K
 *                      (without that room they run the last round unsplit;
 *                      results agree to rounding either way)
 * fp32 accumulation; silu(g)*u is rounded once to act_dtype between the two
 * GEMMs; the gate weight is applied in fp32 before the final rounding.
 * Results are deterministic for a given configuration and routing. */
moe_status moe_grouped_swiglu(const moe_config* cfg, int32_t n_experts, int32_t hidden,
                              const void* x, const int32_t* row_to_assign,
                              const int32_t* expert_offsets, int32_t max_rows,
                              const float* gate_w, const void* w_gate,
                              const void* w_up, const void* w_down, void* y_rows,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Combine ("Full implementation" on the lab page, index_add_ back to token
 * order; "Add a shared expert"; NeMo MoE shared_expert_gate):
 *   out[t] = sum_{s=0..k-1, assign_to_row[t*k+s] >= 0} y_rows[assign_to_row[t*k+s]]
 *            (+ g_t * shared_rows[t]) (+ residual[t]),
 *   g_t = sigmoid(x[t] . shared_expert_gate) when shared_expert_gate [D]
 *   (act_dtype) is given, else 1; x [T, D] is read only in that case;
 *   residual [T, D] act_dtype or NULL: the block's skip connection (may be
 *   x itself; it must not alias out unless it is out).
 * accumulated in fp32 in slot order, one rounding to act_dtype.  No atomics:
 * the result is deterministic.  A token with every slot dropped gets 0
 * (plus its shared-expert row). */
moe_status moe_combine(const moe_config* cfg, const void* y_rows,
                       const int32_t* assign_to_row, const void* shared_rows,
                       const void* x, const void* shared_expert_gate,
                       const void* residual, void* out, hipStream_t stream);

/* RMSNorm of the residual stream ahead of the layer ("Lab: build a tiny MoE
 * in PyTorch", "Put the MoE into a decoder block": the MoE branch of the
 * block takes the RMS-normalised stream; st-moe-pytorch "rms-norm": RMSNorm
 * ahead of the MoE inside SparseMoEBlock):
 *   x_norm[t, d] = x[t, d] / sqrt(mean_d' x[t, d']^2 + cfg->norm_eps) * w[d]
 *   x            [T, D] act_dtype
 *   norm_weight  [D] f32, or NULL for w = 1
 *   x_norm       [T, D] act_dtype out; may be x itself (in place)
 * x, norm_weight and x_norm must be 16-byte aligned (else MOE_ERR_INVALID_ARG).
 * The mean square and the formula are evaluated in fp64 and each output is
 * rounded once to act_dtype (bf16: nearest, ties to even), so the result is
 * the correctly rounded value of the formula up to fp64 summation order.
 * Deterministic.  A row of zeros with eps = 0 gives NaN (0/0). */
moe_status moe_rmsnorm(const moe_config* cfg, const void* x, const float* norm_weight,
                       void* x_norm, hipStream_t stream);

/* The whole forward: moe_route, moe_permute, moe_grouped_swiglu (routed and
 * shared expert) and moe_combine, stream-ordered, with no host
 * synchronisation.  With cfg->pre_norm the forward first runs moe_rmsnorm on
 * x with norm_weight (NULL: w = 1) into the workspace, and router, experts
 * and shared-expert gate take those rows; x itself is not changed (pass it
 * as residual for the block's out = x + MoE(RMSNorm(x))); norm_weight must
 * be NULL without pre_norm, and 16-byte aligned.  w_shared_* may be NULL when cfg->H_shared == 0;
 * shared_expert_gate [D] (optional, needs a shared expert) scales its output
 * per token as in moe_combine; token_mask as in moe_route; residual [T, D]
 * (optional) is added to the output as in moe_combine.  The optional
 * outputs expert_ids [T,k], gate_w [T,k], counts [E] and aux [2] receive the
 * routing results when non-NULL.  saved (optional, bf16 only; device memory
 * of moe_saved_bytes(cfg) bytes, 256-byte aligned, caller-owned) receives the
 * SwiGLU state of every routed row and of the shared expert for
 * moe_backward, which then skips recomputing it: silu(g)*u (the forward's
 * own hidden rows) and the factors d act/d g, d act/d u, bf16. */
moe_status moe_forward(const moe_config* cfg, const void* x, const float* norm_weight,
                       const void* w_router,
                       const float* logit_bias, const float* select_bias,
                       const uint8_t* token_mask, const void* w_gate, const void* w_up,
                       const void* w_down, const void* w_shared_gate,
                       const void* w_shared_up, const void* w_shared_down,
                       const void* shared_expert_gate, const void* residual, void* out,
                       int32_t* expert_ids,
                       float* gate_w, int32_t* counts, float* aux, void* saved,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes that moe_forward_noalloc holds on each GPU it runs on. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving
 * (decode) loops, harnesses that forbid hipMalloc.  Arguments, results and
 * errors are those of moe_forward; the call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  Its scratch is a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held until the process ends; a configuration whose forward needs more
 * (moe_workspace_bytes counts a larger split-K area, so it is an upper bound
 * only) returns MOE_ERR_UNSUPPORTED before anything is enqueued.  Decode-sized
 * layers fit: e.g. T = 64 tokens, D = 4096, H = 1536, E = 128, top_k = 8.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or different host threads without stream
 * order) race and give undefined results; stream-ordered calls are safe.
 * Nothing in the array needs to start at zero (each call writes what it
 * reads).  Outputs agree with moe_forward to rounding: decode-sized grouped
 * GEMMs split their last round along K exactly as moe_forward does, larger
 * tiles run it unsplit. */
moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const float* norm_weight,
                               const void* w_router, const float* logit_bias,
                               const float* select_bias, const uint8_t* token_mask,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const void* w_shared_gate, const void* w_shared_up,
                               const void* w_shared_down, const void* shared_expert_gate,
                               const void* residual, void* out, int32_t* expert_ids,
                               float* gate_w, int32_t* counts, float* aux, void* saved,
                               hipStream_t stream);

/* Bytes of the forward's saved SwiGLU state (0 if the configuration is
 * invalid or not bf16): act, d act/d g and d act/d u of moe_max_rows(cfg)
 * routed rows x H, then of T rows x H_shared. */
size_t moe_saved_bytes(const moe_config* cfg);

/* Workspace bytes of moe_backward (0 if the configuration is invalid or not
 * covered by the backward: bf16 activations only). */
size_t moe_backward_workspace_bytes(const moe_config* cfg);

/* Backward pass of the layer ("Lab: build a tiny MoE in PyTorch", "Smoke test
 * and backward pass": the loss is a task term plus alpha*balance + beta*z).
 * Gradients of  L = <dout, out> + balance_coef*balance + z_coef*z  with the
 * routes, the capacity drops and the counts f of the forward held constant
 * ("2.9 Mixture-of-Experts (MoE) Architectures": top-k is a stop-gradient on
 * the index decision ("The Router"), f is detached ("The auxiliary
 * load-balancing loss")); gradients reach the router through the gate weights
 * of the kept slots, through P_e and through z.
 *   x, norm_weight, w_router, logit_bias, w_gate, w_up, w_down, w_shared_*,
 *   shared_expert_gate: as moe_forward (x is the layer input before the
 *                       pre-norm when cfg->pre_norm = 1)
 *   expert_ids, gate_w  [T, k]: the routes and gate weights of the forward
 *                       (moe_route / moe_forward outputs; -1 marks a masked
 *                       token)
 *   dout                [T, D] act_dtype: gradient of the layer output
 *   dx                  [T, D] act_dtype out
 *   dw_router           [E, D] f32 out; dw_gate, dw_up [E, H, D] f32 out;
 *   dw_down             [E, D, H] f32 out; dws_* (shared expert) f32 out in
 *                       the shapes of w_shared_* (required when H_shared > 0)
 *   d_gate_w            [T, k] f32 out or NULL: dL/d gate weight per slot
 *                       (0 for dropped and masked slots)
 *   d_norm_weight       [D] f32 out or NULL (pre_norm only): dL/d norm weight
 *   d_shared_gate       [D] f32 out or NULL (needs shared_expert_gate):
 *                       dL/d shared-expert gate vector
 *   saved               NULL, or the state moe_forward saved for these same
 *                       inputs and routes (then the gate/up GEMMs are not
 *                       recomputed)
 * With the gated shared expert (NeMo MoE.shared_expert_gate, read as
 * g_t = sigmoid(x_t . w_sg) scaling the shared expert's output), the shared
 * expert receives g_t dout_t and the gate's logit g_t (1 - g_t) <dout_t, S_t>,
 * formed from the shared down dgrad and the saved SwiGLU output without
 * recomputing S; it reaches w_sg (fixed-order column sums) and dx.
 * With the pre-norm ("Lab: build a tiny MoE in PyTorch", "Put the MoE into a
 * decoder block": the MoE branch takes the RMS-normalised stream;
 * st-moe-pytorch "rms-norm": RMSNorm ahead of the MoE in SparseMoEBlock), the
 * rows are renormalised with the forward's kernel and the gradient passes
 * back through the norm:
 * with s = sqrt(mean(x^2) + eps) and g = norm_weight * dL/dy,
 *   dx = g / s - x * sum(g x) / (D s^3),   dL/dw_d = sum_t dL/dy_td x_td / s_t,
 * dL/dy kept fp32, dx rounded once.
 * bf16 activations only.  fp32 accumulation; intermediates (the SwiGLU factors, dL/dg and
 * dL/du, dL/dh) are rounded to bf16 between GEMMs.  Deterministic: no float
 * atomics, every sum runs in a fixed order. */
moe_status moe_backward(const moe_config* cfg, const void* x, const float* norm_weight,
                        const void* w_router, const float* logit_bias, const void* w_gate,
                        const void* w_up, const void* w_down, const void* w_shared_gate,
                        const void* w_shared_up, const void* w_shared_down,
                        const void* shared_expert_gate, const int32_t* expert_ids,
                        const float* gate_w, const void* dout, float balance_coef, float z_coef,
                        void* dx, float* dw_router, float* dw_gate, float* dw_up,
                        float* dw_down, float* dws_gate, float* dws_up, float* dws_down,
                        float* d_shared_gate, float* d_gate_w, float* d_norm_weight,
                        const void* saved, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Auxiliary-loss-free balancer step ("DeepSeek-MoE and the fine-grained +
 * shared-expert idea" and "Exercises" 6 on the book page; NeMo
 * Gate.update_bias), in place on the selection bias that moe_route adds for
 * selection only:
 *   select_bias[e] += gamma * sign(mean_e' counts[e'] - counts[e])
 * with the comparison taken exactly on integers.  counts [E] int32 (e.g. the
 * counts output of moe_route), select_bias [E] f32, both device memory;
 * gamma finite. */
moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma,
                           float* select_bias, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
