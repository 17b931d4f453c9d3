/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer library (libmoe_mi355x.so):
 * the forward pass, its fixed-capacity variant and router variants, and the
 * backward pass.
 *
 * The layer: a router picks, for every token, the k best of E experts; the
 * token is sent through those experts' MLPs and their outputs are summed with
 * the renormalised gate weights.  Sources (page titles, with sections):
 *   [OPS]  aicoding.csdn.net article on the ops-transformer MoE operators:
 *          "原理：MoE的稀疏路由是怎么工作的" Steps 1-4; "坑1：负载均衡";
 *          "实现" (MoEGatingForward); "使用" (MyMoELayer, MoEForward,
 *          MoELoadBalance).
 *   [RTR]  "MoE Router：谁来决定 Token 去哪个 Expert": MoERouter snippet,
 *          load-balancing passage, capacity-limit passage.
 *   [MB]   "01 · MoE 为什么难算：变长专家输入" (MegaBlocks chapter 1):
 *          sections 3, 4.1-4.6.
 *   [CAI]  "在 Colossal-AI 中为你的模型集成混合专家（MoE）...": SparseMLP data
 *          flow, MoeLoss.
 *   [CANN] "MoE 路由算子到底在做什么？一次拆透 ops-transformer 的核心机制":
 *          sections 2-3, 7 (SwiGLU experts).
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers to row-major, contiguous arrays,
 *     16-byte aligned.  The caller allocates and owns all memory, including
 *     the workspace `ws`; the library never allocates, frees, synchronises,
 *     prints or keeps state between calls.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns before it runs.  Concurrent calls on
 *     different streams with different workspaces are independent.
 *   - Arguments are checked on the host before any HIP call.  On an error
 *     nothing is enqueued and no output is written.  T == 0 returns MOE_OK
 *     and does nothing.
 *   - Expert ids must lie in [0, E).  Logits must be finite (NaN/Inf give
 *     unspecified routing).
 *   - dtype MOE_BF16: x, W1, W3, W2, x_perm, out_perm and y are bf16 (raw
 *     16-bit patterns); the router (W_gate, logit_bias, logits, weights) is
 *     always fp32.  MOE_F32: everything fp32.
 *   - Limits: 1 <= k <= E; E <= 256 (MOE_ERR_UNSUPPORTED beyond: one 8-bit
 *     digit for the sort by expert id); k <= 16; h and f multiples of 64.  The
 *     expert GEMMs address their left operand with 32-bit element offsets, so the
 *     entry points that run them return MOE_ERR_UNSUPPORTED when T*h, R*h or R*f
 *     reaches 2^32 (R: the rows the GEMMs may get, min(T*k, E*C), or R_max).
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
  MOE_ERR_ARG = 1,          /* null required pointer, bad size, k out of range, non-finite factor */
  MOE_ERR_UNSUPPORTED = 2,  /* E > 256, k > 16, h or f not a multiple of 64, misaligned pointer */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the entry point needs */
  MOE_ERR_DEVICE = 4        /* a kernel launch failed (hipGetLastError) */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act_t;

/* moe_route flag: `logits` is an input (fp32 [T,E]); x, W_gate, logit_bias are ignored. */
#define MOE_ROUTE_LOGITS_IN 1u

/* Per-expert capacity C = floor(cf * (T*k/E)) ([MB] sections 3 and 4.2: tokens per
 * expert first, then the factor, then truncation).  Returns INT32_MAX ("never drop")
 * when cf <= 0 or the computed C is 0 ([MB] section 4.6), and -1 for invalid
 * arguments (T < 0, E < 1, k < 1, cf not finite).  The factor is widened to double
 * before the product.  Host only. */
int32_t moe_capacity(int32_t T, int32_t E, int32_t k, float capacity_factor);

/* Bytes of workspace that suffice for every entry point below at these sizes
 * (the amount moe_layer_forward needs).  0 for invalid sizes. */
size_t moe_workspace_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                           float capacity_factor, moe_dtype_t dt, moe_act_t act);

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status_t s);

/* Router: logits = x . W_gate (+ logit_bias), softmax, top-k selection, renormalised
 * weights ([OPS] Steps 1-2 and MoEGatingForward; [RTR] MoERouter; routing in fp32 per
 * [CAI] SparseMLP step 2).
 *   x        [T,h] (dt)          W_gate [h,E] fp32        logit_bias [E] fp32 or NULL
 *   logits   [T,E] fp32: output (input with MOE_ROUTE_LOGITS_IN)
 *   topk_idx [T,k] int32: slot j = j-th best expert; order (logit desc, expert asc)
 *   topk_w   [T,k] fp32: softmax of the selected logits (sums to 1 per token)
 *   prob_sum [E] fp32 or NULL: sum over tokens of the full softmax (for the aux loss)
 *   ws: at least moe_route_workspace_bytes(T,h,E,dt,flags,prob_sum != NULL) bytes: for
 *       bf16 x the split router weights (from 32 experts up) and, for few tokens, partial
 *       logits; per-block softmax sums (prob_sum); may be NULL when that is 0. */
size_t moe_route_workspace_bytes(int32_t T, int32_t h, int32_t E, moe_dtype_t dt, uint32_t flags,
                                 int32_t with_prob_sum);  /* 0 for invalid sizes */
moe_status_t moe_route(const void* x, const float* W_gate, const float* logit_bias,
                       int32_t T, int32_t h, int32_t E, int32_t k, moe_dtype_t dt, uint32_t flags,
                       float* logits, int32_t* topk_idx, float* topk_w, float* prob_sum,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Router variants, for training and benchmarking (all optional; NULL options = the plain
 * router).  Random numbers are inputs: the caller draws them.
 *   jitter      [T,h] in x's dtype or NULL: the router sees x * jitter, rounded to the
 *               dtype (bf16: to nearest even); the experts still read x.  Multiplicative
 *               noise in [1-eps, 1+eps] on the router input ([MB] section 5, jitter).
 *   logit_noise [T,E] fp32 or NULL: added (in fp32) to the logits before the softmax and
 *               the top-k ([CAI] Top2Router with a NormalNoiseGenerator); the logits
 *               returned by moe_route_ex are the router's own, without the noise.
 *   temperature > 0: probabilities p = softmax(logits / temperature), used for the
 *               weights and the aux loss; the selection still ranks the (noisy) logits,
 *               the same order for any temperature.  1 = plain.
 *   uniform_assignment nonzero: the expert id of slot j of token t is replaced by
 *               (t*k + j) % E; the weights stay those of the real top-k ([MB] section 5,
 *               the benchmark-only uniform assignment).
 *   soft_topk nonzero: soft top-K ([OPS] "坑3：数值稳定性": instead of a hard top-K, a
 *               softmax with a temperature over all experts, so that the experts that are
 *               not selected keep a little probability and receive gradient).  The k best
 *               experts still run, weighted by p at the selection WITHOUT renormalising
 *               over the k: topk_w[t,j] = p[t, topk_idx[t,j]], summing to less than 1; the
 *               rest of the mass belongs to the unselected experts, whose logits get
 *               gradient through the softmax's denominator (moe_layer_backward_ex).
 *               0 = renormalised weights (the plain router).
 * Errors: MOE_ERR_ARG for a temperature that is not finite and > 0, or jitter together
 * with MOE_ROUTE_LOGITS_IN; MOE_ERR_UNSUPPORTED for a jitter buffer or x not 16-byte
 * aligned.  With jitter the entry points need moe_router_opts_workspace_bytes(...) bytes
 * of workspace beyond their usual amount (the jittered router input). */
typedef struct {
  const void* jitter;
  const float* logit_noise;
  float temperature;
  int32_t uniform_assignment;
  int32_t soft_topk;
} moe_router_opts_t;
size_t moe_router_opts_workspace_bytes(int32_t T, int32_t h, moe_dtype_t dt, const moe_router_opts_t* opts);
moe_status_t moe_route_ex(const void* x, const float* W_gate, const float* logit_bias,
                          int32_t T, int32_t h, int32_t E, int32_t k, moe_dtype_t dt, uint32_t flags,
                          const moe_router_opts_t* opts, float* logits, int32_t* topk_idx,
                          float* topk_w, float* prob_sum, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Permutation: histogram, capacity, prefix sum and a STABLE sort of the T*k assignments
 * s = t*k+j by expert id, then the gather of token rows ([MB] sections 4.1, 4.2, 4.5, 4.6).
 *   topk_idx [T,k] int32 (ids in [0,E)),  x [T,h] (dt) -- may be NULL when x_perm is NULL
 *   counts   [E] int32: assignments per expert BEFORE any drop
 *   offsets  [E+1] int32: exclusive starts over the KEPT rows; offsets[E] = R rows kept
 *   sorted_slot [T*k] int32: row r -> assignment s (first R entries valid)
 *   slot_pos [T*k] int32: assignment s -> row, -1 if dropped (rank >= C in ascending s)
 *   x_perm   [T*k,h] (dt) or NULL: row r = x[sorted_slot[r]/k] for r < R
 *   prob_sum [E] fp32 or NULL (from moe_route), aux_loss: device fp32 scalar or NULL --
 *            when both are given, aux = E * sum_e (counts_e/(T*k)) * (prob_sum_e/T),
 *            unscaled ([OPS] 坑1; [RTR] load-balancing passage; [CAI] MoeLoss).
 *   ws: at least moe_permute_workspace_bytes(T,E,k) bytes (per-block expert counts and
 *       scatter bases, and the row -> token map). */
size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t k);  /* 0 for invalid sizes */
moe_status_t moe_permute(const int32_t* topk_idx, const void* x, int32_t T, int32_t h, int32_t E,
                         int32_t k, float capacity_factor, moe_dtype_t dt,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                         void* x_perm, const float* prob_sum, float* aux_loss,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Experts: for the rows r in segment e = [offsets[e], offsets[e+1]) of x_perm,
 *   SwiGLU: out_perm[r] = (silu(x_perm[r] W1[e]) * (x_perm[r] W3[e])) W2[e]
 *   GELU:   out_perm[r] = gelu(x_perm[r] W1[e]) W2[e]     (exact erf form)
 * ([MB] section 4.3: matmul, activation, matmul per expert; SwiGLU per the
 * ops-transformer operator list).  Offsets are read on the device; experts with no rows
 * read no weights.  In bf16 the hidden activation is rounded to bf16 before W2.
 *   x_perm [R_max,h], W1/W3 [E,h,f], W2 [E,f,h] (dt); W3 must be NULL iff GELU.
 *   offsets [E+1] int32 (device), R_max >= offsets[E] (rows allocated in x_perm/out_perm)
 *   out_perm [R_max,h] (dt): rows >= offsets[E] are not written.
 *   ws: at least moe_expert_ffn_workspace_bytes(R_max,h,f,E,dt,act) bytes (the hidden
 *       activation, plus fp32 partial sums when few rows per expert make the library
 *       split K to fill the GPU, or the raw SwiGLU pre-activations [R_max, 2f] fp32
 *       that the up projection writes when few rows per expert make it stream weights). */
size_t moe_expert_ffn_workspace_bytes(int32_t R_max, int32_t h, int32_t f, int32_t E, moe_dtype_t dt,
                                      moe_act_t act);  /* 0 for invalid sizes */
moe_status_t moe_expert_ffn(const void* x_perm, const int32_t* offsets, int32_t R_max,
                            int32_t h, int32_t f, int32_t E, const void* W1, const void* W3,
                            const void* W2, moe_act_t act, moe_dtype_t dt, void* out_perm,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine: y[t] = sum over j with slot_pos[t*k+j] >= 0 of topk_w[t,j] * out_perm[slot_pos[t*k+j]],
 * fp32 accumulation in ascending j; a token whose slots were all dropped gets 0
 * ([OPS] Step 4; [MB] sections 4.3 and 4.5).  No workspace.
 *   out_perm [*,h] (dt), slot_pos [T*k] int32, topk_w [T,k] fp32, y [T,h] (dt). */
moe_status_t moe_unpermute(const void* out_perm, const int32_t* slot_pos, const float* topk_w,
                           int32_t T, int32_t h, int32_t k, moe_dtype_t dt, void* y,
                           hipStream_t stream);

/* The whole layer: route -> permute (with capacity) -> experts -> combine, plus the aux
 * loss from the same histogram.  x [T,h]; W_gate [h,E] fp32; logit_bias [E] fp32 or NULL;
 * W1/W3 [E,h,f], W2 [E,f,h] (dt; W3 NULL iff GELU); y [T,h] (dt).
 * aux_loss: device fp32 scalar or NULL.  counts: device int32 [E] (pre-drop) or NULL.
 * ws: at least moe_workspace_bytes(T,h,f,E,k,capacity_factor,dt,act) bytes. */
moe_status_t moe_layer_forward(const void* x, const float* W_gate, const float* logit_bias,
                               const void* W1, const void* W3, const void* W2,
                               int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                               float capacity_factor, moe_act_t act, moe_dtype_t dt,
                               void* y, float* aux_loss, int32_t* counts,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Where a moe_layer_forward (or _ex, _train) call left its routing in its workspace:
 * device pointers into `ws`, valid until the workspace is reused.  The pieces are the
 * router's and the permutation's results ([OPS] Steps 2-4; [MB] sections 4.1-4.6):
 *   logits [T,E] fp32 (the router's own, without gate noise), topk_idx [T,k] int32,
 *   topk_w [T,k] fp32, counts [E] int32 pre-drop (only when the call's `counts` argument
 *   was NULL; otherwise the counts went there), offsets [E+1] int32 over the kept rows,
 *   slot_pos [T*k] int32 (-1 = dropped), sorted_slot [>= offsets[E]] int32 (row -> s).
 * Host only: pointer arithmetic on `ws`, nothing is read or launched.  Errors as for
 * moe_layer_forward's size checks; MOE_ERR_WORKSPACE when ws_bytes is smaller than
 * moe_workspace_bytes(...); MOE_ERR_ARG for a NULL ws or out. */
typedef struct {
  const float* logits;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* slot_pos;
  const int32_t* sorted_slot;
} moe_layer_routing_t;
moe_status_t moe_layer_routing(const void* ws, size_t ws_bytes, int32_t T, int32_t h, int32_t f, int32_t E,
                               int32_t k, float capacity_factor, moe_dtype_t dt, moe_act_t act,
                               moe_layer_routing_t* out);

/* moe_layer_forward with the router variants of moe_router_opts_t (NULL = plain).  ws:
 * moe_workspace_bytes(...) + moe_router_opts_workspace_bytes(T,h,dt,opts) bytes. */
moe_status_t moe_layer_forward_ex(const void* x, const float* W_gate, const float* logit_bias,
                                  const void* W1, const void* W3, const void* W2,
                                  int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                  float capacity_factor, moe_act_t act, moe_dtype_t dt,
                                  const moe_router_opts_t* opts, void* y, float* aux_loss,
                                  int32_t* counts, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward pass of moe_layer_forward: the gradients of L = <dy, y> + d_aux * aux_loss.
 * The pages name a backward pass for the gating operator ([OPS] operator list) and
 * autograd wrappers for the permutation ([MB] section 5) without writing them out; this
 * is the exact adjoint of the forward as the library defines it:
 *   dw[t,j] = <dy[t], O[r]>, dO[r] = w[t,j] dy[t] (kept slots; dropped ones get nothing);
 *   dHm = dO W2[e]^T; SwiGLU da = dHm g silu'(a), dg = dHm silu(a); GELU da = dHm gelu'(a);
 *   dW2[e] = Hm^T dO, dW1[e] = X^T da, dW3[e] = X^T dg, dX = da W1^T (+ dg W3^T);
 *   dx[t] = sum_j dX[slot of (t,j)] + dl[t] W_gate^T, dW_gate = x^T dl, with
 *   dl[t,S_j] = w_j (dw_j - sum_j' w_j' dw_j') + d_aux (E/T) p (f - <f, p>) (p the full
 *   softmax, f_e = counts_e / (T k)).
 * Selection and capacity are piecewise constant (no gradient); in bf16 the rounding of
 * Hm passes gradients unchanged, while dW2 uses the rounded Hm.  The plain router; for
 * the variants of moe_router_opts_t see moe_layer_backward_ex.
 *   fwd_ws / fwd_ws_bytes: the workspace of the moe_layer_forward (or
 *     moe_layer_forward_train) call being differentiated, untouched since (it holds the
 *     routing, Hm and the expert outputs); the other inputs must be that call's.
 *   preact / preact_bytes: NULL, or the pre-activations that moe_layer_forward_train wrote
 *     in that call (at least moe_layer_preact_bytes(...) bytes, else MOE_ERR_WORKSPACE).
 *     With NULL the pre-activations a (| g) are recomputed with the up projection's GEMM.
 *   dy [T,h] (dt); d_aux: host scalar.
 *   dx [T,h] (dt); dW_gate [h,E] fp32 or NULL (skipped); dW1, dW3 [E,h,f], dW2 [E,f,h]
 *     fp32 (dW3 NULL iff GELU).  The weight gradients are overwritten, not accumulated.
 *   ws: at least moe_layer_backward_workspace_bytes(...) bytes (the same with or without
 *     preact). */
size_t moe_layer_backward_workspace_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                          float capacity_factor, moe_dtype_t dt, moe_act_t act);
moe_status_t moe_layer_backward(const void* x, const float* W_gate, const void* W1, const void* W3,
                                const void* W2, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                float capacity_factor, moe_act_t act, moe_dtype_t dt, const void* dy,
                                float d_aux, const void* fwd_ws, size_t fwd_ws_bytes,
                                const float* preact, size_t preact_bytes, void* dx,
                                float* dW_gate, float* dW1, float* dW3, float* dW2, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* moe_layer_backward for a moe_layer_forward_ex call with router variants: the gradients
 * of the same L through the variant router ([OPS] "坑3" soft top-K and temperature; [CAI]
 * gate noise; [MB] section 5 jitter).  With p = softmax((logits + noise) / tau):
 *   renormalised weights: dl[t,S_j] = w_j (dw_j - sum_j' w_j' dw_j') / tau, 0 elsewhere;
 *   soft top-K: dl[t,b] = p_b (dw_b - sum_j w_j dw_j) / tau for every expert b (dw_b = 0
 *     when b was not selected, so unselected experts get -p_b sum_j w_j dw_j / tau);
 *   aux: + d_aux (E/T) p_b (f_b - <f, p>) / tau.
 * Gate noise is an input: the gradient with respect to the noisy logits is the one with
 * respect to the logits.  Jitter u: dW_gate = (x u)^T dl and the router's share of dx is
 * (dl W_gate^T) * u (the rounding of the product passes gradients unchanged).
 *   opts: the options of that forward call (the same noise and jitter buffers), or NULL
 *         (= moe_layer_backward).  fwd_ws must be that call's workspace: with jitter it
 *         holds the router's input after the layer's pieces.
 *   preact must be NULL when opts is not (MOE_ERR_ARG): the training forward has no
 *   router variants.  uniform_assignment: MOE_ERR_UNSUPPORTED (a benchmarking mode whose
 *   ids are not the router's choice).  Other arguments as moe_layer_backward. */
moe_status_t moe_layer_backward_ex(const void* x, const float* W_gate, const void* W1, const void* W3,
                                   const void* W2, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                   float capacity_factor, moe_act_t act, moe_dtype_t dt,
                                   const moe_router_opts_t* opts, const void* dy, float d_aux, const void* fwd_ws,
                                   size_t fwd_ws_bytes, const float* preact, size_t preact_bytes, void* dx,
                                   float* dW_gate, float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Training forward: moe_layer_forward (same arguments and results) that also writes the
 * up projection's fp32 pre-activations a (| g) of every kept assignment to `preact`, so
 * that moe_layer_backward can read them instead of recomputing them.  (They are the
 * inputs of the expert's activation: x W1[e] and, for SwiGLU, x W3[e], [CANN] section 7
 * and [MB] section 4.3.)  The buffer is an
 * opaque context of moe_layer_preact_bytes(...) bytes (R_max * f * 4, twice that for
 * SwiGLU, R_max the bound on kept assignments), 16-byte aligned (MOE_ERR_UNSUPPORTED
 * otherwise), caller-owned.  Its values equal the recomputed ones when the up projection
 * runs without K parts, and agree to fp32 rounding otherwise.  `events`: NULL, or as for
 * moe_layer_forward_timed.  preact NULL: MOE_ERR_ARG; too small: MOE_ERR_WORKSPACE. */
size_t moe_layer_preact_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                              float capacity_factor, moe_act_t act);  /* 0 for invalid sizes */
moe_status_t moe_layer_forward_train(const void* x, const float* W_gate, const float* logit_bias,
                                     const void* W1, const void* W3, const void* W2,
                                     int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                     float capacity_factor, moe_act_t act, moe_dtype_t dt,
                                     void* y, float* aux_loss, int32_t* counts,
                                     void* ws, size_t ws_bytes, float* preact, size_t preact_bytes,
                                     hipStream_t stream, hipEvent_t* events);

/* Measurement variant of moe_layer_backward: events[0] before the first kernel, then one
 * after each stage (combine adjoint with the counts and tile lists, router adjoint,
 * pre-activation recompute (empty with preact), down-projection data gradient with the
 * activation's derivative, down-projection weight gradient, up-projection data gradient,
 * up-projection weight gradients, router GEMMs, dx).  `events` (not null: MOE_ERR_ARG) holds
 * MOE_BACKWARD_STAGES + 1 entries, each a hipEvent_t or null (nothing recorded there). */
#define MOE_BACKWARD_STAGES 9
moe_status_t moe_layer_backward_timed(const void* x, const float* W_gate, const void* W1, const void* W3,
                                      const void* W2, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                      float capacity_factor, moe_act_t act, moe_dtype_t dt, const void* dy,
                                      float d_aux, const void* fwd_ws, size_t fwd_ws_bytes,
                                      const float* preact, size_t preact_bytes, void* dx,
                                      float* dW_gate, float* dW1, float* dW3, float* dW2, void* ws,
                                      size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/* The layer with fixed-capacity buckets ("binned" layout: [MB] sections 3, 4.3 and 4.5;
 * [CAI] SparseMLP data flow step 4 and its capacity parameters).  Every expert gets a
 * bucket of C rows: C = max(floor(cf * T*k/E), min_capacity) when cf > 0, else (or if that
 * is 0) the largest expert count of this call ([MB] section 4.6).  An expert's first C
 * assignments, in ascending t*k + j, fill its bucket; later ones are dropped (they add
 * nothing to y); the bucket rows past its count are zero and still go through the
 * expert MLP -- the padding cost of the layout.  y equals moe_layer_forward's output for
 * the same capacity.
 *   capacity: device int32 scalar or NULL: the C used.
 *   x_bins: [E*Cmax, h] (dt) or NULL (then kept in ws), Cmax = moe_binned_capacity_max(...):
 *           bucket e occupies rows [e*C, e*C + C); rows >= E*C are not written.
 *   ws: at least moe_binned_workspace_bytes(...) bytes.  Other arguments as in
 *   moe_layer_forward.  MOE_ERR_UNSUPPORTED when E*Cmax*max(h,f) >= 2^32. */
int32_t moe_binned_capacity_max(int32_t T, int32_t E, int32_t k, float capacity_factor,
                                int32_t min_capacity);  /* -1 for invalid sizes */
size_t moe_binned_workspace_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                  float capacity_factor, int32_t min_capacity, moe_dtype_t dt,
                                  moe_act_t act);
moe_status_t moe_layer_forward_binned(const void* x, const float* W_gate, const float* logit_bias,
                                      const void* W1, const void* W3, const void* W2,
                                      int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                      float capacity_factor, int32_t min_capacity, moe_act_t act,
                                      moe_dtype_t dt, void* y, float* aux_loss, int32_t* counts,
                                      int32_t* capacity, void* x_bins, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* Measurement variant of moe_layer_forward_binned, as moe_layer_forward_timed: events[0]
 * before the router, then one after each stage (router logits, selection + histogram,
 * scan, scatter, bucket gather, expert up-projection, expert down-projection, combine).
 * `events` (not null: MOE_ERR_ARG) holds MOE_BINNED_STAGES + 1 entries, each a hipEvent_t or
 * null (nothing recorded there). */
#define MOE_BINNED_STAGES 8
moe_status_t moe_layer_forward_binned_timed(const void* x, const float* W_gate, const float* logit_bias,
                                            const void* W1, const void* W3, const void* W2,
                                            int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                            float capacity_factor, int32_t min_capacity, moe_act_t act,
                                            moe_dtype_t dt, void* y, float* aux_loss, int32_t* counts,
                                            int32_t* capacity, void* x_bins, void* ws, size_t ws_bytes,
                                            hipStream_t stream, hipEvent_t* events);

/* Measurement variant of moe_layer_forward: the same kernels on the same stream, with
 * caller-created HIP events recorded between the stages, so a profiler-free caller can
 * time each kernel: events[0] before the router, then one after each stage in order
 * (router logits, selection + histogram, scan, scatter, expert up-projection, expert
 * down-projection, combine).  `events` (not null: MOE_ERR_ARG) holds MOE_LAYER_STAGES + 1
 * entries, each a hipEvent_t or null: nothing is recorded there, so a caller can time one
 * kernel without the idle gaps that every event record adds between kernels. */
#define MOE_LAYER_STAGES 7
moe_status_t moe_layer_forward_timed(const void* x, const float* W_gate, const float* logit_bias,
                                     const void* W1, const void* W3, const void* W2,
                                     int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                     float capacity_factor, moe_act_t act, moe_dtype_t dt,
                                     void* y, float* aux_loss, int32_t* counts,
                                     void* ws, size_t ws_bytes, hipStream_t stream,
                                     hipEvent_t* events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
