/*
 * rudnn_moe.h -- local mixture-of-experts forward pass on AMD Instinct MI355X (gfx950).
 *
 * The operation is the local MoE sequence of the ruDNN user guide (docs.rs, ruDNN 0.1.72):
 *   section 3 "MoE workflow":   logits -> softmax/top-k -> compact dispatch -> SwiGLU experts
 *                                -> weighted combine, each step also callable on its own;
 *   section 4 "Routing contract", section 5 "Expert weights and dispatch",
 *   section 6 "Calling MoE"     (the staged call forms, shapes and error rules).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers (memory of the device the stream belongs to),
 *     row-major and contiguous.  The caller owns every buffer, workspace included; the
 *     library never allocates, frees or keeps a pointer after returning.
 *   - Calls only enqueue work on `stream` (NULL = the null stream).  Nothing is synchronised
 *     and nothing is copied to the host: results are valid once the stream reaches them,
 *     like a readback that waits for the device (section 6).
 *   - Inputs are read-only.  Outputs must not overlap any input or each other
 *     (RUDNN_MOE_ERR_ARGUMENT otherwise).
 *   - Every argument is validated on the host before anything is enqueued.  A status other
 *     than RUDNN_MOE_OK means nothing was enqueued and no output was touched, except for
 *     RUDNN_MOE_ERR_RUNTIME (the HIP runtime refused a launch after earlier launches of the
 *     same call were enqueued).
 *   - T = 0 (no tokens) is a successful no-op.
 *   - Calls are reentrant and may run concurrently on different streams with different
 *     buffers.  The library keeps only set-once process state (each kernel's LDS-size
 *     attribute, each device's compute-unit count, both written once with the same value),
 *     and for rudnn_moe_dispatch_no_alloc its per-device scratch array (calls of that entry
 *     point that overlap on one GPU race on it).  The optional timing hook at the end is per
 *     host thread.
 */
#ifndef RUDNN_MOE_H
#define RUDNN_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below travel as 32-bit ints, and a C caller may pass any int.  C++ gives
 * them int as their fixed underlying type, so such a value is still a value of the type and the
 * entry points can reject it with an error (without it, an int outside the enumerators would be
 * undefined behaviour on the library's side). */
#ifdef __cplusplus
#define RUDNN_MOE_ENUM enum : int
#else
#define RUDNN_MOE_ENUM enum
#endif

/* Floating-point storage types (section 4: unquantised F32, F16 or BF16). */
typedef RUDNN_MOE_ENUM {
    RUDNN_MOE_F32 = 0,
    RUDNN_MOE_F16 = 1,
    RUDNN_MOE_BF16 = 2
} rudnn_moe_dtype;

/* Result of every entry point; the counterpart of the guide's MoeError (sections 3 and 6). */
typedef RUDNN_MOE_ENUM {
    RUDNN_MOE_OK = 0,
    RUDNN_MOE_ERR_SHAPE = 1,       /* a size < 1 where one is required; E/H/I disagree */
    RUDNN_MOE_ERR_DTYPE = 2,       /* not F32/F16/BF16; tokens and expert weights differ */
    RUDNN_MOE_ERR_ARGUMENT = 3,    /* top_k outside [1, E]; NULL pointer; overlapping buffers */
    RUDNN_MOE_ERR_DEVICE = 4,      /* a pointer is not device memory of the stream's device */
    RUDNN_MOE_ERR_UNSUPPORTED = 5, /* beyond the kernels' limits: E > 1024, top_k > 64,
                                      T*top_k >= 2^31, rows*max(H,I) >= 2^31 elements */
    RUDNN_MOE_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the size query returns */
    RUDNN_MOE_ERR_RUNTIME = 7      /* HIP reported an error for a launch */
} rudnn_moe_status;

/* RoutingOptions of section 4: 1 <= top_k <= E; renormalize != 0 rescales the k selected
 * probabilities of a row to sum to one before the cast to the logits dtype. */
typedef struct {
    int64_t top_k;
    int32_t renormalize;
} rudnn_moe_routing_options;

/* Borrowed view of the expert weights (SwiGluExperts::new of section 3; shapes and dtype
 * rules of section 5): bias-free SwiGLU experts
 *     y = down_e . ( silu(gate_e . x) * (up_e . x) ),   silu(z) = z / (1 + exp(-z)),
 * gate and up [E, I, H], down [E, H, I] (rows are output features; the contraction axis is
 * contiguous).  All three tensors and the tokens share one float dtype.  The view may be
 * reused for any number of batches; the weights must stay alive until the stream has
 * consumed every call that used them. */
typedef struct {
    const void* gate;
    const void* up;
    const void* down;
    int64_t num_experts;   /* E */
    int64_t hidden;        /* H */
    int64_t intermediate;  /* I */
    rudnn_moe_dtype dtype;
} rudnn_moe_experts;

/*
 * route -- section 4 "Routing contract" (RoutingPlan, expert_indices(), weights()).
 * For each row t of logits [T, E]: p = softmax over all E experts, computed in FP32; the k
 * largest p are selected and listed by descending p.  Softmax is strictly increasing, so the
 * selection is made on the exact logits: equal logits (a true tie) favour the lower expert
 * id, and of two distinct logits the larger wins even where their FP32 probabilities round
 * (or underflow) to the same value.  weights[t, j] = p of the j-th selected expert, divided by the
 * sum of the k selected p when opt.renormalize, then cast (round to nearest even) to the
 * logits dtype.  A row holding a NaN, a +inf, or nothing but -inf gets weights NaN and
 * indices 0..k-1.
 *   logits          [T, E]  logits_dtype (F32/F16/BF16)
 *   expert_indices  [T, k]  uint32, written
 *   weights         [T, k]  logits_dtype, written
 * Errors: SHAPE (T < 0, E < 1), ARGUMENT (top_k outside [1, E], NULL, overlap),
 * DTYPE, UNSUPPORTED (E > 1024 or top_k > 64), DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_route(const void* logits, rudnn_moe_dtype logits_dtype, int64_t T, int64_t E,
                                 rudnn_moe_routing_options opt, uint32_t* expert_indices, void* weights,
                                 hipStream_t stream);

/* Bytes of device workspace rudnn_moe_dispatch needs for T tokens, top_k, E experts. */
size_t rudnn_moe_dispatch_workspace_size(int64_t T, int64_t top_k, int64_t E);

/*
 * dispatch -- section 5 "Expert weights and dispatch" (RoutingPlan::dispatch).
 * Capacity-free grouping of the T*k (token, slot) pairs by expert; no token is dropped.
 *   expert_indices  [T, k] uint32 (as written by rudnn_moe_route)
 *   input           [T, H] dtype
 *   dispatched      [T*k, H] dtype, written: rows [expert_offsets[e], expert_offsets[e+1])
 *                   hold the tokens routed to expert e
 *   expert_offsets  [E+1] int32, written: exclusive prefix sum of the per-expert counts;
 *                   expert_offsets[E] = number of pairs with an index < E (T*k normally)
 *   token_map       [T, k] int32, written: the dispatched row holding copy j of token t
 *                   (the stored map that restores token order); -1 for an index >= E
 * Inside one expert this implementation orders rows by (t, j); the guide leaves that order
 * open, so callers must rely only on token_map.  Indices >= E are a caller error that is
 * contained: such a pair is not copied and combine yields a NaN row for its token.
 * workspace: at least rudnn_moe_dispatch_workspace_size(T, top_k, E) bytes, 256-B aligned (per-chunk
 * expert counts, the expert totals, and a 4-byte rank per pair).
 * Errors: SHAPE, ARGUMENT, DTYPE, UNSUPPORTED (E > 1024, T*k >= 2^31), WORKSPACE, DEVICE,
 * RUNTIME.
 */
rudnn_moe_status rudnn_moe_dispatch(const uint32_t* expert_indices, int64_t T, int64_t top_k, int64_t E,
                                    const void* input, rudnn_moe_dtype dtype, int64_t H, void* dispatched,
                                    int32_t* expert_offsets, int32_t* token_map, void* workspace,
                                    size_t workspace_size, hipStream_t stream);

/*
 * route_dispatch -- section 4 routing followed by section 5 dispatch of the plan, in one call
 * (route(logits, options) and then plan.dispatch(input)).  Writes exactly what rudnn_moe_route and
 * then rudnn_moe_dispatch on its indices write: expert_indices and weights as rudnn_moe_route,
 * dispatched, expert_offsets and token_map as rudnn_moe_dispatch (the same map).  Where the routing
 * blocks can serve as dispatch chunks, the routing kernel also does dispatch's per-chunk counting
 * and ranking, saving a pass.
 *   logits [T, E] logits_dtype; input [T, H] dtype; outputs as in the two calls.
 * workspace: at least rudnn_moe_dispatch_workspace_size(T, top_k, E) bytes, 256-B aligned.
 * Errors: those of rudnn_moe_route and rudnn_moe_dispatch; overlapping buffers are ARGUMENT.
 */
rudnn_moe_status rudnn_moe_route_dispatch(const void* logits, rudnn_moe_dtype logits_dtype, int64_t T, int64_t E,
                                          rudnn_moe_routing_options opt, const void* input, rudnn_moe_dtype dtype,
                                          int64_t H, uint32_t* expert_indices, void* weights, void* dispatched,
                                          int32_t* expert_offsets, int32_t* token_map, void* workspace,
                                          size_t workspace_size, hipStream_t stream);

/*
 * dispatch_no_alloc -- rudnn_moe_dispatch for callers that cannot allocate: code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that forbid it.  Same
 * arguments, results and errors as rudnn_moe_dispatch, without the workspace: the per-chunk
 * expert counts live in a device array of RUDNN_MOE_DISPATCH_NO_ALLOC_MAX_BYTES that the library
 * holds on every GPU it runs on until the process ends (its device address is looked up on the
 * first call on each device).  The call allocates nothing.  A call whose
 * rudnn_moe_dispatch_workspace_size(T, top_k, E) exceeds that size returns
 * RUDNN_MOE_ERR_UNSUPPORTED (e.g. E = 128 allows T * top_k up to about 4 million pairs).
 * All calls on one GPU share the array: calls that may overlap on one GPU (several host threads
 * or streams) race and must be ordered by the caller.
 */
#define RUDNN_MOE_DISPATCH_NO_ALLOC_MAX_BYTES ((size_t)16 << 20)
rudnn_moe_status rudnn_moe_dispatch_no_alloc(const uint32_t* expert_indices, int64_t T, int64_t top_k, int64_t E,
                                             const void* input, rudnn_moe_dtype dtype, int64_t H, void* dispatched,
                                             int32_t* expert_offsets, int32_t* token_map, hipStream_t stream);

/* Bytes of device workspace rudnn_moe_experts_forward needs for `rows` dispatched rows
 * (the hidden activation [rows, I] plus the tile schedule). */
size_t rudnn_moe_experts_workspace_size(const rudnn_moe_experts* ex, int64_t rows);

/*
 * experts_forward -- sections 3 and 5 (SwiGluExperts::forward_dispatched).
 * For every expert e and every row r in [expert_offsets[e], expert_offsets[e+1]):
 *   h = dtype( silu(gate_e . x_r) * (up_e . x_r) )    (FP32 accumulation, one rounding)
 *   expert_output[r] = dtype( down_e . h )             (FP32 accumulation, one rounding)
 *   dispatched      [rows, H] dtype;   expert_offsets [E+1] int32 (device, as written by
 *                   rudnn_moe_dispatch; never read on the host); rows = T*k
 *   expert_output   [rows, H] dtype, written for rows < expert_offsets[E]
 * BF16/F16 run on the matrix cores (MFMA) with FP32 accumulators; F32 runs in FP32 FMA.
 * In the BF16/F16 path silu takes the hardware exp and reciprocal (a few FP32 ulps from
 * z / (1 + exp(-z)), below the 16-bit rounding of h).
 * workspace: at least rudnn_moe_experts_workspace_size(ex, rows) bytes, 256-B aligned.
 * Errors: SHAPE, DTYPE, ARGUMENT, UNSUPPORTED, WORKSPACE, DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_experts_forward(const rudnn_moe_experts* ex, const void* dispatched,
                                           const int32_t* expert_offsets, int64_t rows, void* expert_output,
                                           void* workspace, size_t workspace_size, hipStream_t stream);

/*
 * combine -- sections 3 and 6 (DispatchedTokens::combine).
 *   output[t] = dtype( sum_{j=0..k-1} weights[t, j] * expert_output[token_map[t, j]] )
 * accumulated in FP32 with j ascending.  A token with a map entry outside [0, T*k) (dispatch
 * writes -1 for an expert id >= E) gets a NaN row; no row outside expert_output is read.
 *   expert_output [T*k, H] dtype;  token_map [T, k] int32;  weights [T, k] weights_dtype
 *   output        [T, H] dtype, written
 * Errors: SHAPE, DTYPE, ARGUMENT, UNSUPPORTED (top_k > 64, T*k >= 2^31), DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_combine(const void* expert_output, rudnn_moe_dtype dtype, const int32_t* token_map,
                                   const void* weights, rudnn_moe_dtype weights_dtype, int64_t T, int64_t top_k,
                                   int64_t H, void* output, hipStream_t stream);

/* Bytes of device workspace rudnn_moe_forward needs. */
size_t rudnn_moe_forward_workspace_size(const rudnn_moe_experts* ex, int64_t T, int64_t top_k,
                                        rudnn_moe_dtype logits_dtype);

/*
 * forward -- section 6 (SwiGluExperts::forward(input, logits, options)): the whole local
 * sequence route -> dispatch -> experts -> combine on one stream, bit-identical to calling
 * the four stages in turn.  The gate projection producing the logits is the caller's
 * (section 5).
 *   input [T, H] ex->dtype;  logits [T, E] logits_dtype;  output [T, H] ex->dtype, written
 * workspace: at least rudnn_moe_forward_workspace_size(ex, T, opt.top_k, logits_dtype) bytes.
 */
rudnn_moe_status rudnn_moe_forward(const rudnn_moe_experts* ex, const void* input, const void* logits,
                                   rudnn_moe_dtype logits_dtype, int64_t T, rudnn_moe_routing_options opt,
                                   void* output, void* workspace, size_t workspace_size, hipStream_t stream);

/* GroupRoutingOptions of section 10 (group-limited sigmoid routing).  Experts are split into
 * `groups` contiguous id ranges of E / groups experts.  Valid: 1 <= E <= 1024, 1 <= groups <=
 * 128 with E % groups == 0, 1 <= selected_groups <= groups, 1 <= top_k <= 64 and top_k <=
 * selected_groups * (E / groups), E / groups >= 2 when group_top_two, scale finite and > 0. */
typedef struct {
    int64_t top_k;
    int64_t groups;
    int64_t selected_groups;
    int32_t group_top_two;  /* != 0: a group's score is the sum of its two largest corrected scores */
    int32_t renormalize;    /* != 0: selected weights are divided by their sum (before `scale`) */
    double scale;           /* multiplies the (renormalised) weights */
} rudnn_moe_group_routing_options;

/*
 * route_sigmoid_grouped -- section 10 (route_sigmoid_grouped(logits, bias, options) ->
 * RoutingPlan).  For each row t of logits [T, E], in FP32: s_e = 1 / (1 + exp(-x_e)),
 * evaluated in FP64 and rounded once to FP32 (so the same on every run and device); the
 * corrected score c_e = s_e + bias[e] in FP32 (bias only steers the selection).  A group's score is
 * its largest c, or the sum of its two largest with group_top_two; the selected_groups
 * highest-scoring groups are chosen (equal scores: lower group id), then the top_k experts
 * of those groups by c (equal c: lower id), listed by descending c.  weights[t, j] = s of
 * the j-th selected expert, divided by the sum of the selected s when renormalising, times
 * scale, cast (round to nearest even) to the logits dtype.  A row with a NaN corrected score
 * or a NaN group score (e.g. +inf and -inf biases summed) gets weights NaN, indices 0..k-1.
 *   logits          [T, E]  logits_dtype (F32/F16/BF16)
 *   bias            [E]     FP32 device memory, or NULL for no correction
 *   expert_indices  [T, k]  uint32, written
 *   weights         [T, k]  logits_dtype, written
 * The outputs feed rudnn_moe_dispatch / rudnn_moe_combine exactly like rudnn_moe_route's.
 * Errors: SHAPE (T < 0, E < 1), ARGUMENT (options outside the ranges above, NULL, overlap),
 * DTYPE, UNSUPPORTED (T * top_k >= 2^31), DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_route_sigmoid_grouped(const void* logits, rudnn_moe_dtype logits_dtype, int64_t T,
                                                 int64_t E, const float* bias, rudnn_moe_group_routing_options opt,
                                                 uint32_t* expert_indices, void* weights, hipStream_t stream);

/*
 * forward_sigmoid_grouped -- section 10 (SwiGluExperts::forward_sigmoid_grouped(input,
 * logits, bias, options, strategy)): route_sigmoid_grouped -> dispatch -> experts ->
 * combine on one stream.  One strategy here: the MFMA (BF16/F16) or FP32 kernels.
 *   input [T, H] ex->dtype;  logits [T, E] logits_dtype;  bias [E] FP32 or NULL;
 *   output [T, H] ex->dtype, written
 * workspace: at least rudnn_moe_forward_workspace_size(ex, T, opt.top_k, logits_dtype) bytes.
 * Errors: as rudnn_moe_forward, with the option checks of rudnn_moe_route_sigmoid_grouped.
 */
rudnn_moe_status rudnn_moe_forward_sigmoid_grouped(const rudnn_moe_experts* ex, const void* input,
                                                   const void* logits, rudnn_moe_dtype logits_dtype, int64_t T,
                                                   const float* bias, rudnn_moe_group_routing_options opt,
                                                   void* output, void* workspace, size_t workspace_size,
                                                   hipStream_t stream);

/* Bytes of device workspace rudnn_moe_route_projected needs (0 when it needs none): FP32
 * partial logits when few token tiles make the kernel split the H axis over several blocks. */
size_t rudnn_moe_route_projected_workspace_size(int64_t T, int64_t H, int64_t E, rudnn_moe_dtype dtype);

/*
 * route_projected -- the gate projection that section 5 leaves to the caller, fused with the
 * section 4 routing (rudnn_moe_route) of its result:
 *   logits[t, e] = dtype( sum_h input[t, h] * router[e, h] )   FP32 accumulation, one rounding
 * then routed exactly as rudnn_moe_route routes logits [T, E] of that dtype.  The logits stay
 * on chip; logits_out, when not NULL, receives a copy (the values that were routed).
 *   input           [T, H]  dtype (F32/F16/BF16), 16-byte aligned
 *   router          [E, H]  dtype, 16-byte aligned (one row of gate weights per expert)
 *   logits_out      [T, E]  dtype, written, or NULL
 *   expert_indices  [T, k]  uint32, written;  weights [T, k] dtype, written
 * BF16/F16 run on the matrix cores (v_mfma_f32_32x32x16), F32 on v_mfma_f32_32x32x2f32.
 * workspace: at least rudnn_moe_route_projected_workspace_size(T, H, E, dtype) bytes, 256-B
 * aligned (may be NULL when that size is 0).
 * Errors: SHAPE (T < 0, H < 1, E < 1), ARGUMENT (top_k outside [1, E], NULL, overlap), DTYPE,
 * UNSUPPORTED (E > 256, top_k > 64, H * sizeof(dtype) not a multiple of 16, H >= 2^20,
 * unaligned input or router, T * top_k >= 2^31), WORKSPACE, DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_route_projected(const void* input, rudnn_moe_dtype dtype, const void* router,
                                           int64_t T, int64_t H, int64_t E, rudnn_moe_routing_options opt,
                                           void* logits_out, uint32_t* expert_indices, void* weights,
                                           void* workspace, size_t workspace_size, hipStream_t stream);

/* Bytes of device workspace rudnn_moe_forward_projected needs. */
size_t rudnn_moe_forward_projected_workspace_size(const rudnn_moe_experts* ex, int64_t T, int64_t top_k);

/*
 * forward_projected -- the local forward from the hidden states: route_projected (router
 * [E, H] in ex->dtype) -> dispatch -> experts -> combine on one stream, bit-identical to
 * rudnn_moe_route_projected followed by rudnn_moe_dispatch, rudnn_moe_experts_forward and
 * rudnn_moe_combine.
 *   input [T, H] ex->dtype;  router [E, H] ex->dtype;  output [T, H] ex->dtype, written
 * workspace: at least rudnn_moe_forward_projected_workspace_size(ex, T, opt.top_k) bytes.
 * Errors: as rudnn_moe_forward, with the limits of rudnn_moe_route_projected.
 */
rudnn_moe_status rudnn_moe_forward_projected(const rudnn_moe_experts* ex, const void* input, const void* router,
                                             int64_t T, rudnn_moe_routing_options opt, void* output,
                                             void* workspace, size_t workspace_size, hipStream_t stream);

/* ---- First-order training (section 12 "MoE-Training erster Ordnung") ---- */

/* Integer type of caller-provided expert indices (section 12: U32, I32 or I64). */
typedef RUDNN_MOE_ENUM { RUDNN_MOE_U32 = 0, RUDNN_MOE_I32 = 1, RUDNN_MOE_I64 = 2 } rudnn_moe_index_type;

/* RouterWeightOptions of section 12: RouterScoring::Softmax (0) or Sigmoid (1), optional
 * renormalisation of the selected weights, then a finite positive scale. */
typedef struct {
    int32_t scoring;      /* 0: softmax over all E experts, 1: sigmoid of each logit */
    int32_t renormalize;  /* != 0: divide by the sum of the selected scores */
    double scale;
} rudnn_moe_router_weight_options;

/*
 * selected_router_weights -- section 12 (selected_router_weights(&logits, &indices, options)).
 * For each row t: w[t, j] = scale * score(indices[t, j]) / S, score = the FP32 softmax over all
 * E experts of the row (or the sigmoid of each logit), S = sum_j score(indices[t, j]) when
 * renormalising (gather semantics: a repeated index counts each time), else 1.
 *   logits [T, E] logits_dtype;  indices [T, top_k] index_type;  weights [T, top_k] FP32, written
 * An index outside [0, E) makes the row's weights NaN; nothing is read through it.
 * Errors: SHAPE (T < 0, E < 1), ARGUMENT (top_k outside [1, min(E, 64)], scoring not 0/1, scale
 * not finite and > 0, NULL, overlap), DTYPE (logits or index type), DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_selected_router_weights(const void* logits, rudnn_moe_dtype logits_dtype, int64_t T,
                                                   int64_t E, const void* indices, rudnn_moe_index_type index_type,
                                                   int64_t top_k, rudnn_moe_router_weight_options opt,
                                                   float* weights, hipStream_t stream);

/*
 * selected_router_backward -- section 12 (selected_router_backward(&logits, &indices,
 * &grad_weights, options); RouterTrainingPlan::backward).  grad_logits[t, e] = sum_j
 * grad_weights[t, j] * d w[t, j] / d logits[t, e] for the weights above: the gradient of the
 * continuous weights of the fixed selection (not of the selection itself), computed in FP32 and
 * rounded once to the logits dtype.  An index outside [0, E) makes the row NaN.
 *   grad_weights [T, top_k] FP32;  grad_logits [T, E] logits_dtype, written
 * Errors: as rudnn_moe_selected_router_weights.
 */
rudnn_moe_status rudnn_moe_selected_router_backward(const void* logits, rudnn_moe_dtype logits_dtype, int64_t T,
                                                    int64_t E, const void* indices, rudnn_moe_index_type index_type,
                                                    int64_t top_k, rudnn_moe_router_weight_options opt,
                                                    const float* grad_weights, void* grad_logits,
                                                    hipStream_t stream);

/*
 * combine_backward -- section 12 step 1 (dispatched.combine_backward(&expert_output,
 * grad_output) -> (dexpert, dweights)), the backward of rudnn_moe_combine:
 *   grad_expert_output[token_map[t, j]] = dtype(weights[t, j] * grad_output[t])
 *   grad_weights[t, j] = sum_h grad_output[t, h] * expert_output[token_map[t, j], h]   (FP32)
 *   expert_output, grad_expert_output [T*k, H] dtype;  token_map [T, k] int32;
 *   weights [T, k] weights_dtype;  grad_output [T, H] dtype;  grad_weights [T, k] FP32
 * Rows of grad_expert_output named by no valid map entry are not written.  A token with a map
 * entry outside [0, T*k) gets NaN grad_weights and no row for that entry.  One strategy here.
 * Errors: SHAPE, ARGUMENT, DTYPE, UNSUPPORTED (top_k > 64, H * sizeof(dtype) not a multiple
 * of 16 or unaligned rows, T*k >= 2^31), DEVICE, RUNTIME.
 */
rudnn_moe_status rudnn_moe_combine_backward(const void* expert_output, rudnn_moe_dtype dtype,
                                            const int32_t* token_map, const void* weights,
                                            rudnn_moe_dtype weights_dtype, const void* grad_output, int64_t T,
                                            int64_t top_k, int64_t H, void* grad_expert_output, float* grad_weights,
                                            hipStream_t stream);

/*
 * dispatch_backward -- section 12 step 3 (dispatched.dispatch_backward(dinput)): the selected
 * rows summed back into their token, without the routing weights:
 *   grad_input[t] = dtype(sum_{j ascending} grad_dispatched[token_map[t, j]])   (FP32)
 *   grad_dispatched [T*k, H] dtype;  token_map [T, k] int32;  grad_input [T, H] dtype, written
 * A token with a map entry outside [0, T*k) gets a NaN row.
 * Errors: as rudnn_moe_combine_backward.
 */
rudnn_moe_status rudnn_moe_dispatch_backward(const void* grad_dispatched, rudnn_moe_dtype dtype,
                                             const int32_t* token_map, int64_t T, int64_t top_k, int64_t H,
                                             void* grad_input, hipStream_t stream);

/*
 * experts_forward_training -- section 12 (SwiGluExperts::forward_dispatched_training ->
 * (output, cache)).  rudnn_moe_experts_forward, and in the same pass the cache the backward
 * reads instead of recomputing the gate and up products:
 *   cache[r] = [ gate_e . x_r | up_e . x_r ]   [rows, 2*I] FP32, the FP32 accumulations the
 *                                              forward's silu(g) * u is formed from
 * expert_output is bit-identical to rudnn_moe_experts_forward's.  Same workspace.  The cache
 * belongs to the caller and must stay unchanged until the backward has run (section 12: stored
 * inputs stay unmodified).
 * Errors: as rudnn_moe_experts_forward; ARGUMENT for a NULL cache (rows > 0) or one that
 * overlaps another buffer; UNSUPPORTED for a cache that is not 16-byte aligned.
 */
rudnn_moe_status rudnn_moe_experts_forward_training(const rudnn_moe_experts* ex, const void* dispatched,
                                                    const int32_t* expert_offsets, int64_t rows, void* expert_output,
                                                    float* cache, void* workspace, size_t workspace_size,
                                                    hipStream_t stream);

/* Bytes of device workspace rudnn_moe_experts_backward needs for `rows` dispatched rows; with
 * cached != 0 (a cache from rudnn_moe_experts_forward_training is passed) it leaves out the
 * recomputed [rows, 2*I] FP32 pre-activations. */
size_t rudnn_moe_experts_backward_workspace_size(const rudnn_moe_experts* ex, int64_t rows, int cached);

/*
 * experts_backward -- section 12 step 2 (cache.backward(dexpert) -> dinput for the dispatched
 * rows and FP32 dgate, dup, ddown), the backward of rudnn_moe_experts_forward.  cache: the
 * [rows, 2*I] FP32 pre-activations [g | u] written by rudnn_moe_experts_forward_training for
 * the same dispatched rows and offsets, or NULL, and then g = gate . x and u = up . x are
 * recomputed in FP32.  For every expert e and row r in [expert_offsets[e], expert_offsets[e+1]):
 *   dh = down_e^T dy_r (FP32);  dg = dtype(dh * u * silu'(g)),  du = dtype(dh * silu(g))
 *   grad_dispatched[r] = dtype(gate_e^T dg + up_e^T du)
 *   grad_gate[e] = sum_r dg_r x_r^T,  grad_up[e] = sum_r du_r x_r^T,
 *   grad_down[e] = sum_r dy_r h_r^T with h = dtype(silu(g) * u)            (all FP32)
 *   dispatched, grad_expert_output, grad_dispatched [rows, H] dtype
 *   grad_gate, grad_up [E, I, H] FP32, grad_down [E, H, I] FP32, every entry written (an
 *   expert without rows gets zeros); rows of grad_dispatched outside the experts' ranges are
 *   not written.  BF16/F16 on the matrix cores, F32 on v_mfma_f32_32x32x2f32.
 * workspace: at least rudnn_moe_experts_backward_workspace_size(ex, rows, cache != NULL) bytes,
 * 256-B aligned.
 * Errors: as rudnn_moe_experts_forward; also UNSUPPORTED when H or I is not a multiple of
 * 16 / sizeof(dtype) or a pointer is not 16-byte aligned.
 */
rudnn_moe_status rudnn_moe_experts_backward(const rudnn_moe_experts* ex, const void* dispatched,
                                            const int32_t* expert_offsets, int64_t rows, const float* cache,
                                            const void* grad_expert_output, void* grad_dispatched, float* grad_gate,
                                            float* grad_up, float* grad_down, void* workspace, size_t workspace_size,
                                            hipStream_t stream);

/* Static, human-readable name of a status. */
const char* rudnn_moe_status_string(rudnn_moe_status s);

/*
 * Optional timing hook (measurement only; not part of the method).  The library's kernels,
 * as launched by the entry points above:
 */
typedef RUDNN_MOE_ENUM {
    RUDNN_MOE_KERNEL_ROUTE = 0,
    RUDNN_MOE_KERNEL_DISPATCH_COUNT = 1, /* per-chunk counts and ranks (a dispatch of its own; routing
                                            with dispatch does this step in the routing kernel) */
    RUDNN_MOE_KERNEL_DISPATCH_SCAN = 2,
    RUDNN_MOE_KERNEL_DISPATCH_RANK = 3,  /* not launched: the copy kernel forms the map (the number
                                            is kept so the others keep theirs) */
    RUDNN_MOE_KERNEL_DISPATCH_COPY = 4,  /* the rows and the token map */
    RUDNN_MOE_KERNEL_EXPERTS_PLAN = 5,
    RUDNN_MOE_KERNEL_EXPERTS_GATE_UP = 6,
    RUDNN_MOE_KERNEL_EXPERTS_DOWN = 7,
    RUDNN_MOE_KERNEL_COMBINE = 8,
    RUDNN_MOE_KERNEL_EXPERTS_GATE_UP_REDUCE = 9, /* sums the K-split partials of gate_up tail tiles */
    RUDNN_MOE_KERNEL_EXPERTS_DOWN_REDUCE = 10,   /* the same for down */
    RUDNN_MOE_KERNEL_ROUTE_SIGMOID_GROUPED = 11, /* group-limited sigmoid routing */
    RUDNN_MOE_KERNEL_ROUTE_PROJECTED = 12,        /* gate projection + routing */
    RUDNN_MOE_KERNEL_ROUTE_PROJECTED_REDUCE = 13, /* adds its H-split partials and routes */
    RUDNN_MOE_KERNEL_SELECTED_ROUTER = 14,        /* router weights of a fixed selection, or their gradient */
    RUDNN_MOE_KERNEL_COMBINE_BACKWARD = 15,
    RUDNN_MOE_KERNEL_DISPATCH_BACKWARD = 16,
    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_PLAN = 17,  /* m-tiles per expert */
    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_GU = 18,    /* gate . x and up . x recomputed in FP32 */
    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DH = 19,    /* dh = down^T dy with the dg / du / h epilogue */
    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DX = 20,    /* grad_dispatched */
    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW = 21,    /* the weight gradients (three launches) */
    RUDNN_MOE_KERNEL_COUNT = 22
} rudnn_moe_kernel;

/* For the calling host thread: record `before` on the launch stream immediately before the
 * next launch of `kernel` and `after` immediately after it, then forget the pair (one-shot).
 * Passing NULL events clears a pending pair.  Events are created and destroyed by the
 * caller.  Errors: ARGUMENT (unknown kernel). */
rudnn_moe_status rudnn_moe_time_next_launch(rudnn_moe_kernel kernel, hipEvent_t before, hipEvent_t after);

#ifdef __cplusplus
}
#endif

#endif /* RUDNN_MOE_H */
