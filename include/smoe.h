/*
 * smoe.h - C ABI of the scattered mixture-of-experts hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  A sparse mixture-of-experts (SMoE) layer sends every
 * token t to k of E experts; assignment p = t*k + j is token t's j-th choice
 * with expert e_p and gate g[t][j]; M = T*k.  The layer output is the
 * gate-weighted sum of the chosen experts' outputs (article "This Machine
 * Learning Research Presents ScatterMoE: An Implementation of Sparse
 * Mixture-of-Experts (SMoE) on GPUs", body, para. 1).  ParallelLinear runs
 * the expert linear transforms as one grouped product fused with the
 * reordering of rows (ScatterMoE project page, "How It Works"; review page
 * "Scattered Mixture-of-Experts Implementation", first review, Summary):
 * its input and its output are each either GROUPED (M rows sorted by expert,
 * ties in ascending p) or SCATTERED (token order), giving the four
 * group/scatter-to-group/scatter combinations (same page, second review,
 * Summary), with no padded or copied grouped input (catalogue record
 * "Scattered Mixture-of-Experts Implementation", abstract).  The backward
 * pass runs through the same machinery and yields per-expert weight
 * gradients (article, para. 4).  Around that path the library also exports
 * the router that produces the expert choices and gates (smoe_router_*)
 * and the Mixture-of-Attention core between the Q and O projections
 * (smoe_moa_attention_*), each with its backward.
 *
 * Conventions for every entry point.
 *  - Pointers to tensors are DEVICE pointers owned by the caller.  The
 *    library never allocates device memory, frees or synchronises, and
 *    creates no stream or event; it only enqueues work on `stream` (a
 *    hipStream_t; NULL = the default stream) and returns.  The MLP entry
 *    points can also use a second stream that the caller passes in (struct
 *    smoe_aux below); every output is ordered on `stream` when they return.
 *  - Tensors are row-major.  Weights are [E, d_in, d_out]: y = x W[e].
 *    Index arrays are int32; gates and gradients of gates are fp32 [T, k].
 *  - `dtype` is SMOE_F32 or SMOE_BF16 and applies to x, weights, y, dx and
 *    saved activations unless an entry point takes a separate dx_dtype.
 *    Weight gradients are fp32 by default; the backward entry points take a
 *    dw_dtype (SMOE_BF16: accumulated in fp32, rounded once).
 *  - Feature sizes (d_in, d_out, d_model, d_ff) must be multiples of 8 and
 *    rows must be 16-byte aligned; T*k must fit in int32.
 *  - bf16: T*k rows of any feature size, and one expert's weights, must
 *    each be under 4 GiB (the grouped products address their operands
 *    with 32-bit byte offsets); larger calls fail with SMOE_ERR_SHAPE.
 *  - Scratch memory comes from the caller as (ws, ws_bytes); the matching
 *    *_workspace_bytes() gives the size needed.
 *  - Return value: SMOE_OK or an error status.  A failed host-side check
 *    enqueues nothing.  A launch failure returns SMOE_ERR_HIP.  The text of
 *    the last failure on the calling thread is smoe_last_error().
 *  - Calls that share a workspace, or write the same outputs, must be
 *    ordered on one stream by the caller.
 */
#ifndef SMOE_H
#define SMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum smoe_status {
  SMOE_OK = 0,
  SMOE_ERR_NULL = 1,        /* a required pointer is NULL                  */
  SMOE_ERR_SHAPE = 2,       /* sizes out of range or inconsistent          */
  SMOE_ERR_DTYPE = 3,       /* unknown dtype or activation                 */
  SMOE_ERR_WORKSPACE = 4,   /* ws/saved buffer smaller than required       */
  SMOE_ERR_UNSUPPORTED = 5, /* valid request this build does not implement */
  SMOE_ERR_HIP = 6          /* a HIP launch failed                         */
};

enum smoe_dtype { SMOE_F32 = 0, SMOE_BF16 = 1 };

/* GELU: exact erf form, two matrices W1 -> act -> W2.
 * SWIGLU: silu(x W1[e]) * (x W3[e]) -> W2. */
enum smoe_act { SMOE_ACT_GELU = 0, SMOE_ACT_SWIGLU = 1 };

/* A second stream for the entry points that can run part of their work
 * beside the rest (smoe_mlp_fwd, smoe_mlp_fwd_fused_combine, smoe_mlp_bwd).
 * The caller creates and owns all three handles: `stream` (a hipStream_t of
 * default priority) and two events (hipEvent_t; timing may be disabled).
 * The library records fork_event on the caller's stream and makes `stream`
 * wait for it, enqueues the side work, then records join_event on `stream`
 * and makes the caller's stream wait for it before returning (also when it
 * returns an error after the fork).  Calls that share one smoe_aux must be
 * enqueued from one host thread at a time.  Passing NULL (or a struct with
 * a NULL member) runs everything on the caller's stream. */
typedef struct smoe_aux {
  void* stream;
  void* fork_event;
  void* join_event;
} smoe_aux;

/* Static description of a status code. */
const char* smoe_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* smoe_last_error(void);
/* ABI version of this library. */
int smoe_abi_version(void);

/* ------------------------------------------------------------------------
 * smoe_route - routing indices from the top-k expert choices.
 *
 * Implements the reordering that ParallelLinear fuses with the expert
 * transforms (project page, "How It Works").  With e_p = expert_idxs[p]:
 *   counts[e]   = #{p : e_p = e}
 *   offsets[e]  = sum_{e' < e} counts[e'],  offsets[E] = number of valid p
 *   sorted_scattered_idxs[r] = the p at grouped row r, rows sorted by
 *                  (e_p, p) ascending (a stable sort; bit-exact)
 *   sorted_expert_idxs[r]    = e_p of that row
 * expert_idxs: [T, k] int32.  Outputs: [T*k], [T*k], [E], [E+1] int32.
 * 1 <= E <= 1024, 1 <= k.  Choices outside [0, E) are dropped (never
 * written); offsets[E] < T*k then tells the caller.  Rows past offsets[E]
 * of the sorted arrays are left untouched.
 * ------------------------------------------------------------------------ */
size_t smoe_route_workspace_bytes(int64_t T, int32_t k, int32_t E);
int smoe_route(const int32_t* expert_idxs, int64_t T, int32_t k, int32_t E,
               int32_t* sorted_expert_idxs, int32_t* sorted_scattered_idxs,
               int32_t* counts, int32_t* offsets,
               void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * smoe_route_noalloc - smoe_route for callers that cannot allocate device
 * memory (code under stream capture into a HIP graph, tight serving loops,
 * harnesses that forbid allocation): the same kernels, outputs and errors,
 * with the chunk histograms in a static device array of the library
 * (4 MiB per device, held until the process ends) instead of a workspace.
 * Sizes with ceil(T*k / 4096) * E > 2^20 are rejected (SMOE_ERR_SHAPE,
 * nothing enqueued); nothing is allocated or freed.  Every call on one
 * device shares that array (each call writes what it reads, so nothing
 * carries over between calls): calls that overlap on one device (on
 * different streams, or from several host threads) race and must be
 * ordered by the caller.
 * ------------------------------------------------------------------------ */
int smoe_route_noalloc(const int32_t* expert_idxs, int64_t T, int32_t k, int32_t E,
                       int32_t* sorted_expert_idxs, int32_t* sorted_scattered_idxs,
                       int32_t* counts, int32_t* offsets, void* stream);

/* ------------------------------------------------------------------------
 * smoe_parallel_linear_fwd - scatter2scatter forward (all four layouts).
 *
 * For every grouped row r (expert e, assignment p = sorted_scattered_idxs[r]):
 *   u_r = x_grouped ? x[r] : x[p / fan]     fan = k if x_rows == T, else 1
 *   v_r = u_r W[e]
 * Without gates: y is [T*k, d_out]; row r if y_grouped, row p otherwise.
 * With gates (y_grouped must be 0): y is [T, d_out] and
 *   y[t] = sum_j gates[t][j] v_(row of t*k+j)     (fp32 combine)
 * x: [x_rows, d_in], x_rows = T*k if x_grouped, else T or T*k.
 * w: [E, d_in, d_out].  Routing arrays as produced by smoe_route.
 * Review page, first and second review, Summary; article, para. 3-4.
 * ------------------------------------------------------------------------ */
size_t smoe_parallel_linear_fwd_workspace_bytes(int64_t T, int32_t k, int32_t E,
                                                int64_t d_in, int64_t d_out,
                                                int32_t with_gates, int32_t dtype);
int smoe_parallel_linear_fwd(const void* x, int64_t x_rows, int64_t d_in,
                             const void* w, int64_t d_out, int32_t E,
                             int64_t T, int32_t k,
                             const int32_t* sorted_scattered_idxs,
                             const int32_t* offsets,
                             int32_t x_grouped, int32_t y_grouped,
                             const float* gates, void* y, int32_t dtype,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * smoe_parallel_linear_bwd - backward of smoe_parallel_linear_fwd.
 *
 * dy has the forward output's shape.  Per grouped row r (expert e, p, t):
 *   dy_r = gates ? gates[t][j] * dy[t] : dy[row of r]
 *   dx[input row of r] += dy_r W[e]^T   (k contributions summed, fp32,
 *                                        when a T-row x was read k times)
 *   dw[e]   = sum_r u_r^T dy_r          (experts with no rows get 0)
 *   dgates[t][j] = <dy[t], u_r W[e]>    (only with gates)
 * Any of dx, dw, dgates may be NULL to skip it (dgates needs gates).
 * dgates comes from the dx product as <dy[t] W[e]^T, u_r>, so no saved
 * forward output is needed.
 * dx_dtype: dx in SMOE_BF16 or SMOE_F32 (fp32 keeps the exact sum unrounded;
 * fp32 runs need fp32).  dw_dtype: dw [E, d_in, d_out] in SMOE_F32 or
 * SMOE_BF16 (summed in fp32, rounded once); accumulate_dw != 0 adds the
 * gradient to what dw holds instead of overwriting it.
 * With gates, dw[e] = sum (g u_r)^T dy[t]: the weight-gradient product
 * scales each row it reads from x by the row's gate in registers (x is read
 * in place; no scaled copy exists), and in bf16 runs g*u_r is rounded to
 * bf16 before it enters the contraction.
 * Same page, first review, Summary (forward and backward through
 * ParallelLinear); article, para. 4 (per-expert gradients); catalogue
 * record, abstract (no copied or padded input).
 * ------------------------------------------------------------------------ */
size_t smoe_parallel_linear_bwd_workspace_bytes(int64_t T, int32_t k, int32_t E,
                                                int64_t x_rows, int64_t d_in,
                                                int64_t d_out, int32_t x_grouped,
                                                int32_t with_gates, int32_t dtype);
int smoe_parallel_linear_bwd(const void* x, int64_t x_rows, int64_t d_in,
                             const void* w, int64_t d_out, int32_t E,
                             int64_t T, int32_t k,
                             const int32_t* sorted_scattered_idxs,
                             const int32_t* offsets,
                             int32_t x_grouped, int32_t y_grouped,
                             const float* gates, const void* dy,
                             void* dx, int32_t dx_dtype,
                             void* dw, int32_t dw_dtype, int32_t accumulate_dw,
                             float* dgates, int32_t dtype,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * smoe_mlp_fwd - SMoE-MLP block: route, W1 (and W3) with the activation
 * fused, W2 with scattered output, gate-weighted combine.
 *
 *   out[t] = sum_j gates[t][j] * MLP_e(x[t]),
 *   GELU:   MLP_e(x) = gelu(x W1[e]) W2[e]
 *   SWIGLU: MLP_e(x) = (silu(x W1[e]) * (x W3[e])) W2[e]
 * x: [T, d_model]; w1, w3: [E, d_model, d_ff]; w2: [E, d_ff, d_model];
 * w3 must be NULL unless SWIGLU.  expert_idxs, gates: [T, k].
 * out: [T, d_model].  `saved` (size smoe_mlp_saved_bytes) receives what the
 * backward needs: the routing arrays and the grouped pre-activations h
 * (h1, h3); the activation a is recomputed from them in the backward.  Its
 * layout is given by smoe_mlp_saved_offsets.
 * In bf16 runs h (h1, h3) and a are stored in bf16; a is computed from the
 * stored h; expert outputs and the combine stay fp32 until the final
 * rounding of out.
 * With `aux` (bf16 runs), both layers' routing-dependent m-tiles (those
 * past the whole groups that exist whatever the routing) run on aux's
 * stream beside the rest, so that layer 2's last, partly filled round
 * overlaps layer 1's work.
 * Article, para. 1 and 5 (SMoE MLP); project page, "How It Works".
 * ------------------------------------------------------------------------ */
size_t smoe_mlp_saved_bytes(int64_t T, int32_t k, int32_t E, int64_t d_model,
                            int64_t d_ff, int32_t act, int32_t dtype);
/* Byte offsets inside `saved`: off[0] sorted_expert_idxs, off[1]
 * sorted_scattered_idxs, off[2] counts, off[3] offsets, off[4] h (h1),
 * off[5] h3 (SIZE_MAX unless SWIGLU).  Returns SMOE_OK. */
int smoe_mlp_saved_offsets(int64_t T, int32_t k, int32_t E, int64_t d_model,
                           int64_t d_ff, int32_t act, int32_t dtype, size_t off[6]);
size_t smoe_mlp_fwd_workspace_bytes(int64_t T, int32_t k, int32_t E,
                                    int64_t d_model, int64_t d_ff, int32_t act,
                                    int32_t dtype);
int smoe_mlp_fwd(const void* x, const void* w1, const void* w3, const void* w2,
                 int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                 const int32_t* expert_idxs, const float* gates,
                 int32_t act, int32_t dtype, void* out,
                 void* saved, size_t saved_bytes,
                 void* ws, size_t ws_bytes, const smoe_aux* aux, void* stream);

/* smoe_mlp_fwd_fused_combine - smoe_mlp_fwd with the combine folded into the
 * W2 product: each expert output row is scaled by its gate in the product's
 * epilogue and added with fp32 atomics into an fp32 [T, d_model] token
 * buffer (the front of the workspace), which one pass then rounds to `out`.
 * This drops the [T*k, d_model] fp32 per-assignment rows' write and read.
 * Same arguments, saved layout, limits and error codes as smoe_mlp_fwd;
 * `saved` is interchangeable with it for smoe_mlp_bwd.  The workspace
 * (smoe_mlp_fwd_fused_combine_workspace_bytes) holds T fp32 rows of
 * d_model where smoe_mlp_fwd's holds T*k: the variant trades speed (one
 * 4-byte atomic per element instead of 16-byte stores) for memory.  The
 * order of the k fp32 additions per element is not fixed, so for k > 2
 * results can differ between runs in the last fp32 bits before the final
 * rounding (k <= 2 is exact: 0 + a + b = 0 + b + a).
 * Article, para. 1 and 5 (the SMoE output as the gate-weighted sum of the
 * chosen experts' outputs); project page, "How It Works" (scattered output).
 * ------------------------------------------------------------------------ */
size_t smoe_mlp_fwd_fused_combine_workspace_bytes(int64_t T, int32_t k,
                                                  int32_t E, int64_t d_model,
                                                  int64_t d_ff, int32_t act,
                                                  int32_t dtype);
int smoe_mlp_fwd_fused_combine(const void* x, const void* w1, const void* w3,
                               const void* w2, int64_t T, int64_t d_model,
                               int64_t d_ff, int32_t E, int32_t k,
                               const int32_t* expert_idxs, const float* gates,
                               int32_t act, int32_t dtype, void* out,
                               void* saved, size_t saved_bytes,
                               void* ws, size_t ws_bytes, const smoe_aux* aux,
                               void* stream);

/* ------------------------------------------------------------------------
 * smoe_mlp_bwd - backward of smoe_mlp_fwd for upstream dout [T, d_model].
 *
 * Per assignment (token t, choice j, expert e, gate g), with a = act(h):
 *   dgates[t][j] = <dout[t], a W2[e]>
 *   dA = g * dout[t] W2[e]^T
 *   GELU:   dh = dA * gelu'(h)
 *   SWIGLU: dh1 = dA * h3 * silu'(h1);  dh3 = dA * silu(h1)
 *   dx[t] += dh W1[e]^T (+ dh3 W3[e]^T)            (fp32 k-sum)
 *   dw2[e] += (g a)^T dout[t];  dw1[e] += x[t]^T dh;  dw3[e] += x[t]^T dh3
 * Weight gradients are fully written (experts with no tokens get 0), in
 * dw_dtype: SMOE_F32, or SMOE_BF16 (summed in fp32, rounded once; bf16 runs
 * only).  dw3 must be NULL unless SWIGLU.  dgates may be NULL.  `saved` is
 * the buffer filled by smoe_mlp_fwd with the same arguments.  In bf16 runs
 * dh (dh1, dh3) and g*a are rounded to bf16 before they enter the
 * weight-gradient and dx contractions.
 * With `aux` (bf16 runs), dw1 runs on aux's stream, forked after the dx
 * product's whole rounds of tiles so that it fills the CUs that the last,
 * partly filled round leaves idle, and joined back before dw2.  Every
 * output is ordered on `stream` when the call returns (and a capture of
 * `stream` records both branches).
 * ------------------------------------------------------------------------ */
size_t smoe_mlp_bwd_workspace_bytes(int64_t T, int32_t k, int32_t E,
                                    int64_t d_model, int64_t d_ff, int32_t act,
                                    int32_t dtype);
int smoe_mlp_bwd(const void* dout, const void* x, const void* w1,
                 const void* w3, const void* w2,
                 int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                 const int32_t* expert_idxs, const float* gates,
                 int32_t act, int32_t dtype,
                 const void* saved, size_t saved_bytes,
                 void* dx, void* dw1, void* dw3, void* dw2, int32_t dw_dtype,
                 float* dgates, void* ws, size_t ws_bytes,
                 const smoe_aux* aux, void* stream);

/* ------------------------------------------------------------------------
 * Measurement hook for benchmarks and profilers (not thread-safe).
 *
 * While a role has events attached, each launch of that role is bracketed
 * on its stream by hipEventRecord(start_event) and hipEventRecord(stop_event)
 * (hipEvent_t handles owned by the caller; a role launched several times in
 * one call keeps the last launch).  NULL, NULL detaches.  The GEMM roles
 * cover exactly one kernel launch each.
 * ------------------------------------------------------------------------ */
enum smoe_role {
  SMOE_ROLE_ROUTE = 0,      /* the routing kernels of smoe_mlp_fwd          */
  SMOE_ROLE_UP = 1,         /* MLP W1 (and W3) product, activation fused    */
  SMOE_ROLE_DOWN = 2,       /* MLP W2 product, scattered fp32 output        */
  SMOE_ROLE_COMBINE = 3,    /* gate-weighted combine                        */
  SMOE_ROLE_DA = 4,         /* MLP dout W2^T, activation backward fused     */
  SMOE_ROLE_DW2 = 5,        /* MLP dW2 product                              */
  SMOE_ROLE_DX = 6,         /* MLP dh W1^T (+ dh3 W3^T) product             */
  SMOE_ROLE_KSUM = 7,       /* k-sum of dx contributions                    */
  SMOE_ROLE_DW1 = 8,        /* MLP dW1 product                              */
  SMOE_ROLE_DW3 = 9,        /* MLP dW3 product                              */
  SMOE_ROLE_DW_REDUCE = 10, /* split weight-gradient reduction              */
  SMOE_ROLE_DG_REDUCE = 11, /* gate-gradient reduction                      */
  SMOE_ROLE_PL_FWD = 12,    /* ParallelLinear forward product               */
  SMOE_ROLE_PL_DX = 13,     /* ParallelLinear dx product                    */
  SMOE_ROLE_PL_DW = 14,     /* ParallelLinear dw product                    */
  SMOE_ROLE_ROUTER_FWD = 15, /* router logits, top-k and softmax            */
  SMOE_ROLE_ROUTER_DX = 16, /* router dx                                    */
  SMOE_ROLE_ROUTER_DW = 17, /* router dw product                            */
  SMOE_ROLE_ATTN_FWD = 18,  /* MoA attention forward                        */
  SMOE_ROLE_ATTN_DQ = 19,   /* MoA attention dq                             */
  SMOE_ROLE_ATTN_DKV = 20,  /* MoA attention dk, dv                         */
  SMOE_ROLE_COUNT = 21
};
int smoe_set_role_events(int32_t role, void* start_event, void* stop_event);

/* ------------------------------------------------------------------------
 * smoe_router_fwd - the SMoE router (article "This Machine Learning Research
 * Presents ScatterMoE", body, para. 1: each token goes to k of E experts and
 * its output is their gate-weighted sum):
 *   logits = x w^T            x [T, d_model] (dtype), gate weight w
 *                             [E, d_model] (dtype; a linear layer's layout)
 *   expert_idxs[t, j] = the j-th largest logit's expert (descending, ties to
 *                      the lower expert id)        int32 [T, k]
 *   gates[t, :] = softmax over the k chosen logits (max subtracted), fp32
 *   logits (fp32 [T, E]) is written if not NULL.
 * Logits accumulate in fp32 (bf16: on the matrix cores from exact bf16
 * products); a choice between logits closer than their rounding error may
 * differ from an exact evaluation.  1 <= k <= min(E, 8), E <= 64.
 * expert_idxs and gates are the inputs of the other entry points.
 * ------------------------------------------------------------------------ */
int smoe_router_fwd(const void* x, const void* w, int64_t T, int64_t d_model, int32_t E, int32_t k,
                    int32_t dtype, int32_t* expert_idxs, float* gates, float* logits, void* stream);

/* ------------------------------------------------------------------------
 * smoe_router_bwd - backward of smoe_router_fwd for upstream dgates [T, k]
 * (fp32; e.g. smoe_mlp_bwd's dgates).  The choice carries no gradient; the
 * softmax gives
 *   dlogits[t, e_j] = g_j (dg_j - sum_i g_i dg_i)   (0 for unchosen experts;
 *                            the sum runs over all k choices)
 *   dw_out = dlogits^T x     fp32 [E, d_model], fully written, summed over
 *                            tokens in a fixed order (deterministic)
 *   dx (+)= dlogits w        dtype [T, d_model]: written, or added to what
 *                            dx holds when accumulate_dx != 0 (to put the
 *                            router's part beside smoe_mlp_bwd's dx)
 * Choices with an expert id outside [0, E) contribute nothing.  Scratch:
 * smoe_router_bwd_workspace_bytes(...).  Limits as smoe_router_fwd.
 * ------------------------------------------------------------------------ */
size_t smoe_router_bwd_workspace_bytes(int64_t T, int64_t d_model, int32_t E);
int smoe_router_bwd(const void* x, const void* w, int64_t T, int64_t d_model, int32_t E, int32_t k,
                    int32_t dtype, const int32_t* expert_idxs, const float* gates, const float* dgates,
                    float* dw_out, void* dx, int32_t accumulate_dx, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * smoe_moa_attention_fwd - the Mixture-of-Attention core (article "This
 * Machine Learning Research Presents ScatterMoE", body, para. 4: the head
 * experts of MoA run on the same grouped products, with no extra memory):
 * grouped query rows against keys and values shared by all experts.
 *   q [T*k, head_dim] in grouped order (row r = assignment
 *     sorted_scattered_idxs[r], as smoe_parallel_linear_fwd writes it
 *     scattered-in / grouped-out); row r is token t = s_r / k's query for
 *     its expert head
 *   k, v [T, head_dim] token order, T = B * seq_len tokens (B sequences)
 *   o[r] = softmax_t'(q_r . k_t' / sqrt(head_dim)) v over the keys t' of
 *     t's sequence with t' <= t (causal); o [T*k, head_dim], grouped order
 *   lse[r] = log sum_t' exp(q_r . k_t' / sqrt(head_dim)), fp32 [T*k] (the
 *     backward's input)
 * bf16 only (SMOE_ERR_UNSUPPORTED otherwise), head_dim 128; fp32
 * accumulation, the probabilities enter the P v product in bf16.
 * ------------------------------------------------------------------------ */
int smoe_moa_attention_fwd(const void* q, const void* k_, const void* v, const int32_t* sorted_scattered_idxs,
                           int64_t T, int32_t k, int64_t seq_len, int64_t head_dim, int32_t dtype, void* o, float* lse,
                           void* stream);

/* ------------------------------------------------------------------------
 * smoe_moa_attention_bwd - backward of smoe_moa_attention_fwd for upstream
 * dout [T*k, head_dim] (grouped order).  With p the row's probabilities
 * (recomputed from lse) and D_r = dout_r . o_r:
 *   dz = p (dout_r . v_t' - D_r)          (gradient of the scaled score)
 *   dq_r = dz k / sqrt(head_dim)          [T*k, head_dim], grouped order
 *   dk_t' = sum over rows of dz q_r / sqrt(head_dim),  dv_t' = sum p dout_r
 *                                          [T, head_dim] each
 * dk and dv are summed over every row that reads them in a fixed order
 * (deterministic).  Outputs in the input dtype (bf16), fp32 accumulation.
 * Scratch: smoe_moa_attention_bwd_workspace_bytes(...).  Limits as the
 * forward.
 * ------------------------------------------------------------------------ */
size_t smoe_moa_attention_bwd_workspace_bytes(int64_t T, int32_t k, int64_t seq_len, int64_t head_dim);
int smoe_moa_attention_bwd(const void* q, const void* k_, const void* v, const int32_t* sorted_scattered_idxs,
                           int64_t T, int32_t k, int64_t seq_len, int64_t head_dim, int32_t dtype, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * smoe_probe_mfma_loop - diagnostic (for the caller's measurement of the
 * device, not part of the method): enqueues on `stream` one kernel of
 * `blocks` workgroups of 256 threads in which every wave issues `iters`
 * rounds of 16 independent bf16 v_mfma_f32_32x32x16 on registers (no memory
 * traffic in the loop) and writes one float per thread to out[blocks*256]
 * (device, caller-owned).  FLOP = blocks * 4 * iters * 16 * 32768; timing it
 * gives the matrix cores' reachable rate (and the clock the chip then
 * holds), the reference for the products' utilisation.  blocks and iters
 * must be positive; nothing is enqueued otherwise (SMOE_ERR_SHAPE).
 * ------------------------------------------------------------------------ */
int smoe_probe_mfma_loop(float* out, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SMOE_H */
