/*
 * switch_moe.h -- C ABI of the Switch Transformer sparse expert FFN layer
 * (forward pass) on one AMD MI355X (gfx950).
 *
 * The layer (sources: "042 Switch Transformer" teaching note, wq-win.github.io,
 * sec. 1-3; "MoE routing load collapse" reproduction note, zffjzz.top,
 * "core idea and formulas" and "official code reading route"; paper card
 * "Switch Transformers", ai-papers.xuzou.cn, "bottleneck" and "method
 * adaptation"; "Mixture of experts" explainer, world.lapla.si, "what is inside
 * an expert" and "full means turned back"):
 *
 *   z_te     = sum_i x_ti W_r[i,e] + b_r[e]                  fp32 router
 *   p_te     = softmax_e(z_t),  e*_t = argmax_e z_te (lowest index on ties)
 *   C        = ceil(c T / E)                                 expert capacity
 *   pos_t    = #{s < t : e*_s = e*_t},  keep_t = pos_t < C   slots in token order
 *   buf[e,s] = x_t  for the token t in slot s of expert e    dispatch, bf16
 *   y[e,s]   = ReLU(buf[e,s] W1_e^T) W2_e^T                  expert FFN
 *   out_t    = x_t + keep_t p_{t,e*} y[e*_t, pos_t]          gate not renormalised
 *   f_e = counts_e / T,  P_e = (1/T) sum_t p_te,  L = alpha E sum_e f_e P_e
 *   dL/dz_tj = (alpha E / T) p_tj (f_j - sum_e f_e p_te)     (f held constant)
 *
 * Conventions for every device entry point
 *   - Every pointer is a device pointer owned by the caller; the library keeps
 *     no reference after the call returns.  All arrays are row-major and
 *     contiguous.  bf16 arrays must be 16-byte aligned, others 4-byte aligned.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the host, allocates device memory or
 *     copies device data to the host.
 *   - Arguments are validated before any HIP call: a bad argument returns
 *     SWITCH_E_INVALID / SWITCH_E_UNSUPPORTED / SWITCH_E_WORKSPACE with a
 *     message in switch_last_error() and nothing is enqueued.  A failed
 *     launch returns SWITCH_E_HIP.  Faults while kernels run surface at the
 *     caller's next synchronisation.  Nothing is thrown across the ABI.
 *   - Results are bitwise reproducible run to run (fixed-order reductions,
 *     no floating-point atomics).
 *   - Scratch space is the caller's `ws` of `ws_bytes` bytes, 256-byte
 *     aligned, sized by the matching *_workspace_bytes() helper; its contents
 *     on entry do not matter.  Calls that share a workspace must not overlap.
 *   - Non-finite inputs are outside the contract.
 *   - Limits: 0 <= T < 2^31, 1 <= E <= 4096, 0 <= C, E*C < 2^31; d and d_ff
 *     multiples of 64 (the router alone needs d a multiple of 32, dispatch
 *     and combine need d a multiple of 8).
 */
#ifndef SWITCH_MOE_H
#define SWITCH_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SWITCH_OK = 0,
    SWITCH_E_INVALID = 1,      /* NULL required pointer, bad size, misaligned pointer */
    SWITCH_E_UNSUPPORTED = 2,  /* sizes outside the limits above */
    SWITCH_E_WORKSPACE = 3,    /* ws_bytes smaller than required */
    SWITCH_E_HIP = 4           /* a HIP runtime call failed (text in switch_last_error) */
} switch_status;

typedef uint16_t switch_bf16;  /* raw bf16 bits (torch.bfloat16 storage) */

/* ------------------------------------------------------------ host helpers */

/* C = ceil(c * T / E), exact on the binary value of c (no float rounding).
 * Sources: zffjzz.top note, "core idea and formulas" (C = ceil(cT/E));
 * wq-win note sec. 1 (C = (T/E) c).  Returns SWITCH_E_INVALID for T < 0,
 * E <= 0, c negative or not finite, or a result above 2^31 - 1. */
switch_status switch_capacity(int64_t T, int32_t E, double c, int32_t *C_out);

/* Workspace bytes for each entry point, and for switch_layer_fwd (which
 * covers every other call with the same sizes).  Return 0 for invalid sizes. */
size_t switch_route_workspace_bytes(int64_t T, int32_t d, int32_t E);
size_t switch_dispatch_workspace_bytes(int64_t T, int32_t E);
size_t switch_expert_ffn_workspace_bytes(int32_t E, int32_t C, int32_t d_ff);
size_t switch_aux_loss_workspace_bytes(int64_t T, int32_t E);
size_t switch_workspace_bytes(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C);

const char *switch_status_string(switch_status s);
/* Detail of the last failing call on this host thread ("" if none). */
const char *switch_last_error(void);
/* Hash of the sources the library was built from (32 hex digits; "unknown"
 * when built without it).  The Python binding compares it with the sources
 * beside the library and refuses a stale build. */
const char *switch_build_source_hash(void);

/* ------------------------------------------------------- device entry points */

/* Router, softmax and top-1.  Sources: wq-win note sec. 1 (p = softmax(W_r x),
 * e* = argmax p) and sec. 2 (fp32 inside the router); zffjzz.top note, "core
 * idea and formulas" (Z = XW, p_ti = softmax(Z_t)_i, a_t = argmax, ties to the
 * first index); ai-papers.xuzou.cn card, "method adaptation" (router input,
 * logits and softmax in float32).
 *
 *   x         [T, d]  bf16   tokens                      (unused if logits_in)
 *   w_r       [d, E]  fp32   router weights              (unused if logits_in)
 *   b_r       [E]     fp32   router bias, may be NULL    (unused if logits_in)
 *   logits_in [T, E]  fp32   if not NULL the GEMM is skipped and these logits
 *                            are routed as given (dispatch-only runs)
 *   logits_out[T, E]  fp32   may be NULL; receives z (in GEMM mode)
 *   expert    [T]     int32  e*_t, the raw choice (also for dropped tokens)
 *   gate      [T]     fp32   p_{t,e*_t}
 *   lse       [T]     fp32   log sum_e exp(z_te)
 *   prob_sum  [E]     fp32   sum_t p_te
 *
 * The logits equal an fp32 GEMM up to rounding order: W_r is split into three
 * bf16 terms whose products with bf16 x are exact, accumulated in fp32 on MFMA.
 * The argmax is taken over the logits (equal to the argmax of the exact
 * probabilities).  Workspace: switch_route_workspace_bytes(T, d, E). */
switch_status switch_route(const switch_bf16 *x, const float *w_r, const float *b_r,
                           const float *logits_in, int64_t T, int32_t d, int32_t E,
                           float *logits_out, int32_t *expert, float *gate, float *lse,
                           float *prob_sum, void *ws, size_t ws_bytes, void *stream);

/* Capacity-truncated dispatch in token order.  Sources: zffjzz.top note,
 * "official code reading route" (positions are the cumulative count along the
 * sequence; the raw choice must be kept apart from the capacity mask);
 * wq-win note sec. 3 (truncate by capacity, build the dispatch tensor, cast
 * to low precision and send tokens to their expert); ai-papers.xuzou.cn card,
 * "bottleneck" (fixed capacity; overflow skips the expert layer).
 *
 *   x          [T, d]    bf16   tokens
 *   expert     [T]       int32  e*_t in [0, E)
 *   C                           capacity (switch_capacity); 0 drops every token
 *   position   [T]       int32  pos_t = #{s < t : e*_s = e*_t}
 *   keep       [T]       uint8  pos_t < C
 *   counts     [E]       int32  raw choices per expert
 *   accepted   [E]       int32  min(counts, C)
 *   slot_token [E, C]    int32  token in each slot, -1 if empty; may be NULL
 *   buf        [E, C, d] bf16   buf[e, pos_t] = x_t for kept t, zero rows in
 *                               empty slots
 * Workspace: switch_dispatch_workspace_bytes(T, E). */
switch_status switch_dispatch(const switch_bf16 *x, const int32_t *expert, int64_t T, int32_t d,
                              int32_t E, int32_t C, int32_t *position, uint8_t *keep,
                              int32_t *counts, int32_t *accepted, int32_t *slot_token,
                              switch_bf16 *buf, void *ws, size_t ws_bytes, void *stream);

/* switch_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results, without a workspace.  Its scratch (the
 * per-tile expert counts of the slot scan, ceil(T / 256) * E * 4 bytes) is a
 * fixed device array inside the library, one per GPU, of
 * switch_dispatch_noalloc_max_scratch_bytes() = 4 MiB, held until the
 * process ends; larger T * E return SWITCH_E_UNSUPPORTED with nothing
 * enqueued.  The call makes no hipMalloc/hipFree or other allocating call.
 * Every entry of the scratch is written before it is read, so nothing in it
 * must start at zero; all calls on one GPU share it, so calls that overlap on
 * one GPU (other streams, other host threads) race and must be serialised by
 * the caller.  The first call on a device looks up that device's scratch
 * address (hipGetSymbolAddress) on the current device. */
size_t switch_dispatch_noalloc_max_scratch_bytes(void);
switch_status switch_dispatch_noalloc(const switch_bf16 *x, const int32_t *expert, int64_t T, int32_t d,
                                      int32_t E, int32_t C, int32_t *position, uint8_t *keep,
                                      int32_t *counts, int32_t *accepted, int32_t *slot_token,
                                      switch_bf16 *buf, void *stream);

/* The experts: per expert e and row s < accepted[e],
 *   y[e, s] = ReLU(buf[e, s] W1_e^T) W2_e^T
 * Sources: dmxsf.com essay, "core structure" (experts replace the FFN
 * sublayer); world.lapla.si explainer, "what is inside an expert"
 * (d -> d_ff with ReLU -> d).  bf16 MFMA with fp32 accumulation; the hidden
 * activation is rounded to bf16 once after the ReLU; no expert biases.
 *
 *   buf      [E, C, d]     bf16  expert inputs (switch_dispatch)
 *   accepted [E]           int32 rows in use per expert (0 <= accepted <= C)
 *   w1       [E, d_ff, d]  bf16  first layer, out-features major
 *   w2       [E, d, d_ff]  bf16  second layer, out-features major
 *   y        [E, C, d]     fp32  rows >= accepted[e] are left unwritten
 * Workspace: switch_expert_ffn_workspace_bytes(E, C, d_ff) (the hidden
 * activations, bf16 [E, C, d_ff]). */
switch_status switch_expert_ffn(const switch_bf16 *buf, const int32_t *accepted,
                                const switch_bf16 *w1, const switch_bf16 *w2, int32_t E,
                                int32_t C, int32_t d, int32_t d_ff, float *y, void *ws,
                                size_t ws_bytes, void *stream);

/* Gate-scaled combine back to each token's row.  Sources: wq-win note sec. 1
 * (y = p_e* f_e*(x); overflow tokens continue on the residual) and sec. 2
 * (the selected probability, e.g. 0.7, stays on the output; no
 * renormalisation to 1); sec. 3 (multiply by the routing probability, put
 * back at the original position, add the residual).
 *
 *   out_t = residual_t + keep_t * gate_t * y[expert_t, position_t]
 * computed in fp32 and rounded to bf16 once.  Dropped tokens get
 * out_t = residual_t bit for bit.  residual == NULL gives the branch alone
 * (zero rows for dropped tokens).  y rows are read only for kept tokens.
 *   y [E, C, d] fp32; expert, position [T] int32; keep [T] uint8; gate [T] fp32;
 *   residual [T, d] bf16 or NULL; out [T, d] bf16 (must not alias residual). */
switch_status switch_combine(const float *y, const int32_t *expert, const int32_t *position,
                             const uint8_t *keep, const float *gate, const switch_bf16 *residual,
                             int64_t T, int32_t d, int32_t E, int32_t C, switch_bf16 *out,
                             void *stream);

/* Load-balancing statistics, aux loss and its gradient.  Sources: wq-win note
 * sec. 2 (L = alpha E sum_e f_e P_e; f from the hard choice, not
 * differentiated; P differentiable; alpha = 1e-2 in the paper's recipe);
 * zffjzz.top note, "core idea and formulas" (f counts choices before the
 * capacity limit) and "official code reading route" (the aux statistics are
 * taken before capacity modifies the masks).
 *
 *   counts   [E]    int32 raw choices (switch_dispatch)
 *   prob_sum [E]    fp32  sum_t p_te (switch_route)
 *   logits   [T, E] fp32  needed only when dlogits != NULL
 *   lse      [T]    fp32  needed only when dlogits != NULL
 *   f [E], P [E], loss [1] fp32 outputs; dlogits [T, E] fp32 or NULL
 * For T == 0: f = P = 0 and loss = 0.  loss is reduced in fp64 in a fixed
 * order.  Workspace: switch_aux_loss_workspace_bytes(T, E). */
switch_status switch_aux_loss(const int32_t *counts, const float *prob_sum, const float *logits,
                              const float *lse, int64_t T, int32_t E, float alpha, float *f,
                              float *P, float *loss, float *dlogits, void *ws, size_t ws_bytes,
                              void *stream);

/* Router z-loss (a NEXT row beyond the forward layer).  Source: "MoE routing
 * load collapse" (zffjzz.top), "core idea and formulas": the ST-MoE z-loss
 * L_z = (1/T) sum_t (log sum_i exp z_ti)^2 penalises the log normaliser of the
 * scores; "minimal experiment": a +100 shift of all scores changes it while
 * the probabilities and choices stay the same.
 *
 *   lse      [T]    fp32  log-sum-exp per token (switch_route)
 *   logits   [T, E] fp32  needed only when dlogits != NULL
 *   beta            coefficient, applied to both outputs (z_loss = beta L_z)
 *   z_loss   [1]    fp32  beta (1/T) sum_t lse_t^2, reduced in fp64 in a fixed order
 *   dlogits  [T, E] fp32  or NULL: beta (2/T) lse_t p_tj, written (accumulate = 0)
 *                         or added to the array's contents (accumulate = 1)
 * For T == 0: z_loss = 0. */
switch_status switch_router_z_loss(const float *lse, const float *logits, int64_t T, int32_t E, float beta,
                                   float *z_loss, float *dlogits, int32_t accumulate, void *stream);

/* The whole layer on one stream: route, dispatch, experts, combine, aux loss.
 * Sources: wq-win note sec. 3 (the layer as a step list).  Required pointers
 * are marked (R); optional outputs may be NULL, in which case intermediates
 * live in the workspace (switch_workspace_bytes(T, d, d_ff, E, C)). */
typedef struct switch_layer_args {
    /* inputs */
    const switch_bf16 *x;        /* (R) [T, d] */
    const float *w_r;            /* (R) [d, E] */
    const float *b_r;            /*     [E] or NULL */
    const switch_bf16 *w1;       /* (R) [E, d_ff, d] */
    const switch_bf16 *w2;       /* (R) [E, d, d_ff] */
    /* outputs */
    switch_bf16 *out;            /* (R) [T, d] */
    int32_t *expert;             /* (R) [T] */
    float *gate;                 /* (R) [T] */
    int32_t *position;           /* (R) [T] */
    uint8_t *keep;               /* (R) [T] */
    int32_t *counts;             /* (R) [E] */
    int32_t *accepted;           /* (R) [E] */
    float *f;                    /* (R) [E] */
    float *P;                    /* (R) [E] */
    float *loss;                 /* (R) [1] */
    float *logits;               /*     [T, E] */
    float *lse;                  /*     [T] */
    float *prob_sum;             /*     [E] */
    float *dlogits;              /*     [T, E]; NULL = gradient not computed.  With z_loss
                                  *     set it is the gradient of aux loss + z-loss */
    int32_t *slot_token;         /*     [E, C] */
    switch_bf16 *buf;            /*     [E, C, d] */
    float *y;                    /*     [E, C, d] */
    float *z_loss;               /*     [1]: beta-weighted router z-loss; NULL = not computed */
    /* sizes */
    int64_t T;
    int32_t d, d_ff, E, C;
    float alpha;
    float z_beta;                /* z-loss coefficient (used when z_loss != NULL) */
    int32_t residual;            /* 1: out = x + branch; 0: out = branch only */
    /* routing groups and top-k (see the extended entry points below); zero
     * selects the Switch layer: k = 0 means 1, group = 0 one group of T tokens.
     * With k > 1, expert/gate/position/keep are [T, k]; with several groups,
     * counts/accepted/f/P/prob_sum are [T / group, E], C is the capacity of one
     * group and the buffer has (T / group) * C rows per expert. */
    int32_t k;                   /* choices per token, 1 .. 4 */
    int32_t priority;            /* slot order inside a group: 0 token, 1 rank */
    int64_t group;               /* tokens per routing group */
    int32_t *slot;               /*     [T, k] buffer row of each kept choice, -1 if dropped */
    int32_t *accepted_total;     /*     [E] filled buffer rows per expert */
    switch_bf16 *h;              /*     [E, rows, d_ff] hidden activations relu(buf W1^T) in bf16,
                                  *     kept for switch_layer_bwd */
} switch_layer_args;

switch_status switch_layer_fwd(const switch_layer_args *a, void *ws, size_t ws_bytes, void *stream);
size_t switch_workspace_bytes_ex(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C, int32_t k,
                                 int64_t group);

/* ------------------------------------------- routing groups and top-k choices
 *
 * Routing groups.  Sources: paper card "Switch Transformers" (xuzou.cn),
 * "method adaptation": the input is reshaped to cores x tokens per core and
 * the dispatch/combine tensors carry that group axis; "MoE routing load
 * collapse" (zffjzz.top), "evaluation protocol": every 64 rows apply the
 * capacity limit on their own and the batch metrics are averaged, and
 * "follow-up questions": per-group against merged statistics.  Group g is the
 * `group` consecutive tokens g*group ..; T must be a multiple of `group`, and
 * with more than one group `group` must be a multiple of 64.  Every group has
 * its own capacity C per expert and its own slot counters.
 *
 * Top-k.  Sources: "Mixture of experts" (world.lapla.si), "full means turned
 * back": capacity = tokens per batch / experts x choices per token x capacity
 * factor (so C = switch_capacity(k * group, E, c)); the card's "method
 * adaptation": Switch is the k = 1 case of the earlier top-2 MoE.  A token's
 * choices are its k largest logits in decreasing order, ties to the lower
 * index; each keeps its raw probability as its gate (no renormalisation).
 *
 * Slot order inside a group (priority): 0 = (token, choice) in lexicographic
 * order; 1 = (choice, token), all first choices before any second choice.
 * Buffer rows: each expert's kept choices are packed group after group, so
 * row = (kept choices of that expert in earlier groups) + in-group position,
 * the buffer has groups * C rows per expert and rows 0 .. accepted_total[e]-1
 * of expert e are filled.  One group and k = 1 give the Switch layer exactly.
 */

/* switch_route with k choices per token and per-group probability sums.
 *   expert, gate [T, k]; lse [T]; prob_sum [T / group, E] (one row for one group)
 * Workspace: switch_route_workspace_bytes(T, d, E). */
switch_status switch_route_ex(const switch_bf16 *x, const float *w_r, const float *b_r,
                              const float *logits_in, int64_t T, int32_t d, int32_t E, int32_t k,
                              int64_t group, float *logits_out, int32_t *expert, float *gate,
                              float *lse, float *prob_sum, void *ws, size_t ws_bytes, void *stream);

/* switch_dispatch over the T*k choices with routing groups.
 *   expert [T, k] int32; C capacity of one group per expert;
 *   position [T, k] in-group rank (-1 for ids outside [0, E)); keep [T, k];
 *   slot [T, k] buffer row or -1 (may be NULL with one group);
 *   counts, accepted [T / group, E]; accepted_total [E] (may be NULL with one group);
 *   slot_token [E, groups * C] or NULL; buf [E, groups * C, d] bf16, empty rows zero.
 * Workspace: switch_dispatch_workspace_bytes_ex(T, E, k, group). */
size_t switch_dispatch_workspace_bytes_ex(int64_t T, int32_t E, int32_t k, int64_t group);
switch_status switch_dispatch_ex(const switch_bf16 *x, const int32_t *expert, int64_t T, int32_t d, int32_t E,
                                 int32_t k, int64_t group, int32_t C, int32_t priority, int32_t *position,
                                 uint8_t *keep, int32_t *slot, int32_t *counts, int32_t *accepted,
                                 int32_t *accepted_total, int32_t *slot_token, switch_bf16 *buf, void *ws,
                                 size_t ws_bytes, void *stream);

/* switch_combine over k choices: out_t = residual_t + sum_i keep_ti gate_ti
 * y[expert_ti, slot_ti], the choices added in rank order in fp32, one bf16
 * rounding; a token with every choice dropped gets its residual bit for bit.
 *   y [E, rows, d] fp32; expert, slot [T, k]; keep [T, k]; gate [T, k]. */
switch_status switch_combine_ex(const float *y, const int32_t *expert, const int32_t *slot, const uint8_t *keep,
                                const float *gate, const switch_bf16 *residual, int64_t T, int32_t d, int32_t E,
                                int32_t k, int32_t rows, switch_bf16 *out, void *stream);

/* switch_aux_loss per routing group: f_ge = counts_ge / (k group),
 * P_ge = prob_sum_ge / group, loss = alpha E (1 / groups) sum_g sum_e f_ge P_ge;
 * dlogits_tj = (alpha E / T) p_tj (f_{g(t) j} - sum_e f_{g(t) e} p_te).
 *   counts, prob_sum, f, P [T / group, E]. */
switch_status switch_aux_loss_ex(const int32_t *counts, const float *prob_sum, const float *logits,
                                 const float *lse, int64_t T, int32_t E, int32_t k, int64_t group, float alpha,
                                 float *f, float *P, float *loss, float *dlogits, void *stream);

/* ------------------------------------------------------------- backward
 *
 * Gradients of  J = sum_t <dout_t, out_t> + L_aux (+ L_z)  for the Switch
 * layer, and for its routing-group / top-k form, with the choices and
 * capacity masks of the forward held fixed: argmax has no gradient and the
 * router learns through the selected gates.  Sources: wq-win note sec. 2 (the router stays
 * differentiable through p_e*; the balance loss is added to the training
 * loss); zffjzz.top note, "troubleshooting" (finite differences that keep the
 * discrete choices and masks).
 *
 * For a kept token t with expert e and slot s, a_t = W1_e x_t, g_t = gate_t:
 *   dgate_t = <dout_t, y[e, s]>;  dy = g_t dout_t;  dA = (dy W2_e) * [a_t > 0]
 *   dW2_e = sum dy relu(a)^T;  dW1_e = sum dA x^T;  dx_t = dout_t + dA W1_e
 *   dz_tj = dgate_t g_t (delta_{j e} - p_tj) + dL_aux/dz_tj (+ dL_z/dz_tj)
 *   dW_r = x^T dz;  db_r = sum_t dz_t;  dx_t += W_r dz_t
 * Dropped tokens: dx_t = dout_t + W_r dz_t.
 * With k choices every kept choice (t, i) is one buffer row and follows the
 * rule above with its own gate g_ti = p_{t, e_ti}; dx_t adds the dA W1 terms
 * of all kept choices and dz_tj = sum_i dgate_ti g_ti (delta_{j e_ti} - p_tj)
 * + dL_aux/dz_tj (+ dL_z/dz_tj), the aux term with the f of the token's group.
 * Sources for that form: "Mixture of experts" (world.lapla.si), "full means
 * turned back" (top-k gates, no renormalisation); zffjzz.top note,
 * "evaluation protocol" (per-group statistics).
 *
 * Precision: dy and dA are rounded to bf16 (the MFMA inputs), the GEMMs
 * accumulate in fp32, weight and router gradients are fp32, dx is rounded to
 * bf16 once; its router term W_r dz_t is formed from two-term bf16 splits of
 * W_r and dz (relative error about 2^-15, below that rounding).  dz, dgate and the reductions over tokens (db_r, dW_r) are fp32
 * with fp64 sums in a fixed order.  The aux gradient treats f as constant. */
typedef struct switch_layer_bwd_args {
    /* saved by switch_layer_fwd (with logits and h requested) */
    const switch_bf16 *x;        /* [T, d] */
    const float *w_r;            /* [d, E] */
    const switch_bf16 *w1;       /* [E, d_ff, d] */
    const switch_bf16 *w2;       /* [E, d, d_ff] */
    const int32_t *expert;       /* [T] */
    const float *gate;           /* [T] */
    const int32_t *position;     /* [T] */
    const uint8_t *keep;         /* [T] */
    const int32_t *accepted;     /* [E] */
    const float *f;              /* [E] load fractions of the aux loss */
    const float *logits;         /* [T, E] */
    const float *lse;            /* [T] */
    const switch_bf16 *buf;      /* [E, C, d] */
    const switch_bf16 *h;        /* [E, C, d_ff] */
    const float *y;              /* [E, C, d] */
    const switch_bf16 *dout;     /* [T, d] gradient at the layer output */
    /* outputs */
    switch_bf16 *dx;             /* [T, d] */
    float *dw_r;                 /* [d, E] */
    float *db_r;                 /* [E] */
    float *dw1;                  /* [E, d_ff, d] */
    float *dw2;                  /* [E, d, d_ff] */
    float *dz;                   /*     [T, E] total gradient at the logits, or NULL */
    float *dgate;                /*     [T] (or [T, k]) <dout_t, y[e, s]> for kept choices (0 if
                                  *     dropped), or NULL */
    /* sizes */
    int64_t T;
    int32_t d, d_ff, E, C;
    float alpha;                 /* aux-loss weight of the forward */
    float z_beta;                /* z-loss weight (0: no z-loss term) */
    /* routing groups and top-k, as in switch_layer_args; zero selects the
     * Switch layer (k = 0 means 1, group = 0 one group of T tokens).  With
     * k > 1, expert/gate/position/keep/dgate are [T, k]; with several groups
     * f is [T / group, E], C is the capacity of one group, buf/h/y have
     * (T / group) * C rows per expert, and slot and accepted_total replace
     * position and accepted (which are then not read). */
    int32_t k;                   /* choices per token, 1 .. 4 */
    int64_t group;               /* tokens per routing group */
    const int32_t *slot;         /* [T, k] buffer row of each kept choice (several groups) */
    const int32_t *accepted_total; /* [E] filled buffer rows per expert (several groups) */
    /* 0: dx = dout + (expert and router terms), the layer's input gradient.
     * 1: dx = the expert and router terms alone (sum of the kept choices'
     *    dA W1 rows plus W_r dz_t), rounded to bf16 once; the identity path
     *    of the residual is left to the caller.  Other values are rejected. */
    int32_t dx_branch_only;
} switch_layer_bwd_args;

/* Workspace of switch_layer_bwd: switch_layer_bwd_workspace_bytes_ex(T, d, d_ff,
 * E, C, k, group) with C the capacity of one group; the plain query is its
 * k = 1, one-group case.  Both return 0 for sizes the layer rejects. */
size_t switch_layer_bwd_workspace_bytes(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C);
size_t switch_layer_bwd_workspace_bytes_ex(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C, int32_t k,
                                           int64_t group);
switch_status switch_layer_bwd(const switch_layer_bwd_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------- measurement */

/* A plain device-to-device copy kernel (16-byte vectors); the reference
 * point for bandwidth and hardware-counter calibration.  nbytes must be a
 * multiple of 16 and both pointers 16-byte aligned. */
switch_status switch_stream_copy(void *dst, const void *src, size_t nbytes, void *stream);

/* Rows per token tile of the first expert GEMM for an expert FFN over E
 * experts with `rows` buffer rows each (the capacity, or groups x capacity
 * with routing groups), `assignments` routed choices (T k in a layer; 0 when
 * unknown, as in switch_expert_ffn) and hidden width d_ff, on the current
 * device: 32, 64 or 128 rows by the buffer rows, or 320 ("tall" tiles, one per
 * expert and weight block) when experts are expected to fill more than one
 * 128-row tile and the grid holds at least four tiles per compute unit.
 * Informational (no device work); switch_layer_fwd (any k and group) and
 * switch_expert_ffn choose their tiles with this function.  Returns 0 for
 * E, rows or d_ff <= 0. */
int32_t switch_ffn_gemm1_token_tile(int32_t E, int32_t rows, int64_t assignments, int32_t d_ff);

/* Per-launch timing.  While enabled, every kernel launch made by this library
 * is bracketed by two HIP events recorded on the launch's own stream.
 * switch_profile_collect waits for the recorded events, writes up to `max`
 * (kernel id, milliseconds) pairs in launch order, clears the record and
 * returns how many were written (negative on a HIP error).  Not thread safe. */
void switch_profile_enable(int on);
int switch_profile_collect(int max, int32_t *kernel_ids, float *ms);
const char *switch_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* SWITCH_MOE_H */
