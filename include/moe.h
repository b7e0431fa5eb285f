/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN forward.
 *
 * The layer (sources are page titles as printed on the pages):
 *   1. router logits  l = x . W_r + b            (linear router: "AMD MI300X平台上的MoE
 *      模型训练实践", section 3.2; zero-initialised gate bias: TorchTitan 1K-GPU MoE
 *      article, section 4.2)
 *   2. p = softmax(l / tau) over all experts      (router temperature: "AMD GPU深度学习优化
 *      与ZAYA1大模型实践", section 7; gate temperature 0.3: TorchTitan article, section 2.1)
 *   3. top-k experts per token, gates = p of the chosen experts, optionally
 *      renormalised over them                    (top-1: ZAYA1 page, section 2; top-2:
 *      TorchTitan article, section 2.1)
 *   4. capacity C per expert from a capacity factor, overflow dropped in token
 *      order                                     (capacity factor 1.25: TorchTitan article,
 *      section 2.1)
 *   5. token permutation grouped by expert
 *   6. per-expert GeGLU FFN h = GELU(x W_gate) * (x W_up), o = h W_down
 *                                                 (expert-FFN kernel: MI300X page, section 4.2;
 *      GeGLU fused with the matmul: ZAYA1 page, section 3.2)
 *   7. gate-weighted un-permute and combine      y_t = sum_j g_tj o_(t,j)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (memory of the current HIP device) unless
 *     the comment says "host".  Arrays are row-major and contiguous.  Device
 *     arrays must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream), passed as void*
 *     so that this header needs no HIP header and plain C callers can include
 *     it.  Every call only enqueues work on that stream and returns; nothing
 *     synchronises with the host.  Results are visible after the caller
 *     synchronises the stream.
 *   - The caller owns every buffer.  The library allocates no memory, frees
 *     nothing and keeps no pointer after a call returns.
 *   - Errors are reported by the returned moe_status; nothing is thrown across
 *     the ABI.  Arguments are validated on the host before anything is
 *     enqueued, so an invalid call enqueues nothing.  On any error the output
 *     contents are unspecified.  moe_last_error() gives a message for the
 *     calling thread's most recent failure.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified results.
 *   - Floating-point results are deterministic: the same inputs on the same
 *     device give bit-identical outputs (no float atomics anywhere).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,  /* a size, pointer, alignment or config field is out of range */
    MOE_ERR_UNSUPPORTED = -2,  /* a valid layer this build does not run (dtype) */
    MOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the *_workspace_size() */
    MOE_ERR_HIP = -4           /* the HIP runtime reported an error when enqueuing */
} moe_status;

typedef enum {
    MOE_F32 = 0,   /* activations and weights fp32 */
    MOE_BF16 = 1   /* activations and weights bf16; accumulation is always fp32 */
} moe_dtype;

/* Layer shape and routing parameters.  Limits (checked by every call):
 *   0 <= T, T * k < 2^31           tokens (T = 0 is a valid empty batch)
 *   d % 64 == 0, 64 <= d <= 16384  model width (64-multiple rule of the ZAYA1
 *                                  page's parameter table, section 2)
 *   d_ff % 64 == 0, 64 <= d_ff <= 65536
 *   1 <= E <= 256, 1 <= k <= min(E, 8)
 *   temperature > 0 and finite
 *   cap_den == 0: no capacity limit (C = T); else cap_num >= 0, cap_den > 0
 *   renormalize: 0 or 1;  dtype: a moe_dtype
 *   drop_policy: a moe_drop_policy (appended field; zero = the default)
 *   layout: a moe_layout (appended field; zero = the default); the padded
 *           layout needs a capacity limit (cap_den > 0) and E * C < 2^31
 *   route_threshold, k_min (appended fields; zero = a fixed k): see below */
typedef struct {
    int64_t T;
    int32_t d;
    int32_t E;
    int32_t k;
    int32_t d_ff;
    float temperature;
    int32_t cap_num;
    int32_t cap_den;
    int32_t renormalize;
    int32_t dtype;
    int32_t drop_policy;
    int32_t layout;
    /* Dynamic number of experts per token (a variant: the TorchTitan 1K-GPU
     * article, section 2.1, has each token activate 2-4 experts).  With
     * route_threshold in (0, 1], token t takes k_t experts: the fewest of its
     * k highest-ranked ones, at least k_min (1 <= k_min <= k), whose softmax
     * probabilities sum to at least route_threshold (k when none do).  Gates
     * are p of those k_t experts (renormalised over them when renormalize);
     * topk_idx / topk_gate slots j >= k_t hold -1 and 0, and no row.  The
     * decision is evaluated in fp64 from the fp32 logits.  The capacity then
     * scales the realised mean load: C = ceil(cap_num * A / (cap_den * E))
     * for the A assignments of the batch, computed on the device
     * (moe_capacity and moe_max_rows give the bound for A = T * k).  Not with
     * the padded layout (MOE_ERR_UNSUPPORTED).  In moe_backward the count is
     * piecewise constant in the logits, like the top-k choice: the unused
     * slots carry no gradient (dgate 0) and renormalised gates are
     * differentiated over the k_t experts taken.
     * route_threshold = 0 (with k_min = 0): every token takes k experts. */
    float route_threshold;
    int32_t k_min;
} moe_config;

/* Which assignments fill an expert's C slots first when it overflows. */
typedef enum {
    /* token order: (t', j') before (t, j) iff t' < t -- the reading of the
     * TorchTitan 1K-GPU article's "drop the overflow in token order"
     * (section 2.1) */
    MOE_DROP_TOKEN_ORDER = 0,
    /* choice order (GShard-style priority, a variant): every first choice, in
     * token order, before every second choice, and so on: (t', j') before
     * (t, j) iff j' < j, or j' == j and t' < t */
    MOE_DROP_CHOICE_ORDER = 1
} moe_drop_policy;

/* Row layout of the expert-grouped buffers (x_perm, h, y_perm). */
typedef enum {
    /* compact: expert e's kept rows at offset[e] .. offset[e+1]-1, offset the
     * exclusive prefix of the kept counts; no empty rows */
    MOE_LAYOUT_COMPACT = 0,
    /* padded to capacity (a variant: the fixed per-expert buffer that a
     * capacity factor implies, TorchTitan 1K-GPU article, section 2.1):
     * expert e owns rows e C .. e C + C - 1 (C the effective capacity), its
     * kept rows first; the others are empty (token_of_row -1, x_perm zero).
     * The grouped GEMMs then run C rows for every expert. */
    MOE_LAYOUT_PADDED = 1
} moe_layout;

/* Host.  Expert capacity C = ceil(cap_num * k * T / (cap_den * E)) in exact
 * integer arithmetic, or T when cap_den == 0.  Returns -1 for an invalid
 * config.  (The pages give only the factor, 1.25; tokens-per-expert times the
 * factor, rounded up, is the reading used.) */
int64_t moe_capacity(const moe_config* cfg);

/* Host.  Rows of the expert-grouped buffers: min(T * k, C * E) in the compact
 * layout (an upper bound on rows kept), E * min(C, T) in the padded one.  -1
 * if the config is invalid.  x_perm, h and y_perm need this many rows;
 * token_of_row needs max(T * k, this) entries. */
int64_t moe_max_rows(const moe_config* cfg);

/* Host.  Bytes of workspace moe_forward needs for this config (on the
 * current device), written to *bytes.  It is also enough for moe_dispatch. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Host.  Bytes of workspace moe_dispatch needs for this config (at most
 * moe_workspace_size's), written to *bytes. */
moe_status moe_dispatch_workspace_size(const moe_config* cfg, size_t* bytes);

/* Host.  Static, human-readable name of a status code. */
const char* moe_status_string(moe_status s);

/* Host.  Message describing the calling thread's most recent failed call
 * ("" if none).  The string is owned by the library and valid until the
 * thread's next call into it. */
const char* moe_last_error(void);

/* Steps 1-3: router logits, softmax with temperature, top-k and gates.
 *   x        [T, d]   dtype       input activations
 *   w_router [d, E]   dtype       router weight
 *   bias     [E]      fp32        router bias, or NULL for none
 *   logits   [T, E]   fp32  out   l = x W_r + b, fp32 accumulation
 *   topk_idx [T, k]   int32 out   chosen experts, largest logit first; equal
 *                                 logits order the lower expert index first.
 *                                 Ranking uses the fp32 logits themselves.
 *   topk_gate[T, k]   fp32  out   p of each chosen expert, divided by the sum
 *                                 of the chosen p when cfg->renormalize. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* bias, float* logits, int32_t* topk_idx,
                     float* topk_gate, void* stream);

/* Steps 2-3 only, from given fp32 logits [T, E] (same top-k and gate code as
 * moe_route; lets callers and tests route exactly-known logits, e.g. ties). */
moe_status moe_route_from_logits(const moe_config* cfg, const float* logits,
                                 int32_t* topk_idx, float* topk_gate, void* stream);

/* Variant of steps 1-3: the ZAYA1 MLP router ("AMD MI300X平台上的MoE模型训练实践",
 * section 3.2), forward.  Per token:
 *   u  = x W_down + b_down                  [r]
 *   z  = RMSnorm(u + gamma * prev)          v / sqrt(mean_j v_j^2 + eps), no scale
 *   h1 = GELU(z W1 + b1), h2 = GELU(h1 W2 + b2)   [m], GELU in its erf form
 *   l  = h2 W3 + b3 + pid_bias              [E]
 * then the temperature softmax, top-k and gates of moe_route (same code, same
 * outputs).  The page gives r = 256 and m = 1024 and leaves gamma, eps and the
 * load-balance controller's update rule open: gamma and eps are parameters
 * here, and the controller enters through its output, pid_bias.  bf16 only
 * (MOE_ERR_UNSUPPORTED for fp32); fp32 accumulation, u, z, h1 and h2 rounded
 * once each to bf16, logits fp32.  Weights row-major in the layer's dtype,
 * biases fp32 and optional (NULL = zero). */
typedef struct {
    int32_t r;              /* down-projection width, 64 <= r <= 1024, r % 64 == 0 */
    int32_t m;              /* hidden width, 64 <= m <= 16384, m % 64 == 0 */
    float gamma;            /* weight of prev, finite */
    float eps;              /* RMS-norm epsilon, finite, >= 0 */
    const void* w_down;     /* [d, r] */
    const float* b_down;    /* [r] or NULL */
    const void* w1;         /* [r, m] */
    const float* b1;        /* [m] or NULL */
    const void* w2;         /* [m, m] */
    const float* b2;        /* [m] or NULL */
    const void* w3;         /* [m, E] */
    const float* b3;        /* [E] or NULL */
    const float* pid_bias;  /* [E] or NULL */
} moe_mlp_router;

/* Host.  Workspace bytes moe_route_mlp needs (u, z [T, r], h1, h2 [T, m]
 * bf16 and E fp32). */
moe_status moe_mlp_router_workspace_size(const moe_config* cfg, const moe_mlp_router* router,
                                         size_t* bytes);

/*   x         [T, d]  dtype in
 *   prev      [T, r]  dtype in   the previous layer's router state, or NULL
 *   logits    [T, E]  fp32  out
 *   topk_idx, topk_gate  as for moe_route
 *   workspace ws_bytes >= moe_mlp_router_workspace_size(cfg, router, .) */
moe_status moe_route_mlp(const moe_config* cfg, const moe_mlp_router* router, const void* x,
                         const void* prev, float* logits, int32_t* topk_idx, float* topk_gate,
                         void* workspace, size_t ws_bytes, void* stream);

/* Steps 4-5: capacity, token-order drops and the expert-grouped permutation.
 *   topk_idx      [T, k]         int32  in
 *   x             [T, d]         dtype  in
 *   x_perm        [max_rows, d]  dtype  out  row r = x[token_of_row[r]]; rows of
 *                                            expert e are offset[e]..offset[e+1)-1,
 *                                            in cfg->drop_policy's priority order
 *                                            (token order: ascending token)
 *   expert_count  [E]            int32  out  assignments per expert before drops
 *   expert_offset [E + 1]        int32  out  compact: exclusive prefix of kept counts
 *                                            min(count, C), [E] = rows kept;
 *                                            padded: e * C
 *   row_of        [T, k]         int32  out  row of assignment (t, j), -1 if dropped
 *   token_of_row  [max(T * k, max_rows)]
 *                                int32  out  token of each kept row; empty rows and
 *                                            entries past offset[E] are set to -1
 * In the padded layout the empty rows of x_perm are set to zero.
 *   workspace     ws_bytes >= moe_dispatch_workspace_size(cfg, .)
 * An assignment (t, j) to expert e is kept iff fewer than C assignments to e
 * come before it in cfg->drop_policy's order; with MOE_DROP_TOKEN_ORDER, iff
 * fewer than C earlier tokens (t' < t, at any rank) chose e ("drop overflow
 * in token order"). */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                        void* x_perm, int32_t* expert_count, int32_t* expert_offset,
                        int32_t* row_of, int32_t* token_of_row, void* workspace,
                        size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels, results bit-identical to moe_dispatch's, with its
 * workspace (the per-block expert-count tables, at most 2 * 256 * E int32)
 * in a static device buffer of the library instead of a caller's buffer.
 * That buffer, MOE_DISPATCH_SCRATCH_BYTES (512 KiB) per device, is held until
 * the process ends; a config whose tables need more is rejected with
 * MOE_ERR_INVALID_ARG (no valid config does: blocks <= 256, E <= 256).
 * Nothing here allocates: no hipMalloc, no hipFree.  Every call on one device
 * shares that device's buffer and leaves its contents behind (no call relies
 * on them), so calls that overlap on one device race; calls must be ordered
 * (e.g. on one stream).  Arguments and results as for moe_dispatch. */
#define MOE_DISPATCH_SCRATCH_BYTES (512u * 1024u)
moe_status moe_dispatch_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                                void* x_perm, int32_t* expert_count, int32_t* expert_offset,
                                int32_t* row_of, int32_t* token_of_row, void* stream);

/* Expert-load telemetry from the per-expert assignment counts before drops
 * (expert_count as written by moe_dispatch).  The ZAYA1 page keeps the expert
 * load balance within +-5% (section 3.2) and monitors it during training; the
 * balance figure here is the largest deviation of an expert's load from the
 * mean, relative to the mean.
 *   expert_count [E]  int32 in
 *   stats        [8]  fp64  out  (device)
 *     [0] mean load m = sum_e count_e / E  [1] max count   [2] min count
 *     [3] max / m                          [4] max_e |count_e - m| / m
 *     [5] population std / m               [6] dropped assignments
 *         sum_e max(0, count_e - C)        [7] experts with no assignment
 *     (the three ratios are 0 when there are no assignments)
 * One workgroup; fp64 throughout, so the integers are exact. */
moe_status moe_load_stats(const moe_config* cfg, const int32_t* expert_count, double* stats,
                          void* stream);

/* The MLP router's load-balance controller: one step of a PID controller on
 * the expert load ("AMD MI300X平台上的MoE模型训练实践", section 3.2, puts a
 * PID balance controller on the router logits; its training notes raise the
 * PID gains over a warmup).  The page gives no update rule; the one here is
 * the textbook discrete PID loop, one per expert, on the relative load error,
 * and its output is the additive logit bias that moe_mlp_router.pid_bias
 * takes.  Called once per training step with that step's counts before drops
 * (expert_count as written by moe_dispatch):
 *   m = sum_e count_e / E;  err_e = (m - count_e) / m  (0 when m = 0)
 *   I_e <- I_e + err_e;     D_e = err_e - prev_e;      prev_e <- err_e
 *   pid_bias_e = scale * ((kp err_e + ki I_e) + kd D_e), rounded once to fp32
 * An expert below the mean load gets a positive error, so its bias rises.
 *   expert_count [E]     int32 in
 *   state        [2, E]  fp64  in/out  row 0 the integrals I, row 1 the
 *                                      previous errors; zero before the first
 *                                      step (its D is then err itself)
 *   pid_bias     [E]     fp32  out
 * gains: kp, ki, kd and scale finite (MOE_ERR_INVALID_ARG otherwise); scale
 * ramps the controller's output during a warmup (0 = off, 1 = full gains).
 * One workgroup, fp64 throughout, each operation rounded once in the order
 * written. */
typedef struct {
    double kp, ki, kd;
    double scale;
} moe_pid_gains;
moe_status moe_pid_update(const moe_config* cfg, const moe_pid_gains* gains,
                          const int32_t* expert_count, double* state, float* pid_bias,
                          void* stream);

/* Step 6: grouped GeGLU expert FFN over the permuted rows.
 *   x_perm        [max_rows, d]    dtype in   (rows past expert_offset[E] ignored)
 *   expert_offset [E + 1]          int32 in   as written by moe_dispatch
 *   w_gate, w_up  [E, d, d_ff]     dtype in
 *   w_down        [E, d_ff, d]     dtype in
 *   h             [max_rows, d_ff] dtype out  GELU_erf(x W_gate) * (x W_up), fp32
 *                                             epilogue rounded once to dtype
 *   y_perm        [max_rows, d]    dtype out  h W_down, fp32 accumulation
 * Rows at and past expert_offset[E] of h and y_perm are not written. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm,
                          const int32_t* expert_offset, const void* w_gate,
                          const void* w_up, const void* w_down, void* h, void* y_perm,
                          void* stream);

/* Step 6, first half only: h = GELU_erf(x_perm W_gate) * (x_perm W_up)
 * (same arguments and results as in moe_expert_ffn; one kernel launch). */
moe_status moe_expert_gate_up(const moe_config* cfg, const void* x_perm,
                              const int32_t* expert_offset, const void* w_gate,
                              const void* w_up, void* h, void* stream);

/* Step 6, second half only: y_perm = h W_down (one kernel launch). */
moe_status moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offset,
                           const void* w_down, void* y_perm, void* stream);

/* Step 7: y[t] = sum over kept j (ascending) of topk_gate[t][j] * y_perm[row_of[t][j]],
 * accumulated in fp32 and rounded once to dtype; a token with nothing kept
 * gets y = 0.
 *   y_perm [max_rows, d] dtype in;  row_of [T, k] int32 in;
 *   topk_gate [T, k] fp32 in;       y [T, d] dtype out */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of,
                       const float* topk_gate, void* y, void* stream);

/* Steps 1-7 on one stream, intermediates in the workspace
 * (ws_bytes >= moe_workspace_size(cfg, .), sized for the current device).
 * Same arguments and results as the four calls above in sequence, bit for bit,
 * with one exception below.  Some intermediates are never formed: bf16 layers
 * gather their x rows inside the gate/up GEMM (no x_perm), and bf16 top-1
 * layers whose capacity keeps every token have the down GEMM write y itself
 * (no y_perm, no combine).  When such a layer has too few experts to fill the
 * device's CUs with down-GEMM tiles, the down GEMM runs in two K slices whose
 * fp32 partial sums a second kernel adds (rounding and gating as the combine
 * does); its y then differs from the staged calls' by that fp32 summation
 * order only.  The workspace's contents after the call are unspecified. */
moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* bias, const void* w_gate, const void* w_up,
                       const void* w_down, void* y, void* workspace, size_t ws_bytes,
                       void* stream);

/* Host.  Bytes of workspace moe_backward needs (the recomputed routing and
 * dispatch maps, the expert pre-activations, the per-row gradients). */
moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes);

/* Backward of steps 1-7 for an upstream gradient dy = dL/dy (training, the
 * step that follows the forward on every page: the TorchTitan 1K-GPU article
 * trains this layer, section 2; "AMD MI300X平台上的MoE模型训练实践" trains it
 * too, section 4).  Both dtypes and either layout (the padded layout's
 * empty rows are zero in every product, so the gradients equal the compact
 * layout's).  The forward's routing and expert
 * pre-activations are recomputed from the inputs, as the activation
 * recomputation of that training page's section 4.1 does (same kernels, same
 * values as moe_forward);
 * top-k selection, the dynamic expert count and capacity drops are piecewise
 * constant, so no gradient passes through them.  With
 * p = softmax(logits / temperature), per kept
 * assignment (t, j) of expert e, g = x_t W_gate[e], u = x_t W_up[e],
 * h = GELU_erf(g) u, o = h W_down[e]:
 *   dgate[t][j] = dy_t . o (0 for a dropped assignment)
 *   dh = gate dy_t W_down[e]^T; du = dh GELU(g); dg = dh u GELU'(g)
 *   dw_down[e] += (gate h)^T dy_t, dw_gate[e] += x_t^T dg, dw_up[e] += x_t^T du
 *   gates: renormalised (gate_j = p_j / S, S over the experts the token
 *   took): dp_j = (dgate_j - sum dgate gate) / S,
 *   raw: dp_j = dgate_j; dlogit = p (dp - p . dp) / temperature
 *   dw_router = x^T dlogit, dbias = sum_t dlogit,
 *   dx_t = sum_j (dg W_gate[e]^T + du W_up[e]^T) + dlogit_t W_router^T
 *   x, dy       [T, d]          dtype in     dx [T, d] dtype out
 *   w_router    [d, E]          dtype in     dw_router [d, E] fp32 out
 *   bias        [E]             fp32 in, may be NULL (zero bias)
 *   dbias       [E]             fp32 out, may be NULL (not written)
 *   w_gate, w_up [E, d, d_ff]   dtype in     dw_gate, dw_up [E, d, d_ff] fp32 out
 *   w_down      [E, d_ff, d]    dtype in     dw_down [E, d_ff, d] fp32 out
 *   dgate       [T, k]          fp32 out, may be NULL (not written)
 * Gradients overwrite their outputs (no accumulation); an expert with no kept
 * rows gets zero weight gradients.  Products accumulate in fp32; in bf16
 * layers the expert pre-activations and the per-row gradients fed to the
 * next product are rounded to bf16 (fp32 layers keep them in fp32); the sums
 * over tokens and experts run in a fixed order (the results are
 * deterministic). */
moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const float* bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* dy, void* dx, float* dw_router,
                        float* dbias, float* dw_gate, float* dw_up, float* dw_down, float* dgate,
                        void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
