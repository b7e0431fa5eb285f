/*
 * moe_oracle.c -- plain fp64 CPU oracle of the sparse Mixture-of-Experts FFN
 * forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the HIP library; it is written from the definition
 * of the layer, one step per function, with no blocking, fusion or reordering
 * of any sum beyond what the definition states.  Loops over independent
 * tokens (or independent rows) are spread over OpenMP threads; every single
 * sum runs in ascending index order in one thread.
 *
 * Sources (page titles as printed on the pages):
 *  - linear router logits: "AMD MI300X平台上的MoE模型训练实践", section 3.2
 *    (a conventional MoE uses a simple linear router); zero-initialised gate
 *    bias: TorchTitan 1K-GPU MoE article, section 4.2.
 *  - softmax with a router temperature: "AMD GPU深度学习优化与ZAYA1大模型实践",
 *    section 7 (router_temp), and the TorchTitan article, section 2.1
 *    (gate temperature 0.3).
 *  - top-1 routing: ZAYA1 page, section 2; top-2 with a capacity factor of
 *    1.25: TorchTitan article, section 2.1.
 *  - GeGLU expert FFN: ZAYA1 page, section 3.2 (GeGLU fused with the matmul);
 *    GELU in its erf form (the router listing on the MI300X page, section 3.2,
 *    uses nn.GELU, whose default is the erf form).
 *
 * Readings taken where the pages are silent (each one stated again at the
 * function that applies it):
 *  - top-k ranks the logits themselves, ties go to the lower expert index;
 *  - p = softmax(l / tau) over all E experts; with renormalisation the k chosen
 *    gates are p divided by the sum of the chosen p, otherwise the raw p;
 *  - capacity C = ceil(cap_num * k * T / (cap_den * E)) in exact integers,
 *    C = T when there is no limit;
 *  - overflow is dropped in token order: for each expert the first C tokens
 *    (ascending t, whatever the rank j at which they chose it) are kept;
 *  - dropped assignments contribute nothing and the kept gates are not
 *    renormalised again; a token with every assignment dropped gets y = 0.
 *
 * dtype codes: 0 = fp32, 1 = bf16 (raw 16-bit patterns, the upper half of an
 * IEEE fp32).  Every input value is widened exactly to fp64 before use.
 */
#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact fp64 value of element i of an fp32 or bf16 array. */
static double load(const void* p, int64_t i, int dtype) {
    float f;
    if (dtype == 0) {
        f = ((const float*)p)[i];
    } else {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        memcpy(&f, &u, sizeof f);
    }
    return (double)f;
}

/* GELU, erf form: v * Phi(v) = 0.5 * v * (1 + erf(v / sqrt(2))). */
static double gelu(double v) { return 0.5 * v * (1.0 + erf(v / sqrt(2.0))); }

/* Step 1 -- router logits l[t][e] = sum_i x[t][i] * Wr[i][e] + b[e].
 * x is [T][d], Wr is [d][E] (row-major); bias may be NULL (zero). */
void orc_logits(int64_t T, int64_t d, int64_t E, int dtype, const void* x,
                const void* wr, const float* bias, double* logits) {
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t i = 0; i < d; ++i)
                s += load(x, t * d + i, dtype) * load(wr, i * E + e, dtype);
            if (bias) s += (double)bias[e];
            logits[t * E + e] = s;
        }
    }
}

/* Variant of step 1 -- ZAYA1's MLP router ("AMD MI300X平台上的MoE模型训练实践",
 * section 3.2), forward, per token:
 *   u  = x Wd + bd                          down-projection to r (256 there)
 *   v  = u + gamma * prev                   depth averaging with the previous
 *                                           layer's router state (prev may be NULL)
 *   z  = v / sqrt(sum_j v_j^2 / r + eps)    RMS norm without a learned scale
 *   h1 = GELU(z W1 + b1), h2 = GELU(h1 W2 + b2)   two layers m wide (1024 there)
 *   l  = h2 W3 + b3 + pid                   pid: the load-balance controller's
 *                                           per-expert bias on the logits
 * Wd [d][r], W1 [r][m], W2 [m][m], W3 [m][E] row-major in dtype; prev [T][r]
 * in dtype; biases fp32, each may be NULL (zero).  The page leaves gamma, eps
 * and the controller's update rule open: gamma and eps are parameters and the
 * controller enters only through its output, pid.  z, h1, h2 may be NULL. */
void orc_mlp_router(int64_t T, int64_t d, int64_t r, int64_t m, int64_t E, int dtype,
                    const void* x, const void* prev, double gamma, double eps,
                    const void* wd, const float* bd, const void* w1, const float* b1,
                    const void* w2, const float* b2, const void* w3, const float* b3,
                    const float* pid, double* logits, double* z_out, double* h1_out,
                    double* h2_out) {
    #pragma omp parallel
    {
        double* v = (double*)malloc(sizeof(double) * (size_t)r);
        double* a = (double*)malloc(sizeof(double) * (size_t)m);
        double* b = (double*)malloc(sizeof(double) * (size_t)m);
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t j = 0; j < r; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < d; ++i) s += load(x, t * d + i, dtype) * load(wd, i * r + j, dtype);
                if (bd) s += (double)bd[j];
                if (prev) s += gamma * load(prev, t * r + j, dtype);
                v[j] = s;
            }
            double ss = 0.0;
            for (int64_t j = 0; j < r; ++j) ss += v[j] * v[j];
            double inv = 1.0 / sqrt(ss / (double)r + eps);
            for (int64_t j = 0; j < r; ++j) {
                v[j] *= inv;
                if (z_out) z_out[t * r + j] = v[j];
            }
            for (int64_t n = 0; n < m; ++n) {
                double s = 0.0;
                for (int64_t j = 0; j < r; ++j) s += v[j] * load(w1, j * m + n, dtype);
                if (b1) s += (double)b1[n];
                a[n] = gelu(s);
                if (h1_out) h1_out[t * m + n] = a[n];
            }
            for (int64_t n = 0; n < m; ++n) {
                double s = 0.0;
                for (int64_t j = 0; j < m; ++j) s += a[j] * load(w2, j * m + n, dtype);
                if (b2) s += (double)b2[n];
                b[n] = gelu(s);
                if (h2_out) h2_out[t * m + n] = b[n];
            }
            for (int64_t e = 0; e < E; ++e) {
                double s = 0.0;
                for (int64_t j = 0; j < m; ++j) s += b[j] * load(w3, j * E + e, dtype);
                if (b3) s += (double)b3[e];
                if (pid) s += (double)pid[e];
                logits[t * E + e] = s;
            }
        }
        free(v);
        free(a);
        free(b);
    }
}

/* Step 2 -- top-k expert choice and gate weights, per token.
 * Experts are ranked by their logit (largest first); equal logits rank the
 * lower expert index first.  The ranking uses the logits themselves, never
 * l / tau or p: tau > 0 keeps the order, and ranking rounded quotients could
 * merge distinct logits.
 * p[e] = exp((l[e] - max l) / tau) / sum_e' exp((l[e'] - max l) / tau).
 * renorm != 0: gate[j] = p[idx[j]] / sum_j' p[idx[j']]; else gate[j] = p[idx[j]]. */
void orc_route(int64_t T, int64_t E, int64_t k, double tau, int renorm,
               const double* logits, int32_t* idx, double* gate) {
    #pragma omp parallel
    {
        char* taken = (char*)calloc((size_t)E, 1);
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* l = logits + t * E;
            memset(taken, 0, (size_t)E);
            for (int64_t j = 0; j < k; ++j) {
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e) {
                    if (taken[e]) continue;
                    if (best < 0 || l[e] > l[best]) best = e;   /* strict: ties keep the lower e */
                }
                taken[best] = 1;
                idx[t * k + j] = (int32_t)best;
            }
            double m = l[0];
            for (int64_t e = 1; e < E; ++e) if (l[e] > m) m = l[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) { p[e] = exp((l[e] - m) / tau); z += p[e]; }
            for (int64_t e = 0; e < E; ++e) p[e] /= z;
            double s = 0.0;
            for (int64_t j = 0; j < k; ++j) s += p[idx[t * k + j]];
            for (int64_t j = 0; j < k; ++j)
                gate[t * k + j] = renorm ? p[idx[t * k + j]] / s : p[idx[t * k + j]];
        }
        free(taken);
        free(p);
    }
}

/* Variant of step 2 -- a dynamic number of experts per token: the TorchTitan
 * 1K-GPU article (section 2.1) has each token activate 2-4 experts, with no
 * rule for the count.  Reading taken (cumulative-probability, or "top-p",
 * routing): the experts are ranked as in orc_route; with p = softmax(l / tau)
 * over all E experts, token t takes the k_t highest-ranked experts, k_t the
 * smallest j in [kmin, kmax] whose j largest p sum to at least theta (kmax
 * when none does).  Gates: p of the k_t chosen experts, divided by their sum
 * when renorm.  Slots j >= k_t hold idx -1 and gate 0 (no assignment). */
void orc_route_dynamic(int64_t T, int64_t E, int64_t kmax, int64_t kmin, double theta,
                       double tau, int renorm, const double* logits, int32_t* idx,
                       double* gate) {
    #pragma omp parallel
    {
        char* taken = (char*)calloc((size_t)E, 1);
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* l = logits + t * E;
            int32_t* it = idx + t * kmax;
            double* gt = gate + t * kmax;
            memset(taken, 0, (size_t)E);
            for (int64_t j = 0; j < kmax; ++j) {           /* the kmax best, in rank order */
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e)
                    if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
                taken[best] = 1;
                it[j] = (int32_t)best;
            }
            double mx = l[0];
            for (int64_t e = 1; e < E; ++e) if (l[e] > mx) mx = l[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) { p[e] = exp((l[e] - mx) / tau); z += p[e]; }
            for (int64_t e = 0; e < E; ++e) p[e] /= z;
            int64_t kt = kmax;                             /* how many this token takes */
            double mass = 0.0;
            for (int64_t j = 0; j < kmax; ++j) {
                mass += p[it[j]];
                if (j + 1 >= kmin && mass >= theta) { kt = j + 1; break; }
            }
            double s = 0.0;
            for (int64_t j = 0; j < kt; ++j) s += p[it[j]];
            for (int64_t j = 0; j < kmax; ++j) {
                if (j < kt) {
                    gt[j] = renorm ? p[it[j]] / s : p[it[j]];
                } else {
                    it[j] = -1;
                    gt[j] = 0.0;
                }
            }
        }
        free(taken);
        free(p);
    }
}

/* Capacity of a layer whose tokens take a varying number of experts: the
 * capacity factor scales the realised mean load, C = ceil(cap_num * A /
 * (cap_den * E)) for A assignments in the batch (exact integers); no limit
 * (cap_den == 0) gives C = T. */
int64_t orc_capacity_realised(int64_t A, int64_t T, int64_t E, int64_t cap_num, int64_t cap_den) {
    if (cap_den == 0) return T;
    int64_t num = cap_num * A, den = cap_den * E;
    return num / den + (num % den != 0);
}

/* Step 3 -- expert capacity C = ceil(cap_num * k * T / (cap_den * E)),
 * exact integer arithmetic; cap_den == 0 means no limit, C = T (a token picks
 * an expert at most once, so no expert can receive more than T). */
int64_t orc_capacity(int64_t T, int64_t E, int64_t k, int64_t cap_num, int64_t cap_den) {
    if (cap_den == 0) return T;
    int64_t num = cap_num * k * T, den = cap_den * E;
    return (num + den - 1) / den;
}

/* Step 4 -- positions, capacity drops and the permutation.
 * An assignment (t, j) of token t to expert e = idx[t][j] is kept when fewer
 * than C assignments to e come before it in the priority order:
 *  - policy 0, token order (the reading of "drop the overflow in token order",
 *    TorchTitan 1K-GPU article, section 2.1): (t', j') comes first when t' < t
 *    (a token never picks an expert twice, so j does not matter);
 *  - policy 1, choice order (GShard-style priority, a variant): all first
 *    choices in token order, then all second choices, ...: (t', j') comes
 *    first when j' < j, or j' == j and t' < t.
 * pos[t][j] = number of assignments to the same expert before (t, j) in that
 * order.  count = assignments per expert before drops, kept_e = min(count_e,
 * C).  Rows are grouped by expert in priority order, row = offset[e] + pos
 * (-1 if dropped), token_of_row[row] = t, in one of two layouts:
 *  - layout 0, compact: offset = exclusive prefix sum of kept (E + 1 entries,
 *    offset[E] = rows kept in total), no empty rows;
 *  - layout 1, padded to capacity (the fixed per-expert buffer that a
 *    capacity factor implies, a variant): offset[e] = e C, offset[E] = E C;
 *    the C - kept_e rows after an expert's kept rows are empty
 *    (token_of_row = -1, which the caller pre-fills). */
void orc_dispatch(int64_t T, int64_t E, int64_t k, int64_t C, const int32_t* idx,
                  int32_t* count, int32_t* kept, int32_t* offset, int32_t* pos,
                  int32_t* row_of, int32_t* token_of_row, int policy, int layout) {
    for (int64_t e = 0; e < E; ++e) count[e] = 0;
    /* a slot with idx -1 (dynamic routing: the token took fewer experts) is
     * no assignment: it gets pos -1 and row -1 */
    if (policy == 0) {
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < k; ++j) {
                int32_t e = idx[t * k + j];
                if (e < 0) { pos[t * k + j] = -1; continue; }
                pos[t * k + j] = count[e];
                count[e] += 1;
            }
    } else {
        for (int64_t j = 0; j < k; ++j)
            for (int64_t t = 0; t < T; ++t) {
                int32_t e = idx[t * k + j];
                if (e < 0) { pos[t * k + j] = -1; continue; }
                pos[t * k + j] = count[e];
                count[e] += 1;
            }
    }
    offset[0] = 0;
    for (int64_t e = 0; e < E; ++e) {
        kept[e] = count[e] < C ? count[e] : (int32_t)C;
        offset[e + 1] = layout == 1 ? (int32_t)((e + 1) * C) : offset[e] + kept[e];
    }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            int64_t a = t * k + j;
            if (pos[a] >= 0 && pos[a] < C) {
                int32_t row = offset[idx[a]] + pos[a];
                row_of[a] = row;
                token_of_row[row] = (int32_t)t;
            } else {
                row_of[a] = -1;
            }
        }
}

/* Expert-load telemetry from the per-expert assignment counts before drops.
 * The ZAYA1 page (section 3.2) reports keeping the expert load balance within
 * +-5%, and advises monitoring the load balance during training (section on
 * routing practice); the balance figure read here is the largest deviation of
 * an expert's load from the mean load, relative to the mean.
 * out[0] mean load m = sum_e count_e / E
 * out[1] max_e count_e            out[2] min_e count_e
 * out[3] max / m                  out[4] max_e |count_e - m| / m
 * out[5] sqrt(sum_e (count_e - m)^2 / E) / m   (coefficient of variation)
 * out[6] dropped assignments = sum_e max(0, count_e - C)
 * out[7] experts with no assignment
 * With no assignments at all (m = 0) the three ratios are 0. */
void orc_load_stats(int64_t E, const int32_t* count, int64_t C, double* out) {
    double sum = 0.0, mx = (double)count[0], mn = (double)count[0], dropped = 0.0, empty = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        double c = (double)count[e];
        sum += c;
        if (c > mx) mx = c;
        if (c < mn) mn = c;
        if (c > (double)C) dropped += c - (double)C;
        if (count[e] == 0) empty += 1.0;
    }
    double m = sum / (double)E;
    double dev = 0.0, ss = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        double diff = (double)count[e] - m;
        double ad = diff < 0 ? -diff : diff;
        if (ad > dev) dev = ad;
        ss += diff * diff;
    }
    out[0] = m;
    out[1] = mx;
    out[2] = mn;
    out[3] = m > 0 ? mx / m : 0.0;
    out[4] = m > 0 ? dev / m : 0.0;
    out[5] = m > 0 ? sqrt(ss / (double)E) / m : 0.0;
    out[6] = dropped;
    out[7] = empty;
}

/* The MLP router's load-balance controller: a PID controller on the expert
 * load ("AMD MI300X平台上的MoE模型训练实践", section 3.2, names a PID balance
 * controller acting on the router logits; its training notes raise the PID
 * gains over a warmup).  The page gives no update rule; the reading here is
 * the textbook discrete PID loop, one per expert, on the relative load error,
 * whose output is the additive logit bias.  One update per training step
 * from that step's counts before drops:
 *   m = sum_e count_e / E;  err_e = (m - count_e) / m  (0 for every e when m = 0)
 *   I_e <- I_e + err_e;  D_e = err_e - prev_e
 *   bias_e = scale * (kp * err_e + ki * I_e + kd * D_e);  prev_e <- err_e
 * state [2][E]: row 0 holds I, row 1 prev (zero before the first step).  An
 * expert below the mean load gets a positive error, so its bias rises. */
void orc_pid_update(int64_t E, double kp, double ki, double kd, double scale,
                    const int32_t* count, double* state, double* bias) {
    double sum = 0.0;
    for (int64_t e = 0; e < E; ++e) sum += (double)count[e];
    double mean = sum / (double)E;
    for (int64_t e = 0; e < E; ++e) {
        double err = mean > 0 ? (mean - (double)count[e]) / mean : 0.0;
        double integral = state[e] + err;
        double deriv = err - state[E + e];
        double p_term = kp * err;
        double i_term = ki * integral;
        double d_term = kd * deriv;
        bias[e] = scale * ((p_term + i_term) + d_term);
        state[e] = integral;
        state[E + e] = err;
    }
}

/* Step 5 -- the GeGLU expert FFN for a list of (token, expert) rows.
 * For row r (token t = tok[r], expert e = ex[r]):
 *   g[n] = sum_i x[t][i] * Wg[e][i][n],  u[n] = sum_i x[t][i] * Wu[e][i][n],
 *   h[n] = GELU(g[n]) * u[n],            o[c] = sum_n h[n] * Wd[e][n][c].
 * Wg, Wu are [E][d][d_ff], Wd is [E][d_ff][d].  Each sum runs over its index
 * in ascending order (the loops visit i, then n, outermost so that the weight
 * rows are read in order; that does not change any sum).  h may be NULL. */
void orc_ffn_rows(int64_t n_rows, const int64_t* tok, const int32_t* ex, int64_t d,
                  int64_t d_ff, int dtype, const void* x, const void* wg,
                  const void* wu, const void* wd, double* h_out, double* o_out) {
    #pragma omp parallel
    {
        double* g = (double*)malloc(sizeof(double) * (size_t)d_ff);
        double* u = (double*)malloc(sizeof(double) * (size_t)d_ff);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t t = tok[r], e = ex[r];
            for (int64_t n = 0; n < d_ff; ++n) { g[n] = 0.0; u[n] = 0.0; }
            for (int64_t i = 0; i < d; ++i) {
                double xi = load(x, t * d + i, dtype);
                int64_t wrow = (e * d + i) * d_ff;
                for (int64_t n = 0; n < d_ff; ++n) {
                    g[n] += xi * load(wg, wrow + n, dtype);
                    u[n] += xi * load(wu, wrow + n, dtype);
                }
            }
            for (int64_t n = 0; n < d_ff; ++n) g[n] = gelu(g[n]) * u[n];  /* g now holds h */
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            for (int64_t n = 0; n < d_ff; ++n) {
                int64_t wrow = (e * d_ff + n) * d;
                for (int64_t c = 0; c < d; ++c) o[c] += g[n] * load(wd, wrow + c, dtype);
            }
            if (h_out) memcpy(h_out + r * d_ff, g, sizeof(double) * (size_t)d_ff);
            memcpy(o_out + r * d, o, sizeof(double) * (size_t)d);
        }
        free(g); free(u); free(o);
    }
}

/* GELU'(v) = Phi(v) + v phi(v), the derivative of the erf form. */
static double gelu_grad(double v) {
    return 0.5 * (1.0 + erf(v / sqrt(2.0))) + v * exp(-0.5 * v * v) / sqrt(2.0 * M_PI);
}

/* Backward of the whole layer for an upstream gradient dy = dL/dy [T][d]
 * (the step after the forward: every page trains this layer).  Routing is
 * given (idx, gate, row_of from the forward, logits the values it ranked):
 * the top-k choice and the drops are piecewise constant, so no gradient flows
 * through them; the same holds for a dynamic expert count, whose slots past
 * a token's count hold -1 and take no part in any sum below.  With
 * p = softmax(l / tau) and, per kept assignment (t, j) of
 * expert e: g = x Wg[e], u = x Wu[e], a = GELU(g), h = a * u, o = h Wd[e],
 * y_t = sum_j gate_tj o_tj:
 *   dO = gate_tj dy_t, dgate_tj = dy_t . o_tj (0 for a dropped assignment)
 *   dh = dO Wd[e]^T, dWd[e] += h^T dO
 *   du = dh * a, dg = dh * u * GELU'(g)
 *   dWg[e] += x^T dg, dWu[e] += x^T du, dx_t += dg Wg[e]^T + du Wu[e]^T
 * gates: renormalised, gate_j = p_j / S (S = sum of the chosen p):
 *   dp_j = (dgate_j - sum_j' dgate_j' gate_j') / S; raw: dp_j = dgate_j;
 *   dp = 0 for experts not chosen;
 * softmax with temperature: dl_e = p_e (dp_e - sum_e' p_e' dp_e') / tau;
 * router: dWr += x^T dl, db += dl, dx_t += dl Wr^T.
 * Every sum in ascending index order; expert gradients are built one expert
 * per thread (tokens ascending), token gradients one token per thread
 * (choices ascending).  dgate may be NULL. */
void orc_backward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t d_ff, int dtype,
                  double tau, int renorm, const void* x, const void* wr, const double* logits,
                  const int32_t* idx, const double* gate, const int32_t* row_of,
                  const void* wg, const void* wu, const void* wd, const double* dy,
                  double* dx, double* dwr, double* db, double* dwg, double* dwu, double* dwd,
                  double* dgate) {
    double* dxa = (double*)calloc((size_t)(T * k * d), sizeof(double));   /* per assignment */
    double* dga = (double*)calloc((size_t)(T * k), sizeof(double));
    double* dl = (double*)calloc((size_t)(T * E), sizeof(double));
    if (dwg) memset(dwg, 0, sizeof(double) * (size_t)(E * d * d_ff));
    if (dwu) memset(dwu, 0, sizeof(double) * (size_t)(E * d * d_ff));
    if (dwd) memset(dwd, 0, sizeof(double) * (size_t)(E * d_ff * d));
    #pragma omp parallel
    {
        double* g = (double*)malloc(sizeof(double) * (size_t)d_ff);
        double* u = (double*)malloc(sizeof(double) * (size_t)d_ff);
        double* h = (double*)malloc(sizeof(double) * (size_t)d_ff);
        double* dh = (double*)malloc(sizeof(double) * (size_t)d_ff);
        double* dO = (double*)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t e = 0; e < E; ++e) {
            for (int64_t t = 0; t < T; ++t)
                for (int64_t j = 0; j < k; ++j) {
                    int64_t a = t * k + j;
                    if (idx[a] != e || row_of[a] < 0) continue;
                    for (int64_t n = 0; n < d_ff; ++n) { g[n] = 0.0; u[n] = 0.0; }
                    for (int64_t i = 0; i < d; ++i) {
                        double xi = load(x, t * d + i, dtype);
                        int64_t wrow = (e * d + i) * d_ff;
                        for (int64_t n = 0; n < d_ff; ++n) {
                            g[n] += xi * load(wg, wrow + n, dtype);
                            u[n] += xi * load(wu, wrow + n, dtype);
                        }
                    }
                    for (int64_t n = 0; n < d_ff; ++n) h[n] = gelu(g[n]) * u[n];
                    double dgt = 0.0;
                    for (int64_t c = 0; c < d; ++c) {
                        double o = 0.0;
                        for (int64_t n = 0; n < d_ff; ++n) o += h[n] * load(wd, (e * d_ff + n) * d + c, dtype);
                        dgt += dy[t * d + c] * o;
                        dO[c] = gate[a] * dy[t * d + c];
                    }
                    dga[a] = dgt;
                    for (int64_t n = 0; n < d_ff; ++n) {
                        double s = 0.0;
                        int64_t wrow = (e * d_ff + n) * d;
                        for (int64_t c = 0; c < d; ++c) {
                            s += dO[c] * load(wd, wrow + c, dtype);
                            if (dwd) dwd[wrow + c] += h[n] * dO[c];
                        }
                        dh[n] = s;
                    }
                    for (int64_t n = 0; n < d_ff; ++n) {
                        double du = dh[n] * gelu(g[n]);
                        double dg = dh[n] * u[n] * gelu_grad(g[n]);
                        g[n] = dg;   /* g now holds dg, u holds du */
                        u[n] = du;
                    }
                    for (int64_t i = 0; i < d; ++i) {
                        double xi = load(x, t * d + i, dtype), s = 0.0;
                        int64_t wrow = (e * d + i) * d_ff;
                        for (int64_t n = 0; n < d_ff; ++n) {
                            s += g[n] * load(wg, wrow + n, dtype) + u[n] * load(wu, wrow + n, dtype);
                            if (dwg) dwg[wrow + n] += xi * g[n];
                            if (dwu) dwu[wrow + n] += xi * u[n];
                        }
                        dxa[a * d + i] = s;
                    }
                }
        }
        free(g); free(u); free(h); free(dh); free(dO);
    }
    #pragma omp parallel
    {
        double* dp = (double*)malloc(sizeof(double) * (size_t)E);
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* l = logits + t * E;
            double m = l[0];
            for (int64_t e = 1; e < E; ++e) if (l[e] > m) m = l[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                const double q = (l[e] - m) / tau;
                p[e] = exp(q);
                z += p[e];
            }
            for (int64_t e = 0; e < E; ++e) { p[e] /= z; dp[e] = 0.0; }
            /* slots holding -1 (a token that took fewer than k experts) carry
             * no gate and no gradient: the sums run over the chosen experts */
            if (renorm) {
                double S = 0.0, sg = 0.0;
                for (int64_t j = 0; j < k; ++j) if (idx[t * k + j] >= 0) S += p[idx[t * k + j]];
                for (int64_t j = 0; j < k; ++j) sg += dga[t * k + j] * gate[t * k + j];
                for (int64_t j = 0; j < k; ++j)
                    if (idx[t * k + j] >= 0) dp[idx[t * k + j]] = (dga[t * k + j] - sg) / S;
            } else {
                for (int64_t j = 0; j < k; ++j)
                    if (idx[t * k + j] >= 0) dp[idx[t * k + j]] = dga[t * k + j];
            }
            double pd = 0.0;
            for (int64_t e = 0; e < E; ++e) pd += p[e] * dp[e];
            for (int64_t e = 0; e < E; ++e) dl[t * E + e] = p[e] * (dp[e] - pd) / tau;
            for (int64_t i = 0; i < d; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < k; ++j) s += dxa[(t * k + j) * d + i];
                for (int64_t e = 0; e < E; ++e) s += dl[t * E + e] * load(wr, i * E + e, dtype);
                dx[t * d + i] = s;
            }
            if (dgate) for (int64_t j = 0; j < k; ++j) dgate[t * k + j] = dga[t * k + j];
        }
        free(dp); free(p);
    }
    if (dwr) {
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < d; ++i)
            for (int64_t e = 0; e < E; ++e) {
                double s = 0.0;
                for (int64_t t = 0; t < T; ++t) s += load(x, t * d + i, dtype) * dl[t * E + e];
                dwr[i * E + e] = s;
            }
    }
    if (db) {
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t t = 0; t < T; ++t) s += dl[t * E + e];
            db[e] = s;
        }
    }
    free(dxa); free(dga); free(dl);
}

/* Router part of the backward on its own: dlogit [T][E] from the gate
 * gradients dgate [T][k] (0 for a dropped assignment), the same formulas as
 * in orc_backward: with p = softmax(l / tau),
 *   renormalised gates gate_j = p_j / S: dp_j = (dgate_j - sum_j' dgate_j' gate_j') / S,
 *   raw gates: dp_j = dgate_j; dp = 0 for experts not chosen (slots
 *   holding -1 choose none);
 *   dl_e = p_e (dp_e - sum_e' p_e' dp_e') / tau.
 * One token per thread, every sum in ascending index order. */
void orc_router_backward(int64_t T, int64_t E, int64_t k, double tau, int renorm,
                         const double* logits, const int32_t* idx, const double* gate,
                         const double* dgate, double* dl) {
    #pragma omp parallel
    {
        double* dq = (double*)malloc(sizeof(double) * (size_t)E);   /* dL/dp */
        double* q = (double*)malloc(sizeof(double) * (size_t)E);    /* p */
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* lt = logits + t * E;
            const int32_t* it = idx + t * k;
            double mx = lt[0];
            for (int64_t e = 1; e < E; ++e) if (lt[e] > mx) mx = lt[e];
            double zs = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                q[e] = exp((lt[e] - mx) / tau);
                zs += q[e];
            }
            for (int64_t e = 0; e < E; ++e) { q[e] = q[e] / zs; dq[e] = 0.0; }
            if (renorm) {   /* over the chosen experts: slots holding -1 are skipped */
                double S = 0.0, dot = 0.0;
                for (int64_t j = 0; j < k; ++j) if (it[j] >= 0) S += q[it[j]];
                for (int64_t j = 0; j < k; ++j) dot += dgate[t * k + j] * gate[t * k + j];
                for (int64_t j = 0; j < k; ++j)
                    if (it[j] >= 0) dq[it[j]] = (dgate[t * k + j] - dot) / S;
            } else {
                for (int64_t j = 0; j < k; ++j) if (it[j] >= 0) dq[it[j]] = dgate[t * k + j];
            }
            double qd = 0.0;
            for (int64_t e = 0; e < E; ++e) qd += q[e] * dq[e];
            for (int64_t e = 0; e < E; ++e) dl[t * E + e] = q[e] * (dq[e] - qd) / tau;
        }
        free(dq); free(q);
    }
}

/* Single entries of the expert weight gradients, each summed straight from
 * its definition over the kept assignments (t, j) of expert e, tokens
 * ascending (same quantities as in orc_backward):
 *   which 0: dWg[e][a][b] = sum x_t[a] dg_t[b]
 *   which 1: dWu[e][a][b] = sum x_t[a] du_t[b]
 *   which 2: dWd[e][a][b] = sum gate_tj h_t[a] dy_t[b]
 * where for column n: g_t[n] = sum_i x_t[i] Wg[e][i][n], u_t[n] likewise,
 * h = GELU(g) u, dh_t[n] = gate_tj sum_c dy_t[c] Wd[e][n][c],
 * du = dh GELU(g), dg = dh u GELU'(g).  Costs O(rows of e * d) per entry,
 * so a few entries can be checked at any layer size. */
void orc_backward_wentries(int64_t T, int64_t d, int64_t k, int64_t d_ff, int dtype,
                           const void* x, const int32_t* idx, const double* gate,
                           const int32_t* row_of, const void* wg, const void* wu, const void* wd,
                           const double* dy, int64_t n_ent, const int64_t* which,
                           const int64_t* ent_e, const int64_t* ent_a, const int64_t* ent_b,
                           double* out) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_ent; ++q) {
        const int64_t e = ent_e[q], a = ent_a[q], b = ent_b[q];
        const int64_t n = which[q] == 2 ? a : b;   /* the d_ff column involved */
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < k; ++j) {
                const int64_t s = t * k + j;
                if (idx[s] != e || row_of[s] < 0) continue;
                double g = 0.0, u = 0.0;
                for (int64_t i = 0; i < d; ++i) {
                    const double xi = load(x, t * d + i, dtype);
                    g += xi * load(wg, (e * d + i) * d_ff + n, dtype);
                    u += xi * load(wu, (e * d + i) * d_ff + n, dtype);
                }
                const double act = gelu(g);
                if (which[q] == 2) {
                    acc += gate[s] * (act * u) * dy[t * d + b];
                    continue;
                }
                double dh = 0.0;
                for (int64_t c = 0; c < d; ++c) dh += dy[t * d + c] * load(wd, (e * d_ff + n) * d + c, dtype);
                dh *= gate[s];
                const double xa = load(x, t * d + a, dtype);
                acc += which[q] == 0 ? xa * dh * u * gelu_grad(g) : xa * dh * act;
            }
        out[q] = acc;
    }
}

/* Step 6 -- gate-weighted combine for a list of tokens.
 * y[t] = sum over j = 0..k-1 with row_of[t][j] >= 0 of gate[t][j] * o[slot][.],
 * where o holds one row per (t, j) of the listed tokens: o[(s * k + j) * d + c]
 * for the s-th listed token.  A token with nothing kept gets y = 0. */
void orc_combine(int64_t n_tok, const int64_t* toks, int64_t k, int64_t d,
                 const int32_t* row_of, const double* gate, const double* o, double* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < n_tok; ++s) {
        int64_t t = toks[s];
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                if (row_of[t * k + j] >= 0) acc += gate[t * k + j] * o[(s * k + j) * d + c];
            y[s * d + c] = acc;
        }
    }
}
