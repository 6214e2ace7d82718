/*
 * oracle.c -- plain, slow, obviously correct CPU reference of the local MoE forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no source, header, helper or table with the
 * GPU library and includes nothing from it.
 *
 * Source: "ruDNN" user guide (docs.rs, ruDNN 0.1.72, German README):
 *   section 3 "MoE-Workflow"        -- the sequence logits -> softmax/top-k -> compact
 *                                      dispatch -> SwiGLU experts -> weighted combine;
 *   section 4 "Routing-Vertrag"     -- logits [T,E] in F32/F16/BF16, 1 <= top_k <= E, FP32
 *                                      softmax over all experts before top-k, ties to the
 *                                      lower expert id, optional renormalisation then a cast
 *                                      to the logits dtype, NaN weights for rows with NaN,
 *                                      +inf or only -inf, indices U32 [T,top_k];
 *   section 5 "Expertengewichte und Verteilung" -- tokens [T,H], gate/up [E,I,H],
 *                                      down [E,H,I], no capacity drops, order inside an
 *                                      expert unspecified, a stored map restores order;
 *   section 6 "MoE aufrufen"        -- the staged call forms and the full forward;
 *   section 12 "MoE-Training erster Ordnung" -- FP32 weights of a fixed selection and their
 *                                      logits gradients (softmax or sigmoid scoring, optional
 *                                      renormalisation, then scale; gather semantics), and the
 *                                      backward chain combine -> experts -> dispatch -> router;
 *   section 10 "Gruppenbeschraenktes Sigmoid-MoE-Routing" -- sigmoid scores, an optional FP32
 *                                      correction bias [E] that only steers the selection,
 *                                      group scores (maximum, or the sum of the two largest
 *                                      corrected scores), a choice of groups, top-k inside
 *                                      them, weights = the original sigmoid values,
 *                                      optionally renormalised, times `scale`, lower ids
 *                                      winning ties.
 *
 * Arithmetic: every value is widened exactly to double; sums, exp and divisions run in
 * double; a result is rounded once (round-to-nearest-even) to its storage dtype at the
 * points where the method stores a tensor (routing weights, the SwiGLU hidden activation,
 * the expert output, the combined output).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - A "NaN row" is a row with any NaN, any +inf, or all entries -inf.  Its k indices are
 *    0..k-1 (all probabilities are NaN, none exceeds another: treated as tied, lower id
 *    first) and its k weights are NaN, with or without renormalisation.
 *  - The k selected experts of a row are listed by descending probability, equal
 *    probabilities by ascending id.
 *  - The weight cast to the logits dtype happens whether or not renormalisation is on.
 *  - Rows inside one expert are ordered by (token, slot) ascending -- one of the valid
 *    orders; any order is correct per section 5.
 *  - token_map[t][j] is the dispatched row that holds copy j of token t (combine gathers).
 *  - SwiGLU: h = silu(gate . x) * (up . x), silu(z) = z / (1 + exp(-z)); y = down . h;
 *    no biases (section 5: "bias-freie Expertengewichte").
 *  - An index >= E given to dispatch gets map -1 and its token's combined row is NaN.
 *  - The fused router projection (section 5 leaves the gate projection to the caller; this is
 *    that caller step): logits[t, e] = sum_h input[t, h] * router[e, h] with the router [E, H]
 *    in the token dtype, summed in double and rounded once to the token dtype, which is then
 *    the logits dtype; routing follows section 4 unchanged.
 *  - Training (section 12 "MoE-Training erster Ordnung"): the weights of a fixed selection are
 *    w_j = scale * score(idx_j) / S, score = the softmax over all E (or the sigmoid) of the
 *    row, S = the sum of score(idx_j') over the k selected entries when renormalising (a
 *    repeated index counts each time it appears), else 1; they are FP32.  Their logits
 *    gradient is the chain rule through that formula, rounded once to the logits dtype.  An
 *    index outside [0, E) makes the whole row NaN (weights and gradient).
 *  - combine_backward: dexpert[map[t,j]] = dt(w[t,j] * dout[t]), dweights[t,j] = FP32 of
 *    sum_h dout[t,h] * y[map[t,j],h]; a token with a map entry outside [0, rows) gets NaN
 *    dweights (its forward output is NaN) and no dexpert row for that entry.
 *  - dispatch_backward: dinput[t] = dt(sum_j ddispatched[map[t,j]]), j ascending, no weights;
 *    NaN row for a token with an invalid map entry, as in combine.
 *  - experts backward, per dispatched row of expert e: dh = down_e^T dy; dg = dt(dh * u *
 *    silu'(g)), du = dt(dh * silu(g)) (stored in the dtype, like h in the forward, because
 *    they are the operands of the products that follow); dx = dt(gate_e^T dg + up_e^T du);
 *    dgate_e = FP32(sum_r dg_r x_r^T), dup_e likewise with du, ddown_e = FP32(sum_r dy_r h_r^T)
 *    with h the forward's stored activation.  silu'(z) = s (1 + z (1 - s)), s = 1/(1 + e^-z).
 *  - Sigmoid routing decides in FP32, the precision the guide gives the bias: s32 = the
 *    sigmoid rounded once to FP32, corrected score c = s32 + bias in FP32, a group score is the
 *    largest c of the group or the FP32 sum of its two largest; groups and then experts are
 *    taken by descending score, equal scores by ascending group / expert id.  The weights use
 *    the double sigmoid.  A row with a NaN corrected score or a NaN group score is a NaN
 *    row: indices 0..k-1, NaN weights.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* ------------------------------------------------------------------------------------ */
/* Codecs, written from the IEEE 754-2008 binary16 definition and the bfloat16 definition  */
/* (the upper 16 bits of an IEEE binary32).                                                */
/* ------------------------------------------------------------------------------------ */

static double dec_f16(uint16_t b) {
    int s = b >> 15, e = (b >> 10) & 0x1f, m = b & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/2^10) * 2^(e-15) */
    return s ? -v : v;
}

static double dec_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round x to the nearest number with p significand bits and minimum normal exponent emin
 * (values below 2^emin share the fixed quantum 2^(emin-p+1)), ties to even; beyond maxval
 * the result is +-inf. */
static double round_fmt(double x, int p, int emin, double maxval) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    frexp(fabs(x), &e);                 /* |x| = f * 2^e with f in [0.5, 1) */
    int lead = e - 1;                    /* exponent of the leading bit */
    if (lead < emin) lead = emin;
    double q = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(x / q) * q;     /* x / q is exact; nearbyint rounds half to even */
    if (fabs(r) > maxval) r = copysign(INFINITY, x);
    return r;
}

static uint16_t enc_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    double r = round_fmt(x, 8, -126, ldexp(255.0, 120)); /* max = (2 - 2^-7) * 2^127 */
    float f = (float)r;                   /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint16_t enc_f16(double x) {
    if (isnan(x)) return 0x7e00;
    double r = round_fmt(x, 11, -14, 65504.0);
    uint16_t s = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a)) return s | 0x7c00;
    if (a == 0.0) return s;
    if (a < ldexp(1.0, -14)) return s | (uint16_t)(a / ldexp(1.0, -24)); /* subnormal */
    int e;
    frexp(a, &e);
    int lead = e - 1;
    uint16_t m = (uint16_t)(a / ldexp(1.0, lead - 10) - 1024.0);
    return s | (uint16_t)((lead + 15) << 10) | m;
}

static double load_val(const void* p, int dt, int64_t i) {
    switch (dt) {
    case OR_F32: return (double)((const float*)p)[i];
    case OR_F16: return dec_f16(((const uint16_t*)p)[i]);
    default: return dec_bf16(((const uint16_t*)p)[i]);
    }
}

/* One rounding of a double to the storage dtype, returned as the stored value (double). */
static double round_to(double x, int dt) {
    switch (dt) {
    case OR_F32: return (double)(float)x;  /* C conversion rounds to nearest even */
    case OR_F16: return dec_f16(enc_f16(x));
    default: return dec_bf16(enc_bf16(x));
    }
}

static void store_val(void* p, int dt, int64_t i, double x) {
    switch (dt) {
    case OR_F32: ((float*)p)[i] = (float)x; break;
    case OR_F16: ((uint16_t*)p)[i] = enc_f16(x); break;
    default: ((uint16_t*)p)[i] = enc_bf16(x); break;
    }
}

static size_t dt_size(int dt) { return dt == OR_F32 ? 4 : 2; }

int oracle_dtype_size(int dt) { return (int)dt_size(dt); }

void oracle_decode(const void* src, int dt, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = load_val(src, dt, i);
}

void oracle_encode(const double* src, int dt, int64_t n, void* dst) {
    for (int64_t i = 0; i < n; ++i) store_val(dst, dt, i, src[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------------------ */
/* Route (user guide section 4).                                                          */
/* ------------------------------------------------------------------------------------ */

/* Softmax over all E experts of one row, in double: p_e = exp(x_e - m) / sum exp(x_i - m),
 * m = max_i x_i.  Returns 1 and leaves p untouched for a NaN row. */
static int row_softmax(const double* x, int64_t E, double* p) {
    int any_nan_or_posinf = 0, all_neginf = 1;
    for (int64_t e = 0; e < E; ++e) {
        if (isnan(x[e]) || x[e] == INFINITY) any_nan_or_posinf = 1;
        if (x[e] != -INFINITY) all_neginf = 0;
    }
    if (any_nan_or_posinf || all_neginf) return 1;
    double m = -INFINITY;
    for (int64_t e = 0; e < E; ++e)
        if (x[e] > m) m = x[e];
    double s = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        p[e] = exp(x[e] - m); /* exp(-inf) = 0 exactly */
        s += p[e];
    }
    for (int64_t e = 0; e < E; ++e) p[e] /= s;
    return 0;
}

/* Top-k by brute force: k passes, each taking the largest not-yet-taken probability; a
 * strictly-greater test while scanning ids upward makes the lower id win a tie. */
static void row_topk(const double* p, int64_t E, int64_t k, unsigned char* taken, uint32_t* idx) {
    memset(taken, 0, (size_t)E);
    for (int64_t j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || p[e] > p[best]) best = e;
        }
        taken[best] = 1;
        idx[j] = (uint32_t)best;
    }
}

/* logits [T,E] (ldt) -> expert_indices [T,k] u32, weights [T,k] (ldt).  If weights_exact is
 * not NULL it receives the double weights before the cast.  Returns 0, or -1 on bad args. */
int oracle_route(const void* logits, int ldt, int64_t T, int64_t E, int64_t k, int renormalize,
                 uint32_t* expert_indices, void* weights, double* weights_exact) {
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)E);
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t e = 0; e < E; ++e) x[e] = load_val(logits, ldt, t * E + e);
            uint32_t* idx = expert_indices + t * k;
            if (row_softmax(x, E, p)) {
                for (int64_t j = 0; j < k; ++j) {
                    idx[j] = (uint32_t)j;
                    store_val(weights, ldt, t * k + j, NAN);
                    if (weights_exact) weights_exact[t * k + j] = NAN;
                }
                continue;
            }
            row_topk(p, E, k, taken, idx);
            double den = 0.0;
            for (int64_t j = 0; j < k; ++j) den += p[idx[j]];
            for (int64_t j = 0; j < k; ++j) {
                double v = p[idx[j]];
                if (renormalize) v /= den;
                store_val(weights, ldt, t * k + j, v);
                if (weights_exact) weights_exact[t * k + j] = v;
            }
        }
        free(x);
        free(p);
        free(taken);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Router projection + route: the caller's gate projection (section 5) followed by the     */
/* section 4 routing.                                                                     */
/* ------------------------------------------------------------------------------------ */

/* input [T,H] and router [E,H] in dt -> logits [T,E] in dt (double sum, one rounding). */
int oracle_project(const void* input, int dt, const void* router, int64_t T, int64_t H, int64_t E, void* logits) {
    if (T < 0 || H < 1 || E < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h) acc += load_val(input, dt, t * H + h) * load_val(router, dt, e * H + h);
            store_val(logits, dt, t * E + e, acc);
        }
    }
    return 0;
}

/* logits = project(input, router); then oracle_route on them.  logits_out (may be NULL)
 * receives the rounded logits. */
int oracle_route_projected(const void* input, int dt, const void* router, int64_t T, int64_t H, int64_t E,
                           int64_t k, int renormalize, uint32_t* expert_indices, void* weights, void* logits_out) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || k > E) return -1;
    void* lg = logits_out ? logits_out : malloc(dt_size(dt) * (size_t)(T * E > 0 ? T * E : 1));
    int rc = oracle_project(input, dt, router, T, H, E, lg);
    if (!rc) rc = oracle_route(lg, dt, T, E, k, renormalize, expert_indices, weights, NULL);
    if (!logits_out) free(lg);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* Group-limited sigmoid routing (user guide section 10).                                 */
/* ------------------------------------------------------------------------------------ */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* logits [T,E] (ldt), bias [E] FP32 or NULL -> expert_indices [T,k] u32, weights [T,k] (ldt).
 * E = groups * (E / groups); groups are contiguous id ranges.  weights_exact (may be NULL)
 * receives the double weights before the cast.  Returns 0, or -1 on bad arguments. */
int oracle_route_sigmoid_grouped(const void* logits, int ldt, int64_t T, int64_t E, const float* bias,
                                 int64_t k, int64_t groups, int64_t selected_groups, int top_two,
                                 int renormalize, double scale, uint32_t* expert_indices, void* weights,
                                 double* weights_exact) {
    if (T < 0 || E < 1 || groups < 1 || E % groups != 0 || selected_groups < 1 || selected_groups > groups)
        return -1;
    const int64_t per = E / groups;
    if (k < 1 || k > selected_groups * per || (top_two && per < 2) || !(scale > 0.0) || isinf(scale)) return -1;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)E);
        float* c = (float*)malloc(sizeof(float) * (size_t)E);
        float* gs = (float*)malloc(sizeof(float) * (size_t)groups);
        unsigned char* gsel = (unsigned char*)malloc((size_t)groups);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            uint32_t* idx = expert_indices + t * k;
            int nan_row = 0;
            /* scores: sigmoid of the logit; corrected score in FP32 */
            for (int64_t e = 0; e < E; ++e) {
                s[e] = sigmoid(load_val(logits, ldt, t * E + e));
                const float s32 = (float)s[e];
                c[e] = bias ? (float)((double)s32 + (double)bias[e]) : s32;
                if (isnan(c[e])) nan_row = 1;
            }
            /* group scores: the largest corrected score, or the FP32 sum of the two largest */
            for (int64_t g = 0; g < groups && !nan_row; ++g) {
                const float* cg = c + g * per;
                int64_t b1 = 0;
                for (int64_t i = 1; i < per; ++i)
                    if (cg[i] > cg[b1]) b1 = i;
                if (!top_two) {
                    gs[g] = cg[b1];
                } else {
                    int64_t b2 = -1;
                    for (int64_t i = 0; i < per; ++i)
                        if (i != b1 && (b2 < 0 || cg[i] > cg[b2])) b2 = i;
                    gs[g] = (float)((double)cg[b1] + (double)cg[b2]);
                }
                if (isnan(gs[g])) nan_row = 1;
            }
            if (nan_row) {
                for (int64_t j = 0; j < k; ++j) {
                    idx[j] = (uint32_t)j;
                    store_val(weights, ldt, t * k + j, NAN);
                    if (weights_exact) weights_exact[t * k + j] = NAN;
                }
                continue;
            }
            /* groups by descending score, lower group id on ties */
            memset(gsel, 0, (size_t)groups);
            for (int64_t r = 0; r < selected_groups; ++r) {
                int64_t best = -1;
                for (int64_t g = 0; g < groups; ++g)
                    if (!gsel[g] && (best < 0 || gs[g] > gs[best])) best = g;
                gsel[best] = 1;
            }
            /* experts of the chosen groups by descending corrected score, lower id on ties */
            memset(taken, 0, (size_t)E);
            for (int64_t j = 0; j < k; ++j) {
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e) {
                    if (taken[e] || !gsel[e / per]) continue;
                    if (best < 0 || c[e] > c[best]) best = e;
                }
                taken[best] = 1;
                idx[j] = (uint32_t)best;
            }
            /* weights: the original sigmoid values, optionally renormalised, then scaled */
            double den = 0.0;
            for (int64_t j = 0; j < k; ++j) den += s[idx[j]];
            for (int64_t j = 0; j < k; ++j) {
                double v = s[idx[j]];
                if (renormalize) v /= den;
                v *= scale;
                store_val(weights, ldt, t * k + j, v);
                if (weights_exact) weights_exact[t * k + j] = v;
            }
        }
        free(s);
        free(c);
        free(gs);
        free(gsel);
        free(taken);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Dispatch (user guide section 5): capacity-free grouping by expert plus the stored map. */
/* ------------------------------------------------------------------------------------ */

/* counts[e] = number of (t,j) with index e; offsets = exclusive prefix sum (E+1 entries);
 * rows of one expert are assigned in (t,j) order.  token_map[t*k+j] = assigned row, or -1
 * for an index >= E.  dispatched[token_map[t*k+j]] = input[t], bytes copied verbatim. */
int oracle_dispatch(const uint32_t* expert_indices, int64_t T, int64_t k, int64_t E,
                    const void* input, int dt, int64_t H, void* dispatched,
                    int32_t* expert_offsets, int32_t* token_map, int32_t* counts) {
    if (T < 0 || k < 1 || E < 1 || H < 1) return -1;
    int64_t* cnt = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t a = 0; a < T * k; ++a)
        if (expert_indices[a] < (uint64_t)E) cnt[expert_indices[a]]++;
    int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
    int64_t run = 0;
    for (int64_t e = 0; e < E; ++e) {
        expert_offsets[e] = (int32_t)run;
        if (counts) counts[e] = (int32_t)cnt[e];
        cursor[e] = run;
        run += cnt[e];
    }
    expert_offsets[E] = (int32_t)run;
    size_t row_bytes = (size_t)H * dt_size(dt);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            uint32_t e = expert_indices[t * k + j];
            if (e >= (uint64_t)E) {
                token_map[t * k + j] = -1;
                continue;
            }
            int64_t row = cursor[e]++;
            token_map[t * k + j] = (int32_t)row;
            if (dispatched)
                memcpy((char*)dispatched + (size_t)row * row_bytes,
                       (const char*)input + (size_t)t * row_bytes, row_bytes);
        }
    free(cnt);
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* SwiGLU experts (user guide sections 3 and 5).                                          */
/* ------------------------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Rows x[0..n) (dtype dt, [n,H]) all go through expert e:
 *   g_i = sum_h gate[e,i,h] x[h],  u_i = sum_h up[e,i,h] x[h]   (i < I)
 *   h_i = dt(silu(g_i) * u_i)
 *   y_c = dt(sum_i down[e,c,i] h_i)                              (c < H)
 * hidden (optional, [n,I], dt) receives h.  Rows are taken in blocks so that each weight row
 * is decoded once per block; every sum is still the plain sum over its index. */
#define ROW_BLOCK 64
static void expert_rows(const void* x, int64_t n, int dt, const void* gate, const void* up,
                        const void* down, int64_t e, int64_t H, int64_t I, void* y, void* hidden) {
    for (int64_t r0 = 0; r0 < n; r0 += ROW_BLOCK) {
        int64_t nb = n - r0 < ROW_BLOCK ? n - r0 : ROW_BLOCK;
        double* xb = (double*)malloc(sizeof(double) * (size_t)(nb * H));
        double* hb = (double*)malloc(sizeof(double) * (size_t)(nb * I));
        for (int64_t r = 0; r < nb; ++r)
            for (int64_t c = 0; c < H; ++c) xb[r * H + c] = load_val(x, dt, (r0 + r) * H + c);
#pragma omp parallel
        {
            double* wg = (double*)malloc(sizeof(double) * (size_t)H);
            double* wu = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
            for (int64_t i = 0; i < I; ++i) {
                for (int64_t c = 0; c < H; ++c) {
                    wg[c] = load_val(gate, dt, (e * I + i) * H + c);
                    wu[c] = load_val(up, dt, (e * I + i) * H + c);
                }
                for (int64_t r = 0; r < nb; ++r) {
                    const double* xr = xb + r * H;
                    double g = 0.0, u = 0.0;
                    for (int64_t c = 0; c < H; ++c) {
                        g += wg[c] * xr[c];
                        u += wu[c] * xr[c];
                    }
                    hb[r * I + i] = round_to(silu(g) * u, dt);
                }
            }
            free(wg);
            free(wu);
        }
        if (hidden)
            for (int64_t r = 0; r < nb; ++r)
                for (int64_t i = 0; i < I; ++i) store_val(hidden, dt, (r0 + r) * I + i, hb[r * I + i]);
#pragma omp parallel
        {
            double* wd = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(static)
            for (int64_t c = 0; c < H; ++c) {
                for (int64_t i = 0; i < I; ++i) wd[i] = load_val(down, dt, (e * H + c) * I + i);
                for (int64_t r = 0; r < nb; ++r) {
                    const double* hr = hb + r * I;
                    double s = 0.0;
                    for (int64_t i = 0; i < I; ++i) s += wd[i] * hr[i];
                    store_val(y, dt, (r0 + r) * H + c, s);
                }
            }
            free(wd);
        }
        free(xb);
        free(hb);
    }
}

/* Arbitrary rows through arbitrary experts: row r of x goes through expert expert_of_row[r].
 * Used to check sampled rows of large workloads one by one. */
int oracle_expert_rows(const void* x, int64_t n, int dt, const void* gate, const void* up,
                       const void* down, int64_t E, int64_t H, int64_t I,
                       const int32_t* expert_of_row, void* y, void* hidden) {
    size_t es = dt_size(dt);
    for (int64_t r = 0; r < n; ++r)
        if (expert_of_row[r] < 0 || expert_of_row[r] >= E) return -1;
    /* consecutive rows of one expert go through it together */
    for (int64_t r = 0; r < n;) {
        int64_t r1 = r + 1;
        while (r1 < n && expert_of_row[r1] == expert_of_row[r]) ++r1;
        expert_rows((const char*)x + (size_t)r * H * es, r1 - r, dt, gate, up, down, expert_of_row[r], H, I,
                    (char*)y + (size_t)r * H * es, hidden ? (char*)hidden + (size_t)r * I * es : NULL);
        r = r1;
    }
    return 0;
}

/* Grouped form: rows [offsets[e], offsets[e+1]) of dispatched go through expert e. */
int oracle_experts_forward(const void* dispatched, const int32_t* expert_offsets, int64_t E, int dt,
                           const void* gate, const void* up, const void* down, int64_t H, int64_t I,
                           void* expert_output, void* hidden) {
    size_t es = dt_size(dt);
    for (int64_t e = 0; e < E; ++e) {
        int64_t a = expert_offsets[e], b = expert_offsets[e + 1];
        if (b < a) return -1;
        if (b == a) continue;
        expert_rows((const char*)dispatched + (size_t)a * H * es, b - a, dt, gate, up, down, e, H, I,
                    (char*)expert_output + (size_t)a * H * es,
                    hidden ? (char*)hidden + (size_t)a * I * es : NULL);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Combine (user guide sections 3 and 6): restore token order through the map and sum the */
/* k expert outputs weighted by the routing weights, j ascending, in double.              */
/* ------------------------------------------------------------------------------------ */

int oracle_combine(const void* expert_output, int dt, const int32_t* token_map, const void* weights,
                   int wdt, int64_t T, int64_t k, int64_t H, void* output) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int bad = 0;
        for (int64_t j = 0; j < k; ++j)
            if (token_map[t * k + j] < 0) bad = 1;
        for (int64_t c = 0; c < H; ++c) {
            double s = 0.0;
            if (bad) {
                s = NAN;
            } else {
                for (int64_t j = 0; j < k; ++j) {
                    double w = load_val(weights, wdt, t * k + j);
                    s += w * load_val(expert_output, dt, (int64_t)token_map[t * k + j] * H + c);
                }
            }
            store_val(output, dt, t * H + c, s);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Full local forward (user guide sections 3 and 6): route -> dispatch -> experts ->      */
/* combine.  gate == NULL means identity experts (expert output = dispatched rows).       */
/* ------------------------------------------------------------------------------------ */

static int forward_routed(const void* input, int dt, const uint32_t* idx, const void* w, int ldt, int64_t T,
                          int64_t E, int64_t k, const void* gate, const void* up, const void* down, int64_t H,
                          int64_t I, void* output) {
    size_t es = dt_size(dt);
    int32_t* offs = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* map = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
    void* disp = malloc(es * (size_t)(T * k * H));
    void* y = gate ? malloc(es * (size_t)(T * k * H)) : disp;
    int rc = oracle_dispatch(idx, T, k, E, input, dt, H, disp, offs, map, NULL);
    if (!rc && gate) rc = oracle_experts_forward(disp, offs, E, dt, gate, up, down, H, I, y, NULL);
    if (!rc) rc = oracle_combine(y, dt, map, w, ldt, T, k, H, output);
    if (gate) free(y);
    free(disp);
    free(map);
    free(offs);
    return rc;
}

/* Full local forward with group-limited sigmoid routing (user guide section 10:
 * forward_sigmoid_grouped = sigmoid routing -> dispatch -> experts -> combine). */
int oracle_forward_sigmoid_grouped(const void* input, int dt, const void* logits, int ldt, int64_t T, int64_t E,
                                   const float* bias, int64_t k, int64_t groups, int64_t selected_groups,
                                   int top_two, int renormalize, double scale, const void* gate, const void* up,
                                   const void* down, int64_t H, int64_t I, void* output) {
    if (T < 0) return -1;
    if (T == 0) return 0;
    uint32_t* idx = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(T * k));
    void* w = malloc(dt_size(ldt) * (size_t)(T * k));
    int rc = oracle_route_sigmoid_grouped(logits, ldt, T, E, bias, k, groups, selected_groups, top_two, renormalize,
                                          scale, idx, w, NULL);
    if (!rc) rc = forward_routed(input, dt, idx, w, ldt, T, E, k, gate, up, down, H, I, output);
    free(w);
    free(idx);
    return rc;
}

/* Full local forward from the hidden states: project -> route -> dispatch -> experts -> combine. */
int oracle_forward_projected(const void* input, int dt, const void* router, int64_t T, int64_t E, int64_t k,
                             int renormalize, const void* gate, const void* up, const void* down, int64_t H,
                             int64_t I, void* output) {
    if (T < 0 || E < 1 || k < 1 || k > E || H < 1) return -1;
    if (T == 0) return 0;
    uint32_t* idx = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(T * k));
    void* w = malloc(dt_size(dt) * (size_t)(T * k));
    int rc = oracle_route_projected(input, dt, router, T, H, E, k, renormalize, idx, w, NULL);
    if (!rc) rc = forward_routed(input, dt, idx, w, dt, T, E, k, gate, up, down, H, I, output);
    free(w);
    free(idx);
    return rc;
}

int oracle_forward(const void* input, int dt, const void* logits, int ldt, int64_t T, int64_t E,
                   int64_t k, int renormalize, const void* gate, const void* up, const void* down,
                   int64_t H, int64_t I, void* output) {
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
    if (T == 0) return 0;
    size_t es = dt_size(dt);
    uint32_t* idx = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(T * k));
    void* w = malloc(dt_size(ldt) * (size_t)(T * k));
    int32_t* offs = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* map = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
    void* disp = malloc(es * (size_t)(T * k * H));
    void* y = gate ? malloc(es * (size_t)(T * k * H)) : disp;
    int rc = oracle_route(logits, ldt, T, E, k, renormalize, idx, w, NULL);
    if (!rc) rc = oracle_dispatch(idx, T, k, E, input, dt, H, disp, offs, map, NULL);
    if (!rc && gate) rc = oracle_experts_forward(disp, offs, E, dt, gate, up, down, H, I, y, NULL);
    if (!rc) rc = oracle_combine(y, dt, map, w, ldt, T, k, H, output);
    if (gate) free(y);
    free(disp);
    free(map);
    free(offs);
    free(w);
    free(idx);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* First-order training (user guide section 12).                                          */
/* ------------------------------------------------------------------------------------ */

enum { OR_SCORE_SOFTMAX = 0, OR_SCORE_SIGMOID = 1 };

/* Scores of one row: the softmax over all E experts (max-subtracted, double) or the sigmoid of
 * each logit.  No NaN-row rule here: NaN and infinities propagate by IEEE arithmetic. */
static void row_scores(const double* x, int64_t E, int scoring, double* sc) {
    if (scoring == OR_SCORE_SIGMOID) {
        for (int64_t e = 0; e < E; ++e) sc[e] = sigmoid(x[e]);
        return;
    }
    double m = -INFINITY;
    for (int64_t e = 0; e < E; ++e)
        if (x[e] > m) m = x[e];
    double z = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        sc[e] = exp(x[e] - m);
        z += sc[e];
    }
    for (int64_t e = 0; e < E; ++e) sc[e] /= z;
}

/* d score_i / d x_e of one row. */
static double score_partial(const double* sc, int scoring, int64_t i, int64_t e) {
    if (scoring == OR_SCORE_SIGMOID) return i == e ? sc[i] * (1.0 - sc[i]) : 0.0;
    return sc[i] * ((i == e ? 1.0 : 0.0) - sc[e]);
}

/* FP32 weights of a fixed selection idx [T,k] (int64; outside [0, E) = invalid): w_j = scale *
 * score(idx_j) / S.  weights_exact (may be NULL) receives the double values. */
int oracle_selected_router_weights(const void* logits, int ldt, int64_t T, int64_t E, const int64_t* idx,
                                   int64_t k, int scoring, int renormalize, double scale, float* weights,
                                   double* weights_exact) {
    if (T < 0 || E < 1 || k < 1 || (scoring != OR_SCORE_SOFTMAX && scoring != OR_SCORE_SIGMOID)) return -1;
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)E);
        double* sc = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const int64_t* ix = idx + t * k;
            int bad = 0;
            for (int64_t j = 0; j < k; ++j)
                if (ix[j] < 0 || ix[j] >= E) bad = 1;
            for (int64_t e = 0; e < E; ++e) x[e] = load_val(logits, ldt, t * E + e);
            if (!bad) row_scores(x, E, scoring, sc);
            double S = 1.0;
            if (!bad && renormalize) {
                S = 0.0;
                for (int64_t j = 0; j < k; ++j) S += sc[ix[j]];
            }
            for (int64_t j = 0; j < k; ++j) {
                double v = bad ? NAN : scale * sc[ix[j]] / S;
                weights[t * k + j] = (float)v;
                if (weights_exact) weights_exact[t * k + j] = v;
            }
        }
        free(x);
        free(sc);
    }
    return 0;
}

/* Logits gradient [T,E] (ldt) of the weights above, given grad_weights [T,k] (FP32):
 * dx_e = sum_j g_j d w_j / d x_e with the quotient rule written out,
 * d w_j / d x_e = scale * (d score_{i_j}/d x_e * S - score_{i_j} * d S / d x_e) / S^2,
 * d S / d x_e = sum_j' d score_{i_j'} / d x_e (0 without renormalisation). */
int oracle_selected_router_backward(const void* logits, int ldt, int64_t T, int64_t E, const int64_t* idx,
                                    int64_t k, int scoring, int renormalize, double scale,
                                    const float* grad_weights, void* grad_logits) {
    if (T < 0 || E < 1 || k < 1 || (scoring != OR_SCORE_SOFTMAX && scoring != OR_SCORE_SIGMOID)) return -1;
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)E);
        double* sc = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const int64_t* ix = idx + t * k;
            int bad = 0;
            for (int64_t j = 0; j < k; ++j)
                if (ix[j] < 0 || ix[j] >= E) bad = 1;
            if (bad) {
                for (int64_t e = 0; e < E; ++e) store_val(grad_logits, ldt, t * E + e, NAN);
                continue;
            }
            for (int64_t e = 0; e < E; ++e) x[e] = load_val(logits, ldt, t * E + e);
            row_scores(x, E, scoring, sc);
            double S = 1.0;
            if (renormalize) {
                S = 0.0;
                for (int64_t j = 0; j < k; ++j) S += sc[ix[j]];
            }
            for (int64_t e = 0; e < E; ++e) {
                double dS = 0.0;
                if (renormalize)
                    for (int64_t j = 0; j < k; ++j) dS += score_partial(sc, scoring, ix[j], e);
                double acc = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    const double dw = scale * (score_partial(sc, scoring, ix[j], e) * S - sc[ix[j]] * dS) / (S * S);
                    acc += (double)grad_weights[t * k + j] * dw;
                }
                store_val(grad_logits, ldt, t * E + e, acc);
            }
        }
        free(x);
        free(sc);
    }
    return 0;
}

/* Backward of combine: dexpert [rows,H] (dt, only rows named by valid map entries are written)
 * and dweights [T,k] FP32. */
int oracle_combine_backward(const void* expert_output, int dt, const int32_t* token_map, const void* weights,
                            int wdt, const void* grad_output, int64_t T, int64_t k, int64_t H, int64_t rows,
                            void* grad_expert, float* grad_weights) {
    if (T < 0 || k < 1 || H < 1 || rows < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int bad = 0;
        for (int64_t j = 0; j < k; ++j)
            if (token_map[t * k + j] < 0 || token_map[t * k + j] >= rows) bad = 1;
        for (int64_t j = 0; j < k; ++j) {
            const int64_t r = token_map[t * k + j];
            const int ok = r >= 0 && r < rows;
            const double w = load_val(weights, wdt, t * k + j);
            double dw = 0.0;
            for (int64_t c = 0; c < H; ++c) {
                const double go = load_val(grad_output, dt, t * H + c);
                if (ok) {
                    store_val(grad_expert, dt, r * H + c, w * go);
                    dw += go * load_val(expert_output, dt, r * H + c);
                }
            }
            grad_weights[t * k + j] = bad ? NAN : (float)dw;
        }
    }
    return 0;
}

/* Backward of dispatch: dinput[t] = dt(sum_j ddispatched[map[t,j]]), j ascending. */
int oracle_dispatch_backward(const void* grad_dispatched, int dt, const int32_t* token_map, int64_t T, int64_t k,
                             int64_t H, int64_t rows, void* grad_input) {
    if (T < 0 || k < 1 || H < 1 || rows < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int bad = 0;
        for (int64_t j = 0; j < k; ++j)
            if (token_map[t * k + j] < 0 || token_map[t * k + j] >= rows) bad = 1;
        for (int64_t c = 0; c < H; ++c) {
            double s = 0.0;
            if (bad)
                s = NAN;
            else
                for (int64_t j = 0; j < k; ++j) s += load_val(grad_dispatched, dt, (int64_t)token_map[t * k + j] * H + c);
            store_val(grad_input, dt, t * H + c, s);
        }
    }
    return 0;
}

static double silu_grad(double z) {
    const double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

/* Backward of the SwiGLU experts on the dispatched rows: rows [offsets[e], offsets[e+1]) of
 * dispatched/grad_expert_output belong to expert e.  Writes grad_dispatched [rows,H] (dt) for
 * those rows and the FP32 weight gradients dgate, dup [E,I,H] and ddown [E,H,I] (all entries). */
int oracle_experts_backward(const void* dispatched, const int32_t* expert_offsets, int64_t E, int dt,
                            const void* gate, const void* up, const void* down, int64_t H, int64_t I,
                            const void* grad_expert_output, void* grad_dispatched, float* dgate, float* dup,
                            float* ddown) {
    if (E < 1 || H < 1 || I < 1) return -1;
    for (int64_t e = 0; e < E; ++e)
        if (expert_offsets[e + 1] < expert_offsets[e]) return -1;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t a = expert_offsets[e], n = expert_offsets[e + 1] - a;
        double* X = (double*)calloc((size_t)(n * H) + 1, sizeof(double));
        double* DY = (double*)calloc((size_t)(n * H) + 1, sizeof(double));
        double* Hh = (double*)calloc((size_t)(n * I) + 1, sizeof(double)); /* h, as stored (dt) */
        double* DG = (double*)calloc((size_t)(n * I) + 1, sizeof(double));
        double* DU = (double*)calloc((size_t)(n * I) + 1, sizeof(double));
        for (int64_t r = 0; r < n; ++r)
            for (int64_t c = 0; c < H; ++c) {
                X[r * H + c] = load_val(dispatched, dt, (a + r) * H + c);
                DY[r * H + c] = load_val(grad_expert_output, dt, (a + r) * H + c);
            }
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < I; ++i) {
            for (int64_t r = 0; r < n; ++r) {
                double g = 0.0, u = 0.0, dh = 0.0;
                for (int64_t c = 0; c < H; ++c) {
                    g += load_val(gate, dt, (e * I + i) * H + c) * X[r * H + c];
                    u += load_val(up, dt, (e * I + i) * H + c) * X[r * H + c];
                    dh += load_val(down, dt, (e * H + c) * I + i) * DY[r * H + c];
                }
                Hh[r * I + i] = round_to(silu(g) * u, dt);
                DG[r * I + i] = round_to(dh * u * silu_grad(g), dt);
                DU[r * I + i] = round_to(dh * silu(g), dt);
            }
        }
        /* dx = gate^T dg + up^T du */
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < H; ++c)
            for (int64_t r = 0; r < n; ++r) {
                double s = 0.0;
                for (int64_t i = 0; i < I; ++i)
                    s += load_val(gate, dt, (e * I + i) * H + c) * DG[r * I + i] +
                         load_val(up, dt, (e * I + i) * H + c) * DU[r * I + i];
                store_val(grad_dispatched, dt, (a + r) * H + c, s);
            }
        /* weight gradients: sums over the expert's rows */
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < I; ++i)
            for (int64_t c = 0; c < H; ++c) {
                double sg = 0.0, su = 0.0, sd = 0.0;
                for (int64_t r = 0; r < n; ++r) {
                    sg += DG[r * I + i] * X[r * H + c];
                    su += DU[r * I + i] * X[r * H + c];
                    sd += DY[r * H + c] * Hh[r * I + i];
                }
                dgate[(e * I + i) * H + c] = (float)sg;
                dup[(e * I + i) * H + c] = (float)su;
                ddown[(e * H + c) * I + i] = (float)sd;
            }
        free(X);
        free(DY);
        free(Hh);
        free(DG);
        free(DU);
    }
    return 0;
}
