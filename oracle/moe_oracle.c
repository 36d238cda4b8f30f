/*
 * CPU oracle for the forward pass of one Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header, table or constant with the GPU library.
 *
 * Plain, slow, single-threaded C.  All arithmetic is in double precision;
 * values are rounded to bf16 only where the precision contract of
 * "Extend MoEPacked for Bolt ReLU-square routing and BF16 IQ2 precision"
 * (onnxruntime PR 33963, Description: BF16 store boundaries, FP32 final
 * routing/reduction) puts a bf16 store, i.e. the expert intermediate h that
 * feeds the second projection.  Everything else is returned in double.
 *
 * The steps, in the order of the layer:
 *   1. softmax top-k routing              oracle_route
 *      or sigmoid top-k routing with a     oracle_route_sigmoid
 *      selection-only correction bias
 *      (either one, then the route scale:  oracle_route_scored)
 *   2. count-first dispatch metadata       oracle_dispatch
 *      (counts, prefix sums, rows at known offsets; the afdEP count-first
 *      validation record, "change" and the fault list naming late counts,
 *      late prefix sums and late rows)
 *   3. row gather into expert order        oracle_gather_rows
 *   4. expert FFN (SwiGLU or ReLU-square)  oracle_expert_rows
 *   5. weighted combine to token order     oracle_combine
 *   oracle_forward chains 1-5 for a whole (small) layer.
 *
 * Readings where the pages leave a step open are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { O_F32 = 0, O_BF16 = 1, O_E4M3 = 2 };
enum { O_SWIGLU = 0, O_RELU2 = 1 };
enum { O_SOFTMAX = 0, O_SIGMOID = 1 };

/* ---- storage formats ------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("fn") variant: 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 holds subnormals
 * (m/8 * 2^-6); the all-ones pattern S.1111.111 is NaN; there is no
 * infinity.  Written from the format definition. */
double oracle_e4m3_to_double(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round a double to the nearest bf16 value, ties to even (8 significant
 * bits, binary32 exponent range, subnormal spacing 2^-133). */
double oracle_round_bf16(double v) {
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    double a = fabs(v);
    double r;
    if (a < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(a, 133)), -133);
    } else {
        int ex;
        double mant = frexp(a, &ex);          /* a = mant * 2^ex, 0.5 <= mant < 1 */
        r = ldexp(nearbyint(ldexp(mant, 8)), ex - 8);
        if (r > ldexp(255.0, 120)) r = INFINITY;  /* beyond the largest bf16 */
    }
    return v < 0 ? -r : r;
}

static double widen(const void *p, int fmt, int64_t i) {
    if (fmt == O_F32) return (double)((const float *)p)[i];
    if (fmt == O_BF16) return oracle_bf16_to_double(((const uint16_t *)p)[i]);
    return oracle_e4m3_to_double(((const uint8_t *)p)[i]);
}

/* ---- 1. softmax top-k routing ---------------------------------------- */

/* Does logit a at index ia rank before logit b at index ib?
 * Larger value first; equal values (so -0 == +0) by lower index; NaN ranks
 * below every number, including -inf. */
static int ranks_before(float a, int ia, float b, int ib) {
    int na = isnan(a), nb = isnan(b);
    if (na && nb) return ia < ib;
    if (na) return 0;
    if (nb) return 1;
    if (a > b) return 1;
    if (a < b) return 0;
    return ia < ib;
}

/* Softmax over all E logits of a token, then the k experts with the
 * largest logits (MoEPacked "internal softmax routing", PR 33963
 * Description; the router is handed logits directly, as in its latency
 * table where selected logits are +16 and the others -16).
 * Slot j = 0 holds the largest logit; ties go to the lower expert index.
 * w[t,j] is the softmax probability of the selected expert; with
 * `renormalize` it is instead the softmax over the k selected logits.
 * A row whose largest finite logit is -inf, or that holds a NaN, yields NaN
 * weights. */
int oracle_route(int T, int E, int k, int renormalize, const float *logits,
                 int32_t *ids, double *w) {
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!taken) return -1;
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (int64_t)t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (!isnan(l[e]) && (double)l[e] > m) m = (double)l[e];
        double S = 0.0;
        for (int e = 0; e < E; ++e) S += exp((double)l[e] - m);
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        double Ssel = 0.0;
        for (int j = 0; j < k; ++j) Ssel += exp((double)l[ids[(int64_t)t * k + j]] - m);
        for (int j = 0; j < k; ++j) {
            double num = exp((double)l[ids[(int64_t)t * k + j]] - m);
            w[(int64_t)t * k + j] = num / (renormalize ? Ssel : S);
        }
    }
    free(taken);
    return 0;
}

/* ---- 1b. sigmoid top-k routing with a correction bias ------------------ */

/* Sigmoid routing (PR 33963, Description and the commit adding "projected
 * sigmoid routing"): each expert gets the score s_e = sigma(l_e) =
 * 1 / (1 + e^-l_e); a float32 correction bias b_e enters the selection only.
 * Readings where the pages leave the step open:
 *   - the selection key is a float32: s_e is sigma rounded once to float32,
 *     and key_e = s_e + b_e is a float32 addition (the pages fix an FP32
 *     bias; the comparison is then done in the precision the bias lives in);
 *   - the k largest keys are taken, slot 0 first, ties to the lower index,
 *     NaN below every number (as for softmax routing);
 *   - the weights come from the unbiased scores: w[t,j] = sigma(l_id) (no
 *     renormalize) or sigma(l_id) / sum over the selected sigma (renormalize),
 *     in double;
 *   - `bias` may be NULL (no correction).
 * A NaN logit gets a NaN score and ranks last. */
int oracle_route_sigmoid(int T, int E, int k, int renormalize, const float *logits,
                         const float *bias, int32_t *ids, double *w) {
    float *key = (float *)malloc(sizeof(float) * (size_t)(E > 0 ? E : 1));
    unsigned char *taken = (unsigned char *)malloc((size_t)(E > 0 ? E : 1));
    if (!key || !taken) { free(key); free(taken); return -1; }
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) {
            float s = (float)(1.0 / (1.0 + exp(-(double)l[e])));
            float b = bias ? bias[e] : 0.0f;
            volatile float sum = s + b;   /* one float32 rounding */
            key[e] = bias ? sum : s;
        }
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(key[e], e, key[best], best)) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        double ssel = 0.0;
        for (int j = 0; j < k; ++j)
            ssel += 1.0 / (1.0 + exp(-(double)l[ids[(int64_t)t * k + j]]));
        for (int j = 0; j < k; ++j) {
            double sj = 1.0 / (1.0 + exp(-(double)l[ids[(int64_t)t * k + j]]));
            w[(int64_t)t * k + j] = renormalize ? sj / ssel : sj;
        }
    }
    free(key);
    free(taken);
    return 0;
}

/* Either router, then every weight times `route_scale` (the route scaling
 * the sigmoid-routing commit of PR 33963 keeps; 1 for plain softmax
 * routing).  `bias` is only meaningful for sigmoid routing. */
int oracle_route_scored(int T, int E, int k, int score_func, int renormalize,
                        double route_scale, const float *logits, const float *bias,
                        int32_t *ids, double *w) {
    int rc = score_func == O_SIGMOID
                 ? oracle_route_sigmoid(T, E, k, renormalize, logits, bias, ids, w)
                 : oracle_route(T, E, k, renormalize, logits, ids, w);
    if (rc != 0) return rc;
    if (route_scale != 1.0)
        for (int64_t q = 0; q < (int64_t)T * k; ++q) w[q] *= route_scale;
    return 0;
}

/* ---- 2. count-first dispatch metadata -------------------------------- */

/* Routes are numbered q = t*k + j.  A route is malformed when its expert id
 * is outside [0, E) or repeats an id of an earlier slot of the same token
 * (the negative / wide / duplicate route classes of the count-first
 * validation record).  A malformed route is neither counted nor placed
 * (route_dst = -2, distinct from a capacity drop) and its token is marked
 * bad: its output row becomes NaN (MoEPacked's isolation of malformed
 * routes, PR 33963 commit text).
 *
 * Count first: counts[e] = number of well-formed routes to expert e (raw,
 * before capacity).  Then prefix sums of the kept counts:
 * offsets[0] = 0, offsets[e+1] = offsets[e] + min(counts[e], C).
 * Then rows at known offsets: walking routes in ascending q, the r-th route
 * of expert e (r counted from 0) is kept iff r < C and goes to row
 * offsets[e] + r; later routes of an overflowing expert are dropped
 * (route_dst = -1).  row_src is the inverse map; rows offsets[E] .. r_max-1
 * are -1.  Returns the number of malformed routes, or -1 on bad arguments. */
int64_t oracle_dispatch(int T, int E, int k, int C, const int32_t *ids,
                        int32_t *counts, int32_t *offsets, int32_t *row_src,
                        int64_t r_max, int32_t *route_dst, uint8_t *token_bad) {
    int64_t nq = (int64_t)T * k, n_bad = 0;
    unsigned char *ok = (unsigned char *)malloc((size_t)(nq > 0 ? nq : 1));
    int64_t *seen = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    if (!ok || !seen) { free(ok); free(seen); return -1; }
    for (int t = 0; t < T; ++t) token_bad[t] = 0;
    for (int64_t q = 0; q < nq; ++q) {
        int t = (int)(q / k), j = (int)(q % k);
        int32_t e = ids[q];
        int good = (e >= 0 && e < E);
        for (int jj = 0; good && jj < j; ++jj)
            if (ids[(int64_t)t * k + jj] == e) good = 0;
        ok[q] = (unsigned char)good;
        if (!good) { token_bad[t] = 1; ++n_bad; }
    }
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t q = 0; q < nq; ++q)
        if (ok[q]) counts[ids[q]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + (counts[e] < C ? counts[e] : C);
    if ((int64_t)offsets[E] > r_max) { free(ok); free(seen); return -1; }
    for (int64_t q = 0; q < nq; ++q) {
        if (!ok[q]) { route_dst[q] = -2; continue; }
        int32_t e = ids[q];
        int64_t r = seen[e]++;
        if (r < C) {
            int32_t row = offsets[e] + (int32_t)r;
            route_dst[q] = row;
            row_src[row] = (int32_t)q;
        } else {
            route_dst[q] = -1;
        }
    }
    for (int64_t r = offsets[E]; r < r_max; ++r) row_src[r] = -1;
    free(ok);
    free(seen);
    return n_bad;
}

/* ---- 3. gather rows into expert-contiguous order ---------------------- */

/* x_disp[r] = x[row_src[r] / k], a byte copy of one token row. */
void oracle_gather_rows(int64_t R, int k, int64_t row_bytes, const uint8_t *x,
                        const int32_t *row_src, uint8_t *x_disp) {
    for (int64_t r = 0; r < R; ++r) {
        int64_t t = row_src[r] / k;
        memcpy(x_disp + r * row_bytes, x + t * row_bytes, (size_t)row_bytes);
    }
}

/* ---- 4. expert FFN ---------------------------------------------------- */

/* n rows of one expert.  w13 is [rows, H] with K (=H) contiguous: for SwiGLU
 * rows 0..I-1 are the gate projection and rows I..2I-1 the up projection;
 * for ReLU-square it is [I, H].  w2 is [H, I].
 *   SwiGLU:      h_i = silu(g_i) * u_i, silu(a) = a / (1 + e^-a)
 *   ReLU-square: h_i = max(g_i, 0)^2
 *   y_o = sum_i h_i * w2[o, i]
 * (MoEPacked default SwiGLU and ReLU-square gate/down experts, PR 33963.)
 * For e4m3 weights, s13 / s2 are per-output-row scales: the row's value is
 * scale * code.  With round_h the intermediate h is rounded to bf16 before
 * the second projection (the bf16 store boundary). */
int oracle_expert_rows(int n, int H, int I, int act, int x_fmt, const void *x,
                       int w_fmt, const void *w13, const void *w2,
                       const float *s13, const float *s2, int round_h,
                       double *y) {
    double *xr = (double *)malloc(sizeof(double) * (size_t)H);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    if (!xr || !h) { free(xr); free(h); return -1; }
    for (int r = 0; r < n; ++r) {
        for (int c = 0; c < H; ++c) xr[c] = widen(x, x_fmt, (int64_t)r * H + c);
        for (int i = 0; i < I; ++i) {
            double g = 0.0;
            for (int c = 0; c < H; ++c) g += xr[c] * widen(w13, w_fmt, (int64_t)i * H + c);
            if (w_fmt == O_E4M3) g *= (double)s13[i];
            double v;
            if (act == O_SWIGLU) {
                double u = 0.0;
                for (int c = 0; c < H; ++c)
                    u += xr[c] * widen(w13, w_fmt, (int64_t)(I + i) * H + c);
                if (w_fmt == O_E4M3) u *= (double)s13[I + i];
                v = g / (1.0 + exp(-g)) * u;
            } else {
                v = g > 0.0 ? g * g : 0.0;
            }
            h[i] = round_h ? oracle_round_bf16(v) : v;
        }
        for (int o = 0; o < H; ++o) {
            double acc = 0.0;
            for (int i = 0; i < I; ++i) acc += h[i] * widen(w2, w_fmt, (int64_t)o * I + i);
            if (w_fmt == O_E4M3) acc *= (double)s2[o];
            y[(int64_t)r * H + o] = acc;
        }
    }
    free(xr);
    free(h);
    return 0;
}

/* ---- 5. combine ------------------------------------------------------- */

/* out[t] = sum over slots j (ascending) of w[t,j] * y[route_dst[t,j]],
 * skipping dropped routes (route_dst = -1, contributing zero; the kept
 * weights are not renormalised), plus y_shared[t] when given (shared experts
 * enter with weight 1).  A token holding a malformed route (route_dst = -2)
 * gets a NaN row. */
void oracle_combine(int T, int k, int H, const int32_t *route_dst,
                    const double *w, const double *y, const double *y_shared,
                    double *out) {
    for (int t = 0; t < T; ++t) {
        int bad = 0;
        for (int j = 0; j < k; ++j)
            if (route_dst[(int64_t)t * k + j] == -2) bad = 1;
        for (int o = 0; o < H; ++o) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t row = route_dst[(int64_t)t * k + j];
                if (row >= 0) acc += w[(int64_t)t * k + j] * y[(int64_t)row * H + o];
            }
            if (y_shared) acc += y_shared[(int64_t)t * H + o];
            out[(int64_t)t * H + o] = bad ? NAN : acc;
        }
    }
}

/* ---- the whole layer -------------------------------------------------- */

static int64_t fmt_bytes(int fmt) { return fmt == O_F32 ? 4 : (fmt == O_BF16 ? 2 : 1); }

/* Route (unless ids_in / w_in are given: preselected routes), dispatch,
 * run every non-empty expert on its rows, run the shared experts on every
 * token, combine.  The expert weights are full [E, ...] tensors in w_fmt;
 * shared weights are bf16 (or f32 when x is f32).  round_h is applied when
 * x is bf16.  Outputs: ids, w (double), counts, offsets, row_src
 * (r_max = min(T*k, E*C) entries), route_dst, out [T, H] double.
 * Returns the number of malformed routes, or a negative value on failure. */
int64_t oracle_forward(int T, int H, int E, int k, int I, int C, int act,
                       int x_fmt, int w_fmt, int n_shared, int I_shared,
                       int renormalize, int score_func, double route_scale,
                       const void *x, const float *logits, const float *score_bias,
                       const int32_t *ids_in, const double *w_in,
                       const void *w13, const void *w2, const float *s13,
                       const float *s2, const void *w13_sh, const void *w2_sh,
                       int32_t *ids, double *w, int32_t *counts,
                       int32_t *offsets, int32_t *row_src, int32_t *route_dst,
                       double *out) {
    int64_t nq = (int64_t)T * k;
    int64_t r_max = nq < (int64_t)E * C ? nq : (int64_t)E * C;
    int rows13 = act == O_SWIGLU ? 2 * I : I;
    int round_h = (x_fmt == O_BF16);
    if (ids_in) {
        memcpy(ids, ids_in, sizeof(int32_t) * (size_t)nq);
        memcpy(w, w_in, sizeof(double) * (size_t)nq);
    } else if (oracle_route_scored(T, E, k, score_func, renormalize, route_scale, logits,
                                   score_bias, ids, w) != 0) {
        return -2;
    }
    uint8_t *bad = (uint8_t *)malloc((size_t)(T > 0 ? T : 1));
    if (!bad) return -2;
    int64_t n_bad = oracle_dispatch(T, E, k, C, ids, counts, offsets, row_src,
                                    r_max, route_dst, bad);
    if (n_bad < 0) { free(bad); return -3; }
    int64_t R = offsets[E];
    int64_t xb = fmt_bytes(x_fmt) * H;
    uint8_t *xd = (uint8_t *)malloc((size_t)(R > 0 ? R * xb : 1));
    double *y = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R * H : 1));
    double *ysh = n_shared ? (double *)calloc((size_t)T * H, sizeof(double)) : NULL;
    double *ytmp = n_shared ? (double *)malloc(sizeof(double) * (size_t)T * H) : NULL;
    if (!xd || !y || (n_shared && (!ysh || !ytmp))) {
        free(bad); free(xd); free(y); free(ysh); free(ytmp);
        return -2;
    }
    oracle_gather_rows(R, k, xb, (const uint8_t *)x, row_src, xd);
    int64_t wb = fmt_bytes(w_fmt);
    for (int e = 0; e < E; ++e) {
        int n = offsets[e + 1] - offsets[e];
        if (n == 0) continue;
        const uint8_t *a = (const uint8_t *)w13 + (int64_t)e * rows13 * H * wb;
        const uint8_t *b = (const uint8_t *)w2 + (int64_t)e * H * I * wb;
        oracle_expert_rows(n, H, I, act, x_fmt, xd + (int64_t)offsets[e] * xb,
                           w_fmt, a, b,
                           s13 ? s13 + (int64_t)e * rows13 : NULL,
                           s2 ? s2 + (int64_t)e * H : NULL, round_h,
                           y + (int64_t)offsets[e] * H);
    }
    if (n_shared) {
        int sfmt = (x_fmt == O_F32) ? O_F32 : O_BF16;
        int64_t sb = fmt_bytes(sfmt);
        for (int s = 0; s < n_shared; ++s) {
            const uint8_t *a = (const uint8_t *)w13_sh + (int64_t)s * 2 * I_shared * H * sb;
            const uint8_t *b = (const uint8_t *)w2_sh + (int64_t)s * H * I_shared * sb;
            oracle_expert_rows(T, H, I_shared, O_SWIGLU, x_fmt, x, sfmt, a, b,
                               NULL, NULL, round_h, ytmp);
            for (int64_t i = 0; i < (int64_t)T * H; ++i) ysh[i] += ytmp[i];
        }
    }
    oracle_combine(T, k, H, route_dst, w, y, ysh, out);
    free(bad); free(xd); free(y); free(ysh); free(ytmp);
    return n_bad;
}
