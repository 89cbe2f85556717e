/*
 * CPU oracle for the single-GPU MoE layer: softmax top-k gating, capacity-bounded
 * slot assignment, index-based encode, per-expert FFN, gate-weighted decode, and
 * the backward of encode/FFN/decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do. It is written to be read against the pages, not to be fast: plain loops,
 * one accumulator per output, fp64 accumulation, no blocking and no reordering.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (the contraction flag
 * keeps every multiply and add separately rounded, as written).
 *
 * Sources (pages as printed; sections named on the page):
 *  - Tutel catalogue page (diedong.com), "key configuration" table and FAQ:
 *    gate_type {'type':'top','k':..,'capacity_factor':..}; capacity_factor > 0
 *    is a fixed factor, 0 is max(needed volumes), < 0 is min(-X, max needed);
 *    experts {'type':'ffn', hidden size per expert, has_fc1_bias/has_fc2_bias
 *    (default True)}.
 *  - MoE training blog (DeepSpeed-MoE vs Tutel), part 3 section 3.5 "fast
 *    encode/decode and dynamic capacity factor": encode maps T x M plus the
 *    gate's token-to-expert table into E x C x M, decode maps back; the dense
 *    form is an einsum over a one-hot [T,E,C] mask; kernels K0/K1/K2 are the
 *    combine-forward/encode-backward, encode-forward/combine-backward and the
 *    cross term. Part 1 section 1.4 (third layer, kernels): top-k + cumsum +
 *    scatter with a dense mapping table instead of one-hot einsum.
 *  - DeepSpeed PR #8195 (page of PR #8174), section 1: per-route index,
 *    location and gate values come from the top-k columns, as int32; section 2:
 *    the flat [e*c, m] dispatch buffer; section 3: dispatch and combine by
 *    index, combine accumulated in fp32.
 *
 * Readings where the pages are silent (each one is listed with its reason in the
 * design notes of the repository):
 *  - top-k orders experts by logit, larger first, and among equal logits the
 *    lower expert index first (+0 and -0 are equal); route r = 0 is the largest;
 *  - the softmax is computed in fp64 over all E logits and rounded once to fp32;
 *    gates are the probabilities of the selected experts, not renormalised;
 *  - locations count earlier routes to the same expert in route-major, then
 *    token order; a route is kept iff its location < C; the location of a
 *    dropped route is its raw rank;
 *  - C = ceil(k*S*|f|/E) for f > 0; max needed for f = 0; the smaller of the
 *    two for f < 0; never below 1;
 *  - encode copies token rows (no gate scaling); padding rows are +0;
 *  - FFN: pre = buf . W1[e]^T + b1[e] (W1 is [E,H,M]), h = act(pre) rounded to
 *    the data type, y = h . W2[e]^T + b2[e] (W2 is [E,M,H]) rounded to the data
 *    type; GELU is the exact erf form;
 *  - decode accumulates gate * y in fp32 in route order from +0 with separate
 *    multiply and add, then rounds to the data type; dropped routes add nothing;
 *  - Residual-MoE: the dense branch is an FFN of the same form over every
 *    token (its own W1r, b1r, W2r, b2r), its output y_r rounded to the data
 *    type like an expert's, and decode adds y_r[s] in fp32 after the routes;
 *    the MoE branch is gate-weighted as usual (the pages say only that the two
 *    outputs are added);
 *  - backward: dy = g * dout computed in fp32 (the product rounded to fp32)
 *    and then rounded to the data type, dgate = <dout, y>, dh = dy . W2[e],
 *    dpre = dh * act'(pre) rounded, where pre is the pre-activation as the
 *    forward stored it (rounded to the data type: the value a training step
 *    keeps for its backward), dbuf = dpre . W1[e] rounded, dx = sum of dbuf
 *    over kept routes rounded; weight and bias gradients are fp32 sums over
 *    the expert's filled rows;
 *  - gate backward: the gates are softmax probabilities p of the logits, so
 *    the gradient reaching p is dgates at each route's expert (all k routes as
 *    given; the layer passes 0 for dropped ones) plus the gradient of an
 *    auxiliary load-balance loss. The MoE training blog (part 2 section 2.1,
 *    training settings) fixes only its coefficient, 0.01; its form here is the
 *    usual product of routed fraction and mean probability,
 *      l_aux = alpha * E * sum_e f_e * P_e,  f_e = needed[e] / (k S),
 *      P_e = (1/S) sum_s p[s][e],
 *    with the counts f taken as constants (they come from an argmax). Then
 *    dlogits = p * (g - <p, g>) per token (the softmax Jacobian), dWg = x^T .
 *    dlogits, and the input gradient dx gains dlogits . Wg^T before its one
 *    rounding. All of it in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DT_F32 0
#define DT_BF16 1
#define ACT_RELU 0
#define ACT_GELU 1

/* ------------------------------------------------------------------ scalars */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the upper half of an IEEE binary32. */
static double bf16_value(uint16_t b) { return (double)bits_to_f32((uint32_t)b << 16); }

/* binary32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t f32_to_bf16(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* binary64 -> bf16 with a single rounding to nearest-even: first round to a
 * binary32 by round-to-odd (exact whenever representable, otherwise the
 * truncated value with its last bit set), which has more than two extra bits
 * over bf16, so the second rounding cannot double-round. */
static uint16_t f64_to_bf16(double v) {
    float f = (float)v;
    if ((double)f != v) {
        uint32_t u = f32_to_bits(f);
        if (fabs((double)f) > fabs(v)) u -= 1u; /* step back toward zero */
        u |= 1u;
        f = bits_to_f32(u);
    }
    return f32_to_bf16(f);
}

static double load_elem(const void *p, int dtype, int64_t i) {
    if (dtype == DT_F32) return (double)((const float *)p)[i];
    return bf16_value(((const uint16_t *)p)[i]);
}

/* Store v rounded once to the data type. */
static void store_elem(void *p, int dtype, int64_t i, double v) {
    if (dtype == DT_F32) ((float *)p)[i] = (float)v;
    else ((uint16_t *)p)[i] = f64_to_bf16(v);
}

/* The value the data type holds after storing v. */
static double round_to_dtype(double v, int dtype) {
    if (dtype == DT_F32) return (double)(float)v;
    return bf16_value(f64_to_bf16(v));
}

/* The product of an fp32 gate and a data-type value as fp32 arithmetic gives it:
 * the exact product (it fits in fp64) rounded once to fp32. */
static double fp32_product(float g, double v) { return (double)(float)((double)g * v); }

static double act_f(int act, double v) {
    if (act == ACT_RELU) return v > 0.0 ? v : 0.0;
    return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
}

static double act_grad(int act, double v) {
    if (act == ACT_RELU) return v > 0.0 ? 1.0 : 0.0;
    const double pdf = exp(-0.5 * v * v) / sqrt(2.0 * M_PI);
    return 0.5 * (1.0 + erf(v / sqrt(2.0))) + v * pdf;
}

/* Threads the OpenMP loops below use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Exposed for the tests: the scalar roundings above. */
uint16_t oracle_f64_to_bf16(double v) { return f64_to_bf16(v); }
double oracle_act(int act, double v) { return act_f(act, v); }
double oracle_act_grad(int act, double v) { return act_grad(act, v); }

/* ------------------------------------------------------------------ gating */

/* Gate projection: logit[s][e] = fp32( sum_m x[s][m] * Wg[m][e] ), the plain
 * definition of the product of x (data type, [S,M]) and the fp32 gate matrix
 * Wg [M,E] (Tutel catalogue page, key configuration: the gate scores each token
 * against the E experts). Every product is exact in fp64; the sum runs in fp64
 * from 0 in increasing m and is rounded once to fp32. */
void oracle_gate_logits(int32_t S, int32_t M, int32_t E, int dtype, const void *x,
                        const float *Wg, float *logits) {
    for (int64_t s = 0; s < S; ++s)
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t m = 0; m < M; ++m)
                acc += load_elem(x, dtype, s * M + m) * (double)Wg[(int64_t)m * E + e];
            logits[s * E + e] = (float)acc;
        }
}

/* Order of two experts of one token: larger logit first, equal logits (+0 and
 * -0 included) by lower index first. */
typedef struct { float v; int32_t e; } cand_t;
static int cand_cmp(const void *a, const void *b) {
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->e < y->e) ? -1 : (x->e > y->e);
}

/* Softmax over each token's E logits and the k largest as (expert, prob),
 * route-major outputs idx[r][s], gates[r][s]. Returns 0, or -1 on a
 * non-finite logit (finite logits are a precondition). */
int oracle_softmax_topk(int32_t S, int32_t E, int32_t k, const float *logits,
                        int32_t *idx, float *gates) {
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)E);
    for (int64_t s = 0; s < S; ++s) {
        const float *l = logits + s * E;
        double mx = -INFINITY;
        for (int32_t e = 0; e < E; ++e) {
            if (!isfinite(l[e])) { free(c); return -1; }
            if ((double)l[e] > mx) mx = (double)l[e];
        }
        double sum = 0.0;
        for (int32_t e = 0; e < E; ++e) sum += exp((double)l[e] - mx);
        for (int32_t e = 0; e < E; ++e) { c[e].v = l[e]; c[e].e = e; }
        qsort(c, (size_t)E, sizeof(cand_t), cand_cmp); /* full sort: the comparator is total */
        for (int32_t r = 0; r < k; ++r) {
            idx[(int64_t)r * S + s] = c[r].e;
            gates[(int64_t)r * S + s] = (float)(exp((double)c[r].v - mx) / sum);
        }
    }
    free(c);
    return 0;
}

/* Location of every route: the number of earlier routes (route-major, then
 * token order) that chose the same expert. needed[e] = routes to e. */
void oracle_locations(int32_t S, int32_t E, int32_t k, const int32_t *idx, int32_t *loc,
                      int32_t *needed) {
    for (int32_t e = 0; e < E; ++e) needed[e] = 0;
    for (int32_t r = 0; r < k; ++r)
        for (int64_t s = 0; s < S; ++s) {
            const int32_t e = idx[(int64_t)r * S + s];
            loc[(int64_t)r * S + s] = needed[e];
            needed[e] += 1;
        }
}

/* Capacity from capacity_factor f: f > 0 fixed factor, f == 0 max needed,
 * f < 0 the smaller of the |f| factor and max needed; at least 1. */
int32_t oracle_capacity(int32_t S, int32_t E, int32_t k, double f, const int32_t *needed) {
    int32_t max_needed = 0;
    for (int32_t e = 0; e < E; ++e)
        if (needed[e] > max_needed) max_needed = needed[e];
    const double by_factor = ceil(((double)k * (double)S * fabs(f)) / (double)E);
    int64_t c;
    if (f > 0) c = (int64_t)by_factor;
    else if (f == 0) c = max_needed;
    else c = (int64_t)by_factor < max_needed ? (int64_t)by_factor : max_needed;
    if (c < 1) c = 1;
    return (int32_t)c;
}

/* The whole routing step. fill[e] = min(needed[e], C). slot_route (may be NULL,
 * else E*C entries) gets r*S+s at row e*C+loc for every kept route and -1 on
 * padding rows. Returns C, or -1 on non-finite logits. */
int32_t oracle_route(int32_t S, int32_t E, int32_t k, double f, const float *logits,
                     int32_t *idx, float *gates, int32_t *loc, int32_t *needed,
                     int32_t *fill, int32_t *slot_route) {
    if (oracle_softmax_topk(S, E, k, logits, idx, gates) != 0) return -1;
    oracle_locations(S, E, k, idx, loc, needed);
    const int32_t C = oracle_capacity(S, E, k, f, needed);
    for (int32_t e = 0; e < E; ++e) fill[e] = needed[e] < C ? needed[e] : C;
    if (slot_route) {
        for (int64_t i = 0; i < (int64_t)E * C; ++i) slot_route[i] = -1;
        for (int32_t r = 0; r < k; ++r)
            for (int64_t s = 0; s < S; ++s) {
                const int64_t q = (int64_t)r * S + s;
                if (loc[q] < C) slot_route[(int64_t)idx[q] * C + loc[q]] = (int32_t)q;
            }
    }
    return C;
}

/* ------------------------------------------------------------------ encode */

/* buf[e*C + loc] = x[s] for every kept route (a copy of the bits), every other
 * row of the [E*C, M] buffer = +0. */
void oracle_encode(int32_t S, int32_t M, int32_t E, int32_t k, int32_t C, int dtype,
                   const void *x, const int32_t *idx, const int32_t *loc, void *buf) {
    const size_t eb = dtype == DT_F32 ? 4 : 2;
    memset(buf, 0, eb * (size_t)E * (size_t)C * (size_t)M);
    for (int32_t r = 0; r < k; ++r)
        for (int64_t s = 0; s < S; ++s) {
            const int64_t q = (int64_t)r * S + s;
            if (loc[q] >= C) continue;
            const int64_t row = (int64_t)idx[q] * C + loc[q];
            memcpy((char *)buf + row * M * eb, (const char *)x + s * M * eb, (size_t)M * eb);
        }
}

/* -------------------------------------------------------------- expert FFN */

/* One buffer row `row` = e*C + j through expert e:
 *   pre[h] = sum_m buf[row][m] * W1[e][h][m] + b1[e][h]   (fp64)
 *   hv[h]  = act(pre[h]) rounded to the data type
 *   y[m]   = sum_h hv[h] * W2[e][m][h] + b2[e][m]          (fp64)
 * pre_exact (H doubles) gets the unrounded pre-activation. */
static void ffn_row(int32_t M, int32_t H, int32_t C, int dtype, int act, const void *buf,
                    const void *W1, const void *b1, const void *W2, const void *b2,
                    int64_t row, double *pre_exact, double *hv, double *yv) {
    const int64_t e = row / C;
    for (int32_t h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int32_t m = 0; m < M; ++m)
            acc += load_elem(buf, dtype, row * M + m) * load_elem(W1, dtype, (e * H + h) * M + m);
        if (b1) acc += load_elem(b1, dtype, e * H + h);
        pre_exact[h] = acc;
        hv[h] = round_to_dtype(act_f(act, acc), dtype);
    }
    for (int32_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int32_t h = 0; h < H; ++h)
            acc += hv[h] * load_elem(W2, dtype, (e * M + m) * H + h);
        if (b2) acc += load_elem(b2, dtype, e * M + m);
        yv[m] = acc;
    }
}

/* Forward through the experts for nrows buffer rows (rows[i] = e*C + j).
 * Outputs are compact, one row per listed row, in the data type:
 * pre_out [nrows,H] (may be NULL), h_out [nrows,H] (may be NULL), y_out [nrows,M]. */
void oracle_expert_rows(int32_t M, int32_t H, int32_t E, int32_t C, int dtype, int act,
                        const void *buf, const void *W1, const void *b1, const void *W2,
                        const void *b2, int64_t nrows, const int64_t *rows, void *pre_out,
                        void *h_out, void *y_out) {
    (void)E;
#pragma omp parallel
    {
        double *pre = (double *)malloc(sizeof(double) * (size_t)H);
        double *hv = (double *)malloc(sizeof(double) * (size_t)H);
        double *yv = (double *)malloc(sizeof(double) * (size_t)M);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            ffn_row(M, H, C, dtype, act, buf, W1, b1, W2, b2, rows[i], pre, hv, yv);
            for (int32_t h = 0; h < H; ++h) {
                if (pre_out) store_elem(pre_out, dtype, i * H + h, pre[h]);
                if (h_out) store_elem(h_out, dtype, i * H + h, hv[h]);
            }
            for (int32_t m = 0; m < M; ++m) store_elem(y_out, dtype, i * M + m, yv[m]);
        }
        free(pre); free(hv); free(yv);
    }
}

/* ------------------------------------------------------------------ decode */

/* out[s][m] = sum over kept routes r (in route order) of gates[r][s] * y[slot][m],
 * fp32 from +0 with separate multiply and add, then rounded to the data type.
 * y is the [E*C, M] expert output. tokens (may be NULL = all S) lists the
 * ntok tokens to produce; out is compact [ntok, M].
 * Residual-MoE (MoE training blog, part 1 section 1.2: every token also passes
 * through one fixed dense MLP, and the two branches' outputs are added): with
 * yres (the dense MLP's output [S, M] in the data type, indexed by token) the
 * fp32 sum gains yres[s][m] after the routes, before the one rounding. */
void oracle_decode(int32_t S, int32_t M, int32_t E, int32_t k, int32_t C, int dtype,
                   const void *y, const float *gates, const int32_t *idx, const int32_t *loc,
                   int64_t ntok, const int64_t *tokens, const void *yres, void *out) {
    (void)E;
    for (int64_t i = 0; i < ntok; ++i) {
        const int64_t s = tokens ? tokens[i] : i;
        for (int32_t m = 0; m < M; ++m) {
            float acc = 0.0f;
            for (int32_t r = 0; r < k; ++r) {
                const int64_t q = (int64_t)r * S + s;
                if (loc[q] >= C) continue;
                const int64_t row = (int64_t)idx[q] * C + loc[q];
                const float prod = gates[q] * (float)load_elem(y, dtype, row * M + m);
                acc = acc + prod;
            }
            if (yres != NULL) acc = acc + (float)load_elem(yres, dtype, s * M + m);
            store_elem(out, dtype, i * M + m, (double)acc);
        }
    }
}

/* ---------------------------------------------------------------- backward */

/* Backward of one kept buffer row `row` = e*C + j that holds route q = r*S+s:
 *   dy[m]   = gates[q] * dout[s][m] rounded to fp32, then to the data type
 *   dh[h]   = sum_m dy[m] * W2[e][m][h]                      (fp64)
 *   dpre[h] = dh[h] * act'(pre[h]), rounded, with pre[h] the stored
 *             (rounded) pre-activation
 *   dbuf[m] = sum_h dpre[h] * W1[e][h][m], rounded
 * Outputs (compact, rows in the data type) may each be NULL. */
void oracle_backward_rows(int32_t S, int32_t M, int32_t H, int32_t E, int32_t C, int dtype,
                          int act, const void *buf, const void *W1, const void *b1,
                          const void *W2, const float *gates, const void *dout,
                          int64_t nrows, const int64_t *rows, const int32_t *routes,
                          void *dy_out, void *dpre_out, void *dbuf_out) {
    (void)E; (void)S;
#pragma omp parallel
    {
        double *pre = (double *)malloc(sizeof(double) * (size_t)H);
        double *dy = (double *)malloc(sizeof(double) * (size_t)M);
        double *dpre = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t row = rows[i], e = row / C;
            const int64_t q = routes[i], s = q % S;
            for (int32_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t m = 0; m < M; ++m)
                    acc += load_elem(buf, dtype, row * M + m) * load_elem(W1, dtype, (e * H + h) * M + m);
                if (b1) acc += load_elem(b1, dtype, e * H + h);
                pre[h] = acc;
            }
            for (int32_t m = 0; m < M; ++m) {
                dy[m] = round_to_dtype(fp32_product(gates[q], load_elem(dout, dtype, s * M + m)), dtype);
                if (dy_out) store_elem(dy_out, dtype, i * M + m, dy[m]);
            }
            for (int32_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t m = 0; m < M; ++m)
                    acc += dy[m] * load_elem(W2, dtype, (e * M + m) * H + h);
                dpre[h] = round_to_dtype(acc * act_grad(act, round_to_dtype(pre[h], dtype)), dtype);
                if (dpre_out) store_elem(dpre_out, dtype, i * H + h, dpre[h]);
            }
            if (dbuf_out)
                for (int32_t m = 0; m < M; ++m) {
                    double acc = 0.0;
                    for (int32_t h = 0; h < H; ++h)
                        acc += dpre[h] * load_elem(W1, dtype, (e * H + h) * M + m);
                    store_elem(dbuf_out, dtype, i * M + m, acc);
                }
        }
        free(pre); free(dy); free(dpre);
    }
}

/* The same backward quantities for selected hidden columns only, for sampling
 * the weight gradients of large layers. For each listed kept row (rows[i] =
 * e*C + j holding route routes[i]) and each hidden column hcols[c]:
 *   hv[i][c]   = act(pre) rounded,  dpre[i][c] = (dy . W2[e][:, h]) * act'(stored pre) rounded,
 * and the full dy row dy[i][:] = gates * dout[s] (fp32, then rounded). Every element follows
 * the same definitions as ffn_row / oracle_backward_rows. */
void oracle_backward_cols(int32_t S, int32_t M, int32_t H, int32_t C, int dtype, int act, const void *buf,
                          const void *W1, const void *b1, const void *W2, const float *gates,
                          const void *dout, int64_t nrows, const int64_t *rows, const int32_t *routes,
                          int32_t ncols, const int32_t *hcols, void *dy_out, void *hv_out, void *dpre_out) {
#pragma omp parallel
    {
        double *dy = (double *)malloc(sizeof(double) * (size_t)M);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t row = rows[i], e = row / C;
            const int64_t q = routes[i], s = q % S;
            for (int32_t m = 0; m < M; ++m) {
                dy[m] = round_to_dtype(fp32_product(gates[q], load_elem(dout, dtype, s * M + m)), dtype);
                store_elem(dy_out, dtype, i * M + m, dy[m]);
            }
            for (int32_t c = 0; c < ncols; ++c) {
                const int64_t h = hcols[c];
                double pre = 0.0;
                for (int32_t m = 0; m < M; ++m)
                    pre += load_elem(buf, dtype, row * M + m) * load_elem(W1, dtype, (e * H + h) * M + m);
                if (b1) pre += load_elem(b1, dtype, e * H + h);
                store_elem(hv_out, dtype, i * ncols + c, act_f(act, pre));
                double dh = 0.0;
                for (int32_t m = 0; m < M; ++m) dh += dy[m] * load_elem(W2, dtype, (e * M + m) * H + h);
                store_elem(dpre_out, dtype, i * ncols + c, dh * act_grad(act, round_to_dtype(pre, dtype)));
            }
        }
        free(dy);
    }
}

/* Weight and bias gradients of expert e from its n filled rows (in row order):
 *   dW2[m][h] = sum_j dy[j][m] * hv[j][h]      db2[m] = sum_j dy[j][m]
 *   dW1[h][m] = sum_j dpre[j][h] * buf[j][m]   db1[h] = sum_j dpre[j][h]
 * dy, hv, dpre, bufrows are compact [n, *] arrays in the data type; outputs are
 * fp32 [M,H], [M], [H,M], [H] for this expert. */
void oracle_weight_grads(int32_t M, int32_t H, int dtype, int64_t n, const void *dy,
                         const void *hv, const void *dpre, const void *bufrows, float *dW1,
                         float *db1, float *dW2, float *db2) {
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m) {
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j)
                acc += load_elem(dy, dtype, j * M + m) * load_elem(hv, dtype, j * H + h);
            dW2[(int64_t)m * H + h] = (float)acc;
        }
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += load_elem(dy, dtype, j * M + m);
        db2[m] = (float)acc;
    }
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
        for (int32_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j)
                acc += load_elem(dpre, dtype, j * H + h) * load_elem(bufrows, dtype, j * M + m);
            dW1[(int64_t)h * M + m] = (float)acc;
        }
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += load_elem(dpre, dtype, j * H + h);
        db1[h] = (float)acc;
    }
}

/* dgate of route q: sum_m dout[s][m] * y[slot][m] in fp64, rounded to fp32.
 * yrows holds the kept routes' expert-output rows, compact [n, M]. */
void oracle_dgates(int32_t S, int32_t M, int dtype, int64_t n, const int32_t *routes,
                   const void *dout, const void *yrows, float *dg) {
    for (int64_t i = 0; i < n; ++i) {
        const int64_t s = routes[i] % S;
        double acc = 0.0;
        for (int32_t m = 0; m < M; ++m)
            acc += load_elem(dout, dtype, s * M + m) * load_elem(yrows, dtype, i * M + m);
        dg[i] = (float)acc;
    }
}

/* dx[s][m] = sum over the token's kept routes of dbuf[slot][m] in route order
 * (fp64), rounded to the data type. dbufrows [n, M] holds dbuf rows; for token
 * t, route_rows[t*k + r] is the dbuf row of its route r, or -1 when that route
 * was dropped. dx is [ntok, M]. With dlog_rows, the gate projection's share
 * dlogits[t] . Wg^T is added; with res_rows ([ntok, M] in the data type), the
 * Residual-MoE dense branch's dx_r row (the branch's output is added to the
 * layer output, so its input gradient adds to dx), after the other terms. */
void oracle_dx(int32_t M, int32_t k, int dtype, const void *dbufrows, int64_t ntok,
               const int64_t *route_rows, int32_t E, const double *dlog_rows, const float *Wg,
               const void *res_rows, void *dx) {
    for (int64_t t = 0; t < ntok; ++t)
        for (int32_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int32_t r = 0; r < k; ++r) {
                const int64_t i = route_rows[t * k + r];
                if (i >= 0) acc += load_elem(dbufrows, dtype, i * M + m);
            }
            if (dlog_rows != NULL) /* the gate projection's share: dlogits[t] . Wg[m]^T */
                for (int32_t e = 0; e < E; ++e) acc += dlog_rows[t * E + e] * (double)Wg[(int64_t)m * E + e];
            if (res_rows != NULL) acc += load_elem(res_rows, dtype, t * M + m);
            store_elem(dx, dtype, t * M + m, acc);
        }
}

/* ------------------------------------------------------------------ gate backward */

/* Gradient of the logits (fp64, [S,E]) and the auxiliary loss (reading in the
 * header): p = softmax(logits[s]) in fp64; g[e] = sum of dgates[r][s] over the
 * routes r with idx[r][s] == e, plus alpha * E * f_e / S when needed is given
 * (needed == NULL: no auxiliary term, aux_loss = 0); dlogits[s][e] =
 * p[e] * (g[e] - sum_j p[j] g[j]). */
void oracle_gate_backward(int32_t S, int32_t E, int32_t k, double alpha, const float *logits,
                          const int32_t *idx, const float *dgates, const int32_t *needed,
                          double *dlogits, double *aux_loss) {
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    double *g = (double *)malloc(sizeof(double) * (size_t)E);
    double *colsum = (double *)calloc((size_t)E, sizeof(double));
    for (int64_t s = 0; s < S; ++s) {
        const float *l = logits + s * E;
        double mx = -INFINITY, sum = 0.0;
        for (int32_t e = 0; e < E; ++e)
            if ((double)l[e] > mx) mx = (double)l[e];
        for (int32_t e = 0; e < E; ++e) { p[e] = exp((double)l[e] - mx); sum += p[e]; }
        for (int32_t e = 0; e < E; ++e) p[e] /= sum;
        for (int32_t e = 0; e < E; ++e) {
            g[e] = needed ? alpha * (double)E * ((double)needed[e] / ((double)k * (double)S)) / (double)S : 0.0;
            colsum[e] += p[e];
        }
        for (int32_t r = 0; r < k; ++r) g[idx[(int64_t)r * S + s]] += (double)dgates[(int64_t)r * S + s];
        double dot = 0.0;
        for (int32_t e = 0; e < E; ++e) dot += p[e] * g[e];
        for (int32_t e = 0; e < E; ++e) dlogits[s * E + e] = p[e] * (g[e] - dot);
    }
    double loss = 0.0;
    if (needed != NULL && S > 0)
        for (int32_t e = 0; e < E; ++e)
            loss += ((double)needed[e] / ((double)k * (double)S)) * (colsum[e] / (double)S);
    *aux_loss = alpha * (double)E * loss;
    free(p); free(g); free(colsum);
}

/* dWg[m][e] = sum_s x[s][m] * dlogits[s][e] (fp64, [M,E]), s in increasing order. */
void oracle_gate_weight_grad(int32_t S, int32_t M, int32_t E, int dtype, const void *x,
                             const double *dlogits, double *dWg) {
    for (int32_t m = 0; m < M; ++m)
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t s = 0; s < S; ++s) acc += load_elem(x, dtype, s * M + m) * dlogits[s * E + e];
            dWg[(int64_t)m * E + e] = acc;
        }
}

/* ------------------------------------------------------------------ MX (microscaling) experts */

/* Low-precision experts (Tutel catalogue page: FP8 / MXFP4 / block-wise FP8
 * quantised inference). Format: OCP Microscaling (MX) v1.0 -- blocks of 32
 * consecutive values along the reduction dimension share one E8M0 scale
 * X = 2^(b - 127); each value is an element P with value X * P.
 *   fmt 0: MXFP8, E4M3 elements (bias 7, 3 mantissa bits, max normal 448,
 *          subnormals, S.1111.111 is NaN and never produced), one byte each;
 *   fmt 1: MXFP4, E2M1 elements (bias 1, 1 mantissa bit, values 0, 0.5, 1,
 *          1.5, 2, 3, 4, 6), two per byte, the even index in the low nibble.
 * Quantisation of a block (the MX specification's algorithm): amax = max |v|;
 * shared exponent e = floor(log2 amax) - emax_elem (8 for E4M3, 2 for E2M1),
 * clamped to [-127, 127], e = -127 for an all-zero block; each element is
 * v / 2^e rounded to the nearest element value, ties to the even code, with
 * magnitudes beyond the largest normal clamped to it; the sign bit is the
 * input's (so -0 stays -0). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e4m3_value(int code) {
    const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

double oracle_e2m1_value(int code) {
    const double v = kE2M1[code & 7];
    return (code & 8) ? -v : v;
}

/* Nearest element code of |q| (q >= 0), ties to the even code, saturating. */
static int nearest_code(double q, int fmt) {
    const int ncodes = fmt == 0 ? 127 : 8;  /* E4M3: codes 0..126 are the finite magnitudes */
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < ncodes; ++c) {
        const double v = fmt == 0 ? oracle_e4m3_value(c) : kE2M1[c];
        const double d = fabs(v - q);
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    return best;
}

/* One row of K values (fp64) -> codes (row layout of the format) and K/32 scale bytes. */
static void mx_quantize_row(const double *v, int32_t K, int fmt, uint8_t *codes, uint8_t *scales) {
    const int emax = fmt == 0 ? 8 : 2;
    for (int32_t b = 0; b < K / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[32 * b + i]));
        int e = -127;
        if (amax > 0.0) {
            e = ilogb(amax) - emax;  /* floor(log2 amax) for finite nonzero amax */
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i) {
            const int32_t k = 32 * b + i;
            const double x = v[k];
            const int c = nearest_code(ldexp(fabs(x), -e), fmt) | (signbit(x) ? (fmt == 0 ? 0x80 : 0x8) : 0);
            if (fmt == 0) codes[k] = (uint8_t)c;
            else if (k % 2 == 0) codes[k / 2] = (uint8_t)c;
            else codes[k / 2] |= (uint8_t)(c << 4);
        }
    }
}

static int64_t mx_row_bytes(int32_t K, int fmt) { return fmt == 0 ? K : K / 2; }

static double mx_value(const uint8_t *codes, const uint8_t *scales, int32_t K, int fmt, int64_t row, int32_t k) {
    const double x = ldexp(1.0, (int)scales[row * (K / 32) + k / 32] - 127);
    if (fmt == 0) return x * oracle_e4m3_value(codes[row * K + k]);
    const uint8_t byte = codes[row * (K / 2) + k / 2];
    return x * oracle_e2m1_value((k & 1) ? (byte >> 4) : (byte & 15));
}

/* Quantise a row-major [rows, K] matrix of the data type (K a multiple of 32). */
void oracle_mx_quantize(int fmt, int64_t rows, int32_t K, int dtype, const void *src, uint8_t *codes,
                        uint8_t *scales) {
    double *v = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t k = 0; k < K; ++k) v[k] = load_elem(src, dtype, r * K + k);
        mx_quantize_row(v, K, fmt, codes + r * mx_row_bytes(K, fmt), scales + r * (K / 32));
    }
    free(v);
}

/* Exact values of an MX matrix, fp64 [rows, K]. */
void oracle_mx_dequantize(int fmt, int64_t rows, int32_t K, const uint8_t *codes, const uint8_t *scales,
                          double *out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t k = 0; k < K; ++k) out[r * K + k] = mx_value(codes, scales, K, fmt, r, k);
}

/* Expert FFN on MX operands, for the listed buffer rows (row = e*C + j):
 *   pre = sum_m buf[row][m] W1[e][h][m] + b1[e][h]   (MX values, fp64 sums)
 *   h   = act(pre), rounded to fp32 (the precision the quantisation decision
 *         is taken in), then quantised to MXFP8 in blocks of 32 along H
 *   y   = sum_h hq[h] W2[e][m][h] + b2[e][m], rounded to bf16
 * buf is MXFP8 ([E*C, M] codes, [E*C, M/32] scales); W1 [E*H, M] and W2 [E*M, H]
 * in weight format wfmt; biases bf16 (may be NULL). Outputs compact per listed
 * row: h codes [n, H], h scales [n, H/32] (either may be NULL), y bf16 [n, M]. */
void oracle_expert_rows_mx(int32_t M, int32_t H, int32_t C, int act, int wfmt, const uint8_t *buf_codes,
                           const uint8_t *buf_scales, const uint8_t *w1_codes, const uint8_t *w1_scales,
                           const void *b1, const uint8_t *w2_codes, const uint8_t *w2_scales, const void *b2,
                           int64_t nrows, const int64_t *rows, uint8_t *h_codes, uint8_t *h_scales, void *y_out) {
#pragma omp parallel
    {
        double *xv = (double *)malloc(sizeof(double) * (size_t)M);
        double *hv = (double *)malloc(sizeof(double) * (size_t)H);
        uint8_t *hc = (uint8_t *)malloc((size_t)H);
        uint8_t *hs = (uint8_t *)malloc((size_t)(H / 32));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t row = rows[i];
            const int64_t e = row / C;
            for (int32_t m = 0; m < M; ++m) xv[m] = mx_value(buf_codes, buf_scales, M, 0, row, m);
            for (int32_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t m = 0; m < M; ++m) acc += xv[m] * mx_value(w1_codes, w1_scales, M, wfmt, e * H + h, m);
                if (b1) acc += load_elem(b1, DT_BF16, e * H + h);
                hv[h] = (double)(float)act_f(act, acc);
            }
            mx_quantize_row(hv, H, 0, hc, hs);
            if (h_codes) memcpy(h_codes + i * H, hc, (size_t)H);
            if (h_scales) memcpy(h_scales + i * (H / 32), hs, (size_t)(H / 32));
            for (int32_t h = 0; h < H; ++h) hv[h] = mx_value(hc, hs, H, 0, 0, h);
            for (int32_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int32_t h = 0; h < H; ++h) acc += hv[h] * mx_value(w2_codes, w2_scales, H, wfmt, e * M + m, h);
                if (b2) acc += load_elem(b2, DT_BF16, e * M + m);
                store_elem(y_out, DT_BF16, i * M + m, acc);
            }
        }
        free(xv); free(hv); free(hc); free(hs);
    }
}

/* ------------------------------------------------------------------ block-wise FP8 experts */

/* Block-wise FP8 (the Tutel pages list it beside FP8, NVFP4 and MXFP4 without
 * defining it; the reading is the fine-grained scheme published with DeepSeek-V3,
 * one of the model families the Tutel project summary names): E4M3 elements and
 * one fp32 scale per block of brows x 128 values, 128 x 128 for weights (128
 * output features by 128 steps of the reduction dimension) and 1 x 128 for
 * activations (128 consecutive features of one token). A block is quantised as
 *   amax = max |v|,  s = amax / 448  (fp32 division; 448 is E4M3's largest value),
 *   code = v / s (fp32 division) rounded to the nearest E4M3 value, ties to the
 *          even code, magnitudes beyond 448 clamped to it, the sign kept;
 * an all-zero block has s = 0 and codes 0. A code c of a block of scale s stands
 * for e4m3(c) * s. Scales are laid out [rows / brows][K / 128], row-major. */
static void blk_quantize(const float *v, int64_t rows, int32_t K, int32_t brows, uint8_t *codes, float *scales) {
    const int32_t KB = K / 128;
    for (int64_t rb = 0; rb < rows / brows; ++rb)
        for (int32_t kb = 0; kb < KB; ++kb) {
            float amax = 0.0f;
            for (int32_t i = 0; i < brows; ++i)
                for (int32_t j = 0; j < 128; ++j) amax = fmaxf(amax, fabsf(v[(rb * brows + i) * K + kb * 128 + j]));
            const float s = amax / 448.0f;
            scales[rb * KB + kb] = s;
            for (int32_t i = 0; i < brows; ++i)
                for (int32_t j = 0; j < 128; ++j) {
                    const int64_t at = (rb * brows + i) * K + kb * 128 + j;
                    int c = 0;
                    if (s > 0.0f) {
                        const float q = v[at] / s;
                        c = nearest_code(fabs((double)q), 0) | (signbit(q) ? 0x80 : 0);
                    }
                    codes[at] = (uint8_t)c;
                }
        }
}

static double blk_value(const uint8_t *codes, const float *scales, int32_t K, int32_t brows, int64_t row, int32_t k) {
    return oracle_e4m3_value(codes[row * K + k]) * (double)scales[(row / brows) * (K / 128) + k / 128];
}

/* Quantise a row-major [rows, K] matrix of the data type (rows a multiple of
 * brows, K of 128): codes [rows, K], scales [rows / brows, K / 128]. */
void oracle_blockfp8_quantize(int64_t rows, int32_t K, int32_t brows, int dtype, const void *src, uint8_t *codes,
                              float *scales) {
    float *v = (float *)malloc(sizeof(float) * (size_t)(rows * K > 0 ? rows * K : 1));
    for (int64_t i = 0; i < rows * K; ++i) v[i] = (float)load_elem(src, dtype, i);
    blk_quantize(v, rows, K, brows, codes, scales);
    free(v);
}

/* Exact values of a block-FP8 matrix, fp64 [rows, K]. */
void oracle_blockfp8_dequantize(int64_t rows, int32_t K, int32_t brows, const uint8_t *codes, const float *scales,
                                double *out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t k = 0; k < K; ++k) out[r * K + k] = blk_value(codes, scales, K, brows, r, k);
}

/* Expert FFN on block-FP8 operands, for the listed buffer rows (row = e*C + j):
 *   pre = sum_m buf[row][m] W1[e][h][m] + b1[e][h]   (dequantised values, fp64 sums)
 *   h   = act(pre), rounded to fp32, then quantised in 1 x 128 blocks along H
 *   y   = sum_h hq[h] W2[e][m][h] + b2[e][m], rounded to bf16
 * buf: codes [E*C, M], scales [E*C, M/128] (1 x 128 blocks); W1 [E*H, M] and W2
 * [E*M, H] codes with 128 x 128 block scales [E*H/128, M/128] and [E*M/128, H/128];
 * biases bf16 (may be NULL). Outputs compact per listed row: h codes [n, H], h
 * scales [n, H/128] (either may be NULL), y bf16 [n, M]. */
void oracle_expert_rows_blockfp8(int32_t M, int32_t H, int32_t C, int act, const uint8_t *buf_codes,
                                 const float *buf_scales, const uint8_t *w1_codes, const float *w1_scales,
                                 const void *b1, const uint8_t *w2_codes, const float *w2_scales, const void *b2,
                                 int64_t nrows, const int64_t *rows, uint8_t *h_codes, float *h_scales, void *y_out) {
#pragma omp parallel
    {
        double *xv = (double *)malloc(sizeof(double) * (size_t)M);
        float *hf = (float *)malloc(sizeof(float) * (size_t)H);
        double *hv = (double *)malloc(sizeof(double) * (size_t)H);
        uint8_t *hc = (uint8_t *)malloc((size_t)H);
        float *hs = (float *)malloc(sizeof(float) * (size_t)(H / 128));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t row = rows[i];
            const int64_t e = row / C;
            for (int32_t m = 0; m < M; ++m) xv[m] = blk_value(buf_codes, buf_scales, M, 1, row, m);
            for (int32_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t m = 0; m < M; ++m) acc += xv[m] * blk_value(w1_codes, w1_scales, M, 128, e * H + h, m);
                if (b1) acc += load_elem(b1, DT_BF16, e * H + h);
                hf[h] = (float)act_f(act, acc);
            }
            blk_quantize(hf, 1, H, 1, hc, hs);
            if (h_codes) memcpy(h_codes + i * H, hc, (size_t)H);
            if (h_scales) memcpy(h_scales + i * (H / 128), hs, sizeof(float) * (size_t)(H / 128));
            for (int32_t h = 0; h < H; ++h) hv[h] = blk_value(hc, hs, H, 1, 0, h);
            for (int32_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int32_t h = 0; h < H; ++h) acc += hv[h] * blk_value(w2_codes, w2_scales, H, 128, e * M + m, h);
                if (b2) acc += load_elem(b2, DT_BF16, e * M + m);
                store_elem(y_out, DT_BF16, i * M + m, acc);
            }
        }
        free(xv); free(hf); free(hv); free(hc); free(hs);
    }
}

/* ------------------------------------------------------------------ NVFP4 experts (weights) */

/* NVFP4 (the Tutel pages name it beside FP8, MXFP4 and block-wise FP8 without
 * defining it; the reading is NVIDIA's published two-level 4-bit format): E2M1
 * elements in blocks of 16 consecutive values along the reduction dimension,
 * each block with an E4M3 scale, and one fp32 scale g per tensor (here each
 * expert's weight matrix). The pages list these formats for A100/A800/H100/MI300,
 * which have no 4-bit matrix arithmetic, so the reading is weight-only: the
 * experts' weights are stored NVFP4 and multiplied by bf16 tokens at their exact
 * values. Quantisation of one tensor, fp32 arithmetic in this order:
 *   amax_t = max |v|;  g = amax_t / 2688   (448 * 6: E4M3's and E2M1's largest)
 *   per block of 16: amax_b = max |v|;  d = (amax_b / 6) / g;
 *     q = the E4M3 code nearest d (ties to the even code, saturating at 448);
 *     sd = e4m3(q);  each element: c = the E2M1 code nearest v / (sd * g) (the
 *     product rounded to fp32, then the division), ties to the even code,
 *     saturating at 6, the sign bit the input's;
 *   g == 0 (an all-zero tensor): scale codes 0; a block whose sd * g is 0 in fp32
 *   (sd == 0, or an underflowing product): element codes 0.
 * Element c of a block with scale code q in a tensor of scale g stands for
 * e2m1(c) * e4m3(q) * g. Layout: codes [rows, K/2] (two per byte, the even index
 * in the low nibble), scales [rows, K/16] E4M3 bytes, g [ntensor] fp32. */
static void nvfp4_quantize_tensor(const float *v, int64_t rows, int32_t K, uint8_t *codes, uint8_t *scales,
                                  float *g_out) {
    float amax_t = 0.0f;
    for (int64_t i = 0; i < rows * K; ++i) amax_t = fmaxf(amax_t, fabsf(v[i]));
    const float g = amax_t / 2688.0f;
    *g_out = g;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t b = 0; b < K / 16; ++b) {
            const float *blk = v + r * K + 16 * b;
            float amax_b = 0.0f;
            for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(blk[i]));
            int q = 0;
            if (g > 0.0f) {
                const float d = (amax_b / 6.0f) / g;
                q = nearest_code((double)d, 0);
            }
            const float sd = (float)oracle_e4m3_value(q);
            scales[r * (K / 16) + b] = (uint8_t)q;
            for (int i = 0; i < 16; ++i) {
                int c = 0;
                const float den = sd * g;
                if (den > 0.0f) {
                    const float x = blk[i] / den;
                    c = nearest_code(fabs((double)x), 1) | (signbit(x) ? 0x8 : 0);
                }
                const int64_t k = 16 * b + i;
                uint8_t *byte = codes + r * (K / 2) + k / 2;
                if (k % 2 == 0) *byte = (uint8_t)c;
                else *byte |= (uint8_t)(c << 4);
            }
        }
}

static double nvfp4_value(const uint8_t *codes, const uint8_t *scales, double g, int32_t K, int64_t row, int32_t k) {
    const uint8_t byte = codes[row * (K / 2) + k / 2];
    const int c = (k & 1) ? (byte >> 4) : (byte & 15);
    return oracle_e2m1_value(c) * oracle_e4m3_value(scales[row * (K / 16) + k / 16]) * g;
}

/* Quantise a row-major [rows, K] matrix of the data type (K a multiple of 16) as
 * ntensor tensors of rows / ntensor consecutive rows each (an expert's matrix). */
void oracle_nvfp4_quantize(int64_t rows, int32_t K, int32_t ntensor, int dtype, const void *src, uint8_t *codes,
                           uint8_t *scales, float *g) {
    const int64_t per = rows / ntensor;
    float *v = (float *)malloc(sizeof(float) * (size_t)(per * K > 0 ? per * K : 1));
    for (int32_t t = 0; t < ntensor; ++t) {
        for (int64_t i = 0; i < per * K; ++i) v[i] = (float)load_elem(src, dtype, t * per * K + i);
        nvfp4_quantize_tensor(v, per, K, codes + t * per * (K / 2), scales + t * per * (K / 16), g + t);
    }
    free(v);
}

/* Exact values of an NVFP4 matrix of ntensor tensors, fp64 [rows, K]. */
void oracle_nvfp4_dequantize(int64_t rows, int32_t K, int32_t ntensor, const uint8_t *codes, const uint8_t *scales,
                             const float *g, double *out) {
    const int64_t per = rows / ntensor;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t k = 0; k < K; ++k) out[r * K + k] = nvfp4_value(codes, scales, (double)g[r / per], K, r, k);
}

/* Expert FFN with NVFP4 weights and bf16 tokens, for the listed buffer rows
 * (row = e*C + j), the bf16 expert FFN's definitions on the weights' values:
 *   pre = sum_m buf[row][m] W1[e][h][m] + b1[e][h]   (fp64 sums)
 *   h   = act(pre), rounded to bf16
 *   y   = sum_h h[h] W2[e][m][h] + b2[e][m], rounded to bf16
 * buf bf16 [E*C, M]; W1 codes [E*H, M/2], scales [E*H, M/16], g1 [E]; W2 codes
 * [E*M, H/2], scales [E*M, H/16], g2 [E]; biases bf16 (may be NULL). Outputs
 * compact per listed row: pre and h bf16 [n, H] (either may be NULL), y bf16 [n, M]. */
void oracle_expert_rows_nvfp4(int32_t M, int32_t H, int32_t C, int act, const void *buf, const uint8_t *w1_codes,
                              const uint8_t *w1_scales, const float *g1, const void *b1, const uint8_t *w2_codes,
                              const uint8_t *w2_scales, const float *g2, const void *b2, int64_t nrows,
                              const int64_t *rows, void *pre_out, void *h_out, void *y_out) {
#pragma omp parallel
    {
        double *xv = (double *)malloc(sizeof(double) * (size_t)M);
        double *hv = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t row = rows[i];
            const int64_t e = row / C;
            for (int32_t m = 0; m < M; ++m) xv[m] = load_elem(buf, DT_BF16, row * M + m);
            for (int32_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t m = 0; m < M; ++m)
                    acc += xv[m] * nvfp4_value(w1_codes, w1_scales, (double)g1[e], M, e * H + h, m);
                if (b1) acc += load_elem(b1, DT_BF16, e * H + h);
                if (pre_out) store_elem(pre_out, DT_BF16, i * H + h, acc);
                hv[h] = round_to_dtype(act_f(act, acc), DT_BF16);  /* h as stored feeds fc2 */
                if (h_out) store_elem(h_out, DT_BF16, i * H + h, hv[h]);
            }
            for (int32_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int32_t h = 0; h < H; ++h)
                    acc += hv[h] * nvfp4_value(w2_codes, w2_scales, (double)g2[e], H, e * M + m, h);
                if (b2) acc += load_elem(b2, DT_BF16, e * M + m);
                store_elem(y_out, DT_BF16, i * M + m, acc);
            }
        }
        free(xv); free(hv);
    }
}
