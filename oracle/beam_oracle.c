/*
 * beam_oracle.c -- plain, slow, obviously correct CPU reference of one Beam
 * mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header or constant table with the GPU path.
 *
 * Sources (cited by page title and section):
 *   [GL]  Glonce, "Reflection releases Beam, a 501B open MoE model with 1M context",
 *         the architecture paragraphs ("The first 3 layers ...", "The residual
 *         connections ...").
 *   [TF]  transformers v5.20.1 model doc "Beam", Overview: bullets "Sparse MoE" and
 *         "Sandwich norms with depth-scaled residuals", and the paragraph on FP32
 *         numerics; Notes: "No auxiliary loss".
 *   [UA]  unicornapi.net, "Reflection releases Beam, an open 501B AI model built for
 *         coding agents", section "How Beam is built".
 *
 * What the layer computes, per token (a row u of the layer input):
 *   1. logits l_e = sum_h u_h W_r[e,h]; scores s_e = sigmoid(l_e)          [GL][TF]
 *   2. biased scores s'_e = s_e + b_e, used only to choose experts         [TF]
 *   3. experts form n_group contiguous groups; a group's score is the sum of
 *      its two largest s' (the DeepSeek-V3 group-limited scheme the pages
 *      name; the pages do not print the formula)                           [GL][UA]
 *   4. keep the topk_group best groups; choose the top_k largest s' among
 *      the experts of the kept groups (others are excluded, not zeroed)    [GL][TF]
 *   5. weights w_j = rho * s_{e_j} / sum_i s_{e_i}  (normalised, x rho)     [GL][TF]
 *   6. expert e: SwiGLU MLP  z = W_d[e] (silu(W_g[e] u) * (W_u[e] u)),
 *      silu(a) = a * sigmoid(a); output y = sum_j w_j z_j, no shared expert [GL][TF]
 *   Sublayer (sandwich norm + depth-scaled residual)                       [GL][TF]:
 *      u = RMSNorm_1(x), ..., yhat = RMSNorm_2(y),
 *      out = sqrt((k-1)/k) x + yhat / sqrt(k).
 *
 * Precision.  Floating point is fp64 throughout, except where the pages fix
 * FP32 and the value decides an integer or feeds one:
 *   - routing [TF, FP32 numerics]: logits are accumulated in fp64 and rounded to
 *     fp32; s = fp32(sigmoid(l32)) (evaluated in fp64, rounded once);
 *     s' = s + b as an fp32 add; a group score is an fp32 add of two s'; every
 *     choice is taken on these fp32 values, ties going to the lower index.
 *     The fp64 values are kept too, to report how far each choice is from a tie.
 *   - the pre-RMSNorm output u feeds the router [TF, FP32 RMSNorm scaling]: the
 *     mean square is summed in fp64, r = fp32(1/sqrt(ss/H + eps)) evaluated in
 *     fp64 and rounded once, then u = bf16(fp32(fp32(x*r) * g)), round to nearest
 *     even.
 * Tensors: bf16 arrives as uint16 bit patterns and is widened exactly.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- exact widening / rounding helpers ------------------------------------ */

static double bf16_to_double(uint16_t b) {
    uint32_t w = (uint32_t)b << 16;
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

static uint16_t float_to_bf16_rne(float f) {
    uint32_t w;
    memcpy(&w, &f, 4);
    w += 0x7FFFu + ((w >> 16) & 1u);
    return (uint16_t)(w >> 16);
}

/* element i of a tensor stored as fp32 (is_bf16 == 0) or bf16 (is_bf16 == 1) */
static double elem(const void* p, int64_t i, int is_bf16) {
    return is_bf16 ? bf16_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* ---- 8-bit expert weights ------------------------------------------------------
 * OCP FP8 E4M3: sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
 * holds the subnormals m * 2^-9; S.1111.111 is NaN (no infinities).  One E8M0 scale
 * byte s per 32 consecutive elements of a row multiplies them by 2^(s - 127).
 */
double oracle_e4m3_value(uint8_t code) {
    const int sgn = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* ---- 4-bit expert weights (MXFP4) ----------------------------------------------
 * OCP FP4 E2M1: sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0
 * holds the subnormals 0 and 0.5; no infinities or NaN; largest 6.  Two codes per byte:
 * the element with the even index in bits 0..3, the next one in bits 4..7.  The same E8M0
 * scale byte per 32 consecutive elements of a row.
 */
double oracle_e2m1_value(uint8_t code) {
    const int sgn = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    const double v = e == 0 ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
    return sgn ? -v : v;
}

/* value of one E8M0 scale byte (OCP microscaling formats): an exponent alone with bias
 * 127, 2^(s - 127) for s = 0 .. 254 (0 is 2^-127: no zero), and 0xFF is NaN (no infinity) */
double oracle_e8m0_value(uint8_t s) { return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127); }

/* decoding tables for one call: value of every code and factor of every scale byte */
typedef struct { double code[256], fp4[16], scale[256]; } fp8_tables;

static void fp8_tables_init(fp8_tables* t) {
    for (int i = 0; i < 256; ++i) {
        t->code[i] = oracle_e4m3_value((uint8_t)i);
        t->scale[i] = oracle_e8m0_value((uint8_t)i);
    }
    for (int i = 0; i < 16; ++i) t->fp4[i] = oracle_e2m1_value((uint8_t)i);
}

/* weight element i stored as fp32 (fmt 0), bf16 (fmt 1), or with block scales sc as E4M3
 * codes (fmt 2) or packed E2M1 codes (fmt 3) */
static double wval(const void* p, const uint8_t* sc, int64_t i, int fmt, const fp8_tables* t) {
    if (fmt == 2) return t->code[((const uint8_t*)p)[i]] * t->scale[sc[i >> 5]];
    if (fmt == 3) {
        const uint8_t b = ((const uint8_t*)p)[i >> 1];
        return t->fp4[(i & 1) ? b >> 4 : b & 15] * t->scale[sc[i >> 5]];
    }
    return elem(p, i, fmt);
}

/* ---- pre-RMSNorm with the pinned fp32 rounding ------------------------------ */

/* x [T,H] bf16, gain [H] fp32 -> u [T,H] bf16. */
void oracle_rmsnorm_pinned(const uint16_t* x, const float* gain, float eps, int64_t T, int64_t H, uint16_t* u) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xr = x + t * H;
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double v = bf16_to_double(xr[h]);
            ss += v * v;
        }
        float r = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
        for (int64_t h = 0; h < H; ++h) {
            float xv = (float)bf16_to_double(xr[h]);
            float a = xv * r;
            float b = a * gain[h];
            u[t * H + h] = float_to_bf16_rne(b);
        }
    }
}

/* ---- router ------------------------------------------------------------------ */

/* true when expert a ranks before expert b: larger value first, then lower index */
static int before_f(float va, int a, float vb, int b) { return va > vb || (va == vb && a < b); }
static int before_d(double va, int a, double vb, int b) { return va > vb || (va == vb && a < b); }

/*
 * act [T,H] (fp32 or bf16), w_router [E,H] fp32, bias [E] fp32.
 * Outputs per token t:
 *   idx[t*K + j]       chosen experts, in decision order (descending s', ties -> lower id)
 *   wts[t*K + j]       rho * s / sum(s) over the chosen, fp64
 *   logits[t*E + e]    fp64 logits (may be NULL)
 *   margin[t*2 + 0]    fp64 gap between the last kept and the first dropped group score
 *   margin[t*2 + 1]    fp64 gap between the K-th and (K+1)-th biased score among the
 *                      candidates (+inf where there is no such boundary)   (may be NULL)
 *   agree[t]           1 if deciding on the fp64 values gives the same kept groups and
 *                      the same chosen set as deciding on fp32 (may be NULL)
 * Returns 0, or -1 on an invalid shape.
 */
int oracle_route(const void* act, int act_bf16, int64_t T, int64_t H, const float* w_router, const float* bias,
                 int E, int n_group, int topk_group, int K, double rho, int32_t* idx, double* wts, double* logits,
                 double* margin, int32_t* agree) {
    if (E <= 0 || n_group <= 0 || E % n_group != 0 || topk_group <= 0 || topk_group > n_group || K <= 0 ||
        K > topk_group * (E / n_group))
        return -1;
    const int gsize = E / n_group;
#pragma omp parallel
    {
        double* l64 = (double*)malloc(sizeof(double) * E);
        float* s32 = (float*)malloc(sizeof(float) * E);
        float* sb32 = (float*)malloc(sizeof(float) * E);
        double* s64 = (double*)malloc(sizeof(double) * E);
        double* sb64 = (double*)malloc(sizeof(double) * E);
        float* gs32 = (float*)malloc(sizeof(float) * n_group);
        double* gs64 = (double*)malloc(sizeof(double) * n_group);
        int* kept = (int*)malloc(sizeof(int) * n_group);
        int* kept64 = (int*)malloc(sizeof(int) * n_group);
        int* gorder = (int*)malloc(sizeof(int) * n_group);
        int* cand = (int*)malloc(sizeof(int) * E);
        int* chosen64 = (int*)malloc(sizeof(int) * (K + 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < T; ++t) {
            /* 1-2: logits, scores, biased scores */
            for (int e = 0; e < E; ++e) {
                double acc = 0.0;
                for (int64_t h = 0; h < H; ++h) acc += elem(act, t * H + h, act_bf16) * (double)w_router[e * H + h];
                l64[e] = acc;
                float l32 = (float)acc;
                s32[e] = (float)sigmoid((double)l32);
                sb32[e] = s32[e] + bias[e];
                s64[e] = sigmoid(acc);
                sb64[e] = s64[e] + (double)bias[e];
                if (logits) logits[t * E + e] = acc;
            }
            /* 3: group score = largest + second largest biased score in the group */
            for (int g = 0; g < n_group; ++g) {
                float a1 = -INFINITY, a2 = -INFINITY;
                double d1 = -INFINITY, d2 = -INFINITY;
                for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
                    if (sb32[e] > a1) { a2 = a1; a1 = sb32[e]; } else if (sb32[e] > a2) { a2 = sb32[e]; }
                    if (sb64[e] > d1) { d2 = d1; d1 = sb64[e]; } else if (sb64[e] > d2) { d2 = sb64[e]; }
                }
                gs32[g] = (gsize >= 2) ? a1 + a2 : a1;
                gs64[g] = (gsize >= 2) ? d1 + d2 : d1;
            }
            /* 4: keep the topk_group best groups (rank by fp32 score, ties -> lower g) */
            for (int g = 0; g < n_group; ++g) {
                int rank = 0, rank64 = 0;
                for (int o = 0; o < n_group; ++o) {
                    if (o != g && before_f(gs32[o], o, gs32[g], g)) ++rank;
                    if (o != g && before_d(gs64[o], o, gs64[g], g)) ++rank64;
                }
                kept[g] = rank < topk_group;
                kept64[g] = rank64 < topk_group;
                gorder[rank64] = g;
            }
            /* 5: top-K biased scores among candidates of the kept groups; the other
             * experts are excluded outright (selection by repeated arg-max) */
            int nc = 0;
            for (int e = 0; e < E; ++e)
                if (kept[e / gsize]) cand[nc++] = e;
            double ssum = 0.0;
            for (int j = 0; j < K; ++j) {
                int best = -1;
                for (int c = 0; c < nc; ++c) {
                    int e = cand[c];
                    if (e < 0) continue;
                    if (best < 0 || before_f(sb32[e], e, sb32[best], best)) best = e;
                }
                idx[t * K + j] = best;
                for (int c = 0; c < nc; ++c)
                    if (cand[c] == best) cand[c] = -1;
                ssum += s64[best];
            }
            /* 6: normalised weights of the unbiased scores, scaled by rho */
            for (int j = 0; j < K; ++j) wts[t * K + j] = rho * s64[idx[t * K + j]] / ssum;

            /* distance to the nearest tie, in fp64, and the fp64 decision */
            if (margin || agree) {
                double mg = INFINITY, me = INFINITY;
                if (topk_group < n_group) mg = gs64[gorder[topk_group - 1]] - gs64[gorder[topk_group]];
                /* fp64 top-(K+1) among the fp64-kept groups */
                int nc64 = 0;
                for (int e = 0; e < E; ++e)
                    if (kept64[e / gsize]) cand[nc64++] = e;
                int take = K + 1 <= nc64 ? K + 1 : nc64;
                for (int j = 0; j < take; ++j) {
                    int best = -1;
                    for (int c = 0; c < nc64; ++c) {
                        int e = cand[c];
                        if (e < 0) continue;
                        if (best < 0 || before_d(sb64[e], e, sb64[best], best)) best = e;
                    }
                    chosen64[j] = best;
                    for (int c = 0; c < nc64; ++c)
                        if (cand[c] == best) cand[c] = -1;
                }
                if (take == K + 1) me = sb64[chosen64[K - 1]] - sb64[chosen64[K]];
                if (margin) {
                    margin[t * 2 + 0] = mg;
                    margin[t * 2 + 1] = me;
                }
                if (agree) {
                    int ok = 1;
                    for (int g = 0; g < n_group; ++g) ok &= (kept[g] == kept64[g]);
                    for (int j = 0; j < K && ok; ++j) {
                        int found = 0;
                        for (int q = 0; q < K; ++q) found |= (idx[t * K + q] == chosen64[j]);
                        ok &= found;
                    }
                    agree[t] = ok;
                }
            }
        }
        free(l64); free(s32); free(sb32); free(s64); free(sb64); free(gs32); free(gs64);
        free(kept); free(kept64); free(gorder); free(cand); free(chosen64);
    }
    return 0;
}

/* ---- experts and combine ------------------------------------------------------ */

/*
 * For each listed token tok[n] (n < n_tok): y[n, :] = sum_j wts[t,j] * FFN_{idx[t,j]}(act[t, :]),
 * j ascending, where FFN_e(u) = W_d[e] (silu(W_g[e] u) * (W_u[e] u)).
 * act [T,H]; w_gate, w_up [E,I,H]; w_down [E,H,I], all stored as w_fmt: fp32 (0), bf16 (1),
 * E4M3 codes (2) or E2M1 codes two per byte (3), the last two with E8M0 block scales
 * s_gate, s_up [E,I,H/32] and s_down [E,H,I/32];
 * idx [T,K]; wts [T,K] fp64.  y [n_tok,H] fp64.
 */
void oracle_experts(const void* act, int act_bf16, int64_t H, int64_t I, const void* w_gate, const void* w_up,
                    const void* w_down, int w_fmt, const uint8_t* s_gate, const uint8_t* s_up,
                    const uint8_t* s_down, int K, const int32_t* idx, const double* wts, const int64_t* tok,
                    int64_t n_tok, double* y) {
    fp8_tables tabs;
    fp8_tables_init(&tabs);
#pragma omp parallel
    {
        double* u = (double*)malloc(sizeof(double) * H);
        double* hh = (double*)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_tok; ++n) {
            int64_t t = tok[n];
            for (int64_t h = 0; h < H; ++h) u[h] = elem(act, t * H + h, act_bf16);
            double* yr = y + n * H;
            for (int64_t o = 0; o < H; ++o) yr[o] = 0.0;
            for (int j = 0; j < K; ++j) {
                int64_t e = idx[t * K + j];
                double wj = wts[t * K + j];
                for (int64_t i = 0; i < I; ++i) {
                    double a = 0.0, c = 0.0;
                    int64_t base = (e * I + i) * H;
                    for (int64_t h = 0; h < H; ++h) {
                        a += wval(w_gate, s_gate, base + h, w_fmt, &tabs) * u[h];
                        c += wval(w_up, s_up, base + h, w_fmt, &tabs) * u[h];
                    }
                    hh[i] = a * sigmoid(a) * c;
                }
                for (int64_t o = 0; o < H; ++o) {
                    double z = 0.0;
                    int64_t base = (e * H + o) * I;
                    for (int64_t i = 0; i < I; ++i) z += wval(w_down, s_down, base + i, w_fmt, &tabs) * hh[i];
                    yr[o] += wj * z;
                }
            }
        }
        free(u);
        free(hh);
    }
}

/* ---- post-RMSNorm and depth-scaled residual ---------------------------------- */

/*
 * y [n,H] fp64 (MoE output), x [n,H] (fp32 or bf16, the sublayer input), gain [H] fp32:
 *   yhat = gain * y / sqrt(mean(y^2) + eps);  out = sqrt((k-1)/k) x + yhat / sqrt(k).
 */
void oracle_post_residual(const double* y, const void* x, int x_bf16, const float* gain, float eps, int64_t n,
                          int64_t H, double k, double* out) {
    double a = sqrt((k - 1.0) / k), b = 1.0 / sqrt(k);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const double* yr = y + t * H;
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) ss += yr[h] * yr[h];
        double r = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = a * elem(x, t * H + h, x_bf16) + b * ((double)gain[h] * yr[h] * r);
    }
}

/* threads the oracle's parallel loops use */
int oracle_threads(void) { return omp_get_max_threads(); }

/* sets the number of threads of the oracle's later parallel loops (n >= 1) */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
