/*
 * oracle.c -- plain, slow CPU oracle for one sparse MoE layer's routed expert
 * FFN over a whole prompt, as described in "EStream: Fast and Memory-Efficient
 * MoE Prefill through Expert Virtualization on Mobile NPUs" (arXiv 2609.06551),
 * section 3.2 "Intra-NPU MoE Execution".
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library never
 * links, loads or calls it, and it shares no code, header or table with it.
 *
 * Every function computes its result from the definition, with no blocking,
 * fusion or reordering:
 *   oracle_router_logits  L = X W_r (+ bias): the dot product and the bias
 *                         summed in fp64 (every product of two fp32 values
 *                         is exact there) and rounded once to fp32.  No
 *                         evaluation order is part of the definition.
 *   oracle_topk           top-k of E experts per token (section 2.2: "a router
 *                         assigns each token to the top-k of E experts"), ties
 *                         to the lower expert id; softmax weights in fp64,
 *                         optionally renormalised over the k selected; shared
 *                         experts appended with weight 1.
 *   oracle_route_map      the route map of Algorithm 1: slot resolve psi_i =
 *                         Phi(e_i), per-slot counts, prefix-sum offsets, and a
 *                         cursor pass in ascending route index storing (t_i, i).
 *   oracle_expert_ffn     Eq. (2) Y_t = A_t + sum alpha F_e(X_t) with Eq. (1)
 *                         F_e(x) = W_d (SiLU(W_g x) * (W_u x)), per token and
 *                         per selected expert, accumulated in fp64. With row
 *                         scales, each weight is its stored value times its
 *                         row's scale (weight-only quantised experts).
 *   oracle_fp8e4m3_decode the value of an fp8 e4m3 code (OCP 8-bit floating
 *                         point: sign, 4 exponent bits with bias 7, 3 mantissa
 *                         bits; exponent 0 is subnormal; S.1111.111 is NaN;
 *                         there are no infinities).
 *   oracle_mxfp4_decode   the weights of an OCP MXFP4 slice: 4-bit E2M1 codes
 *                         times one E8M0 power-of-two scale per 32 weights of
 *                         a row (the 4-bit block-scaled weight format standing
 *                         for the pages' 4-bit weight-only blocks).
 *
 * Parity status: every function is pinned by CPU tests (brute force, closed
 * forms, special cases and invariants); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Router logits (section 2.2: the router scores every expert for every
 * token; the scores are the linear map X W_r, plus a per-expert bias when
 * one is given). L[t][e] is the fp32 value nearest to
 *   sum over i = 0..d-1 of X[t][i] * Wr[i][e]  (+ bias[e]),
 * taken as: every product formed in fp64 (exact: two 24-bit significands
 * fit in 53 bits), the products and the bias added in fp64 in ascending i,
 * and the fp64 total rounded once to fp32 (round to nearest even).  The fp64
 * sum differs from the exact one by at most (d + 1) 2^-53 sum |x w|, far
 * below half an fp32 unit, so L is the correctly rounded logit except when
 * the exact value lies that close to an fp32 rounding boundary.
 * X: [T][ldx] fp32 values (bf16 inputs widened exactly), Wr: [d][E], bias: [E]
 * or NULL, L: [T][E].
 */
void oracle_router_logits(int64_t T, int64_t d, int64_t E, const float *X,
                          int64_t ldx, const float *Wr, const float *bias,
                          float *L)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t i = 0; i < d; ++i)
                s += (double)X[t * ldx + i] * (double)Wr[i * E + e];
            if (bias) s += (double)bias[e];
            L[t * E + e] = (float)s;
        }
    }
}

/*
 * Top-k routing for each token t.
 *   A NaN logit is read as -infinity (the pages define no NaN behaviour: such
 *   an expert ranks below every number and gets weight 0).
 *   idx[t][j], j < k: the j-th choice by repeated selection of the largest
 *     logit among the experts not yet chosen; equal logits go to the lower id.
 *   alpha: p_e = exp(L_e - m) / sum_e' exp(L_e' - m) with m = max_e L_e
 *     (the softmax over all E), in fp64; alpha[t][j] = p_{idx[t][j]}, divided
 *     by sum_{j'<k} p_{idx[t][j']} when renorm != 0. When every logit is
 *     -infinity, m is taken as 0 and every weight is 0.
 *   shared experts: idx[t][k + s] = E + s, alpha = 1, for s < n_shared.
 * idx and alpha are [T][k + n_shared].
 */
void oracle_topk(int64_t T, int64_t E, int64_t k, int64_t n_shared, int renorm,
                 const float *L, int32_t *idx, double *alpha)
{
    const int64_t kp = k + n_shared;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        for (int64_t e = 0; e < E; ++e) l[e] = isnan(L[t * E + e]) ? -INFINITY : L[t * E + e];
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;  /* strict: ties keep lower id */
            }
            taken[best] = 1;
            idx[t * kp + j] = (int32_t)best;
        }
        double m = (double)l[0];
        for (int64_t e = 1; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        if (m == -INFINITY) m = 0.0;
        double s = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            s += p[e];
        }
        for (int64_t e = 0; e < E; ++e) p[e] = s > 0.0 ? p[e] / s : 0.0;
        double sel = 0.0;
        for (int64_t j = 0; j < k; ++j) sel += p[idx[t * kp + j]];
        for (int64_t j = 0; j < k; ++j) {
            double a = p[idx[t * kp + j]];
            alpha[t * kp + j] = renorm ? (sel > 0.0 ? a / sel : 0.0) : a;
        }
        for (int64_t s2 = 0; s2 < n_shared; ++s2) {
            idx[t * kp + k + s2] = (int32_t)(E + s2);
            alpha[t * kp + k + s2] = 1.0;
        }
        free(taken);
        free(p);
        free(l);
    }
}

/*
 * Route map of Algorithm 1 (section 3.2, "Composed Sparse Route and Parameter
 * Binding") for the routes of tokens t0 .. t0+nt-1.  Route i = t*kp + j sends
 * token t to logical expert e_i = idx[i].
 *   psi_i = phi[e_i] (-1 = not resident; such routes are left out);
 *   count[s] = number of routes with psi_i = s, s < P;
 *   offset[0] = 0, offset[s+1] = offset[s] + count[s];
 *   cursor = offset; for i ascending: p = cursor[psi_i]; rec[p] = (t_i, i);
 *   cursor[psi_i] = p + 1.
 * route_pos[i] = p for placed routes and -1 for left-out routes of the range;
 * entries outside the range are not touched.  Returns n_valid = offset[P], or
 * -1 if an expert id is outside [0, n_exp) or phi names a slot outside
 * [-1, P).
 */
int64_t oracle_route_map(int64_t kp, int64_t t0, int64_t nt, const int32_t *idx,
                         int64_t n_exp, const int32_t *phi, int64_t P,
                         int32_t *count, int32_t *offset, int32_t *rec_token,
                         int32_t *rec_route, int32_t *route_pos)
{
    const int64_t i0 = t0 * kp, i1 = (t0 + nt) * kp;
    for (int64_t i = i0; i < i1; ++i) {
        if (idx[i] < 0 || idx[i] >= n_exp) return -1;
        if (phi[idx[i]] < -1 || phi[idx[i]] >= P) return -1;
    }
    for (int64_t s = 0; s < P; ++s) count[s] = 0;
    for (int64_t i = i0; i < i1; ++i) {
        int32_t psi = phi[idx[i]];
        if (psi >= 0) count[psi] += 1;
    }
    offset[0] = 0;
    for (int64_t s = 0; s < P; ++s) offset[s + 1] = offset[s] + count[s];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P + 1));
    for (int64_t s = 0; s <= P; ++s) cursor[s] = offset[s];
    for (int64_t i = i0; i < i1; ++i) {
        int32_t psi = phi[idx[i]];
        if (psi < 0) {
            route_pos[i] = -1;
            continue;
        }
        int32_t p = cursor[psi];
        rec_token[p] = (int32_t)(i / kp);
        rec_route[p] = (int32_t)i;
        route_pos[i] = p;
        cursor[psi] = p + 1;
    }
    free(cursor);
    return offset[P];
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * MXFP4 (OCP Microscaling Formats, FP4 E2M1 elements with an E8M0 scale per
 * block of 32). codes: [N][K/2] bytes; element 2i of a row is the low nibble
 * of byte i, element 2i+1 the high nibble. An E2M1 code is sign (bit 3),
 * exponent (bits 2..1, bias 1) and mantissa (bit 0): exponent 0 gives the
 * subnormals 0 and 0.5, exponent e > 0 gives (1 + m/2) * 2^(e-1); there are
 * no infinities or NaN. scales: [N][K/32] bytes, E8M0: 2^(s - 127), s = 255
 * is NaN. out[n][k] = E2M1(code[n][k]) * 2^(scales[n][k/32] - 127).
 */
void oracle_mxfp4_decode(int64_t N, int64_t K, const uint8_t *codes, const uint8_t *scales, float *out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t byte = codes[n * (K / 2) + k / 2];
            const int c = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            const int sgn = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
            const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
            const int sc = scales[n * (K / 32) + k / 32];
            const double v = sc == 255 ? NAN : ldexp(sgn ? -mag : mag, sc - 127);
            out[n * K + k] = (float)v;
        }
}

/*
 * fp8 e4m3 codes to fp32 values (exact: every code's value has at most 4
 * significant bits and an exponent in [-9, 8]).
 *   code = s eeee mmm:  e = 0:        (-1)^s * m/8 * 2^-6
 *                       e = 15, m = 7: NaN
 *                       otherwise:    (-1)^s * (1 + m/8) * 2^(e-7)
 */
void oracle_fp8e4m3_decode(int64_t n, const uint8_t *q, float *out)
{
    for (int64_t i = 0; i < n; ++i) {
        const int sgn = q[i] >> 7, e = (q[i] >> 3) & 15, m = q[i] & 7;
        double v;
        if (e == 15 && m == 7)
            v = NAN;
        else if (e == 0)
            v = ldexp((double)m / 8.0, -6);
        else
            v = ldexp(1.0 + (double)m / 8.0, e - 7);
        out[i] = (float)(sgn ? -v : v);
    }
}

/*
 * Expert FFN and weighted combine for the listed tokens, Eq. (1)-(2):
 *   y = A[t]; for j = 0 .. kp-1 (routes of token t whose mask byte is nonzero,
 *   all of them when route_mask is NULL), with e = idx[t][j]:
 *     g[n] = sum_i Wg[e][n][i] x[i],  u[n] = sum_i Wu[e][n][i] x[i]   (n < f)
 *     h[n] = SiLU(g[n]) * u[n],       SiLU(z) = z / (1 + exp(-z))
 *     o[m] = sum_n Wd[e][m][n] h[n]                                   (m < d)
 *     y[m] += alpha[t][j] * o[m]
 * in fp64.  X: [T][ldx] fp32 values; Wg, Wu: [n_exp][f][d]; Wd: [n_exp][d][f];
 * A: [T][d] fp32 or NULL (zero residual); Y: [n_tok][d] fp64, row r for token
 * tokens[r].  route_mask is indexed by the global route id t*kp + j.
 * Sg, Su: [n_exp][f] and Sd: [n_exp][d] row scales, or all NULL: weight
 * Wg[e][n][i] stands for Wg[e][n][i] * Sg[e][n] (likewise Wu, and Wd with
 * Sd[e][m]), the product taken in fp64.
 */
void oracle_expert_ffn(int64_t d, int64_t f, int64_t kp, int64_t n_tok,
                       const int64_t *tokens, const float *X, int64_t ldx,
                       const int32_t *idx, const double *alpha,
                       const unsigned char *route_mask, const float *Wg,
                       const float *Wu, const float *Wd, const float *Sg,
                       const float *Su, const float *Sd, const float *A,
                       double *Y)
{
    int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < n_tok; ++r) {
        const int64_t t = tokens[r];
        const float *x = X + t * ldx;
        double *y = Y + r * d;
        double *g = (double *)malloc(sizeof(double) * (size_t)f);
        double *u = (double *)malloc(sizeof(double) * (size_t)f);
        double *h = (double *)malloc(sizeof(double) * (size_t)f);
        for (int64_t m = 0; m < d; ++m) y[m] = A ? (double)A[t * d + m] : 0.0;
        for (int64_t j = 0; j < kp; ++j) {
            const int64_t i = t * kp + j;
            if (route_mask && !route_mask[i]) continue;
            const int64_t e = idx[i];
            const float *wg = Wg + e * f * d;
            const float *wu = Wu + e * f * d;
            const float *wd = Wd + e * d * f;
            for (int64_t n = 0; n < f; ++n) {
                const double scg = Sg ? (double)Sg[e * f + n] : 1.0;
                const double scu = Su ? (double)Su[e * f + n] : 1.0;
                double sg = 0.0, su = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    sg += (double)wg[n * d + c] * scg * (double)x[c];
                    su += (double)wu[n * d + c] * scu * (double)x[c];
                }
                g[n] = sg;
                u[n] = su;
            }
            for (int64_t n = 0; n < f; ++n) h[n] = silu(g[n]) * u[n];
            for (int64_t m = 0; m < d; ++m) {
                const double scd = Sd ? (double)Sd[e * d + m] : 1.0;
                double o = 0.0;
                for (int64_t n = 0; n < f; ++n) o += (double)wd[m * f + n] * scd * h[n];
                y[m] += alpha[i] * o;
            }
        }
        free(g);
        free(u);
        free(h);
    }
}
