/*
 * signmuon_oracle.c -- CPU oracle for the Sign-Muon optimizer step.
 *
 * TEST INFRASTRUCTURE. Plain single-threaded C: no BLAS, no SIMD intrinsics,
 * sums accumulated in double precision in ascending index order. It is built
 * with -O2 -ffp-contract=off, so a multiply and an add are fused only where
 * fmaf() is written out. The GPU library shares no code with this file.
 *
 * Citations name sections of the technical summary of "SignMuon: Communication-
 * Efficient Distributed Muon Optimization" (gist.science, paper 2605.16311).
 * Where the summary leaves a step open, the reading taken is stated at the
 * function.
 */
#include "signmuon_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Storage helpers                                                          */
/* ------------------------------------------------------------------------ */

/* Round-to-nearest-even fp32 -> bf16: add half an ulp of the kept part (minus
 * one when the kept part is even) and truncate. NaN keeps its sign and top
 * payload bits and is forced quiet. */
uint16_t orc_bf16_from_f32(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

void orc_bf16_round_array(int64_t n, const float *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_f32(x[i]);
}

static double load_elem(const void *p, int dt, int64_t i)
{
    switch (dt) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return (double)orc_bf16_to_f32(((const uint16_t *)p)[i]);
    default: return ((const double *)p)[i];
    }
}

/* Storage of a value produced in fp32 arithmetic (only ORC_F32 / ORC_BF16). */
static void store_f32_value(void *p, int dt, int64_t i, float v)
{
    if (dt == ORC_BF16)
        ((uint16_t *)p)[i] = orc_bf16_from_f32(v);
    else
        ((float *)p)[i] = v;
}

/* A value computed in fp64 and then stored in the Newton-Schulz working type:
 * it passes through fp32 first (the accumulator type of the device matrix
 * cores), then through bf16 when that is the storage type. */
static double round_ns(double x, int ns_dt)
{
    if (ns_dt == ORC_F64)
        return x;
    float f = (float)x;
    if (ns_dt == ORC_BF16)
        f = orc_bf16_to_f32(orc_bf16_from_f32(f));
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* O1 momentum -- §2 "Algorithmic flow" step 1 (each worker updates its local */
/* momentum from its stochastic gradient). The form is not printed; the       */
/* reading taken is heavy-ball M <- beta*M + G with M starting at zero, one   */
/* correctly rounded fp32 fused multiply-add, stored in the momentum's type.  */
/* ------------------------------------------------------------------------ */
void orc_momentum(int64_t n, float beta, const void *g, int g_dt, void *m, int m_dt)
{
    for (int64_t i = 0; i < n; ++i) {
        float gi = (float)load_elem(g, g_dt, i);
        float mi = (float)load_elem(m, m_dt, i);
        store_f32_value(m, m_dt, i, fmaf(beta, mi, gi));
    }
}

/* ------------------------------------------------------------------------ */
/* O2 normalisation -- §2 "Communication efficiency" (normalisation is local) */
/* and §4 "nanoGPT" (Frobenius scaling is one of the two evaluated). Dividing */
/* by the Frobenius norm bounds the spectral norm by 1 (§3 "Geometry").      */
/* ------------------------------------------------------------------------ */
double orc_normalise(int64_t n, const void *m, int m_dt, double *x0)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = load_elem(m, m_dt, i);
        ss += v * v;
    }
    double nu = sqrt(ss);
    double s = nu > 0.0 ? 1.0 / nu : 0.0;
    for (int64_t i = 0; i < n; ++i)
        x0[i] = s * load_elem(m, m_dt, i);
    return nu;
}

/* ------------------------------------------------------------------------ */
/* O3 Newton-Schulz -- §2 "Core mechanism" (the polar factor of the momentum */
/* is approximated locally by the Newton-Schulz iteration) and §2            */
/* "Algorithmic flow" step 1. Coefficients are not printed; the cubic        */
/* X <- 1.5 X - 0.5 (X X^T) X is used, iterating on the smaller Gram matrix: */
/* X X^T when R <= C, X^T X (and X <- 1.5 X - 0.5 X (X^T X)) when R > C.     */
/* ------------------------------------------------------------------------ */

/* Gram matrix of the current iterate, r x r, rounded to the working type. */
static void gram(int64_t R, int64_t C, const double *x, int ns_dt, double *a)
{
    if (R <= C) {
        /* A[i][l] = sum_k X[i][k] X[l][k] */
        for (int64_t i = 0; i < R; ++i)
            for (int64_t l = 0; l < R; ++l) {
                double acc = 0.0;
                for (int64_t k = 0; k < C; ++k)
                    acc += x[i * C + k] * x[l * C + k];
                a[i * R + l] = acc;
            }
        for (int64_t t = 0; t < R * R; ++t)
            a[t] = round_ns(a[t], ns_dt);
    } else {
        /* A[i][l] = sum_k X[k][i] X[k][l]; k runs outermost, so each entry
         * still sums k = 0, 1, ... in order. */
        memset(a, 0, sizeof(double) * (size_t)(C * C));
        for (int64_t k = 0; k < R; ++k)
            for (int64_t i = 0; i < C; ++i) {
                double xi = x[k * C + i];
                for (int64_t l = 0; l < C; ++l)
                    a[i * C + l] += xi * x[k * C + l];
            }
        for (int64_t t = 0; t < C * C; ++t)
            a[t] = round_ns(a[t], ns_dt);
    }
}

/* P = A X (R <= C) or P = X A (R > C); each P entry sums the contraction
 * index in ascending order (written as row updates). */
static void gram_product(int64_t R, int64_t C, const double *a, const double *x, double *p)
{
    memset(p, 0, sizeof(double) * (size_t)(R * C));
    if (R <= C) {
        for (int64_t i = 0; i < R; ++i)
            for (int64_t l = 0; l < R; ++l) {
                double ail = a[i * R + l];
                for (int64_t j = 0; j < C; ++j)
                    p[i * C + j] += ail * x[l * C + j];
            }
    } else {
        for (int64_t i = 0; i < R; ++i)
            for (int64_t l = 0; l < C; ++l) {
                double xil = x[i * C + l];
                for (int64_t j = 0; j < C; ++j)
                    p[i * C + j] += xil * a[l * C + j];
            }
    }
}

static int newton_schulz(int64_t R, int64_t C, const double *x0, const double *a0, int k,
                         int ns_dt, double *u);

int orc_newton_schulz(int64_t R, int64_t C, const double *x0, int k, int ns_dt, double *u)
{
    return newton_schulz(R, C, x0, NULL, k, ns_dt, u);
}

int orc_newton_schulz_a0(int64_t R, int64_t C, const double *x0, const double *a0, int k,
                         int ns_dt, double *u)
{
    return newton_schulz(R, C, x0, a0, k, ns_dt, u);
}

/* a0 (nullable): the first iteration's Gram matrix, already rounded; the
 * later iterations form their own. */
static int newton_schulz(int64_t R, int64_t C, const double *x0, const double *a0, int k,
                         int ns_dt, double *u)
{
    int64_t n = R * C, r = R <= C ? R : C;
    double *x = (double *)malloc(sizeof(double) * (size_t)n);
    double *p = (double *)malloc(sizeof(double) * (size_t)n);
    double *a = (double *)malloc(sizeof(double) * (size_t)(r * r));
    if (!x || !p || !a) {
        free(x); free(p); free(a);
        return -1;
    }
    memcpy(x, x0, sizeof(double) * (size_t)n);
    for (int j = 0; j < k; ++j) {
        if (j == 0 && a0)
            memcpy(a, a0, sizeof(double) * (size_t)(r * r));
        else
            gram(R, C, x, ns_dt, a);
        gram_product(R, C, a, x, p);
        int last = (j == k - 1);
        for (int64_t t = 0; t < n; ++t) {
            double next = 1.5 * x[t] - 0.5 * p[t];
            x[t] = last ? next : round_ns(next, ns_dt);
        }
    }
    memcpy(u, x, sizeof(double) * (size_t)n);
    free(x); free(p); free(a);
    return 0;
}

int orc_ns1_entries(int64_t R, int64_t C, const double *x0, int ns_dt, int64_t nidx,
                    const int64_t *ri, const int64_t *ci, double *out)
{
    int64_t r = R <= C ? R : C;
    double *arow = (double *)malloc(sizeof(double) * (size_t)r);
    if (!arow)
        return -1;
    for (int64_t t = 0; t < nidx; ++t) {
        int64_t i = ri[t], j = ci[t];
        double p = 0.0;
        if (R <= C) {
            /* row i of A = X X^T, then (A X)[i][j] */
            for (int64_t l = 0; l < R; ++l) {
                double acc = 0.0;
                for (int64_t k = 0; k < C; ++k)
                    acc += x0[i * C + k] * x0[l * C + k];
                arow[l] = round_ns(acc, ns_dt);
            }
            for (int64_t l = 0; l < R; ++l)
                p += arow[l] * x0[l * C + j];
        } else {
            /* column j of A = X^T X, then (X A)[i][j] */
            for (int64_t l = 0; l < C; ++l) {
                double acc = 0.0;
                for (int64_t k = 0; k < R; ++k)
                    acc += x0[k * C + l] * x0[k * C + j];
                arow[l] = round_ns(acc, ns_dt);
            }
            for (int64_t l = 0; l < C; ++l)
                p += x0[i * C + l] * arow[l];
        }
        out[t] = 1.5 * x0[i * C + j] - 0.5 * p;
    }
    free(arow);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Spectral normalisation -- §4 "nanoGPT" (the results hold with spectral as */
/* with Frobenius scaling of the Newton-Schulz input) and §3 "Geometry" (the */
/* polar direction lives in the spectral-norm geometry). The summary gives   */
/* no procedure; readings: ||M||_2^2 is the largest eigenvalue of the Gram   */
/* matrix of the stored M (the Newton-Schulz orientation), estimated by p    */
/* power-iteration steps from the all-ones vector: w = A v, lambda = ||w||,  */
/* v = w / lambda. The Gram is stored (rounded) before its scale is known,   */
/* so A_0 = round(fp32(s^2) * A_raw) with s = 1 / sqrt(lambda), and the      */
/* first iteration starts from X_0 = s M with that A_0. lambda = 0 gives     */
/* s = 0 (U = 0).                                                            */
/* ------------------------------------------------------------------------ */
double orc_power_lambda(int64_t r, const double *a, int p)
{
    double *v = (double *)malloc(sizeof(double) * (size_t)r);
    double *w = (double *)malloc(sizeof(double) * (size_t)r);
    if (!v || !w) {
        free(v); free(w);
        return -1.0;
    }
    for (int64_t i = 0; i < r; ++i)
        v[i] = 1.0 / sqrt((double)r);
    double lambda = 0.0;
    for (int it = 0; it < p; ++it) {
        double ss = 0.0;
        for (int64_t i = 0; i < r; ++i) {
            double acc = 0.0;
            for (int64_t l = 0; l < r; ++l)
                acc += a[i * r + l] * v[l];
            w[i] = acc;
            ss += acc * acc;
        }
        lambda = sqrt(ss);
        if (lambda == 0.0)
            break;
        for (int64_t i = 0; i < r; ++i)
            v[i] = w[i] / lambda;
    }
    free(v); free(w);
    return lambda;
}

double orc_spectral_x0_a0(int64_t R, int64_t C, const void *m, int m_dt, int ns_dt, int p,
                          double *x0, double *a0)
{
    int64_t n = R * C, r = R <= C ? R : C;
    for (int64_t i = 0; i < n; ++i)
        x0[i] = load_elem(m, m_dt, i);
    gram(R, C, x0, ns_dt, a0); /* A_raw of the stored M */
    double lambda = orc_power_lambda(r, a0, p);
    if (lambda < 0.0)
        return lambda;
    double s = lambda > 0.0 ? 1.0 / sqrt(lambda) : 0.0;
    float s2 = lambda > 0.0 ? (float)(1.0 / lambda) : 0.0f;
    for (int64_t i = 0; i < n; ++i)
        x0[i] *= s;
    /* exact mode: no storage, so no fp32 scale either */
    double s2d = ns_dt == ORC_F64 ? (lambda > 0.0 ? 1.0 / lambda : 0.0) : (double)s2;
    for (int64_t t = 0; t < r * r; ++t)
        a0[t] = round_ns(s2d * a0[t], ns_dt);
    return lambda;
}

/* ------------------------------------------------------------------------ */
/* O4 + O5 sign and 1-bit packing -- §2 "Core mechanism" (each worker sends  */
/* only the entrywise signs, values in {-1,+1}), §2 "Algorithmic flow" steps */
/* 2-3 (S = sign(U); signs packed one bit per entry for the all-gather).     */
/* Readings: +1 is bit 1 and is chosen when U >= 0 (so +0 and -0 give +1 and */
/* NaN gives -1); words are uint64, least significant bit first, over the    */
/* row-major flat index, tail bits zero.                                     */
/* ------------------------------------------------------------------------ */
int64_t orc_packed_words(int64_t n)
{
    return (n + 63) / 64;
}

void orc_sign_pack(int64_t n, const void *u, int u_dt, uint64_t *words)
{
    int64_t nw = orc_packed_words(n);
    for (int64_t w = 0; w < nw; ++w)
        words[w] = 0;
    for (int64_t i = 0; i < n; ++i)
        if (load_elem(u, u_dt, i) >= 0.0)
            words[i / 64] |= (uint64_t)1 << (i % 64);
}

/* ------------------------------------------------------------------------ */
/* O6 + O7 majority vote and update -- §2 "Core mechanism" (vote = integer   */
/* sum of the workers' signs, then its sign) and §2 "Algorithmic flow" step  */
/* 4 (W_{t+1} = W_t - eta_t * S-bar_t). Reading: a tie (possible only with   */
/* an even worker count) votes 0 and leaves the entry unchanged.             */
/* ------------------------------------------------------------------------ */
void orc_vote_update(int64_t n, int32_t mw, const uint64_t *packed, float *w, float eta,
                     int8_t *vote)
{
    int64_t nw = orc_packed_words(n);
    for (int64_t i = 0; i < n; ++i) {
        int64_t plus = 0;
        for (int32_t m = 0; m < mw; ++m)
            plus += (int64_t)((packed[m * nw + i / 64] >> (i % 64)) & 1u);
        /* sum of signs = plus - (mw - plus) */
        int64_t sum = 2 * plus - mw;
        int8_t v = sum > 0 ? 1 : (sum < 0 ? -1 : 0);
        if (w && v > 0)
            w[i] = w[i] - eta;
        else if (w && v < 0)
            w[i] = w[i] + eta;
        if (vote)
            vote[i] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* Int8 payload -- §2 "Core mechanism" (the vote as an integer SUM           */
/* all-reduce of the workers' signs followed by a local sign) and §2         */
/* "Communication efficiency" (eight bits per entry with int8). Each worker  */
/* sends its signs as int8 +1 / -1 with the same rule as the packed bits     */
/* (u >= 0 gives +1); the vote is the sign of the plain integer sum of the   */
/* workers' values, and the update is that of O7.                            */
/* ------------------------------------------------------------------------ */
void orc_sign_int8(int64_t n, const void *u, int u_dt, int8_t *s)
{
    for (int64_t i = 0; i < n; ++i)
        s[i] = load_elem(u, u_dt, i) >= 0.0 ? (int8_t)1 : (int8_t)-1;
}

void orc_vote_update_int8(int64_t n, int32_t mw, const int8_t *signs, float *w, float eta,
                          int8_t *vote)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t sum = 0;
        for (int32_t m = 0; m < mw; ++m)
            sum += signs[(int64_t)m * n + i];
        int8_t v = sum > 0 ? 1 : (sum < 0 ? -1 : 0);
        if (w && v > 0)
            w[i] = w[i] - eta;
        else if (w && v < 0)
            w[i] = w[i] + eta;
        if (vote)
            vote[i] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* Full-precision Muon step, the comparison point the summary's §1 "Problem  */
/* statement" and §4 "Empirical results" name (Muon): one worker's momentum, */
/* its normalised Newton-Schulz polar factor U, and W <- W - eta U with no   */
/* sign and no vote. Readings: the same momentum, normalisation (norm,       */
/* power_iters as in orc_step_matrix_norm) and iteration as the Sign-Muon    */
/* step; the update is one fp32 fused multiply-add on the fp32 value of U,   */
/* as in the post-vote polar step.                                           */
/* ------------------------------------------------------------------------ */
int orc_muon_step_matrix(int64_t R, int64_t C, float beta, float eta, int k, int g_dt, int m_dt,
                         int ns_dt, int norm, int power_iters, const void *g, void *m,
                         double *u_out, float *w)
{
    int64_t n = R * C, r = R <= C ? R : C;
    double *x0 = (double *)malloc(sizeof(double) * (size_t)n);
    double *u = (double *)malloc(sizeof(double) * (size_t)n);
    double *a0 = norm == ORC_NORM_SPECTRAL ? (double *)malloc(sizeof(double) * (size_t)(r * r)) : NULL;
    if (!x0 || !u || (norm == ORC_NORM_SPECTRAL && !a0)) {
        free(x0); free(u); free(a0);
        return -1;
    }
    int rc = 0;
    orc_momentum(n, beta, g, g_dt, m, m_dt);
    if (norm == ORC_NORM_SPECTRAL) {
        if (orc_spectral_x0_a0(R, C, m, m_dt, ns_dt, power_iters, x0, a0) < 0.0)
            rc = -1;
        else
            rc = newton_schulz(R, C, x0, a0, k, ns_dt, u);
    } else {
        orc_normalise(n, m, m_dt, x0);
        rc = orc_newton_schulz(R, C, x0, k, ns_dt, u);
    }
    if (rc == 0) {
        for (int64_t i = 0; i < n; ++i)
            w[i] = fmaf(-eta, (float)u[i], w[i]);
        if (u_out)
            memcpy(u_out, u, sizeof(double) * (size_t)n);
    }
    free(x0); free(u); free(a0);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* O8 optional post-vote polar step -- §2 "Algorithmic flow" step 5 (a local */
/* polar step on the aggregated sign matrix, no extra communication).        */
/* Readings: the same Frobenius-normalised Newton-Schulz as O2-O3 applied to */
/* S-bar (||S-bar||_F = sqrt(nnz)), and the update W <- W - eta * Y in one   */
/* fp32 fused multiply-add on the fp32 value of Y. Scale: parity unpinned.   */
/* ------------------------------------------------------------------------ */
int64_t orc_post_polar(int64_t R, int64_t C, const int8_t *vote, int k, int ns_dt, float *w,
                       float eta)
{
    int64_t n = R * C, nnz = 0;
    for (int64_t i = 0; i < n; ++i)
        nnz += vote[i] != 0;
    if (nnz == 0)
        return 0;
    double *y0 = (double *)malloc(sizeof(double) * (size_t)n);
    double *y = (double *)malloc(sizeof(double) * (size_t)n);
    if (!y0 || !y) {
        free(y0); free(y);
        return -1;
    }
    double s = 1.0 / sqrt((double)nnz);
    for (int64_t i = 0; i < n; ++i)
        y0[i] = s * (double)vote[i];
    if (orc_newton_schulz(R, C, y0, k, ns_dt, y) != 0) {
        free(y0); free(y);
        return -1;
    }
    for (int64_t i = 0; i < n; ++i)
        w[i] = fmaf(-eta, (float)y[i], w[i]);
    free(y0); free(y);
    return nnz;
}

/* ------------------------------------------------------------------------ */
/* One step for one matrix -- §2 "Algorithmic flow" steps 1-5 in order. The  */
/* collective of step 3 is not modelled: all workers' packed buffers are     */
/* already local, which is the state every worker holds after the gather.    */
/* ------------------------------------------------------------------------ */
static int elem_bytes(int dt)
{
    return dt == ORC_BF16 ? 2 : (dt == ORC_F32 ? 4 : 8);
}

int orc_step_matrix(int64_t R, int64_t C, int32_t mw, float beta, float eta, int k, int post_k,
                    int g_dt, int m_dt, int ns_dt, const void *g, void *m, double *u_out,
                    uint64_t *packed, float *w, int8_t *vote_out)
{
    return orc_step_matrix_norm(R, C, mw, beta, eta, k, post_k, g_dt, m_dt, ns_dt, ORC_NORM_FROB,
                                0, g, m, u_out, packed, w, vote_out);
}

int orc_step_matrix_norm(int64_t R, int64_t C, int32_t mw, float beta, float eta, int k,
                         int post_k, int g_dt, int m_dt, int ns_dt, int norm, int power_iters,
                         const void *g, void *m, double *u_out, uint64_t *packed, float *w,
                         int8_t *vote_out)
{
    int64_t n = R * C, nw = orc_packed_words(n), r = R <= C ? R : C;
    double *x0 = (double *)malloc(sizeof(double) * (size_t)n);
    double *u = (double *)malloc(sizeof(double) * (size_t)n);
    int8_t *vote = (int8_t *)malloc((size_t)n);
    double *a0 = norm == ORC_NORM_SPECTRAL ? (double *)malloc(sizeof(double) * (size_t)(r * r)) : NULL;
    if (!x0 || !u || !vote || (norm == ORC_NORM_SPECTRAL && !a0)) {
        free(x0); free(u); free(vote); free(a0);
        return -1;
    }
    int rc = 0;
    for (int32_t wk = 0; wk < mw && rc == 0; ++wk) {
        const char *gw = (const char *)g + (size_t)(wk * n) * (size_t)elem_bytes(g_dt);
        char *mwp = (char *)m + (size_t)(wk * n) * (size_t)elem_bytes(m_dt);
        orc_momentum(n, beta, gw, g_dt, mwp, m_dt);
        if (norm == ORC_NORM_SPECTRAL) {
            if (orc_spectral_x0_a0(R, C, mwp, m_dt, ns_dt, power_iters, x0, a0) < 0.0)
                rc = -1;
            else
                rc = newton_schulz(R, C, x0, a0, k, ns_dt, u);
        } else {
            orc_normalise(n, mwp, m_dt, x0);
            rc = orc_newton_schulz(R, C, x0, k, ns_dt, u);
        }
        if (rc == 0) {
            orc_sign_pack(n, u, ORC_F64, packed + wk * nw);
            if (u_out)
                memcpy(u_out + wk * n, u, sizeof(double) * (size_t)n);
        }
    }
    if (rc == 0) {
        if (post_k > 0) {
            /* W moves only by the polar step of the vote. */
            orc_vote_update(n, mw, packed, NULL, eta, vote);
            if (orc_post_polar(R, C, vote, post_k, ns_dt, w, eta) < 0)
                rc = -1;
        } else {
            orc_vote_update(n, mw, packed, w, eta, vote);
        }
        if (rc == 0 && vote_out)
            memcpy(vote_out, vote, (size_t)n);
    }
    free(x0); free(u); free(vote); free(a0);
    return rc;
}
