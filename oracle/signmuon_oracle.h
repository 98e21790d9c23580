/*
 * signmuon_oracle.h -- CPU oracle for the Sign-Muon optimizer step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this code. The GPU library never includes, links or
 * calls it, and this header shares nothing with the GPU library's headers.
 *
 * Source of the method: the technical summary of "SignMuon: Communication-
 * Efficient Distributed Muon Optimization" (gist.science, paper 2605.16311;
 * the es/fr/ar/ko pages carry the same text). Citations below name its
 * sections: §2 "Core mechanism", §2 "Algorithmic flow" steps 1-5, §2
 * "Communication efficiency", §3 "Geometry", §4 "nanoGPT".
 *
 * Conventions
 *  - Matrices are R x C, row-major, contiguous; n = R*C.
 *  - Per-worker buffers are stacked: worker m of a [Mw][n] array starts at m*n.
 *  - Storage codes (ORC_*) say how a buffer's elements are stored. bf16
 *    buffers hold raw 16-bit patterns (uint16_t). ORC_F64 means "exact": the
 *    value is kept in double precision and no storage rounding happens.
 *  - Packed signs: uint64 words, bit j of word w is entry 64*w + j of the
 *    row-major flat index; unused tail bits are zero; ceil(n/64) words per
 *    worker.
 *
 * Parity status: every function here is pinned by a CPU test against a fact
 * that does not come from this file (closed forms, library SVD, brute force,
 * the pages' worked vote example). The only unpinned quantity is the scale of
 * the optional post-vote polar step (the pages give none).
 */
#ifndef SIGNMUON_ORACLE_H
#define SIGNMUON_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };
enum { ORC_NORM_FROB = 0, ORC_NORM_SPECTRAL = 1 };

/* fp32 <-> bf16 bit patterns, round to nearest even. */
uint16_t orc_bf16_from_f32(float x);
float orc_bf16_to_f32(uint16_t h);
/* Round each of n fp32 values to bf16 (bulk helper for tests). */
void orc_bf16_round_array(int64_t n, const float *x, uint16_t *out);

/* O1 momentum, in place: M <- store_m(fmaf(beta, M, G)). */
void orc_momentum(int64_t n, float beta, const void *g, int g_dt, void *m, int m_dt);

/* O2 Frobenius normalisation: returns nu = ||M||_F (fp64 sum of squares of
 * the stored values) and writes x0 = M / nu in fp64 (x0 = 0 when nu = 0). */
double orc_normalise(int64_t n, const void *m, int m_dt, double *x0);

/* O3 Newton-Schulz: k cubic iterations from x0 (R x C, fp64).
 * Rounding points for ns_dt (ORC_F32 / ORC_BF16): each Gram matrix, and each
 * iterate X_j with 1 <= j < k, pass through fp32 and then ns_dt storage.
 * X_k is returned unrounded. ORC_F64 rounds nowhere. Returns 0, or -1 when
 * memory runs out. */
int orc_newton_schulz(int64_t R, int64_t C, const double *x0, int k, int ns_dt, double *u);

/* O3 with the first iteration's Gram matrix given (a0: r x r, rounded). */
int orc_newton_schulz_a0(int64_t R, int64_t C, const double *x0, const double *a0, int k,
                         int ns_dt, double *u);

/* Spectral normalisation: p power-iteration steps on the symmetric r x r
 * matrix a from the all-ones vector (w = a v, lambda = ||w||, v = w/lambda);
 * returns the last lambda (-1 when memory runs out). */
double orc_power_lambda(int64_t r, const double *a, int p);
/* X0 = M / sqrt(lambda) and the first Gram A0 = round(fp32(1/lambda) A_raw),
 * A_raw the stored Gram of M; returns lambda. */
double orc_spectral_x0_a0(int64_t R, int64_t C, const void *m, int m_dt, int ns_dt, int p,
                          double *x0, double *a0);

/* O3 for k = 1, one output entry at a time: out[t] = X_1[ri[t]][ci[t]].
 * Same sums in the same order as orc_newton_schulz with k = 1. */
int orc_ns1_entries(int64_t R, int64_t C, const double *x0, int ns_dt, int64_t nidx,
                    const int64_t *ri, const int64_t *ci, double *out);

/* O4 + O5 sign and 1-bit pack: bit = (u >= 0). */
void orc_sign_pack(int64_t n, const void *u, int u_dt, uint64_t *words);
int64_t orc_packed_words(int64_t n);

/* O6 + O7 majority vote over mw packed buffers ([mw][ceil(n/64)] words) and
 * the sign update of W in place (w nullable: vote only). vote (nullable)
 * receives S-bar in {-1,0,1}. */
void orc_vote_update(int64_t n, int32_t mw, const uint64_t *packed, float *w, float eta,
                     int8_t *vote);

/* Int8 payload: s[i] = +1 if u >= 0 else -1 (as the packed bits), and the
 * vote as the sign of the integer sum of the mw workers' int8 values
 * ([mw][n]), with the update of orc_vote_update. */
void orc_sign_int8(int64_t n, const void *u, int u_dt, int8_t *s);
void orc_vote_update_int8(int64_t n, int32_t mw, const int8_t *signs, float *w, float eta,
                          int8_t *vote);

/* O8 optional post-vote polar step: W <- fmaf(-eta, Y, W) with Y the k-step
 * Newton-Schulz factor of V / ||V||_F. Returns nnz(V); W is unchanged when
 * nnz(V) = 0. Returns -1 when memory runs out. */
int64_t orc_post_polar(int64_t R, int64_t C, const int8_t *vote, int k, int ns_dt, float *w,
                       float eta);

/* One full step for one matrix: every worker's O1-O5, then O6+O7 (or O6+O8
 * when post_k > 0). u_out (nullable) receives each worker's fp64 U, packed
 * receives [mw][ceil(n/64)] words, vote_out (nullable) S-bar.
 * Returns 0, or -1 when memory runs out. */
int orc_step_matrix(int64_t R, int64_t C, int32_t mw, float beta, float eta, int k, int post_k,
                    int g_dt, int m_dt, int ns_dt, const void *g, void *m, double *u_out,
                    uint64_t *packed, float *w, int8_t *vote_out);

/* orc_step_matrix with the normalisation of the Newton-Schulz input chosen:
 * ORC_NORM_FROB, or ORC_NORM_SPECTRAL with power_iters steps. */
int orc_step_matrix_norm(int64_t R, int64_t C, int32_t mw, float beta, float eta, int k,
                         int post_k, int g_dt, int m_dt, int ns_dt, int norm, int power_iters,
                         const void *g, void *m, double *u_out, uint64_t *packed, float *w,
                         int8_t *vote_out);

/* Full-precision Muon step for one worker (no sign, no vote): momentum,
 * normalised Newton-Schulz U (k iterations), W <- fmaf(-eta, (float)U, W).
 * u_out (nullable) receives U in fp64. */
int orc_muon_step_matrix(int64_t R, int64_t C, float beta, float eta, int k, int g_dt, int m_dt,
                         int ns_dt, int norm, int power_iters, const void *g, void *m,
                         double *u_out, float *w);

#ifdef __cplusplus
}
#endif
#endif
