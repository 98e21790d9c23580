/*
 * signmuon.h -- C ABI of the MI355X (gfx950) Sign-Muon optimizer step.
 *
 * The method is the one summarised in "SignMuon: Communication-Efficient
 * Distributed Muon Optimization" (gist.science, paper 2605.16311, technical
 * summary; citations below name its sections). Each of Mw workers updates its
 * own momentum, takes an approximate polar factor of it with Newton-Schulz
 * iterations, and keeps only the entrywise signs, packed one bit per entry;
 * all workers then take the majority vote of the Mw sign matrices and move
 * the weights by eta times the vote.
 *
 * On one GPU the Mw workers' buffers sit side by side in device memory: the
 * vote reads the Mw packed buffers that every worker would hold after the
 * all-gather of the summary's 1-bit variant. No collective is called here.
 *
 * Conventions shared by every entry point
 *  - A matrix is R x C, row-major and contiguous; n = R * C >= 1.
 *  - Per-worker arrays are stacked: [Mw][R][C], worker m at offset m * n.
 *  - All data pointers are DEVICE pointers owned by the caller. The library
 *    allocates no memory, frees nothing and keeps no state between calls
 *    (except signmuon_step_noalloc's static scratch, below); every call may be
 *    made from any host thread.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting for it. The library never synchronises.
 *    The compute entry points enqueue only kernel launches (no allocation, no
 *    memset, no copy), so a call may be captured into a HIP graph and
 *    replayed; the graph keeps the pointers and scalars of the captured call.
 *  - Pointers to device arrays must be 16-byte aligned (SIGNMUON_EALIGN).
 *  - Every argument is checked before anything is enqueued: a call that
 *    returns an error has enqueued no work. A launch failure returns
 *    SIGNMUON_EHIP (signmuon_strerror names the HIP error); a device fault
 *    shows up at the caller's next synchronisation of the stream.
 *  - Buffers written by a call must not overlap any other buffer of the
 *    same call, except where an entry point says "in place".
 *  - bf16 is stored as its 16-bit pattern; fp32 -> bf16 rounds to nearest
 *    even (NaN becomes a quiet NaN of the same sign).
 *
 * Packed signs (summary §2 "Algorithmic flow", step 3, 1-bit variant): one
 * uint64 word per 64 entries, signmuon_packed_words(n) = ceil(n/64) words per
 * worker. Bit j of word w is entry 64*w + j of the row-major flat index; bit
 * 1 means +1, chosen when the value is >= 0 (so +0 and -0 give +1 and NaN
 * gives -1); bits past n are zero.
 */
#ifndef SIGNMUON_H
#define SIGNMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SIGNMUON_ABI_VERSION 4

/* Status codes. */
enum {
    SIGNMUON_OK = 0,
    SIGNMUON_EINVAL = -1,     /* null pointer, size <= 0, workers < 1, bad count */
    SIGNMUON_EDTYPE = -2,     /* dtype code not accepted by this entry point */
    SIGNMUON_EALIGN = -3,     /* a device pointer is not 16-byte aligned */
    SIGNMUON_EWORKSPACE = -4, /* workspace missing or smaller than required */
    SIGNMUON_EHIP = -5,       /* a HIP call failed */
    SIGNMUON_ERANGE = -6,     /* a size exceeds what the kernels index */
    SIGNMUON_ESCRATCH = -7    /* signmuon_step_noalloc: the step's workspace exceeds
                                 SIGNMUON_STATIC_SCRATCH_BYTES */
};

typedef enum { SIGNMUON_F32 = 0, SIGNMUON_BF16 = 1 } signmuon_dtype;

/* Normalisation of the Newton-Schulz input X_0 = s M (summary §4 "nanoGPT":
 * Frobenius and spectral scaling both evaluated). */
typedef enum {
    SIGNMUON_NORM_FROBENIUS = 0, /* s = 1 / ||M||_F */
    SIGNMUON_NORM_SPECTRAL = 1   /* s = 1 / sqrt(lambda), lambda the power-iteration estimate of
                                    ||M||_2^2 on the Gram matrix (see signmuon_params) */
} signmuon_norm;

/* Sign payload of signmuon_step (summary §2 "Communication efficiency": one
 * bit per entry, or eight "for implementation simplicity"). */
typedef enum {
    SIGNMUON_PAYLOAD_BITS = 0, /* packed 1-bit signs in signmuon_matrix.packed; the vote counts
                                  the +1 bits */
    SIGNMUON_PAYLOAD_INT8 = 1  /* int8 +-1 signs in signmuon_matrix.signs_i8; the vote is the
                                  sign of their integer sum (what an integer SUM all-reduce
                                  of the workers' buffers would give) */
} signmuon_payload;

/* A hipStream_t, passed as an opaque pointer so that this header needs no
 * HIP header. */
typedef void *signmuon_stream;

/* One weight matrix and its per-worker buffers. */
typedef struct {
    int64_t rows, cols;  /* R, C >= 1 */
    const void *grad;    /* [Mw][R][C] of params.grad_dtype: each worker's stochastic
                            gradient G (summary §2 "Algorithmic flow", step 1) */
    void *momentum;      /* [Mw][R][C] of params.mom_dtype, in place: each worker's
                            momentum M, the only persistent optimizer state (summary
                            §4 "Memory"); start it at zero */
    float *polar_out;    /* [Mw][R][C] fp32 or NULL: the Newton-Schulz output U of each
                            worker. signmuon_momentum_ns requires it; signmuon_step
                            writes it when non-NULL */
    uint64_t *packed;    /* [Mw][signmuon_packed_words(R*C)]: each worker's packed
                            signs S = sign(U) (required by signmuon_step) */
    float *weight;       /* [R][C] fp32, in place: the weights W (required by
                            signmuon_step) */
    int8_t *vote_out;    /* [R][C] or NULL: the vote S-bar in {-1, 0, +1} */
    int8_t *signs_i8;    /* [Mw][R][C] int8: each worker's signs as +1 / -1 (same rule as
                            the packed bits). Required by signmuon_step with
                            params.payload == SIGNMUON_PAYLOAD_INT8 (then `packed` is not
                            used); ignored otherwise */
} signmuon_matrix;

/* Hyper-parameters of one step (summary §2 "Algorithmic flow"). */
typedef struct {
    int32_t workers;          /* Mw >= 1 */
    float beta;               /* momentum coefficient: M <- beta*M + G (finite) */
    float eta;                /* step size eta_t of W <- W - eta_t * S-bar (finite) */
    int32_t ns_iters;         /* k >= 0 Newton-Schulz iterations (k = 0: U = M/||M||_F) */
    int32_t post_polar_iters; /* 0 = off; > 0: the optional local polar step on S-bar
                                 (summary §2 "Algorithmic flow", step 5) with this many
                                 iterations, which then replaces the sign update */
    signmuon_dtype grad_dtype; /* G storage: F32 or BF16 */
    signmuon_dtype mom_dtype;  /* M storage: F32 or BF16 */
    signmuon_dtype ns_dtype;   /* Newton-Schulz operand storage: F32 or BF16 */
    int32_t norm;              /* signmuon_norm of X_0 (0 = Frobenius) */
    int32_t power_iters;       /* SIGNMUON_NORM_SPECTRAL: power-iteration steps p >= 1 (ignored
                                  otherwise). The summary gives no procedure; the one taken:
                                  A_raw = the stored Gram matrix of the stored M (M M^T if
                                  R <= C, else M^T M); from v = all-ones / sqrt(r), p times
                                  w = A_raw v, lambda = ||w||, v = w / lambda; s = 1/sqrt(lambda);
                                  the first iteration uses A_0 = round(fp32(1/lambda) * A_raw)
                                  and X_0 = s M. lambda = 0 gives U = 0. Needs min(R, C) <= 8192
                                  (SIGNMUON_ERANGE). The post-vote polar step keeps its exact
                                  Frobenius scale. */
    int32_t payload;           /* signmuon_payload of signmuon_step (0 = packed bits). INT8
                                  does not combine with post_polar_iters > 0 (SIGNMUON_EINVAL). */
} signmuon_params;

/* Largest number of matrices one call accepts. */
#define SIGNMUON_MAX_MATRICES 4096

/*
 * signmuon_momentum_ns -- each worker's local computation up to the polar
 * factor (summary §2 "Core mechanism" and "Algorithmic flow" step 1):
 *   M <- store_M(fmaf(beta, M, G))            (one fp32 fused multiply-add)
 *   X0 = M / ||M||_F                          (Frobenius scaling; X0 = 0 if M = 0)
 *   k times: A = X X^T, X <- 1.5 X - 0.5 A X  (R <= C)
 *            A = X^T X, X <- 1.5 X - 0.5 X A  (R > C)
 *   U = X_k written to polar_out as fp32.
 * The Gram matrix A and every iterate before the last are stored in
 * ns_dtype; products accumulate in fp32 on the matrix cores. The summary
 * prints neither the momentum form nor the Newton-Schulz coefficients; the
 * heavy-ball form and the cubic 1.5 / -0.5 are the readings taken.
 * mats[i].grad, .momentum and .polar_out are used; the other fields are
 * ignored. workspace: signmuon_workspace_bytes(mats, n_mats, p) bytes.
 */
int signmuon_momentum_ns(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                         void *workspace, size_t workspace_bytes, signmuon_stream stream);

/*
 * signmuon_sign_pack -- entrywise sign and 1-bit packing (summary §2 "Core
 * mechanism" and "Algorithmic flow" steps 2-3): u is [workers][n] of u_dtype
 * (F32 or BF16); packed receives [workers][signmuon_packed_words(n)] words in
 * the packed-sign layout above.
 */
int signmuon_sign_pack(const void *u, signmuon_dtype u_dtype, int64_t n, int32_t workers,
                       uint64_t *packed, signmuon_stream stream);

/*
 * signmuon_vote_update -- majority vote and update (summary §2 "Core
 * mechanism", and "Algorithmic flow" step 4):
 *   c_i = number of workers whose bit i is 1,  S-bar_i = sign(2 c_i - workers)
 *   W_i <- W_i - eta (S-bar_i = +1),  W_i + eta (S-bar_i = -1),  unchanged (0)
 * Each add is one fp32 operation rounded to nearest even. A tie (even worker
 * count only) votes 0 -- the summary does not say; this is the reading taken.
 * packed is [workers][signmuon_packed_words(n)]; weight [n] fp32 is updated in
 * place (NULL: vote only); vote_out [n] int8 or NULL. At least one of weight
 * and vote_out must be non-NULL.
 */
int signmuon_vote_update(const uint64_t *packed, int32_t workers, int64_t n, float *weight,
                         float eta, int8_t *vote_out, signmuon_stream stream);

/*
 * signmuon_sign_int8 -- the int8 payload of the signs (summary §2
 * "Communication efficiency": eight bits per entry with int8, 4x below fp32):
 * signs[i] = +1 where u[i] >= 0, else -1 -- the rule of the packed bits, so
 * +0 and -0 give +1 and NaN gives -1. u is [workers][n] of u_dtype (F32 or
 * BF16); signs receives [workers][n] int8.
 */
int signmuon_sign_int8(const void *u, signmuon_dtype u_dtype, int64_t n, int32_t workers,
                       int8_t *signs, signmuon_stream stream);

/*
 * signmuon_vote_update_int8 -- the vote from int8 payloads (summary §2 "Core
 * mechanism": an integer SUM all-reduce of the workers' signs followed by a
 * local sign; "Algorithmic flow" step 4 for the update):
 *   t_i = sum over workers m of signs[m][i]   (plain integer sum)
 *   S-bar_i = sign(t_i), and W as in signmuon_vote_update.
 * On one GPU the sum runs over the workers' buffers in memory, as every rank
 * would after an integer all-reduce. With +-1 inputs (signmuon_sign_int8) the
 * vote and W equal those of signmuon_vote_update on the packed bits. signs
 * is [workers][n] int8 (any int8 values are summed as integers); weight [n]
 * fp32 in place (NULL: vote only); vote_out [n] int8 or NULL. At least one of
 * weight and vote_out must be non-NULL; workers <= 255.
 */
int signmuon_vote_update_int8(const int8_t *signs, int32_t workers, int64_t n, float *weight,
                              float eta, int8_t *vote_out, signmuon_stream stream);

/*
 * signmuon_step -- one whole optimizer step for every matrix (summary §2
 * "Algorithmic flow", steps 1-5 with the collective of step 3 replaced by the
 * workers' packed buffers being local): signmuon_momentum_ns, the sign and
 * packing of U fused into the last Newton-Schulz product, then the vote and
 * the update of W. With post_polar_iters > 0 the vote S-bar is not applied
 * directly: W <- fmaf(-eta, Y, W) with Y the post_polar_iters-step
 * Newton-Schulz factor of S-bar / ||S-bar||_F (W unchanged if S-bar = 0).
 * mats[i].grad, .momentum, .packed and .weight are required; .polar_out and
 * .vote_out are written when non-NULL. With params.payload ==
 * SIGNMUON_PAYLOAD_INT8 (summary §2 "Core mechanism" 3 and "Communication
 * efficiency": the integer all-reduce variant), the last product writes each
 * worker's signs as int8 to .signs_i8 (required; .packed is not used) and the
 * vote is the sign of the integer sum over workers; W and the vote then equal
 * the packed path's bit for bit.
 */
int signmuon_step(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                  void *workspace, size_t workspace_bytes, signmuon_stream stream);

/*
 * signmuon_muon_step -- the full-precision Muon step that the summary
 * compares against (§1 "Problem statement", §4 "Empirical results"): for one
 * worker, the momentum and normalised Newton-Schulz factor U of
 * signmuon_momentum_ns, then W <- fmaf(-eta, U, W) on the fp32 value of U,
 * with no sign and no vote. p->workers must be 1 and p->ns_iters >= 1
 * (p->post_polar_iters must be 0; norm and power_iters apply as in
 * signmuon_step). mats[i].grad, .momentum and .weight are required;
 * .polar_out receives U when non-NULL; .packed and .vote_out are ignored.
 * workspace: signmuon_workspace_bytes(mats, n_mats, p) bytes.
 */
int signmuon_muon_step(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                       void *workspace, size_t workspace_bytes, signmuon_stream stream);

/*
 * signmuon_step_noalloc -- signmuon_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same launches and results, with the workspace
 * taken from a static device array inside the library instead of a caller's
 * buffer. The array holds SIGNMUON_STATIC_SCRATCH_BYTES per GPU; it is
 * reserved on each GPU the library runs on and held until the process ends,
 * and its device address is looked up on the first call on each device.
 * Arguments, ownership and errors are those of signmuon_step, plus
 * SIGNMUON_ESCRATCH when signmuon_workspace_bytes(mats, n_mats, p) exceeds
 * the array (checked before any HIP call; nothing is enqueued). The call
 * allocates nothing. No part of the array needs to start at zero: every part
 * a step reads, it has written first in the same stream order. All calls on
 * one GPU share its array, so two calls whose work overlaps in time on the
 * same GPU (different streams or host threads without ordering) race and
 * give undefined results; order them on one stream.
 */
#define SIGNMUON_STATIC_SCRATCH_BYTES (128u << 20)
int signmuon_step_noalloc(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                          signmuon_stream stream);

/* Kernel kinds reported by signmuon_step_traced, one per launch. */
enum {
    SIGNMUON_K_MOMENTUM = 1, /* momentum update + Frobenius partial sums */
    SIGNMUON_K_SCALES = 2,   /* 1/||M||_F per (matrix, worker) */
    SIGNMUON_K_GRAM = 3,     /* Newton-Schulz Gram matrix */
    SIGNMUON_K_PRODUCT = 4,  /* Newton-Schulz product (+ fused sign/pack on the last) */
    SIGNMUON_K_PACK = 5,     /* standalone sign + pack */
    SIGNMUON_K_VOTE = 6,     /* majority vote + update */
    SIGNMUON_K_AUX = 7,      /* post-vote polar step bookkeeping */
    SIGNMUON_K_POWER = 8,    /* spectral normalisation: power steps and scale */
    SIGNMUON_K_VOTE_I8 = 9   /* vote from the int8 payload + update */
};

/* Instrumentation for stage timing: events[0] (a hipEvent_t created by the
 * caller) is recorded on the stream before the first launch and events[i+1]
 * after launch i, while i + 1 < capacity; kinds[i] receives launch i's kind.
 * launches receives the number of launches the call made. */
typedef struct {
    void **events;      /* hipEvent_t[capacity] */
    int32_t capacity;
    int32_t *kinds;     /* [capacity - 1] */
    int32_t launches;   /* out */
} signmuon_trace;

/* signmuon_step with every kernel launch bracketed by trace events (same
 * arguments, same results). trace may be NULL. */
int signmuon_step_traced(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                         void *workspace, size_t workspace_bytes, signmuon_stream stream,
                         signmuon_trace *trace);

/* ceil(n / 64): packed words per worker for n entries (0 for n <= 0). */
size_t signmuon_packed_words(int64_t n);

/* Device workspace, in bytes, that signmuon_step and signmuon_momentum_ns
 * need for these matrices and parameters (0 on invalid arguments). The same
 * workspace serves both entry points. */
size_t signmuon_workspace_bytes(const signmuon_matrix *mats, int32_t n_mats,
                                const signmuon_params *p);

/* Text for a status code; for SIGNMUON_EHIP it names the HIP error of the
 * calling thread's last failure. Never NULL. */
const char *signmuon_strerror(int status);

/* SIGNMUON_ABI_VERSION of the loaded library. */
int signmuon_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
