// sm_internal.h -- launch descriptors shared by the host API and the gfx950
// kernels of the Sign-Muon step. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

namespace sm {

// Matrices per kernel launch: the descriptors travel by value in the kernel
// arguments, which must stay well under the 4 KiB argument limit.
constexpr int kMaxMatsPerLaunch = 48;

// First block (or tile) of each matrix of a launch, packed contiguously so
// that a block finds its matrix with a few wide scalar loads and unrolled
// compares. Entries past the launch's matrices hold INT32_MAX.
struct Starts {
    int32_t v[kMaxMatsPerLaunch];
    __host__ __device__ Starts() {
        for (int i = 0; i < kMaxMatsPerLaunch; ++i) v[i] = INT32_MAX;
    }
};

// Index of the matrix whose range holds block t (starts are non-decreasing
// and start at 0).
__device__ __forceinline__ int find_start(const Starts &s, int t) {
    int mi = 0;
#pragma unroll
    for (int j = 1; j < kMaxMatsPerLaunch; ++j) mi += t >= s.v[j] ? 1 : 0;
    return mi;
}

// ---------------------------------------------------------------------------
// Momentum + Frobenius partial sums.
// ---------------------------------------------------------------------------
constexpr int kMomThreads = 256;
constexpr int kMomElemsPerThread = 32;  // 4 rounds of 8
constexpr int kMomChunk = kMomThreads * kMomElemsPerThread;

struct MomMat {
    const void *g;          // [Mw][n] gradient
    void *m;                // [Mw][n] momentum, in place
    uint64_t *packed;       // k = 0: [Mw][n / 64] signs of the stored M (n % 64 == 0,
                            // n % 8 == 0 path), or nullptr
    int64_t n;
    int32_t block_begin;    // first block of this matrix within the launch
    int32_t blocks_per_worker;
    int32_t partial_begin;  // index of (this matrix, worker 0, chunk 0) in partials
    int32_t unit_begin;     // index of (this matrix, worker 0) in the unit arrays
};

struct MomBatch {
    MomMat mat[kMaxMatsPerLaunch];
    int32_t nmat;
    int32_t workers;
    int32_t total_blocks;
    float beta;
    int32_t g_bf16;
    int32_t m_bf16;
    double *partials;       // sum of squares of the stored momentum, per block
    float2 *scales;         // per unit: {s = 1/||M||_F, s^2} (0 when ||M|| = 0)
    int32_t *pack_fix;      // per unit: 1 where the signs of U = s M differ from those of
                            // M, i.e. ||M||_F is NaN or Inf (set by finalize_scales for
                            // matrices with packed)
    Starts starts;         // first block (tile) of each matrix
};

void launch_momentum(const MomBatch &b, hipStream_t s);
void launch_finalize_scales(const MomBatch &b, hipStream_t s);
// k = 0 with signs packed by the momentum kernel: for each unit flagged in
// b.pack_fix, the signs of s M again from the stored M and its scale (the
// sign_pack arithmetic), over the whole unit; a few blocks per unit, which
// return at once for an unflagged one.
void launch_pack_fixup(const MomBatch &b, bool m_bf16, hipStream_t s);

// ---------------------------------------------------------------------------
// Newton-Schulz GEMMs (matrix cores).
// ---------------------------------------------------------------------------
// EPI_FINAL: U (fp32) and/or packed signs; EPI_FINAL_I8: U (fp32) and/or
// int8 signs (the int8 payload); EPI_WUPD: W <- fmaf(-eta, U, W).
enum NsEpilogue { EPI_GRAM = 0, EPI_ITER = 1, EPI_FINAL = 2, EPI_WUPD = 3, EPI_FINAL_I8 = 4 };

struct NsMat {
    const void *x;      // current iterate, worker 0; worker stride n (ns dtype)
    void *a;            // Gram buffer, worker 0; worker stride r*r (ns dtype)
    void *out;          // EPI_ITER: next iterate (ns dtype); EPI_FINAL: U fp32 or
                        // nullptr; EPI_WUPD: W fp32, W <- fmaf(-eta, U, W) (no worker
                        // stride: one worker)
    uint64_t *packed;   // EPI_FINAL fused sign+pack target or nullptr
    float *u_out;       // EPI_WUPD: U (fp32) as well, or nullptr (one worker)
    int8_t *i8;         // EPI_FINAL_I8: int8 signs [Mw][n]
    int32_t R, C;
    int32_t tile_begin;  // first tile of this matrix within one worker's tiles
    int32_t tiles_per_worker;
    int32_t unit_begin;  // index of (this matrix, worker 0) in scales
    int32_t split;       // split Gram: k chunks per tile (partial tiles in out)
};

// Tiles are numbered worker-major: worker w's tiles of every matrix of the
// launch, then worker w + 1's. The XCDs take contiguous ranges of tiles, so
// each receives the same mix of matrices.
struct NsBatch {
    NsMat mat[kMaxMatsPerLaunch];
    int32_t nmat;
    int32_t workers;
    int32_t total_tiles;
    int32_t tiles_per_worker_all;  // tiles of one worker over all matrices
    int32_t use_scales;   // iteration 0: fold s^2 (Gram) and s (product) in
    const float2 *scales; // per unit {s, s^2}; must cover every unit of the batch even
                          // when use_scales = 0 (the kernels read it unconditionally)
    float eta;            // EPI_WUPD step size
    int32_t id_scaled;    // first product under spectral scaling: A is the unscaled Gram
                          // matrix; the identity coefficient is -3 / s^2 and the
                          // accumulators are multiplied by s^2 before the epilogue
    Starts starts;         // first block (tile) of each matrix
};

// Output tiles of the Newton-Schulz GEMMs: the Gram's are kNsTileM square,
// the product's kNsTileM rows by kNsProdTileN columns.
constexpr int kNsTileM = 256;
constexpr int kNsProdTileN = 256;

// Tiles one worker of an R x C matrix needs.
inline int32_t ns_gram_tiles(int64_t R, int64_t C) {
    int64_t r = R < C ? R : C;
    int64_t t = (r + kNsTileM - 1) / kNsTileM;
    return (int32_t)(t * (t + 1) / 2);
}
// Tiles one worker of an R x C matrix takes in the persistent Gram walk, which
// covers the upper triangle in 64 x 64 blocks: one tile per pair of distinct
// 256-row groups, and two tiles per three groups for the blocks inside a group
// (ten per group: five waves of two blocks), one for each group left over.
inline int32_t ns_gram_walk_tiles(int64_t R, int64_t C) {
    int64_t r = R < C ? R : C;
    int64_t g = (r + kNsTileM - 1) / kNsTileM;
    return (int32_t)(g * (g - 1) / 2 + 2 * (g / 3) + g % 3);
}
inline int32_t ns_product_tiles(int64_t R, int64_t C) {
    // output rows = R, cols = C in both orientations
    return (int32_t)(((R + kNsTileM - 1) / kNsTileM) * ((C + kNsProdTileN - 1) / kNsProdTileN));
}

// ns_bf16 selects the operand storage type; epi the epilogue.
void launch_ns_gram(const NsBatch &b, bool ns_bf16, hipStream_t s);
// The Gram matrices of few-tile matrices with a long k range, in two
// launches: launch_ns_gram_split (tiles_per_worker = Gram tiles x split, one
// block per k chunk of a tile) writes unscaled fp32 partial tiles to each
// matrix's out ([Mw][Gram tiles][split][256][256]); launch_gram_reduce
// (tiles_per_worker = Gram tiles x 16, one block per 16 rows of a tile)
// adds them in chunk order, applies s^2 when use_scales, and stores A and its
// mirror.
constexpr int kGramReduceParts = 16;  // reduce blocks per Gram tile (16 rows each)
void launch_ns_gram_split(const NsBatch &b, bool ns_bf16, hipStream_t s);
void launch_gram_reduce(const NsBatch &b, bool ns_bf16, hipStream_t s);
// K chunks per Gram tile of an R x C matrix (0: not split, the Gram kernel
// stores A itself): for matrices with at most 3 Gram tiles per worker, so
// that the few tiles spread over more blocks. A chunk is a quarter of the k
// slices (BK k each), but at least 4 and at most 24 slices; at most 16
// chunks, and a single chunk means no split. A function of the shape alone,
// so that results do not depend on which matrices share a launch.
inline int32_t ns_gram_split(int64_t R, int64_t C, bool ns_bf16) {
    if (ns_gram_tiles(R, C) > 3) return 0;
    const int64_t c = R > C ? R : C, bk = ns_bf16 ? 32 : 16;
    const int64_t slices = (c + bk - 1) / bk;
    const int64_t len = slices / 4 < 4 ? 4 : (slices / 4 > 24 ? 24 : slices / 4);
    const int64_t s = (slices + len - 1) / len;
    return (int32_t)(s < 2 ? 0 : (s > 16 ? 16 : s));
}
// The bf16 Gram matrices as a persistent walk: grid_blocks workgroups (one
// per CU, at most b.total_tiles) walk the tiles of wide and tall matrices in
// one launch. Tiles are numbered matrix-major: tile_begin of matrix i is the
// number of tiles (all workers) of matrices 0 .. i - 1, tiles_per_worker its
// Gram tiles of one worker; the matrices are listed longest k first. Every
// matrix has C and min(R, C) multiples of 8, each worker's matrix is under
// 2 GiB, and ceil(max(R, C) / 32) is a multiple of 4 and at least 8.
void launch_ns_gram_walk(const NsBatch &b, int grid_blocks, hipStream_t s);
void launch_ns_product(const NsBatch &b, bool ns_bf16, NsEpilogue epi, hipStream_t s);
// A product with bf16 operands as a persistent tile walk: grid_blocks
// workgroups (one per CU, at most b.total_tiles) walk the tiles with the
// load pipeline running across tile boundaries. Every matrix of b is tall
// (R > C) or every one wide; C and min(R, C) are multiples of 8, each
// worker's matrix is under 2 GiB, and ceil(min(R, C) / 32) is a multiple of
// 4 and at least 12. epi: EPI_FINAL (packed set, out null, C % 64 == 0),
// EPI_FINAL_I8 (i8 set, out null, C % 64 == 0) or EPI_ITER (out: the next
// iterate, as for launch_ns_product).
void launch_ns_product_pack(const NsBatch &b, bool tall, NsEpilogue epi, int grid_blocks, hipStream_t s);

// ---------------------------------------------------------------------------
// Sign + pack of a stored U, and scale + sign + pack for k = 0.
// ---------------------------------------------------------------------------
struct PackMat {
    const void *u;       // [Mw][n]
    uint64_t *packed;    // [Mw][words]
    float *u_out;        // optional fp32 copy of the scaled value (k = 0 path)
    int8_t *i8;          // int8 signs [Mw][n] instead of packed bits, or nullptr
    int64_t n;
    int32_t block_begin;
    int32_t blocks_per_worker;
    int32_t unit_begin;
    int32_t pad_;
};

struct PackBatch {
    PackMat mat[kMaxMatsPerLaunch];
    int32_t nmat;
    int32_t workers;
    int32_t total_blocks;
    int32_t u_bf16;
    const float2 *scales;  // nullptr: plain sign of u; else sign of s*u
    Starts starts;         // first block (tile) of each matrix
};

// 256 threads, each packing pack_chunks_per_thread chunks of 8 entries (one
// byte of packed words each): 8 for bf16 U (16 bytes per chunk), 4 for fp32
// U (32 bytes), so 128 bytes of U per thread are in flight together.
constexpr int pack_chunks_per_thread(bool u_bf16) { return u_bf16 ? 8 : 4; }
constexpr int pack_words_per_block(bool u_bf16) { return 256 * pack_chunks_per_thread(u_bf16) / 8; }

void launch_sign_pack(const PackBatch &b, hipStream_t s);

// ---------------------------------------------------------------------------
// Majority vote + update.
// ---------------------------------------------------------------------------
constexpr int kVoteWordsPerWave = 64;                     // 4096 entries
constexpr int kVoteWordsPerBlock = 4 * kVoteWordsPerWave;  // 256 threads

struct VoteMat {
    const uint64_t *packed;  // [Mw][words]
    float *w;                // [n] or nullptr
    int8_t *vote;            // [n] or nullptr
    void *v_ns;              // [n] vote written in the NS storage type, or nullptr
    uint32_t *nnz;           // nonzero count of the vote (added to), or nullptr
    int64_t n;
    int32_t block_begin;
    int32_t pad_;
};

struct VoteBatch {
    VoteMat mat[kMaxMatsPerLaunch];
    int32_t nmat;
    int32_t workers;
    int32_t total_blocks;
    int32_t v_ns_bf16;
    float eta;
    int32_t pad_;
    Starts starts;         // first block (tile) of each matrix
};

void launch_vote_update(const VoteBatch &b, hipStream_t s);

// Int8 payload: signs of a flat [workers][n] array, and the vote as the sign
// of the integer sum over workers with the update of W.
int64_t sign_int8_blocks(int64_t total);
void launch_sign_int8(const void *u, bool u_bf16, int64_t total, int8_t *signs, hipStream_t s);
struct VoteI8Mat {
    const int8_t *signs;  // [Mw][n]
    float *w;             // [n] or nullptr
    int8_t *vote;         // [n] or nullptr
    int64_t n;
    int32_t block_begin;
    int32_t vec;          // n % 16 == 0: 16-byte loads and stores
};

struct VoteI8Batch {
    VoteI8Mat mat[kMaxMatsPerLaunch];
    int32_t nmat;
    int32_t workers;
    int32_t total_blocks;
    float eta;
    Starts starts;  // first block of each matrix
};

int64_t vote_int8_blocks(int64_t n);
void launch_vote_update_int8(const VoteI8Batch &b, hipStream_t s);

// ---------------------------------------------------------------------------
// Spectral normalisation: power iteration on each worker's Gram matrix.
// ---------------------------------------------------------------------------
constexpr int kPowRowsPerBlock = 32;  // rows of A per power-step block (8 per wave)
constexpr int kMaxPowR = 8192;         // the power vector of a Gram lives in LDS
// The one-workgroup power iteration: two 16-byte column chunks per lane at most.
inline int max_fused_pow_r(bool bf16) { return bf16 ? 1016 : 504; }  // (r + 8) / EPC <= 128

struct PowMat {
    const void *a;   // worker 0's Gram matrix [r][r] (ns type); worker stride r*r
    float *w;        // [2][Mw][r] power vectors (ping-pong by step parity)
    double *part;    // [2][Mw][bpw] block sums of squares of w
    int32_t r;
    int32_t bpw;     // blocks per worker of the launch
    int32_t unit_begin;
    int32_t pad_;
};

struct PowBatch {
    PowMat mat[kMaxMatsPerLaunch];
    int32_t nmat;
    int32_t workers;
    int32_t total_blocks;
    int32_t it;      // power step (power_step), or the last step (finalize)
    float2 *scales;  // per unit: {s, s^2}
    Starts starts;   // first block of each matrix
};

int32_t power_blocks_per_worker(int64_t r);
void launch_power_step(const PowBatch &b, bool bf16, hipStream_t s);
void launch_power_finalize(const PowBatch &b, hipStream_t s);
// All it = p power steps and the scales with one workgroup per (matrix,
// worker); every r % 8 == 0 and r <= max_fused_pow_r.
void launch_power_fused(const PowBatch &b, bool bf16, hipStream_t s);

// Post-vote polar step helpers.
void launch_zero_u32(uint32_t *p, int32_t count, hipStream_t s);
// scales[unit_begin + i] = {1/sqrt(nnz[i]), 1/nnz[i]} (0 when nnz = 0)
void launch_nnz_scales(const uint32_t *nnz, int32_t count, float2 *scales, hipStream_t s);

}  // namespace sm

namespace sm {
// Launch descriptors travel as kernel arguments (4 KiB at most).
static_assert(sizeof(MomBatch) <= 4000 && sizeof(NsBatch) <= 4000 && sizeof(PackBatch) <= 4000 &&
                  sizeof(VoteBatch) <= 4000 && sizeof(PowBatch) <= 4000 && sizeof(VoteI8Batch) <= 4000,
              "launch descriptor exceeds the kernel argument space");
}  // namespace sm
