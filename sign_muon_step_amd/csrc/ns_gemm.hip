// ns_gemm.hip -- Newton-Schulz matrix products of the Sign-Muon step on the
// gfx950 matrix cores.
//
// Method: "SignMuon: Communication-Efficient Distributed Muon Optimization"
// (gist.science, paper 2605.16311, technical summary), §2 "Core mechanism"
// and "Algorithmic flow" step 1: each worker approximates the polar factor of
// its momentum by Newton-Schulz iterations. The summary prints no
// coefficients; the cubic X <- 1.5 X - 0.5 (X X^T) X is used, on the smaller
// Gram matrix (X X^T when R <= C, X^T X and X <- 1.5 X - 0.5 X (X^T X) when
// R > C).
//
// One iteration is two launches over every (matrix, worker) of the step:
//   gram:    A = s2 * Y Y^T  (Y = X, or X^T for a tall X), r x r, symmetric:
//            only tiles on or above the diagonal are computed and each is
//            stored twice (itself and its mirror).
//   product: X' = alpha X + gamma * (A X)   (wide)   or
//            X' = alpha X + gamma * (X A)   (tall),
//            alpha = 1.5 s, gamma = -0.5 s; s folds the Frobenius scaling of
//            the first iteration in (s = 1 afterwards).
// The last product's epilogue either stores fp32 U and/or takes the sign of
// each entry and packs 64 signs per uint64 word straight from the wave64
// ballot of the accumulator registers (summary §2 "Algorithmic flow", steps
// 2-3), or (post-vote polar step) applies W <- fmaf(-eta, Y, W).
//
// Every GEMM is C[m][n] = sum_k P[m][k] Q[n][k] on a 256 x 256 output tile
// with 4 waves of 128 x 128. Operands are staged through LDS in a [row][k]
// layout, 128 bytes of k per row (64 bf16 or 32 fp32), 16-byte chunks
// XOR-swizzled by row so that both the MFMA fragment reads and the staging
// writes spread over all banks. An operand whose k index is the strided one
// in memory (X in a wide product, both Gram operands of a tall X) is loaded
// as 8 x 8 (bf16) or 4 x 4 (fp32) blocks and transposed in registers before
// the LDS write.
#include "sm_internal.h"

namespace sm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kRowBytes = 128;
constexpr int kOpBytes = kNsTileM * kRowBytes;  // 32 KiB per operand per stage
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kLdsBytes = 2 * kStageBytes;      // double-buffered: 128 KiB

template <bool BF16> struct Elem;
template <> struct Elem<true> {
    using T = uint16_t;
    static constexpr int BK = 64;   // k per LDS row
    static constexpr int EPC = 8;   // elements per 16-byte chunk
};
template <> struct Elem<false> {
    using T = float;
    static constexpr int BK = 32;
    static constexpr int EPC = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <bool BF16>
__device__ __forceinline__ float load_val(const void *p, int64_t i) {
    if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_val(void *p, int64_t i, float v) {
    if (BF16)
        static_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
    else
        static_cast<float *>(p)[i] = v;
}

// Byte offset of (row, 16-byte chunk) inside one operand's LDS stage.
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
    return (uint32_t)(row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4));
}

// Blocks go to the 8 XCDs round-robin; give each XCD a contiguous run of
// logical tiles so that the tiles of one (matrix, worker) share an L2.
__device__ __forceinline__ int xcd_remap(int b, int g) {
    const int q = g >> 3, rem = g & 7, x = b & 7, p = b >> 3;
    return x * q + (x < rem ? x : rem) + p;
}

// One GEMM operand as seen by a tile: element (mn, k) of the operand, for
// mn in [0, rows) relative to the tile origin, is at
//   base[mn * ld + k]  (k-contiguous)   or   base[k * ld + mn]  (mn-contiguous).
struct Operand {
    const char *base;
    int64_t ld;
    int rows;  // valid rows from the tile origin (may exceed 256)
    int K;
    bool vec;  // 16-byte chunks: every chunk lies wholly inside or outside the operand
};

// Buffer offset beyond every extent: a load there returns zeros.
constexpr uint32_t kOOB = 0x80000000u;

template <bool BF16, bool KC>
__device__ __forceinline__ int64_t operand_extent(const Operand &op) {
    const int64_t sz = sizeof(typename Elem<BF16>::T);
    return KC ? ((int64_t)(op.rows - 1) * op.ld + op.K) * sz : ((int64_t)(op.K - 1) * op.ld + op.rows) * sz;
}

// Stages one operand's BK-wide k-slice (256 rows) from global memory to LDS.
// Loads go through a buffer resource spanning the operand: a chunk outside it
// reads the out-of-bounds offset and comes back as zeros, so edge tiles need
// no branches. KC: k-contiguous rows, 8 chunks of 16 bytes per 128-byte LDS
// row. !KC: 8 x 8 (bf16) or 4 x 4 (fp32) blocks transposed in registers.
template <bool BF16, bool KC>
struct Stager {
    using E = Elem<BF16>;
    using T = typename E::T;
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t off[8];   // byte offset of each chunk at k = 0
    int kofs[8];       // k of each chunk relative to the slice start
    uint32_t valid;    // bit i: chunk i's rows lie inside the operand
    uint32_t kstep;    // bytes per BK of k
    int K;
    uint4 st[8];

    __device__ __forceinline__ void init(const Operand &op) {
        const int tid = threadIdx.x;
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(op.base), (short)0,
                                                 (int)operand_extent<BF16, KC>(op), 0x00020000);
        K = op.K;
        valid = 0;
        const uint32_t sz = sizeof(T);
        if (KC) {
            const int c = tid & 7;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = (tid >> 3) + 32 * i;
                off[i] = (uint32_t)(row * op.ld + c * E::EPC) * sz;
                kofs[i] = c * E::EPC;
                valid |= (uint32_t)(row < op.rows) << i;
            }
            kstep = E::BK * sz;
        } else if (BF16) {
            const int kb = tid >> 5, mb = tid & 31;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                off[j] = (uint32_t)((kb * 8 + j) * op.ld + mb * 8) * sz;
                kofs[j] = kb * 8 + j;
                valid |= (uint32_t)(mb * 8 < op.rows) << j;
            }
            kstep = (uint32_t)(E::BK * op.ld) * sz;
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = tid + kThreads * i;
                const int kb = q >> 6, mb = q & 63;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    off[4 * i + j] = (uint32_t)((kb * 4 + j) * op.ld + mb * 4) * sz;
                    kofs[4 * i + j] = kb * 4 + j;
                    valid |= (uint32_t)(mb * 4 < op.rows) << (4 * i + j);
                }
            }
            kstep = (uint32_t)(E::BK * op.ld) * sz;
        }
    }

    __device__ __forceinline__ void load(int kt) {
        const int k0 = kt * E::BK;
        const uint32_t kb = (uint32_t)kt * kstep;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = ((valid >> i) & 1u) && k0 + kofs[i] < K;
            const uint32_t o = ok ? off[i] + kb : kOOB;
            st[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)o, 0, 0));
        }
    }

    __device__ __forceinline__ void store(char *lds) const {
        const int tid = threadIdx.x;
        if (KC) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + kThreads * i;
                *reinterpret_cast<uint4 *>(lds + lds_off(q >> 3, q & 7)) = st[i];
            }
        } else if (BF16) {
            // Transpose the 8 (k) x 8 (mn) block of 16-bit values: output row
            // e (mn = 8 mb + e) gathers element e of each of the 8 k rows.
            const int kb = tid >> 5, mb = tid & 31;
            uint32_t in[8][4];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                in[j][0] = st[j].x; in[j][1] = st[j].y; in[j][2] = st[j].z; in[j][3] = st[j].w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t o[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t lo = in[2 * d][e >> 1], hi = in[2 * d + 1][e >> 1];
                    o[d] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                *reinterpret_cast<uint4 *>(lds + lds_off(mb * 8 + e, kb)) =
                    make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = tid + kThreads * i;
                const int kb = q >> 6, mb = q & 63;
                const uint4 *r = &st[4 * i];
                *reinterpret_cast<uint4 *>(lds + lds_off(mb * 4 + 0, kb)) = make_uint4(r[0].x, r[1].x, r[2].x, r[3].x);
                *reinterpret_cast<uint4 *>(lds + lds_off(mb * 4 + 1, kb)) = make_uint4(r[0].y, r[1].y, r[2].y, r[3].y);
                *reinterpret_cast<uint4 *>(lds + lds_off(mb * 4 + 2, kb)) = make_uint4(r[0].z, r[1].z, r[2].z, r[3].z);
                *reinterpret_cast<uint4 *>(lds + lds_off(mb * 4 + 3, kb)) = make_uint4(r[0].w, r[1].w, r[2].w, r[3].w);
            }
        }
    }
};

// Slow staging for shapes whose rows break 16-byte chunk alignment: element
// by element with bounds, written to LDS in the same layout.
template <bool BF16, bool KC>
struct SlowStager {
    using E = Elem<BF16>;
    using T = typename E::T;
    const T *p;
    int64_t ld;
    int rows, K;

    __device__ __forceinline__ void init(const Operand &op) {
        p = reinterpret_cast<const T *>(op.base);
        ld = op.ld;
        rows = op.rows;
        K = op.K;
    }

    __device__ __forceinline__ T at(int mn, int k) const {
        if (mn >= rows || k >= K) return (T)0;
        return KC ? p[(int64_t)mn * ld + k] : p[(int64_t)k * ld + mn];
    }

    // Load straight into LDS: thread t fills rows t (and chunks of all k).
    __device__ __forceinline__ void load_store(int kt, char *lds) const {
        const int k0 = kt * E::BK;
        for (int q = threadIdx.x; q < kNsTileM * 8; q += kThreads) {
            const int row = q >> 3, c = q & 7;
            T v[E::EPC];
#pragma unroll
            for (int e = 0; e < E::EPC; ++e) v[e] = at(row, k0 + c * E::EPC + e);
            uint4 u;
            __builtin_memcpy(&u, v, 16);
            *reinterpret_cast<uint4 *>(lds + lds_off(row, c)) = u;
        }
    }
};

// acc[f][g]: 32 x 32 block (f along m, g along n) of the wave's 128 x 128.
// MFMA 32x32 layout: lane l holds column (l & 31) and, in register r, row
// 8*(r/4) + 4*(l/32) + (r%4) of the block. The fragments of the next k16
// step are read from LDS while the current step's 16 MFMAs run.
template <bool BF16>
__device__ __forceinline__ void mma_stage(const char *lds_p, const char *lds_q, int wm0, int wn0,
                                          f32x16_t (&acc)[4][4]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int lrow = lane & 31, half = lane >> 5;
    if (BF16) {
        bf16x8_t pa[2][4], qa[2][4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            pa[0][f] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(lds_p + lds_off(wm0 + f * 32 + lrow, half)));
            qa[0][f] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(lds_q + lds_off(wn0 + f * 32 + lrow, half)));
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int cb = kk & 1, nb = cb ^ 1;
            if (kk < 3) {
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    pa[nb][f] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(lds_p + lds_off(wm0 + f * 32 + lrow, 2 * (kk + 1) + half)));
                    qa[nb][f] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(lds_q + lds_off(wn0 + f * 32 + lrow, 2 * (kk + 1) + half)));
                }
            }
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[cb][f], qa[cb][g], acc[f][g], 0, 0, 0);
        }
        // Schedule: the first step's 8 reads, then each step's 16 MFMAs with
        // the next step's 8 reads slotted between them.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    } else {
        // fp32: each lane reads 4 consecutive k of a chunk; MFMA step s uses
        // element s, so one instruction contracts k = 8c + s (lanes 0-31) and
        // 8c + 4 + s (lanes 32-63). Both operands use the same mapping.
        f32x4_t pa[2][4], qa[2][4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            pa[0][f] = *reinterpret_cast<const f32x4_t *>(lds_p + lds_off(wm0 + f * 32 + lrow, half));
            qa[0][f] = *reinterpret_cast<const f32x4_t *>(lds_q + lds_off(wn0 + f * 32 + lrow, half));
        }
#pragma unroll
        for (int cp = 0; cp < 4; ++cp) {
            const int cb = cp & 1, nb = cb ^ 1;
            if (cp < 3) {
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    pa[nb][f] = *reinterpret_cast<const f32x4_t *>(lds_p + lds_off(wm0 + f * 32 + lrow, 2 * (cp + 1) + half));
                    qa[nb][f] = *reinterpret_cast<const f32x4_t *>(lds_q + lds_off(wn0 + f * 32 + lrow, 2 * (cp + 1) + half));
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int f = 0; f < 4; ++f)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x2f32(pa[cb][f][s], qa[cb][g][s], acc[f][g], 0, 0, 0);
        }
    }
}

// Full K loop of one tile, double-buffered through LDS: the next slice's
// global loads are in flight while the current slice's MFMAs run.
template <bool BF16, bool PKC, bool QKC>
__device__ __forceinline__ void tile_mainloop(const Operand &P, const Operand &Q, char *smem,
                                              f32x16_t (&acc)[4][4]) {
    using E = Elem<BF16>;
    const int wid = threadIdx.x / kWave;
    const int wm0 = (wid >> 1) * 128, wn0 = (wid & 1) * 128;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;
    const int kt_n = (P.K + E::BK - 1) / E::BK;
    if (P.vec && Q.vec) {
        Stager<BF16, PKC> sp;
        Stager<BF16, QKC> sq;
        sp.init(P);
        sq.init(Q);
        sp.load(0);
        sq.load(0);
        sp.store(smem);
        sq.store(smem + kOpBytes);
        __syncthreads();
        for (int kt = 0; kt < kt_n; ++kt) {
            char *cur = smem + (kt & 1) * kStageBytes;
            char *nxt = smem + ((kt + 1) & 1) * kStageBytes;
            const bool more = kt + 1 < kt_n;
            if (more) {
                sp.load(kt + 1);
                sq.load(kt + 1);
            }
            mma_stage<BF16>(cur, cur + kOpBytes, wm0, wn0, acc);
            if (more) {
                sp.store(nxt);
                sq.store(nxt + kOpBytes);
            }
            __syncthreads();
        }
    } else {
        SlowStager<BF16, PKC> sp;
        SlowStager<BF16, QKC> sq;
        sp.init(P);
        sq.init(Q);
        for (int kt = 0; kt < kt_n; ++kt) {
            sp.load_store(kt, smem);
            sq.load_store(kt, smem + kOpBytes);
            __syncthreads();
            mma_stage<BF16>(smem, smem + kOpBytes, wm0, wn0, acc);
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int find_ns_mat(const NsBatch &b, int t) {
    int mi = 0;
    while (mi + 1 < b.nmat && t >= b.mat[mi + 1].tile_begin) ++mi;
    return mi;
}

// ---------------------------------------------------------------------------
// Epilogue helpers. A wave stages 32 rows x 128 columns of fp32 in LDS
// (row stride kStageStride floats) to turn the MFMA register layout into
// row-major 4-column pieces.
// ---------------------------------------------------------------------------
constexpr int kStageStride = 132;
static_assert(4 * 32 * kStageStride * 4 <= kLdsBytes, "epilogue stage exceeds LDS");

__device__ __forceinline__ void stage_rows(const f32x16_t (&acc)[4][4], int f, float *stage,
                                           float scale) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
            stage[row * kStageStride + 32 * g + (lane & 31)] = acc[f][g][rr] * scale;
        }
}

// 4 consecutive values at element index idx. FAST: one vector access (the
// caller guarantees bounds and alignment); otherwise element by element,
// valid while row_ok and t < cols_left.
template <bool BF16, bool FAST>
__device__ __forceinline__ void load4(const void *p, int64_t idx, float (&v)[4], bool row_ok,
                                      int cols_left) {
    if (FAST) {
        if (BF16) {
            const uint2 h = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
            v[0] = bf16_bits_to_f32(h.x & 0xffffu);
            v[1] = bf16_bits_to_f32(h.x >> 16);
            v[2] = bf16_bits_to_f32(h.y & 0xffffu);
            v[3] = bf16_bits_to_f32(h.y >> 16);
        } else {
            const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (row_ok && t < cols_left) ? load_val<BF16>(p, idx + t) : 0.f;
    }
}

template <bool BF16, bool FAST>
__device__ __forceinline__ void store4(void *p, int64_t idx, const float (&v)[4], bool row_ok,
                                       int cols_left) {
    if (FAST) {
        if (BF16) {
            const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
            const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p) + idx) = make_uint2(lo, hi);
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(p) + idx) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (row_ok && t < cols_left) store_val<BF16>(p, idx + t, v[t]);
    }
}

// ---------------------------------------------------------------------------
// Gram tile: A = scale * Y Y^T on the tile (ti <= tj) of the r x r result.
// Each orientation is its own instantiation so that the accumulators stay in
// registers from the main loop through the epilogue.
// ---------------------------------------------------------------------------
template <bool BF16, bool FAST>
__device__ __forceinline__ void gram_epilogue(f32x16_t (&acc)[4][4], char *smem, int ti, int tj,
                                              int r, float scale, void *a) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int m0 = ti * kNsTileM + (wid >> 1) * 128, n0 = tj * kNsTileN + (wid & 1) * 128;
    float *stage = reinterpret_cast<float *>(smem) + wid * 32 * kStageStride;
    const bool mirror = ti < tj;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        stage_rows(acc, f, stage, scale);
        // Mirror (below the diagonal) straight from the registers: lane holds
        // 4 consecutive rows of one column, i.e. 4 consecutive entries of the
        // mirrored row.
        if (mirror) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int gi = m0 + f * 32 + 8 * q + 4 * (lane >> 5);
                    const int gj = n0 + 32 * g + (lane & 31);
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = acc[f][g][4 * q + t] * scale;
                    store4<BF16, FAST>(a, (int64_t)gj * r + gi, v, gj < r, r - gi);
                }
        }
        __syncthreads();
        // Direct tile, row-major: 4 columns per lane, 2 rows per instruction.
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int row = it * 2 + (lane >> 5), c4 = (lane & 31) * 4;
            const int gi = m0 + f * 32 + row, gj = n0 + c4;
            const float4 v4 = *reinterpret_cast<const float4 *>(stage + row * kStageStride + c4);
            float v[4] = {v4.x, v4.y, v4.z, v4.w};
            store4<BF16, FAST>(a, (int64_t)gi * r + gj, v, gi < r, r - gj);
        }
        __syncthreads();
    }
}

template <bool BF16, bool KC>
__device__ __forceinline__ void gram_tile(const Operand &P, const Operand &Q, char *smem, int ti,
                                          int tj, int r, float scale, void *a) {
    f32x16_t acc[4][4];
    tile_mainloop<BF16, KC, KC>(P, Q, smem, acc);
    const bool fast = P.vec && (r % Elem<BF16>::EPC) == 0 && (ti + 1) * kNsTileM <= r &&
                      (tj + 1) * kNsTileN <= r;
    if (fast)
        gram_epilogue<BF16, true>(acc, smem, ti, tj, r, scale, a);
    else
        gram_epilogue<BF16, false>(acc, smem, ti, tj, r, scale, a);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ns_gram_kernel(NsBatch b) {
    using T = typename Elem<BF16>::T;
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    const int lt = xcd_remap(blockIdx.x, gridDim.x);
    const NsMat &M = b.mat[find_ns_mat(b, lt)];
    const int local = lt - M.tile_begin;
    const int w = local / M.tiles_per_worker;
    int t = local - w * M.tiles_per_worker;
    const bool wide = M.R <= M.C;
    const int r = wide ? M.R : M.C, c = wide ? M.C : M.R;
    const int T_ = (r + kNsTileM - 1) / kNsTileM;
    int ti = 0;
    while (t >= T_ - ti) {
        t -= T_ - ti;
        ++ti;
    }
    const int tj = ti + t;
    const int64_t n = (int64_t)M.R * M.C;
    const char *y = static_cast<const char *>(M.x) + (int64_t)w * n * (int64_t)sizeof(T);
    // Buffer offsets are 32-bit: the 16-byte path needs the matrix under 2 GiB.
    const bool vec = (M.C % Elem<BF16>::EPC) == 0 && n * (int64_t)sizeof(T) < ((int64_t)1 << 31);
    const float scale = b.use_scales ? b.scales[M.unit_begin + w].y : 1.0f;
    void *a = static_cast<char *>(M.a) + (int64_t)w * r * r * (int64_t)sizeof(T);
    if (wide) {
        // Y = X (r x c, k-contiguous rows)
        Operand P{y + (int64_t)ti * kNsTileM * M.C * (int64_t)sizeof(T), M.C, r - ti * kNsTileM, c, vec};
        Operand Q{y + (int64_t)tj * kNsTileM * M.C * (int64_t)sizeof(T), M.C, r - tj * kNsTileM, c, vec};
        gram_tile<BF16, true>(P, Q, smem, ti, tj, r, scale, a);
    } else {
        // Y = X^T: element (i, k) of Y is X[k][i]: mn-contiguous, ld = C
        Operand P{y + (int64_t)ti * kNsTileM * (int64_t)sizeof(T), M.C, r - ti * kNsTileM, c, vec};
        Operand Q{y + (int64_t)tj * kNsTileM * (int64_t)sizeof(T), M.C, r - tj * kNsTileM, c, vec};
        gram_tile<BF16, false>(P, Q, smem, ti, tj, r, scale, a);
    }
}

// ---------------------------------------------------------------------------
// Product tile: X' = alpha X + gamma (A X) or (X A), with the epilogue EPI.
// ---------------------------------------------------------------------------
struct ProductArgs {
    const char *x;   // this worker's iterate
    void *out;       // this worker's output (U / next iterate) or W
    uint64_t *pk;    // this worker's packed words or nullptr
    int R, C, ti, tj;
    float alpha, gamma, eta;
};

// Epilogue of the product, 32 rows of the wave's 128 x 128 at a time through
// LDS: u = alpha * X + gamma * acc row-major (4 columns per lane), stored as
// EPI asks; for the fused sign + pack, u goes back to LDS and each packed word
// is the ballot of 64 consecutive columns of one row (needs C % 64 == 0).
template <bool BF16, int EPI, bool FAST>
__device__ __forceinline__ void product_epilogue(const ProductArgs &pa, f32x16_t (&acc)[4][4],
                                                 char *smem) {
    const int R = pa.R, C = pa.C;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int m0 = pa.ti * kNsTileM + (wid >> 1) * 128, n0 = pa.tj * kNsTileN + (wid & 1) * 128;
    float *stage = reinterpret_cast<float *>(smem) + wid * 32 * kStageStride;
    const bool want_out = EPI == EPI_ITER || EPI == EPI_WUPD || (EPI == EPI_FINAL && pa.out);
    const bool want_pack = EPI == EPI_FINAL && pa.pk;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        stage_rows(acc, f, stage, 1.0f);
        __syncthreads();
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int row = it * 2 + (lane >> 5), c4 = (lane & 31) * 4;
            const int gm = m0 + f * 32 + row, gn = n0 + c4;
            const int64_t idx = (int64_t)gm * C + gn;
            float *sp = stage + row * kStageStride + c4;
            const float4 v4 = *reinterpret_cast<const float4 *>(sp);
            const float v[4] = {v4.x, v4.y, v4.z, v4.w};
            float xv[4];
            load4<BF16, FAST>(pa.x, idx, xv, gm < R, C - gn);
            float u[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool ok = FAST || (gm < R && gn + t < C);
                u[t] = ok ? __builtin_fmaf(pa.gamma, v[t], pa.alpha * xv[t]) : 0.f;
            }
            if (want_out) {
                if (EPI == EPI_ITER) {
                    store4<BF16, FAST>(pa.out, idx, u, gm < R, C - gn);
                } else if (EPI == EPI_FINAL) {
                    store4<false, FAST>(pa.out, idx, u, gm < R, C - gn);
                } else {
                    float w[4];
                    load4<false, FAST>(pa.out, idx, w, gm < R, C - gn);
#pragma unroll
                    for (int t = 0; t < 4; ++t) w[t] = __builtin_fmaf(-pa.eta, u[t], w[t]);
                    store4<false, FAST>(pa.out, idx, w, gm < R, C - gn);
                }
            }
            if (want_pack) *reinterpret_cast<float4 *>(sp) = make_float4(u[0], u[1], u[2], u[3]);
        }
        if (want_pack) {
            __syncthreads();
            uint64_t mine = 0;
#pragma unroll 8
            for (int q = 0; q < 64; ++q) {
                const float v = stage[(q >> 1) * kStageStride + 64 * (q & 1) + lane];
                const uint64_t bal = __ballot(v >= 0.f);
                if (lane == q) mine = bal;
            }
            const int gm = m0 + f * 32 + (lane >> 1), gn0 = n0 + 64 * (lane & 1);
            if (gm < R && gn0 < C) pa.pk[((int64_t)gm * C + gn0) >> 6] = mine;
        }
        __syncthreads();
    }
}

template <bool BF16, bool QKC, int EPI>
__device__ __forceinline__ void product_tile(const Operand &P, const Operand &Q, char *smem,
                                             const ProductArgs &pa) {
    f32x16_t acc[4][4];
    tile_mainloop<BF16, true, QKC>(P, Q, smem, acc);
    const bool fast = P.vec && (pa.ti + 1) * kNsTileM <= pa.R && (pa.tj + 1) * kNsTileN <= pa.C;
    if (fast)
        product_epilogue<BF16, EPI, true>(pa, acc, smem);
    else
        product_epilogue<BF16, EPI, false>(pa, acc, smem);
}

template <bool BF16, int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ns_product_kernel(NsBatch b) {
    using T = typename Elem<BF16>::T;
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    const int lt = xcd_remap(blockIdx.x, gridDim.x);
    const NsMat &M = b.mat[find_ns_mat(b, lt)];
    const int local = lt - M.tile_begin;
    const int w = local / M.tiles_per_worker;
    const int t = local - w * M.tiles_per_worker;
    const int R = M.R, C = M.C;
    const bool wide = R <= C;
    const int r = wide ? R : C;
    const int tiles_n = (C + kNsTileN - 1) / kNsTileN;
    const int ti = t / tiles_n, tj = t - ti * tiles_n;
    const int64_t n = (int64_t)R * C;
    const char *x = static_cast<const char *>(M.x) + (int64_t)w * n * (int64_t)sizeof(T);
    const char *a = static_cast<const char *>(M.a) + (int64_t)w * r * r * (int64_t)sizeof(T);
    // Buffer offsets are 32-bit: the 16-byte path needs the matrix under 2 GiB.
    const bool vec = (C % Elem<BF16>::EPC) == 0 && (r % Elem<BF16>::EPC) == 0 &&
                     n * (int64_t)sizeof(T) < ((int64_t)1 << 31);

    ProductArgs pa;
    pa.x = x;
    pa.R = R;
    pa.C = C;
    pa.ti = ti;
    pa.tj = tj;
    const float s = b.use_scales ? b.scales[M.unit_begin + w].x : 1.0f;
    pa.alpha = 1.5f * s;
    pa.gamma = -0.5f * s;
    pa.eta = b.eta;
    if (EPI == EPI_ITER)
        pa.out = static_cast<char *>(M.out) + (int64_t)w * n * (int64_t)sizeof(T);
    else if (EPI == EPI_FINAL)
        pa.out = M.out ? static_cast<void *>(static_cast<float *>(M.out) + (int64_t)w * n) : nullptr;
    else
        pa.out = M.out;
    pa.pk = M.packed ? M.packed + (int64_t)w * ((n + 63) >> 6) : nullptr;

    if (wide) {
        // out[m][n] = sum_k A[m][k] X[k][n]: P = A (k-contiguous), Q(n, k) = X[k][n]
        Operand P{a + (int64_t)ti * kNsTileM * r * (int64_t)sizeof(T), r, R - ti * kNsTileM, r, vec};
        Operand Q{x + (int64_t)tj * kNsTileN * (int64_t)sizeof(T), C, C - tj * kNsTileN, r, vec};
        product_tile<BF16, false, EPI>(P, Q, smem, pa);
    } else {
        // out[m][n] = sum_k X[m][k] A[k][n] = sum_k X[m][k] A[n][k] (A symmetric)
        Operand P{x + (int64_t)ti * kNsTileM * C * (int64_t)sizeof(T), C, R - ti * kNsTileM, r, vec};
        Operand Q{a + (int64_t)tj * kNsTileN * r * (int64_t)sizeof(T), r, C - tj * kNsTileN, r, vec};
        product_tile<BF16, true, EPI>(P, Q, smem, pa);
    }
}

}  // namespace

void launch_ns_gram(const NsBatch &b, bool ns_bf16, hipStream_t s) {
    dim3 grid(b.total_tiles), block(kThreads);
    if (ns_bf16)
        hipLaunchKernelGGL(ns_gram_kernel<true>, grid, block, 0, s, b);
    else
        hipLaunchKernelGGL(ns_gram_kernel<false>, grid, block, 0, s, b);
}

void launch_ns_product(const NsBatch &b, bool ns_bf16, NsEpilogue epi, hipStream_t s) {
    dim3 grid(b.total_tiles), block(kThreads);
#define SM_PROD(BF, E) hipLaunchKernelGGL((ns_product_kernel<BF, E>), grid, block, 0, s, b)
    if (ns_bf16) {
        if (epi == EPI_ITER) SM_PROD(true, EPI_ITER);
        else if (epi == EPI_FINAL) SM_PROD(true, EPI_FINAL);
        else SM_PROD(true, EPI_WUPD);
    } else {
        if (epi == EPI_ITER) SM_PROD(false, EPI_ITER);
        else if (epi == EPI_FINAL) SM_PROD(false, EPI_FINAL);
        else SM_PROD(false, EPI_WUPD);
    }
#undef SM_PROD
}

}  // namespace sm
