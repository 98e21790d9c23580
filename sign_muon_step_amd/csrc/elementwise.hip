// elementwise.hip -- HBM-bound kernels of the Sign-Muon step for gfx950:
// momentum update with Frobenius partial sums, sign + 1-bit pack (or int8
// signs), majority vote + weight update from packed bits or from int8
// signs, and the small helpers of the post-vote polar step.
//
// Method: "SignMuon: Communication-Efficient Distributed Muon Optimization"
// (gist.science, paper 2605.16311, technical summary), cited by section.
#include "sm_internal.h"

namespace sm {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even, NaN quieted with its sign and
// top payload bits: one v_cvt_pk_bf16_f32 per pair of values (the hardware
// conversion gives exactly this rule on every fp32 bit pattern).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) { return pack_bf16x2(x, x) & 0xffffu; }

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Matrix of a flat block index: the descriptors are sorted by block_begin.
template <typename Batch>
__device__ __forceinline__ int find_mat(const Batch &b, int blk) {
    return find_start(b.starts, blk);
}

// ---------------------------------------------------------------------------
// Momentum: M <- store(fmaf(beta, M, G)) in place, one fp32 fused multiply-
// add per entry (summary §2 "Algorithmic flow", step 1; heavy-ball form is
// the reading taken), plus the sum of squares of the stored M per block for
// the Frobenius normalisation (summary §4 "nanoGPT": Frobenius scaling).
// ---------------------------------------------------------------------------
// Raw 16-byte pieces of 8 consecutive entries: fp32 takes two, bf16 one.
// G and M stream through once, so their loads and stores are nontemporal:
// they do not displace cache lines that the next kernels reuse.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct Raw8 {
    u32x4_t v[2];
};

__device__ __forceinline__ u32x4_t load16_nt(const void *p) {
    return __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
}

__device__ __forceinline__ void store16_nt(void *p, u32x4_t v) {
    __builtin_nontemporal_store(v, static_cast<u32x4_t *>(p));
}

template <bool B16>
__device__ __forceinline__ Raw8 load8(const void *p, int64_t e) {
    Raw8 r;
    if (B16) {
        r.v[0] = load16_nt(static_cast<const uint16_t *>(p) + e);
    } else {
        const float *q = static_cast<const float *>(p) + e;
        r.v[0] = load16_nt(q);
        r.v[1] = load16_nt(q + 4);
    }
    return r;
}

template <bool B16>
__device__ __forceinline__ void unpack8(const Raw8 &r, float (&x)[8]) {
    if (B16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(r.v[0][i] & 0xffffu);
            x[2 * i + 1] = bf16_bits_to_f32(r.v[0][i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(r.v[i >> 2][i & 3]);
    }
}

// Sign byte (bit t = (v_t >= 0)) of 8 stored values (the k = 0 signs packed
// by the momentum kernel).
struct Signs8 {
    uint32_t byte = 0;
    __device__ __forceinline__ void add(int t, float v) { byte |= (uint32_t)(v >= 0.0f) << t; }
};

// y = fmaf(beta, m, g) for 8 entries, stored in the momentum's type; returns
// the sum of squares of the stored values, and their signs in sg.
template <bool MB>
__device__ __forceinline__ double update8(float beta, const float (&g)[8], const float (&m)[8], void *mp,
                                          int64_t e, Signs8 &sg) {
    double ss = 0.0;
    if (MB) {
        u32x4_t out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t both = pack_bf16x2(__builtin_fmaf(beta, m[2 * i], g[2 * i]),
                                              __builtin_fmaf(beta, m[2 * i + 1], g[2 * i + 1]));
            const uint32_t lo = both & 0xffffu, hi = both >> 16;
            out[i] = both;
            const float f0 = bf16_bits_to_f32(lo), f1 = bf16_bits_to_f32(hi);
            const double s0 = f0, s1 = f1;
            ss += s0 * s0;
            ss += s1 * s1;
            sg.add(2 * i, f0);
            sg.add(2 * i + 1, f1);
        }
        store16_nt(static_cast<uint16_t *>(mp) + e, out);
    } else {
        u32x4_t y[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = __builtin_fmaf(beta, m[i], g[i]);
            y[i >> 2][i & 3] = __float_as_uint(v);
            const double d = v;
            ss += d * d;
            sg.add(i, v);
        }
        float *q = static_cast<float *>(mp) + e;
        store16_nt(q, y[0]);
        store16_nt(q + 4, y[1]);
    }
    return ss;
}

template <bool GB, bool MB>
__device__ __forceinline__ double momentum_one(const MomBatch &b, const void *gp, void *mp,
                                               int64_t e) {
    float g = GB ? bf16_bits_to_f32(static_cast<const uint16_t *>(gp)[e])
                 : static_cast<const float *>(gp)[e];
    float y;
    if (MB) {
        uint16_t *p = static_cast<uint16_t *>(mp) + e;
        uint32_t bits = f32_to_bf16_bits(__builtin_fmaf(b.beta, bf16_bits_to_f32(*p), g));
        *p = (uint16_t)bits;
        y = bf16_bits_to_f32(bits);
    } else {
        float *p = static_cast<float *>(mp) + e;
        y = __builtin_fmaf(b.beta, *p, g);
        *p = y;
    }
    double d = y;
    return d * d;
}

// With M.packed (k = 0, n % 64 == 0) the kernel also packs the signs of the
// stored M -- bit t of byte c is (M[8c + t] >= 0), the sign-pack layout. For
// k = 0 the factor is U = M / ||M||_F, whose signs are those of M whenever
// ||M||_F is finite (also when it is 0: M is then all +-0, every bit 1);
// finalize_scales flags the units where it is not (a NaN or Inf entry), and
// launch_pack_fixup recomputes those.
template <bool GB, bool MB>
__global__ __launch_bounds__(kMomThreads) void momentum_kernel(MomBatch b) {
    const int blk = blockIdx.x;
    const MomMat &M = b.mat[find_mat(b, blk)];
    const int local = blk - M.block_begin;
    const int w = local / M.blocks_per_worker;
    const int chunk = local - w * M.blocks_per_worker;
    const int64_t n = M.n;
    const size_t gsz = GB ? 2 : 4, msz = MB ? 2 : 4;
    const void *gp = static_cast<const char *>(M.g) + (size_t)w * (size_t)n * gsz;
    void *mp = static_cast<char *>(M.m) + (size_t)w * (size_t)n * msz;
    uint8_t *pk = M.packed ? reinterpret_cast<uint8_t *>(M.packed) + (size_t)w * (size_t)(n >> 3) : nullptr;
    const int64_t begin = (int64_t)chunk * kMomChunk;
    // the block's sign bytes (k = 0, packed here): staged, then stored as
    // 8-byte words (one byte per lane would be 64 bytes per wave store)
    __shared__ __attribute__((aligned(16))) uint8_t sbytes[kMomChunk / 8];
    double ss = 0.0;
    if ((n & 7) == 0) {
        // 8 consecutive entries per thread and round; n % 8 == 0 keeps every
        // worker's slice 16-byte aligned and every 8-group inside the matrix.
        // All rounds' loads are issued before the first store, so they are
        // all in flight together.
        constexpr int kRounds = kMomElemsPerThread / 8;
        Raw8 graw[kRounds], mraw[kRounds];
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int64_t e = begin + (int64_t)(r * kMomThreads + (int)threadIdx.x) * 8;
            if (e < n) {
                graw[r] = load8<GB>(gp, e);
                mraw[r] = load8<MB>(mp, e);
            }
        }
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int64_t e = begin + (int64_t)(r * kMomThreads + (int)threadIdx.x) * 8;
            if (e < n) {
                float g[8], m[8];
                unpack8<GB>(graw[r], g);
                unpack8<MB>(mraw[r], m);
                Signs8 sg;
                ss += update8<MB>(b.beta, g, m, mp, e, sg);
                if (pk) sbytes[(e - begin) >> 3] = (uint8_t)sg.byte;
            }
        }
    } else {
        for (int r = 0; r < kMomElemsPerThread; ++r) {
            int64_t e = begin + (int64_t)r * kMomThreads + threadIdx.x;
            if (e < n) ss += momentum_one<GB, MB>(b, gp, mp, e);
        }
    }
    // Deterministic block sum: waves by shuffle, then the 4 wave sums in order.
    __shared__ double wsum[kMomThreads / kWave];
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) wsum[threadIdx.x / kWave] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < kMomThreads / kWave; ++i) t += wsum[i];
        b.partials[M.partial_begin + local] = t;
    }
    if (pk) {  // n % 64 == 0: the block's byte count is a multiple of 8
        const int64_t nb = (n - begin < kMomChunk ? n - begin : kMomChunk) >> 3;
        for (int64_t o = (int64_t)threadIdx.x * 8; o < nb; o += (int64_t)kMomThreads * 8)
            *reinterpret_cast<uint2 *>(pk + (begin >> 3) + o) = *reinterpret_cast<const uint2 *>(sbytes + o);
    }
}

// s = 1/||M||_F and s^2 per (matrix, worker) (summary §2 "Communication
// efficiency": the normalisation is local to each worker). One wave per
// (matrix, worker): lane l adds the block partial sums l, l + 64, ... in fp64,
// then a fixed butterfly adds the 64 lane sums, so the result does not depend
// on timing.
__global__ __launch_bounds__(256) void finalize_scales_kernel(MomBatch b) {
    const int u = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    if (u >= b.nmat * b.workers) return;
    const MomMat &M = b.mat[u / b.workers];
    const int w = u % b.workers;
    const double *p = b.partials + M.partial_begin + (int64_t)w * M.blocks_per_worker;
    double ss = 0.0;
    for (int i = lane; i < M.blocks_per_worker; i += kWave) ss += p[i];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) {
        float s = 0.f, s2 = 0.f;
        if (ss > 0.0) {
            s = (float)(1.0 / sqrt(ss));
            s2 = (float)(1.0 / ss);
        }
        b.scales[M.unit_begin + w] = make_float2(s, s2);
        // the momentum kernel packed sign(M): the signs of M / ||M||_F unless
        // the sum of squares is NaN or Inf (then s = 0 and U = 0 * M)
        if (M.packed) b.pack_fix[M.unit_begin + w] = (ss - ss == 0.0) ? 0 : 1;
    }
}

// k = 0, packed by the momentum kernel: the units flagged in pack_fix (a NaN
// or Inf in M, so s = 0) get the signs of U = s M recomputed from the stored
// M (bit = (s * M >= 0), the sign_pack arithmetic: +1 for finite entries, -1
// for NaN and Inf), one 64-entry word per thread. kFixBlocks blocks per unit
// (blockIdx.x = unit * kFixBlocks + part); a block of an unflagged unit reads
// its flag and returns.
constexpr int kFixBlocks = 4;

template <bool MB>
__global__ __launch_bounds__(256) void pack_fixup_kernel(MomBatch b) {
    const int u = blockIdx.x / kFixBlocks, part = blockIdx.x % kFixBlocks;
    const MomMat &M = b.mat[u / b.workers];
    const int w = u % b.workers;
    if (!M.packed || !b.pack_fix[M.unit_begin + w]) return;
    const float s = b.scales[M.unit_begin + w].x;
    const int64_t words = M.n >> 6;
    const char *mp = static_cast<const char *>(M.m) + (size_t)w * (size_t)M.n * (MB ? 2 : 4);
    uint64_t *pk = M.packed + (size_t)w * (size_t)words;
    for (int64_t q = (int64_t)part * 256 + threadIdx.x; q < words; q += kFixBlocks * 256) {
        uint64_t word = 0;
        for (int t = 0; t < 64; ++t) {
            const int64_t e = q * 64 + t;
            const float v = MB ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(mp)[e])
                               : reinterpret_cast<const float *>(mp)[e];
            word |= (uint64_t)(s * v >= 0.0f) << t;
        }
        pk[q] = word;
    }
}

// ---------------------------------------------------------------------------
// Sign + 1-bit pack (summary §2 "Core mechanism"; "Algorithmic flow" steps
// 2-3): word w of a worker holds entries 64w..64w+63, bit j = (u >= 0) for
// entry 64w + j. In little-endian byte order, byte c of a worker's words is
// then the 8 signs of entries 8c..8c+7 (bit t = entry 8c + t), so each lane
// packs whole 8-entry chunks: one 16-byte load (bf16) or two (fp32) give one
// byte, stored by its lane (bf16) or gathered with its 7 neighbours into one
// 8-byte word store (fp32). A block's chunks are interleaved by thread, so
// every wave load covers 1 KiB (bf16) of consecutive entries and every wave
// store 64 consecutive bytes. Entries past n, up to the end of the last word, pack as 0. With an
// int8 target the chunk's 8 signs are stored as +1 / -1 bytes instead (one
// 8-byte store per chunk).
// ---------------------------------------------------------------------------
// DPP control of row_shl:N is kDppRowShl1 + N - 1 (lane i reads lane i + N of
// its 16-lane row).
constexpr int kDppRowShl1 = 0x101;

template <bool UB>
__global__ __launch_bounds__(256) void sign_pack_kernel(PackBatch b) {
    const int blk = blockIdx.x;
    const PackMat &M = b.mat[find_mat(b, blk)];
    const int local = blk - M.block_begin;
    const int w = local / M.blocks_per_worker;
    const int wb = local - w * M.blocks_per_worker;
    const int64_t n = M.n;
    const int64_t nbytes = ((n + 63) >> 6) * 8;  // packed bytes of one worker
    const float s = b.scales ? b.scales[M.unit_begin + w].x : 1.0f;
    const size_t usz = UB ? 2 : 4;
    const char *u = static_cast<const char *>(M.u) + (size_t)w * (size_t)n * usz;
    uint8_t *pk = M.packed ? reinterpret_cast<uint8_t *>(M.packed) + (size_t)w * (size_t)nbytes : nullptr;
    float *uo = M.u_out ? M.u_out + (size_t)w * (size_t)n : nullptr;
    int8_t *i8 = M.i8 ? M.i8 + (size_t)w * (size_t)n : nullptr;
    // n % 8 == 0: every chunk is whole and 16-byte aligned (bf16) or
    // 32-byte aligned (fp32) given a 16-byte aligned base.
    const bool vec = (n & 7) == 0;
    constexpr int CPT = pack_chunks_per_thread(UB);
    const int64_t c0 = (int64_t)wb * (256 * CPT) + threadIdx.x;
    // Every chunk's raw 16-byte pieces are loaded first (all in flight
    // together, 128 bytes of U per thread) and unpacked one chunk at a time,
    // so the registers hold raw words rather than CPT x 8 floats.
    u32x4_t raw[CPT][UB ? 1 : 2];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t e0 = (c0 + i * 256) * 8;
        if (vec && e0 < n) {  // read once: nontemporal
            raw[i][0] = load16_nt(u + e0 * usz);
            if (!UB) raw[i][UB ? 0 : 1] = load16_nt(u + e0 * usz + 16);
        }
    }
    // chunk i as 8 values (0 past n)
    auto values = [&](int i, float (&v)[8]) {
        const int64_t e0 = (c0 + i * 256) * 8;
        if (vec && e0 < n) {
            if (UB) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[2 * t] = bf16_bits_to_f32(raw[i][0][t] & 0xffffu);
                    v[2 * t + 1] = bf16_bits_to_f32(raw[i][0][t] >> 16);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[t] = __uint_as_float(raw[i][0][t]);
                    v[4 + t] = __uint_as_float(raw[i][UB ? 0 : 1][t]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int64_t e = e0 + t;
                v[t] = e < n ? (UB ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(u)[e])
                                   : reinterpret_cast<const float *>(u)[e])
                             : 0.0f;
            }
        }
    };
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = c0 + i * 256, e0 = c * 8;
        if (UB && c >= nbytes) continue;
        float v[8];
        values(i, v);
        uint32_t byte = 0;
        if (e0 + 8 <= n) {  // a whole chunk: no per-entry bound (5 % faster for bf16 U)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = b.scales ? s * v[t] : v[t];
                v[t] = x;
                byte |= (uint32_t)(x >= 0.0f) << t;
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = b.scales ? s * v[t] : v[t];
                v[t] = x;
                byte |= (uint32_t)(e0 + t < n && x >= 0.0f) << t;
            }
        }
        if (UB) {
            if (pk) pk[c] = (uint8_t)byte;
        } else {
            // fp32 U: lanes 8k..8k+7 hold the 8 bytes of one word (a wave's
            // chunks start at a multiple of 64). Three row shifts (lane i takes
            // lane i + 1, + 2, + 4 of its 16-lane row) gather them into lane
            // 8k, which stores the word: 8 bytes per store instead of one,
            // 7 % faster here. (With bf16 U the byte stores are as fast.)
            if (pk) {
                const uint32_t h = byte | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)byte, kDppRowShl1, 0xf, 0xf, false) << 8);
                const uint32_t q = h | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, kDppRowShl1 + 1, 0xf, 0xf, false) << 16);
                const uint32_t q1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, kDppRowShl1 + 3, 0xf, 0xf, false);
                if ((lane & 7) == 0 && c < nbytes)
                    *reinterpret_cast<uint64_t *>(pk + c) = (uint64_t)q | ((uint64_t)q1 << 32);
            }
            if (c >= nbytes) continue;
        }
        if (i8 && e0 < n) {
            // bit t set: +1 (0x01), clear: -1 (0xff)
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                lo |= (((byte >> t) & 1u) ? 0x01u : 0xffu) << (8 * t);
                hi |= (((byte >> (t + 4)) & 1u) ? 0x01u : 0xffu) << (8 * t);
            }
            if (vec) {
                *reinterpret_cast<uint2 *>(i8 + e0) = make_uint2(lo, hi);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (e0 + t < n) i8[e0 + t] = (int8_t)((t < 4 ? lo >> (8 * t) : hi >> (8 * (t - 4))) & 0xffu);
            }
        }
        if (uo) {
            if (vec && e0 < n) {
                *reinterpret_cast<float4 *>(uo + e0) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4 *>(uo + e0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (e0 + t < n) uo[e0 + t] = v[t];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Majority vote + update (summary §2 "Core mechanism": the vote is the sign
// of the integer sum of the workers' signs; "Algorithmic flow" step 4:
// W <- W - eta * S-bar). With c the number of +1 bits over Mw workers the
// sum is 2c - Mw; a tie votes 0 and leaves the entry unchanged.
//
// Each wave counts 64 words (4096 entries): lane l holds word l of the group
// for every worker and adds them into NB bit-sliced counters (one counter bit
// per plane, 64 entries per plane word), then compares the counters with the
// two thresholds to get a plus-mask and a minus-mask per word. The masks go
// through LDS so that W is then read and written 16 bytes per lane in
// coalesced order.
// ---------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ uint64_t counter_gt(const uint64_t (&c)[NB], int t) {
    uint64_t gt = 0, eq = ~0ull;
#pragma unroll
    for (int bit = NB - 1; bit >= 0; --bit) {
        if ((t >> bit) & 1) {
            eq &= c[bit];
        } else {
            gt |= eq & c[bit];
            eq &= ~c[bit];
        }
    }
    return gt;
}

template <int NB>
__global__ __launch_bounds__(256) void vote_update_kernel(VoteBatch b) {
    __shared__ uint64_t plus_s[4][kVoteWordsPerWave];
    __shared__ uint64_t minus_s[4][kVoteWordsPerWave];
    const int blk = blockIdx.x;
    const VoteMat &M = b.mat[find_mat(b, blk)];
    const int local = blk - M.block_begin;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t n = M.n;
    const int64_t nw = (n + 63) >> 6;
    const int64_t group = (int64_t)local * 4 + wave;
    const int64_t word = group * kVoteWordsPerWave + lane;
    const int mw = b.workers;

    uint64_t c[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) c[i] = 0;
    if (word < nw) {
        const uint64_t *p = M.packed + word;
        for (int m = 0; m < mw; ++m) {
            uint64_t carry = p[(size_t)m * nw];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                uint64_t t = c[i] & carry;
                c[i] ^= carry;
                carry = t;
            }
        }
    }
    // plus: 2c > mw  <=>  c > floor(mw/2);  minus: 2c < mw  <=>  !(c > ceil(mw/2) - 1)
    uint64_t plus = counter_gt<NB>(c, mw >> 1);
    uint64_t minus = ~counter_gt<NB>(c, ((mw + 1) >> 1) - 1);
    if (word >= nw) {
        plus = 0;
        minus = 0;
    } else if ((word + 1) * 64 > n) {
        uint64_t valid = (1ull << (n & 63)) - 1;
        plus &= valid;
        minus &= valid;
    }
    if (M.nnz) {
        uint32_t cnt = wave_sum_u32((uint32_t)__popcll(plus | minus));
        if (lane == 0 && cnt) atomicAdd(M.nnz, cnt);
    }
    plus_s[wave][lane] = plus;
    minus_s[wave][lane] = minus;
    __syncthreads();

    const float eta = b.eta;
    const int64_t ebase = group * (kVoteWordsPerWave * 64);
#pragma unroll 4
    for (int it = 0; it < kVoteWordsPerWave / 4; ++it) {
        const int64_t e = ebase + it * 256 + lane * 4;
        if (e >= n) break;
        const int wi = it * 4 + (lane >> 4);
        const int sh = (lane & 15) * 4;
        const uint32_t p4 = (uint32_t)(plus_s[wave][wi] >> sh) & 0xfu;
        const uint32_t m4 = (uint32_t)(minus_s[wave][wi] >> sh) & 0xfu;
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (int)((p4 >> j) & 1u) - (int)((m4 >> j) & 1u);
        const bool full = e + 4 <= n;
        if (M.w) {
            if (full) {
                float4 *wp = reinterpret_cast<float4 *>(M.w + e);
                float4 x = *wp;
                float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xs[j] = v[j] > 0 ? xs[j] - eta : (v[j] < 0 ? xs[j] + eta : xs[j]);
                *wp = make_float4(xs[0], xs[1], xs[2], xs[3]);
            } else {
                for (int j = 0; j < 4 && e + j < n; ++j) {
                    float x = M.w[e + j];
                    M.w[e + j] = v[j] > 0 ? x - eta : (v[j] < 0 ? x + eta : x);
                }
            }
        }
        if (M.vote) {
            if (full) {
                uint32_t packed4 = (uint32_t)(uint8_t)(int8_t)v[0] | ((uint32_t)(uint8_t)(int8_t)v[1] << 8) |
                                   ((uint32_t)(uint8_t)(int8_t)v[2] << 16) |
                                   ((uint32_t)(uint8_t)(int8_t)v[3] << 24);
                *reinterpret_cast<uint32_t *>(M.vote + e) = packed4;
            } else {
                for (int j = 0; j < 4 && e + j < n; ++j) M.vote[e + j] = (int8_t)v[j];
            }
        }
        if (M.v_ns) {
            if (b.v_ns_bf16) {
                uint16_t *vp = static_cast<uint16_t *>(M.v_ns) + e;
                for (int j = 0; j < 4 && e + j < n; ++j)
                    vp[j] = v[j] > 0 ? 0x3f80u : (v[j] < 0 ? 0xbf80u : 0u);
            } else {
                float *vp = static_cast<float *>(M.v_ns) + e;
                for (int j = 0; j < 4 && e + j < n; ++j) vp[j] = (float)v[j];
            }
        }
    }
}

__global__ void zero_u32_kernel(uint32_t *p, int32_t count) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

// Frobenius scale of the vote: ||S-bar||_F = sqrt(nnz) exactly.
__global__ void nnz_scales_kernel(const uint32_t *nnz, int32_t count, float2 *scales) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    double c = (double)nnz[i];
    scales[i] = c > 0.0 ? make_float2((float)(1.0 / sqrt(c)), (float)(1.0 / c)) : make_float2(0.f, 0.f);
}

// ---------------------------------------------------------------------------
// Int8 payload (summary §2 "Core mechanism": the vote as an integer SUM
// all-reduce of the workers' signs followed by a local sign; §2
// "Communication efficiency": eight bits per entry with int8). Both kernels
// stream 16 entries per thread.
// ---------------------------------------------------------------------------
constexpr int kI8PerThread = 16;
constexpr int kI8PerBlock = 256 * kI8PerThread;

// signs[i] = +1 where u[i] >= 0, else -1, over the flat [workers][n] array.
template <bool UB>
__global__ __launch_bounds__(256) void sign_int8_kernel(const void *u, int64_t total, int8_t *signs) {
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * kI8PerThread;
    if (e0 >= total) return;
    if (e0 + kI8PerThread <= total) {
        float x[kI8PerThread];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            Raw8 r = load8<UB>(u, e0 + 8 * h);
            float y[8];
            unpack8<UB>(r, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[8 * h + i] = y[i];
        }
        u32x4_t out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t wd = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) wd |= (x[4 * q + b] >= 0.f ? 0x01u : 0xffu) << (8 * b);
            out[q] = wd;
        }
        store16_nt(signs + e0, out);
    } else {
        for (int64_t e = e0; e < total; ++e) {
            const float v = UB ? bf16_bits_to_f32(static_cast<const uint16_t *>(u)[e]) : static_cast<const float *>(u)[e];
            signs[e] = v >= 0.f ? (int8_t)1 : (int8_t)-1;
        }
    }
}

// vote_i = sign(sum over workers of signs[m][i]) and the update of W, for
// every matrix of the batch. Each thread takes 16 entries; with n % 16 == 0
// (vec) every worker's 16 entries are one 16-byte load.
__global__ __launch_bounds__(256) void vote_update_int8_kernel(VoteI8Batch b) {
    const int blk = blockIdx.x;
    const VoteI8Mat &M = b.mat[find_start(b.starts, blk)];
    const int64_t n = M.n;
    const int mw = b.workers;
    const float eta = b.eta;
    float *w = M.w;
    int8_t *vote = M.vote;
    const int64_t e0 = ((int64_t)(blk - M.block_begin) * 256 + threadIdx.x) * kI8PerThread;
    if (e0 >= n) return;
    if (M.vec) {
        int32_t t[kI8PerThread];
#pragma unroll
        for (int i = 0; i < kI8PerThread; ++i) t[i] = 0;
        const int8_t *p = M.signs + e0;
        auto add = [&](const u32x4_t &r) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) t[4 * q + c] += (int32_t)(int8_t)(r[q] >> (8 * c));
        };
        int m = 0;
        for (; m + 4 <= mw; m += 4) {  // four workers' loads in flight together
            u32x4_t r[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = load16_nt(p + (int64_t)(m + k) * n);
#pragma unroll
            for (int k = 0; k < 4; ++k) add(r[k]);
        }
        for (; m < mw; ++m) add(load16_nt(p + (int64_t)m * n));
        if (w) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 *wp = reinterpret_cast<float4 *>(w + e0 + 4 * q);
                float4 v = *wp;
                float *f = &v.x;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int32_t ti = t[4 * q + c];
                    f[c] = ti > 0 ? f[c] - eta : (ti < 0 ? f[c] + eta : f[c]);
                }
                *wp = v;
            }
        }
        if (vote) {
            u32x4_t out;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t wd = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int32_t ti = t[4 * q + c];
                    wd |= (uint32_t)(uint8_t)(int8_t)(ti > 0 ? 1 : (ti < 0 ? -1 : 0)) << (8 * c);
                }
                out[q] = wd;
            }
            *reinterpret_cast<u32x4_t *>(vote + e0) = out;
        }
    } else {
        const int64_t e1 = e0 + kI8PerThread < n ? e0 + kI8PerThread : n;
        for (int64_t e = e0; e < e1; ++e) {
            int32_t ti = 0;
            for (int m = 0; m < mw; ++m) ti += M.signs[(int64_t)m * n + e];
            const int v = ti > 0 ? 1 : (ti < 0 ? -1 : 0);
            if (w && v > 0)
                w[e] = w[e] - eta;
            else if (w && v < 0)
                w[e] = w[e] + eta;
            if (vote) vote[e] = (int8_t)v;
        }
    }
}


// Sign + pack when the packed bits are the only output and n % 8 == 0 (the
// same blocks as sign_pack_kernel: 2048 chunks of 8 entries per block for
// bf16 U, 1024 for fp32). Every load is one 16-byte piece of U, consecutive
// across the lanes (8 bf16 entries: one packed byte; 4 fp32 entries: half a
// byte), and the bits go through 2 KiB of LDS, so that the block writes its
// packed bytes as 8-byte words: byte stores of 64 bytes per wave instruction
// cost more than all the loads.
template <bool UB>
__global__ __launch_bounds__(256) void sign_pack_words_kernel(PackBatch b) {
    constexpr int EPP = UB ? 8 : 4;        // entries per 16-byte piece
    constexpr int PPT = 8;                 // pieces per thread
    constexpr int OUT = 256 * PPT * EPP / 8;  // packed bytes per block
    __shared__ __attribute__((aligned(16))) uint8_t bits[256 * PPT];  // per piece: a byte (bf16) or a nibble (fp32)
    const int blk = blockIdx.x;
    const PackMat &M = b.mat[find_mat(b, blk)];
    const int local = blk - M.block_begin;
    const int w = local / M.blocks_per_worker;
    const int wb = local - w * M.blocks_per_worker;
    const int64_t n = M.n;
    const int64_t nbytes = ((n + 63) >> 6) * 8;
    const float s = b.scales ? b.scales[M.unit_begin + w].x : 1.0f;
    const char *u = static_cast<const char *>(M.u) + (size_t)w * (size_t)n * (UB ? 2 : 4);
    uint8_t *pk = reinterpret_cast<uint8_t *>(M.packed) + (size_t)w * (size_t)nbytes;
    const int64_t q0 = (int64_t)wb * (256 * PPT);  // first piece of the block
    u32x4_t raw[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int64_t e0 = (q0 + i * 256 + threadIdx.x) * EPP;
        if (e0 < n) raw[i] = load16_nt(u + e0 * (UB ? 2 : 4));
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int64_t e0 = (q0 + i * 256 + threadIdx.x) * EPP;
        uint32_t v = 0;
        if (e0 < n) {  // n % 8 == 0: the piece is whole
#pragma unroll
            for (int t = 0; t < EPP; ++t) {
                const float x = UB ? bf16_bits_to_f32(t & 1 ? raw[i][t >> 1] >> 16 : raw[i][t >> 1] & 0xffffu)
                                   : __uint_as_float(raw[i][t]);
                v |= (uint32_t)((b.scales ? s * x : x) >= 0.0f) << t;
            }
        }
        bits[i * 256 + threadIdx.x] = (uint8_t)v;
    }
    __syncthreads();
    // thread t writes packed bytes 8t .. 8t + 7 of the block
    if (threadIdx.x * 8 < OUT) {
        const int64_t c = (int64_t)wb * OUT + threadIdx.x * 8;
        if (c < nbytes) {  // nbytes % 8 == 0: the word is whole
            const uint32_t *b32 = reinterpret_cast<const uint32_t *>(bits);
            uint32_t lo, hi;
            if (UB) {  // one byte per piece already
                lo = b32[threadIdx.x * 2];
                hi = b32[threadIdx.x * 2 + 1];
            } else {   // two nibbles (pieces 2j, 2j + 1, one per byte) per packed byte j
                auto pair = [](uint32_t x) {  // bytes n0 n1 n2 n3 -> (n0 | n1 << 4) | (n2 | n3 << 4) << 8
                    return (x & 0xfu) | ((x >> 4) & 0xf0u) | ((x >> 8) & 0xf00u) | ((x >> 12) & 0xf000u);
                };
                lo = pair(b32[threadIdx.x * 4]) | pair(b32[threadIdx.x * 4 + 1]) << 16;
                hi = pair(b32[threadIdx.x * 4 + 2]) | pair(b32[threadIdx.x * 4 + 3]) << 16;
            }
            *reinterpret_cast<uint2 *>(pk + c) = make_uint2(lo, hi);
        }
    }
}
}  // namespace

void launch_momentum(const MomBatch &b, hipStream_t s) {
    dim3 grid(b.total_blocks), block(kMomThreads);
    if (b.g_bf16 && b.m_bf16)
        hipLaunchKernelGGL((momentum_kernel<true, true>), grid, block, 0, s, b);
    else if (b.g_bf16)
        hipLaunchKernelGGL((momentum_kernel<true, false>), grid, block, 0, s, b);
    else if (b.m_bf16)
        hipLaunchKernelGGL((momentum_kernel<false, true>), grid, block, 0, s, b);
    else
        hipLaunchKernelGGL((momentum_kernel<false, false>), grid, block, 0, s, b);
}

void launch_finalize_scales(const MomBatch &b, hipStream_t s) {
    int units = b.nmat * b.workers;
    hipLaunchKernelGGL(finalize_scales_kernel, dim3((units + 3) / 4), dim3(256), 0, s, b);
}

void launch_pack_fixup(const MomBatch &b, bool m_bf16, hipStream_t s) {
    const dim3 grid(b.nmat * b.workers * kFixBlocks);
    if (m_bf16)
        hipLaunchKernelGGL(pack_fixup_kernel<true>, grid, dim3(256), 0, s, b);
    else
        hipLaunchKernelGGL(pack_fixup_kernel<false>, grid, dim3(256), 0, s, b);
}

void launch_sign_pack(const PackBatch &b, hipStream_t s) {
    dim3 grid(b.total_blocks), block(256);
    bool words = true;  // packed bits the only output, whole chunks
    for (int i = 0; i < b.nmat; ++i)
        words = words && b.mat[i].packed && !b.mat[i].u_out && !b.mat[i].i8 && (b.mat[i].n & 7) == 0;
    if (words) {
        if (b.u_bf16)
            hipLaunchKernelGGL(sign_pack_words_kernel<true>, grid, block, 0, s, b);
        else
            hipLaunchKernelGGL(sign_pack_words_kernel<false>, grid, block, 0, s, b);
        return;
    }
    if (b.u_bf16)
        hipLaunchKernelGGL(sign_pack_kernel<true>, grid, block, 0, s, b);
    else
        hipLaunchKernelGGL(sign_pack_kernel<false>, grid, block, 0, s, b);
}

void launch_vote_update(const VoteBatch &b, hipStream_t s) {
    dim3 grid(b.total_blocks), block(256);
    const int mw = b.workers;
#define SM_VOTE(NBITS) hipLaunchKernelGGL(vote_update_kernel<NBITS>, grid, block, 0, s, b)
    if (mw <= 1) SM_VOTE(1);
    else if (mw <= 3) SM_VOTE(2);
    else if (mw <= 7) SM_VOTE(3);
    else if (mw <= 15) SM_VOTE(4);
    else if (mw <= 31) SM_VOTE(5);
    else if (mw <= 63) SM_VOTE(6);
    else if (mw <= 127) SM_VOTE(7);
    else SM_VOTE(8);
#undef SM_VOTE
}

void launch_zero_u32(uint32_t *p, int32_t count, hipStream_t s) {
    if (count <= 0) return;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((count + 255) / 256), dim3(256), 0, s, p, count);
}

void launch_nnz_scales(const uint32_t *nnz, int32_t count, float2 *scales, hipStream_t s) {
    if (count <= 0) return;
    hipLaunchKernelGGL(nnz_scales_kernel, dim3((count + 255) / 256), dim3(256), 0, s, nnz, count,
                       scales);
}

}  // namespace sm

namespace sm {

int64_t sign_int8_blocks(int64_t total) { return (total + kI8PerBlock - 1) / kI8PerBlock; }

void launch_sign_int8(const void *u, bool u_bf16, int64_t total, int8_t *signs, hipStream_t s) {
    dim3 grid((unsigned)sign_int8_blocks(total)), block(256);
    if (u_bf16)
        hipLaunchKernelGGL(sign_int8_kernel<true>, grid, block, 0, s, u, total, signs);
    else
        hipLaunchKernelGGL(sign_int8_kernel<false>, grid, block, 0, s, u, total, signs);
}

int64_t vote_int8_blocks(int64_t n) { return (n + kI8PerBlock - 1) / kI8PerBlock; }

void launch_vote_update_int8(const VoteI8Batch &b, hipStream_t s) {
    hipLaunchKernelGGL(vote_update_int8_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
}

}  // namespace sm
