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
//   product: X' = -0.5 s * (A X - 3 X)   (wide)   or
//            X' = -0.5 s * (X A - 3 X)   (tall),
//            i.e. s (1.5 X - 0.5 A X); the -3 X term is accumulated on the
//            matrix cores with a -3 I fragment, and s folds the Frobenius
//            scaling of the first iteration in (s = 1 afterwards).
// The last product's epilogue stores fp32 U and/or takes the sign of each
// entry: packed 64 signs per uint64 word straight from the wave64 ballot of
// the accumulator registers, or int8 +1 / -1 (summary §2 "Algorithmic flow",
// steps 2-3, and "Communication efficiency"); or (Muon step, post-vote polar
// step) it applies W <- fmaf(-eta, Y, W).
//
// Kernels: ns_gram_kernel (one block per Gram tile; for matrices with at
// most 3 Gram tiles per worker, one block per k chunk of a tile, writing fp32
// partial tiles that gram_reduce_kernel adds in order, scales and stores);
// ns_product_kernel (one block per output tile, every epilogue); and
// ns_product_pack_kernel, the bf16 products as a persistent walk of one
// workgroup per CU whose direct-to-LDS loads run on across tile boundaries
// (final signs packed or int8 from the accumulators, or the next iterate).
//
// Every GEMM is C[m][n] = sum_k P[m][k] Q[n][k] on a 256 x TN output tile
// computed by waves of 128 x 64, two waves per SIMD (one wave's LDS reads and
// waits overlap the other's matrix instructions). Both kernels use TN = 256:
// 8 waves and 128 KiB of LDS, one workgroup per CU. (The Gram's tiles must be
// square for the mirror; for the product, 256 x 128 tiles with two
// workgroups per CU were faster on single-shape batches but slower on a
// transformer's mixed batch, where the 256 x 256 tile reuses more in L2.)
// Operands stream from global memory straight into LDS, one k-slice of 64
// bytes per row (32 bf16 or 16 fp32) at a time. A k-contiguous operand is
// stored by rows with its 16-byte chunks XOR-swizzled, so that the fragment
// reads spread over all banks. An operand whose k index is the strided one
// in memory (X in a wide product, both Gram operands of a tall X) lands in
// LDS mn-contiguous, in 4 (k) x 16 (mn) blocks for bf16, and its bf16
// fragments come out with the LDS transpose read (ds_read_b64_tr_b16); fp32
// ones are read element by element.
#include <type_traits>
#include <utility>

#include "sm_internal.h"

namespace sm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// Wave tile kWaveM x kWaveN, in 32 x 32 MFMA blocks.
constexpr int kWaveM = 128, kWaveN = 64;
constexpr int kFM = kWaveM / 32, kFN = kWaveN / 32;
constexpr int kRowBytes = 64;  // LDS bytes of one operand row per k-slice

// Where a helper gets the thread's index: HwTid reads threadIdx.x where it is
// used; GivenTid carries a value the caller produced (the persistent product
// makes it afresh per tile, so that the compiler does not keep lane
// arithmetic in registers across its whole walk).
struct HwTid {
    __device__ unsigned operator()() const { return threadIdx.x; }
};
struct GivenTid {
    unsigned v;
    __device__ unsigned operator()() const { return v; }
};

// Workgroup layout of a 256 x TN output tile: two rows of TN / kWaveN waves;
// each LDS stage holds one k-slice of P (256 rows) then of Q (TN rows).
template <int TN>
struct Lay {
    static constexpr int kTileM = 256, kTileN = TN;
    static constexpr int kWavesN = TN / kWaveN;
    static constexpr int kWaves = (kTileM / kWaveM) * kWavesN;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kPBytes = kTileM * kRowBytes, kQBytes = TN * kRowBytes;
    static constexpr int kStageBytes = kPBytes + kQBytes;
    static constexpr int kStages = TN == 256 ? 4 : 3;  // pipeline depth
    static constexpr int kLdsBytes = kStages * kStageBytes;
    static constexpr int kPLoads = kPBytes / 1024 / kWaves;  // 1 KiB loads per wave per slice
    static constexpr int kQLoads = kQBytes / 1024 / kWaves;
    static_assert(kPLoads * kWaves * 1024 == kPBytes && kQLoads * kWaves * 1024 == kQBytes, "loads");
    __device__ static int m0(int wid) { return (wid / kWavesN) * kWaveM; }
    __device__ static int n0(int wid) { return (wid % kWavesN) * kWaveN; }
};
using GramLay = Lay<256>;
using ProdLay = Lay<kNsProdTileN>;
static_assert(GramLay::kLdsBytes <= 160 * 1024 && ProdLay::kLdsBytes <= 160 * 1024, "LDS");

template <bool BF16> struct Elem;
template <> struct Elem<true> {
    using T = uint16_t;
    static constexpr int BK = 32;   // k per stage
    static constexpr int EPC = 8;   // elements per 16-byte chunk
};
template <> struct Elem<false> {
    using T = float;
    static constexpr int BK = 16;
    static constexpr int EPC = 4;
};

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

// LDS layouts of one operand's k-slice (ROWS rows of the tile, 64 bytes each):
//  k-contiguous ("KL"): ROWS rows x 64 bytes (BK of k), 16-byte chunk c of
//    row r stored at chunk c ^ ((r >> 2) & 3): the MFMA reads of 16
//    consecutive rows then hit 16 distinct 16-byte bank groups.
//  mn-contiguous bf16 ("ML"): 4 (k) x 16 (mn) blocks of 128 bytes, block
//    (k/4, mn/16) at ((k/4) * ROWS/16 + mn/16) * 128: one LDS transpose read
//    of a 16-lane group covers exactly one block.
//  mn-contiguous fp32: plain rows of ROWS mn per k.
__device__ __forceinline__ uint32_t kl_off(int row, int chunk) {
    return (uint32_t)(row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4));
}
template <int ROWS>
__device__ __forceinline__ uint32_t ml_off_bf16(int k, int mn) {
    return (uint32_t)((((k >> 2) * (ROWS / 16) + (mn >> 4)) << 7) + ((k & 3) << 5) + ((mn & 15) << 1));
}
template <int ROWS>
__device__ __forceinline__ uint32_t ml_off_f32(int k, int mn) { return (uint32_t)((k * ROWS + mn) * 4); }

// s_waitcnt with vmcnt = N, lgkmcnt = 0 (expcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses without waiting for the
// direct-to-LDS loads still in flight (the caller waits for what it needs).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane load from a buffer straight into LDS: lane L's 16
// bytes land at LDS address lds + 16 L. Written as asm so that the compiler
// does not order later LDS reads behind every load still in flight; the
// caller waits with explicit vmcnt counts. The asm has no outputs: address
// and descriptor are consumed at issue. M0 (the LDS base of the load) is a
// register the compiler reserves and cannot take as a clobber; no code the
// compiler generates for these kernels reads M0, so writing it here is safe.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voffset, v4u32 rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voffset), "s"(rsrc)
                 : "memory");
}

// Direct-to-LDS loads of one operand (ROWS rows of the tile, WAVES waves):
// each wave instruction moves 1 KiB (16 bytes per lane) from global memory
// straight into LDS, so a k-slice costs no registers and several slices can
// be in flight. The LDS destination of lane L is fixed (base + 16 L); the
// lane therefore fetches whichever global chunk the layout (k- or
// mn-contiguous, chosen at init) puts there. Chunks outside the operand read
// the out-of-bounds buffer offset and land as zeros. Each thread issues
// NL = ROWS / 16 / WAVES loads per slice.
template <bool BF16, int ROWS, int WAVES>
struct DmaSlices {
    using E = Elem<BF16>;
    using T = typename E::T;
    static constexpr int NL = ROWS / 16 / WAVES;
    static_assert(NL * 16 * WAVES == ROWS, "loads per wave");
    v4u32 rsrc;
    uint32_t off[NL];  // byte offset of each of the thread's chunks in slice 0
    int kofs[NL];      // k of the chunk relative to the slice start
    uint32_t valid;    // bit i: chunk i's rows lie inside the operand
    uint32_t kstep;    // bytes per slice
    int K;
    int wid;

    template <bool KC, class Tid = HwTid>
    __device__ __forceinline__ void setup(const Operand &op, Tid tid = Tid{}) {
        const int lane = tid() & (kWave - 1);
        wid = __builtin_amdgcn_readfirstlane(tid() / kWave);
        // Buffer descriptor: 48-bit base, stride 0, num_records = extent in
        // bytes, raw 32-bit dword format (0x00020000 on this family).
        const uint64_t base = reinterpret_cast<uint64_t>(op.base);
        rsrc = v4u32{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xffffu)),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)operand_extent<BF16, KC>(op)),
                     0x00020000u};
        K = op.K;
        valid = 0;
        const uint32_t sz = sizeof(T);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int b = i * WAVES + wid;      // 1 KiB block of the slice
            int mn, k;
            if (KC) {                           // 16 rows of 64 bytes
                const int row = b * 16 + (lane >> 2);
                const int c = (lane & 3) ^ ((row >> 2) & 3);
                mn = row;
                k = c * E::EPC;
            } else if (BF16) {                  // 8 blocks of 4 (k) x 16 (mn)
                const int blk = b * 8 + (lane >> 3), w = lane & 7;
                k = (blk / (ROWS / 16)) * 4 + (w >> 1);
                mn = (blk % (ROWS / 16)) * 16 + (w & 1) * 8;
            } else {                            // 256 / ROWS k rows of ROWS fp32
                k = b * (256 / ROWS) + lane / (ROWS / 4);
                mn = (lane % (ROWS / 4)) * 4;
            }
            off[i] = KC ? (uint32_t)(mn * op.ld + k) * sz : (uint32_t)(k * op.ld + mn) * sz;
            kofs[i] = k;
            valid |= (uint32_t)(mn < op.rows) << i;
        }
        kstep = KC ? (uint32_t)E::BK * sz : (uint32_t)(E::BK * op.ld) * sz;
    }

    // A queue with nothing to load: every chunk reads the out-of-bounds offset
    // of an empty buffer and lands as zeros.
    __device__ __forceinline__ void init_empty() {
        wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        rsrc = v4u32{0u, 0u, 0u, 0x00020000u};
#pragma unroll
        for (int i = 0; i < NL; ++i) off[i] = kofs[i] = 0;
        valid = 0;
        kstep = 0;
        K = 0;
    }

    // Buffer offset of load i of slice kt.
    __device__ __forceinline__ uint32_t offset(int kt, int i) const {
        const bool ok = ((valid >> i) & 1u) && kt * E::BK + kofs[i] < K;
        return ok ? off[i] + (uint32_t)kt * kstep : kOOB;
    }

    // lds: LDS byte address of this operand's slice buffer.
    __device__ __forceinline__ void issue_at(uint32_t lds, int i, uint32_t o, v4u32 rs) const {
        dma16(lds + (uint32_t)(i * WAVES + wid) * 1024u, o, rs);
    }

    // Load i (0 .. NL - 1) of slice kt only.
    __device__ __forceinline__ void issue_one(int kt, uint32_t lds, int i) const {
        issue_at(lds, i, offset(kt, i), rsrc);
    }

    __device__ __forceinline__ void issue(int kt, uint32_t lds) const {
        const int k0 = kt * E::BK;
        const uint32_t kb = (uint32_t)kt * kstep;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const bool ok = ((valid >> i) & 1u) && k0 + kofs[i] < K;
            issue_at(lds, i, ok ? off[i] + kb : kOOB, rsrc);
        }
    }
};

template <bool BF16, bool KC, int ROWS, int WAVES>
struct DmaLoader : DmaSlices<BF16, ROWS, WAVES> {
    __device__ __forceinline__ void init(const Operand &op) { this->template setup<KC>(op); }
};

// Element-by-element loader for shapes whose rows break 16-byte alignment:
// writes the same LDS layouts with plain loads and stores (synchronous).
template <bool BF16, bool KC, int ROWS, int THREADS>
struct SlowLoader {
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

    __device__ __forceinline__ void load_store(int kt, char *lds) const {
        const int k0 = kt * E::BK;
        for (int e = threadIdx.x; e < ROWS * E::BK; e += THREADS) {
            const int mn = e / E::BK, k = e % E::BK;
            T v = (T)0;
            if (mn < rows && k0 + k < K) v = KC ? p[(int64_t)mn * ld + k0 + k] : p[(int64_t)(k0 + k) * ld + mn];
            uint32_t o;
            if (KC)
                o = kl_off(mn, k / E::EPC) + (k % E::EPC) * sizeof(T);
            else
                o = BF16 ? ml_off_bf16<ROWS>(k, mn) : ml_off_f32<ROWS>(k, mn);
            *reinterpret_cast<T *>(lds + o) = v;
        }
    }
};

// MFMA fragments of one 32-row (m or n) block for k16 step kk (bf16): lane l
// holds row (l & 31) and k = 16 kk + 8 (l / 32) .. + 7.
template <bool KC, int ROWS, class Tid = HwTid>
__device__ __forceinline__ bf16x8_t frag_bf16(const char *lds, int row0, int kk, Tid tid = Tid{}) {
    const int lane = tid() & (kWave - 1);
    if (KC) {
        const uint4 v = *reinterpret_cast<const uint4 *>(lds + kl_off(row0 + (lane & 31), 2 * kk + (lane >> 5)));
        return __builtin_bit_cast(bf16x8_t, v);
    } else {
        // Two LDS transpose reads: in each 16-lane group g, lane 4j + q points
        // at 4 mn-consecutive values of k row j; lane i gets mn column i of
        // the 4 rows, i.e. 4 k-consecutive values of its own mn.
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const int g = lane >> 4, i = lane & 15;
        const int mn = row0 + 16 * (g & 1) + 4 * (i & 3);
        const int k = 16 * kk + 8 * (g >> 1) + (i >> 2);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds + ml_off_bf16<ROWS>(k, mn)));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds + ml_off_bf16<ROWS>(k + 4, mn)));
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8_t, both);
    }
}

// fp32 fragments for chunk pair cp: lane l holds 4 consecutive k
// (k = 8 cp + 4 (l / 32) .. + 3) of row (l & 31); MFMA step s uses element s.
template <bool KC, int ROWS, class Tid = HwTid>
__device__ __forceinline__ f32x4_t frag_f32(const char *lds, int row0, int cp, Tid tid = Tid{}) {
    const int lane = tid() & (kWave - 1);
    if (KC) return *reinterpret_cast<const f32x4_t *>(lds + kl_off(row0 + (lane & 31), 2 * cp + (lane >> 5)));
    const int mn = row0 + (lane & 31), k = 8 * cp + 4 * (lane >> 5);
    f32x4_t v;
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = *reinterpret_cast<const float *>(lds + ml_off_f32<ROWS>(k + s, mn));
    return v;
}

// Fragments of one half of a k-slice (bf16: one k16 step; fp32: one pair of
// 16-byte chunks) for the wave's kFM m-blocks and kFN n-blocks.
template <bool BF16> struct Frags;
template <> struct Frags<true> { bf16x8_t p[kFM], q[kFN]; };
template <> struct Frags<false> { f32x4_t p[kFM], q[kFN]; };

// Fragment j (0 .. kFM + kFN - 1) of one half: j < kFM is P block j, the
// rest Q block j - kFM.
template <bool BF16, bool PKC, bool QKC, int TN, class Tid = HwTid>
__device__ __forceinline__ void read_frag(Frags<BF16> &fr, const char *lds_p, const char *lds_q,
                                          int wm0, int wn0, int half, int j, Tid tid = Tid{}) {
    if constexpr (BF16) {
        if (j < kFM)
            fr.p[j] = frag_bf16<PKC, 256, Tid>(lds_p, wm0 + j * 32, half, tid);
        else
            fr.q[j - kFM] = frag_bf16<QKC, TN, Tid>(lds_q, wn0 + (j - kFM) * 32, half, tid);
    } else {
        if (j < kFM)
            fr.p[j] = frag_f32<PKC, 256, Tid>(lds_p, wm0 + j * 32, half, tid);
        else
            fr.q[j - kFM] = frag_f32<QKC, TN, Tid>(lds_q, wn0 + (j - kFM) * 32, half, tid);
    }
}

template <bool BF16, bool PKC, bool QKC, int TN, class Tid = HwTid>
__device__ __forceinline__ void read_frags(Frags<BF16> &fr, const char *lds_p, const char *lds_q,
                                           int wm0, int wn0, int half, Tid tid = Tid{}) {
#pragma unroll
    for (int j = 0; j < kFM + kFN; ++j) read_frag<BF16, PKC, QKC, TN, Tid>(fr, lds_p, lds_q, wm0, wn0, half, j, tid);
}

// acc[f][g]: 32 x 32 block (f along m, g along n) of the wave's tile.
// MFMA 32x32 layout: lane l holds column (l & 31) and, in register r, row
// 8*(r/4) + 4*(l/32) + (r%4) of the block.
template <bool BF16>
__device__ __forceinline__ void mma_half(const Frags<BF16> &fr, f32x16_t (&acc)[kFM][kFN]) {
    if constexpr (BF16) {
#pragma unroll
        for (int f = 0; f < kFM; ++f)
#pragma unroll
            for (int g = 0; g < kFN; ++g)
                acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.p[f], fr.q[g], acc[f][g], 0, 0, 0);
    } else {
        // fp32: MFMA step s contracts element s of each lane's 4 k values.
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int f = 0; f < kFM; ++f)
#pragma unroll
                for (int g = 0; g < kFN; ++g)
                    acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.p[f][st], fr.q[g][st], acc[f][g], 0, 0, 0);
    }
}

// Block i (f = i / kFN, g = i % kFN) of mma_half.
template <bool BF16>
__device__ __forceinline__ void mma_step(const Frags<BF16> &fr, f32x16_t (&acc)[kFM][kFN], int i) {
    const int f = i / kFN, g = i % kFN;
    if constexpr (BF16) {
        acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.p[f], fr.q[g], acc[f][g], 0, 0, 0);
    } else {
#pragma unroll
        for (int st = 0; st < 4; ++st)
            acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.p[f][st], fr.q[g][st], acc[f][g], 0, 0, 0);
    }
}

// The product adds -3 X to the accumulators, so that the epilogue's
// -0.5 s * acc is s (1.5 X - 0.5 A X) without reading X again: -3 X is the
// product of -3 I with the X fragments already in registers, issued at the
// slices whose k range holds the output rows (wide: A X, identity on the P
// side) or columns (tall: X A, identity on the Q side). -3 is exact in bf16
// and the products are exact in fp32.
enum IdSide { ID_NONE = 0, ID_P = 1, ID_Q = 2 };

// Coefficient of the identity term: -3, or, in the first iteration under
// spectral scaling, -3 / s^2. There A enters unscaled and the accumulators
// are multiplied by s^2 before the epilogue, so that s^2 (A - 3 / s^2 I) X
// stands for (s^2 A - 3 I) X without a rescaled copy of A. A bf16 fragment
// holds the coefficient as the sum hi + lo of two bf16 values (relative
// error below 2^-17; lo = 0 for -3, and its MFMA is issued only when lo is
// not 0), an fp32 fragment whole. Every field is wave-uniform.
struct IdCoef {
    uint32_t hi, lo;  // bf16 bits
    float f;
};
constexpr IdCoef kIdMinus3{0xc040u, 0u, -3.0f};

// s2: the unit's s^2. It is 0 when lambda is 0 or not finite; then s = 0 as
// well, and -3 keeps the accumulators as finite as they were.
__device__ __forceinline__ IdCoef id_coef_spectral(float s2) {
    const float c = s2 > 0.f ? -3.0f / s2 : -3.0f;
    const uint32_t hi = f32_to_bf16_bits(c);
    const uint32_t lo = f32_to_bf16_bits(c - __uint_as_float(hi << 16));  // c - hi is exact
    return IdCoef{(uint32_t)__builtin_amdgcn_readfirstlane((int)hi),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)lo),
                  __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)))};
}

// One-hot fragment of the bf16 value with bits h: lane l, k index kl (within
// the 32-row block) holds it where kl equals the lane's row (l & 31).
template <class Tid = HwTid>
__device__ __forceinline__ bf16x8_t id_frag_bf16(int roff, int kk, uint32_t h, Tid tid = Tid{}) {
    const int lane = tid() & (kWave - 1);
    const int j = (lane & 31) - roff - 16 * kk - 8 * (lane >> 5);  // element holding h
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        w[e] = (j == 2 * e ? h : 0u) | (j == 2 * e + 1 ? h << 16 : 0u);
    return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

template <class Tid = HwTid>
__device__ __forceinline__ f32x4_t id_frag_f32(int roff, int cp, float c, Tid tid = Tid{}) {
    const int lane = tid() & (kWave - 1);
    const int j = (lane & 31) - roff - 8 * cp - 4 * (lane >> 5);
    f32x4_t v;
#pragma unroll
    for (int st = 0; st < 4; ++st) v[st] = j == st ? c : 0.0f;
    return v;
}

// d = slice index minus the wave's first identity slice.
template <bool BF16, int SIDE>
__device__ __forceinline__ void mma_identity(const Frags<BF16> &fr, f32x16_t (&acc)[kFM][kFN], int d,
                                             int half, const IdCoef &ic) {
    constexpr int RS = Elem<BF16>::BK;  // k rows per slice
    constexpr int WS = SIDE == ID_Q ? kWaveN : kWaveM;  // wave extent on the identity side
    constexpr int NB = WS / 32, NO = SIDE == ID_Q ? kFM : kFN;
    if (SIDE == ID_NONE || d < 0 || d >= WS / RS) return;
    const int blk = d * RS / 32, roff = (d * RS) % 32;
    if constexpr (BF16) {
        for (int part = 0; part < 2; ++part) {
            const uint32_t h = part == 0 ? ic.hi : ic.lo;
            if (part == 1 && h == 0u) break;
            const bf16x8_t id = id_frag_bf16(roff, half, h);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b == blk)
#pragma unroll
                    for (int o = 0; o < NO; ++o) {
                        if constexpr (SIDE == ID_P)
                            acc[b][o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id, fr.q[o], acc[b][o], 0, 0, 0);
                        else
                            acc[o][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.p[o], id, acc[o][b], 0, 0, 0);
                    }
        }
    } else {
        const f32x4_t id = id_frag_f32(roff, half, ic.f);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b == blk)
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int o = 0; o < NO; ++o) {
                        if constexpr (SIDE == ID_P)
                            acc[b][o] = __builtin_amdgcn_mfma_f32_32x32x2f32(id[st], fr.q[o][st], acc[b][o], 0, 0, 0);
                        else
                            acc[o][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.p[o][st], id[st], acc[o][b], 0, 0, 0);
                    }
    }
}

// Identity term of iteration J of a rotated k loop (the tile's own 256 k
// come first, see tile_mainloop): the slice covers k = J * BK .. + BK - 1 of
// the tile, i.e. rows (ID_P) or columns (ID_Q) w0 + 32 b + roff .. of the
// wave's extent WS on that side when J * BK lies in [w0, w0 + WS). Other
// waves have no term at this slice and skip it (a wave-uniform branch: their
// fragment would be all zeros, and adding exact zeros to an accumulator that
// starts at +0 changes no bit).
template <bool BF16, int SIDE, int J, class Tid = HwTid>
__device__ __forceinline__ void mma_identity_at(const Frags<BF16> &fr, f32x16_t (&acc)[kFM][kFN], int w0,
                                                int half, const IdCoef &ic, Tid tid = Tid{}) {
    constexpr int RS = Elem<BF16>::BK;
    constexpr int WS = SIDE == ID_Q ? kWaveN : kWaveM;
    constexpr int NO = SIDE == ID_Q ? kFM : kFN;
    constexpr int kb = J * RS;
    constexpr int b = (kb % WS) / 32, roff = kb % 32;
    if (__builtin_amdgcn_readfirstlane(kb / WS == w0 / WS ? 1 : 0) == 0) return;
    if constexpr (BF16) {
        const bf16x8_t id = id_frag_bf16<Tid>(roff, half, ic.hi, tid);
#pragma unroll
        for (int o = 0; o < NO; ++o) {
            if constexpr (SIDE == ID_P)
                acc[b][o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id, fr.q[o], acc[b][o], 0, 0, 0);
            else
                acc[o][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.p[o], id, acc[o][b], 0, 0, 0);
        }
        if (ic.lo != 0u) {
            const bf16x8_t il = id_frag_bf16<Tid>(roff, half, ic.lo, tid);
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                if constexpr (SIDE == ID_P)
                    acc[b][o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(il, fr.q[o], acc[b][o], 0, 0, 0);
                else
                    acc[o][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.p[o], il, acc[o][b], 0, 0, 0);
            }
        }
    } else {
        const f32x4_t id = id_frag_f32<Tid>(roff, half, ic.f, tid);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                if constexpr (SIDE == ID_P)
                    acc[b][o] = __builtin_amdgcn_mfma_f32_32x32x2f32(id[st], fr.q[o][st], acc[b][o], 0, 0, 0);
                else
                    acc[o][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.p[o][st], id[st], acc[o][b], 0, 0, 0);
            }
    }
}

template <int... Js, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Js...>, F &&f) {
    (f(std::integral_constant<int, Js>{}), ...);
}

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)p);
}

// Full K loop of one tile. S = L::kStages LDS buffers hold k-slices
// kt .. kt + S - 1; the direct-to-LDS loads run up to S slices ahead of the
// MFMAs. Each slice is consumed in two halves; the barrier that hands over
// slice kt + 1 (and frees slice kt's buffer for slice kt + S) sits between
// them, and the first fragments of slice kt + 1 are read while the second
// half of slice kt is still in the MFMA pipe.
// id_origin: tile origin (rows for ID_P, columns for ID_Q) of the identity
// term; unused for ID_NONE.
template <class L, bool BF16, bool PKC, bool QKC, int SIDE = ID_NONE>
__device__ __forceinline__ void tile_mainloop(const Operand &P, const Operand &Q, char *smem,
                                              f32x16_t (&acc)[kFM][kFN], int id_origin = 0,
                                              IdCoef ic = kIdMinus3) {
    using E = Elem<BF16>;
    constexpr int TN = L::kTileN, S = L::kStages;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm0 = L::m0(wid), wn0 = L::n0(wid);
    const int id0 = (id_origin + (SIDE == ID_P ? wm0 : wn0)) / E::BK;  // first identity slice
#pragma unroll
    for (int f = 0; f < kFM; ++f)
#pragma unroll
        for (int g = 0; g < kFN; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;
    const int kt_n = (P.K + E::BK - 1) / E::BK;
    if (P.vec && Q.vec) {
        DmaLoader<BF16, PKC, L::kTileM, L::kWaves> lp;
        DmaLoader<BF16, QKC, TN, L::kWaves> lq;
        lp.init(P);
        lq.init(Q);
        constexpr int PL = L::kPLoads, QL = L::kQLoads, NLD = PL + QL;
        const uint32_t lds0 = lds_addr(smem);
        // The product visits its k slices starting at the tile's own k range
        // on the identity side (rotation), so that the identity term falls on
        // the first NID iterations, which are unrolled. Iteration j reads
        // slice (j + rot) mod kt_n; iterations j >= kt_n, and every load
        // issued past the last iteration, read beyond K and land as zeros, so
        // every iteration issues the same loads and waits for the same count.
        constexpr int NID = SIDE == ID_NONE ? 0 : (SIDE == ID_Q ? TN : L::kTileM) / E::BK;
        const int rot = SIDE == ID_NONE ? 0 : (id_origin / E::BK) % kt_n;
        const int iters = kt_n > NID ? kt_n : NID;
        auto slice_of = [&](int j) {
            const int t = j + rot;
            return j >= kt_n ? kt_n : (t < kt_n ? t : t - kt_n);
        };
        // Slice j + S - 1's Q loads go out in the first half of iteration j
        // and slice j + S's P loads in its second half, so the prologue issues
        // slices 0 .. S - 2 and the P part of slice S - 1.
#pragma unroll
        for (int st = 0; st < S - 1; ++st) {
            lp.issue(slice_of(st), lds0 + st * L::kStageBytes);
            lq.issue(slice_of(st), lds0 + st * L::kStageBytes + L::kPBytes);
        }
        lp.issue(slice_of(S - 1), lds0 + (S - 1) * L::kStageBytes);
        wait_vm_lgkm0<(S - 2) * NLD + PL>();  // slice 0 landed
        lds_barrier();
        Frags<BF16> fa, fb;
        read_frags<BF16, PKC, QKC, TN>(fa, smem, smem + L::kPBytes, wm0, wn0, 0);
        // Iteration j: the MFMAs of the first half (fa) run while the second
        // half's fragments (fb) are read and the Q part of slice j + S - 1 is
        // loaded into the buffer slice j - 1 left; after the barrier that
        // hands over slice j + 1, the MFMAs of fb run while the first half of
        // slice j + 1 is read and the P part of slice j + S is loaded into the
        // buffer slice j leaves. Each MFMA step carries at most one fragment
        // read and one load, so the matrix pipe does not wait behind a run of
        // them.
        constexpr int kSteps = kFM * kFN, kFrag = kFM + kFN;
        constexpr int eQ = kSteps / QL, eP = kSteps / PL;  // MFMA steps per load
        static_assert(kFrag <= kSteps && eQ * QL == kSteps && eP * PL == kSteps, "interleave");
        const int w0 = SIDE == ID_Q ? wn0 : wm0;
        auto iteration = [&](int j, auto jid) {
            constexpr int JID = decltype(jid)::value;  // unrolled identity iteration, or -1
            const char *cur = smem + (j % S) * L::kStageBytes;
            const int late = slice_of(j + S - 1);  // its buffer was freed by barrier j - 1
            const uint32_t late_dst = lds0 + ((j + S - 1) % S) * L::kStageBytes + L::kPBytes;
#pragma unroll
            for (int i = 0; i < kSteps; ++i) {
                mma_step<BF16>(fa, acc, i);
                if (i < kFrag) read_frag<BF16, PKC, QKC, TN>(fb, cur, cur + L::kPBytes, wm0, wn0, 1, i);
                if (i % eQ == eQ - 1) lq.issue_one(late, late_dst, i / eQ);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (JID >= 0) mma_identity_at<BF16, SIDE, JID>(fa, acc, w0, 0, ic);
            wait_vm_lgkm0<(S - 2) * NLD>();
            lds_barrier();
            const char *nxt = smem + ((j + 1) % S) * L::kStageBytes;
            const uint32_t dst = lds0 + (j % S) * L::kStageBytes;
            const int refill = slice_of(j + S);
#pragma unroll
            for (int i = 0; i < kSteps; ++i) {
                mma_step<BF16>(fb, acc, i);
                if (i < kFrag) read_frag<BF16, PKC, QKC, TN>(fa, nxt, nxt + L::kPBytes, wm0, wn0, 0, i);
                if (i % eP == eP - 1) lp.issue_one(refill, dst, i / eP);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (JID >= 0) mma_identity_at<BF16, SIDE, JID>(fb, acc, w0, 1, ic);
        };
        static_for(std::make_integer_sequence<int, NID>{}, [&](auto jid) { iteration(decltype(jid)::value, jid); });
        for (int j = NID; j < iters; ++j) iteration(j, std::integral_constant<int, -1>{});
        wait_vm_lgkm0<0>();  // the zero-fill loads past the end write LDS too
    } else {
        SlowLoader<BF16, PKC, L::kTileM, L::kThreads> lp;
        SlowLoader<BF16, QKC, TN, L::kThreads> lq;
        lp.init(P);
        lq.init(Q);
        for (int kt = 0; kt < kt_n; ++kt) {
            lp.load_store(kt, smem);
            lq.load_store(kt, smem + L::kPBytes);
            __syncthreads();
            Frags<BF16> fa;
            read_frags<BF16, PKC, QKC, TN>(fa, smem, smem + L::kPBytes, wm0, wn0, 0);
            mma_half<BF16>(fa, acc);
            mma_identity<BF16, SIDE>(fa, acc, kt - id0, 0, ic);
            read_frags<BF16, PKC, QKC, TN>(fa, smem, smem + L::kPBytes, wm0, wn0, 1);
            mma_half<BF16>(fa, acc);
            mma_identity<BF16, SIDE>(fa, acc, kt - id0, 1, ic);
            __syncthreads();
        }
    }
    __syncthreads();  // every wave is done with the slices before LDS is reused
}

// Tile -> matrix lookup in two steps, so that the table load goes out at
// kernel entry together with the other kernel-argument loads: lane j reads
// start j of the batch's table (non-decreasing, entry 0 is 0, unused entries
// INT32_MAX) with one vector load straight from the kernel-argument segment
// (the batch is the kernel's only argument); the index of the matrix holding
// tile t is then the count of starts <= t, less one. A scalar scan of the
// table waits for its loads in several dependent batches.
__device__ __forceinline__ int ns_start_of_lane() {
    static_assert(kMaxMatsPerLaunch <= kWave, "one start per lane");
    using CChar = const __attribute__((address_space(4))) char;
    using CInt = const __attribute__((address_space(4))) int;
    CChar *k = (CChar *)__builtin_amdgcn_kernarg_segment_ptr();
    CInt *starts = reinterpret_cast<CInt *>(k + offsetof(NsBatch, starts));
    const int lane = threadIdx.x & (kWave - 1);
    return lane < kMaxMatsPerLaunch ? starts[lane] : INT32_MAX;
}
__device__ __forceinline__ int find_ns_mat(int start_of_lane, int t) {
    return __popcll(__ballot(start_of_lane <= t)) - 1;
}

// Descriptor mi of the batch in one vector load (lane d reads its dword d),
// broadcast back field by field: its fields arrive together, where the
// compiler's scalar loads would come in several batches with a wait each.
__device__ __forceinline__ NsMat load_ns_mat(int mi) {
    constexpr int ND = (int)(sizeof(NsMat) / 4);
    static_assert(sizeof(NsMat) % 4 == 0 && ND <= kWave, "descriptor dwords");
    using CChar = const __attribute__((address_space(4))) char;
    using CInt = const __attribute__((address_space(4))) int;
    CChar *k = (CChar *)__builtin_amdgcn_kernarg_segment_ptr();
    CInt *p = reinterpret_cast<CInt *>(k + offsetof(NsBatch, mat) + (size_t)mi * sizeof(NsMat));
    const int lane = threadIdx.x & (kWave - 1);
    const int v = lane < ND ? p[lane] : 0;
    int d[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) d[i] = __builtin_amdgcn_readlane(v, i);
    NsMat m;
    __builtin_memcpy(&m, d, sizeof(NsMat));
    return m;
}

// Descriptor mi of the batch (mi uniform) and a unit's {s, s^2}, by scalar
// loads: for a kernel that decodes its next tile while its own direct-to-LDS
// loads are in flight, since the waits for scalar loads count only scalar
// and LDS operations, not the vector memory operations those loads are.
__device__ __forceinline__ NsMat load_ns_mat_scalar(int mi) {
    constexpr int ND = (int)(sizeof(NsMat) / 4);
    using CChar = const __attribute__((address_space(4))) char;
    using CInt = const __attribute__((address_space(4))) int;
    CChar *k = (CChar *)__builtin_amdgcn_kernarg_segment_ptr();
    CInt *p = reinterpret_cast<CInt *>(k + offsetof(NsBatch, mat) + (size_t)mi * sizeof(NsMat));
    int d[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) d[i] = p[i];
    NsMat m;
    __builtin_memcpy(&m, d, sizeof(NsMat));
    return m;
}
__device__ __forceinline__ float load_scale_scalar(const float2 *scales, int unit, int which) {
    using CFloat = const __attribute__((address_space(4))) float;
    CFloat *p = (CFloat *)(uintptr_t)scales;
    return p[2 * unit + which];
}

// The first iteration's scale, loaded at the start of a tile but selected
// and used only in its epilogue, so that the load does not hold up the
// tile's start (the array covers every unit, so the read is always valid).
struct LateScale {
    float raw;
    int use;
    __device__ float get() const { return use ? raw : 1.0f; }
};

// ---------------------------------------------------------------------------
// Epilogue helpers. A wave stages 32 rows x kWaveN columns of fp32 in LDS
// (row stride kStageStride floats) to turn the MFMA register layout into
// row-major 4-column pieces: kLanesPerRow lanes cover one staged row, so one
// instruction covers kRowsPerInstr rows.
// ---------------------------------------------------------------------------
constexpr int kStageStride = kWaveN + 8;  // 4 rows apart = 32 banks apart
constexpr int kLanesPerRow = kWaveN / 4, kRowsPerInstr = kWave / kLanesPerRow;
constexpr int kWordsPerRow = kWaveN / 64;  // packed sign words per wave row
static_assert(GramLay::kWaves * 32 * kStageStride * 4 <= GramLay::kLdsBytes &&
                  ProdLay::kWaves * 32 * kStageStride * 4 <= ProdLay::kLdsBytes,
              "epilogue stage exceeds LDS");
static_assert(kWaveN % 64 == 0, "a packed word spans 64 columns of one wave");

__device__ __forceinline__ void stage_rows(const f32x16_t (&acc)[kFM][kFN], int f, float *stage,
                                           float scale) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int g = 0; g < kFN; ++g)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
            stage[row * kStageStride + 32 * g + (lane & 31)] = acc[f][g][rr] * scale;
        }
}

// Orders one wave's LDS staging writes before its reads of other lanes'
// entries (LDS executes a wave's instructions in order; this keeps the
// compiler from reordering them).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
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
            const uint32_t lo = pack_bf16x2(v[0], v[1]);
            const uint32_t hi = pack_bf16x2(v[2], v[3]);
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
// 32 consecutive values at element index idx (one mirrored row segment).
// FAST: 16-byte stores (the caller guarantees bounds and alignment).
template <bool BF16, bool FAST>
__device__ __forceinline__ void store32(void *p, int64_t idx, const float (&v)[32], bool row_ok,
                                        int cols_left) {
    if (FAST && BF16) {
        uint4 *q = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p) + idx);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack_bf16x2(v[8 * c + 2 * e], v[8 * c + 2 * e + 1]);
            q[c] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else if (FAST) {
        float4 *q = reinterpret_cast<float4 *>(static_cast<float *>(p) + idx);
#pragma unroll
        for (int c = 0; c < 8; ++c) q[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float w[4] = {v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
            store4<BF16, false>(p, idx + 4 * c, w, row_ok, cols_left - 4 * c);
        }
    }
}

// Each wave stages its kWaveM x kWaveN result 32 rows at a time in its own
// LDS area, then writes the rows (4 columns per lane) and, above the
// diagonal, the mirrored tile: a lane reads one column of the staged rows,
// which is 32 consecutive entries of a mirrored row, and stores them as one
// run. (Storing the mirror straight from the accumulators, 4 entries of a
// mirrored row per lane, was slower: each store instruction then touches 32
// rows.)
template <bool BF16, bool FAST>
__device__ __forceinline__ void gram_epilogue(f32x16_t (&acc)[kFM][kFN], char *smem, int ti, int tj,
                                              int r, LateScale sc, void *a) {
    const float scale = sc.get();
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int m0 = ti * kNsTileM + GramLay::m0(wid), n0 = tj * kNsTileM + GramLay::n0(wid);
    float *stage = reinterpret_cast<float *>(smem) + wid * 32 * kStageStride;
    const bool mirror = ti < tj;
#pragma unroll
    for (int f = 0; f < kFM; ++f) {
        stage_rows(acc, f, stage, scale);
        wave_lds_fence();
        // Direct tile, row-major: 4 columns per lane.
#pragma unroll 4
        for (int it = 0; it < 32 / kRowsPerInstr; ++it) {
            const int row = it * kRowsPerInstr + lane / kLanesPerRow, c4 = (lane % kLanesPerRow) * 4;
            const int gi = m0 + f * 32 + row, gj = n0 + c4;
            const float4 v4 = *reinterpret_cast<const float4 *>(stage + row * kStageStride + c4);
            float v[4] = {v4.x, v4.y, v4.z, v4.w};
            store4<BF16, FAST>(a, (int64_t)gi * r + gj, v, gi < r, r - gj);
        }
        if (mirror) {
#pragma unroll
            for (int it = 0; it < kWaveN / kWave; ++it) {
                const int col = it * kWave + lane;
                float v[32];
#pragma unroll
                for (int t = 0; t < 32; ++t) v[t] = stage[t * kStageStride + col];
                const int gj = n0 + col, gi = m0 + f * 32;
                store32<BF16, FAST>(a, (int64_t)gj * r + gi, v, gj < r, r - gi);
            }
        }
        wave_lds_fence();
    }
}

template <bool BF16, bool KC>
__device__ __forceinline__ void gram_tile(const Operand &P, const Operand &Q, char *smem, int ti,
                                          int tj, int r, LateScale sc, void *a) {
    f32x16_t acc[kFM][kFN];
    tile_mainloop<GramLay, BF16, KC, KC>(P, Q, smem, acc);
    const bool fast = P.vec && (r % Elem<BF16>::EPC) == 0 && (ti + 1) * kNsTileM <= r &&
                      (tj + 1) * kNsTileM <= r;
    if (fast)
        gram_epilogue<BF16, true>(acc, smem, ti, tj, r, sc, a);
    else
        gram_epilogue<BF16, false>(acc, smem, ti, tj, r, sc, a);
}

// One k chunk of a split Gram tile: the unscaled fp32 sum, stored whole
// (256 x 256, row-major) at its place in M.out.
template <bool BF16, bool KC>
__device__ __forceinline__ void gram_partial_tile(const Operand &P, const Operand &Q, char *smem,
                                                  const NsMat &M, int w, int tile, int chunk) {
    f32x16_t acc[kFM][kFN];
    tile_mainloop<GramLay, BF16, KC, KC>(P, Q, smem, acc);
    const int r = M.R <= M.C ? M.R : M.C;
    const int T_ = (r + kNsTileM - 1) / kNsTileM;
    float *part = static_cast<float *>(M.out) +
                  ((int64_t)(w * (T_ * (T_ + 1) / 2) + tile) * M.split + chunk) * (kNsTileM * kNsTileM);
    gram_epilogue<false, true>(acc, smem, 0, 0, kNsTileM, LateScale{1.0f, 0}, part);
}

// SPLIT: each tile's k range is cut into M.split chunks, one block each;
// a block writes its chunk's unscaled fp32 sum as a full 256 x 256 tile to
// M.out (worker stride tiles * split tiles, tile t's chunks consecutive) and
// gram_reduce_kernel adds the chunks in order, scales and stores A.
template <bool BF16, bool SPLIT = false>
__global__ __launch_bounds__(GramLay::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_gram_kernel(NsBatch b) {
    using T = typename Elem<BF16>::T;
    __shared__ __attribute__((aligned(16))) char smem[GramLay::kLdsBytes];
    const int sv = ns_start_of_lane();
    const int lt = xcd_remap(blockIdx.x, b.total_tiles);  // the grid is one block per tile
    const int w = lt / b.tiles_per_worker_all;
    const int lw = lt - w * b.tiles_per_worker_all;
    const NsMat M = load_ns_mat(find_ns_mat(sv, lw));
    int t = lw - M.tile_begin;
    int chunk = 0;
    if constexpr (SPLIT) {
        chunk = t % M.split;
        t /= M.split;
    }
    const bool wide = M.R <= M.C;
    const int r = wide ? M.R : M.C, c = wide ? M.C : M.R;
    const int T_ = (r + kNsTileM - 1) / kNsTileM;
    const int tile = t;
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
    const LateScale sc{b.scales[M.unit_begin + w].y, b.use_scales};
    void *a = static_cast<char *>(M.a) + (int64_t)w * r * r * (int64_t)sizeof(T);
    int k0 = 0, kn = c;
    if constexpr (SPLIT) {
        // chunk of whole k slices: ceil(slices / split) slices each
        constexpr int BK = Elem<BF16>::BK;
        const int per = ((c + BK - 1) / BK + M.split - 1) / M.split * BK;
        k0 = chunk * per;
        kn = c - k0 < per ? c - k0 : per;
    }
    if (wide) {
        // Y = X (r x c, k-contiguous rows)
        const char *base = y + (int64_t)k0 * (int64_t)sizeof(T);
        Operand P{base + (int64_t)ti * kNsTileM * M.C * (int64_t)sizeof(T), M.C, r - ti * kNsTileM, kn, vec};
        Operand Q{base + (int64_t)tj * kNsTileM * M.C * (int64_t)sizeof(T), M.C, r - tj * kNsTileM, kn, vec};
        if constexpr (SPLIT)
            gram_partial_tile<BF16, true>(P, Q, smem, M, w, tile, chunk);
        else
            gram_tile<BF16, true>(P, Q, smem, ti, tj, r, sc, a);
    } else {
        // Y = X^T: element (i, k) of Y is X[k][i]: mn-contiguous, ld = C
        const char *base = y + (int64_t)k0 * M.C * (int64_t)sizeof(T);
        Operand P{base + (int64_t)ti * kNsTileM * (int64_t)sizeof(T), M.C, r - ti * kNsTileM, kn, vec};
        Operand Q{base + (int64_t)tj * kNsTileM * (int64_t)sizeof(T), M.C, r - tj * kNsTileM, kn, vec};
        if constexpr (SPLIT)
            gram_partial_tile<BF16, false>(P, Q, smem, M, w, tile, chunk);
        else
            gram_tile<BF16, false>(P, Q, smem, ti, tj, r, sc, a);
    }
}

// Sums the split Gram's chunks of 16 rows of one 256 x 256 tile per block,
// in chunk order, then stores A = scale * sum in the storage type (the tile
// and, above the diagonal, its mirror). 256 threads: 4 rows of 64 threads x
// 4 columns per pass.
template <bool BF16>
__global__ __launch_bounds__(256) void gram_reduce_kernel(NsBatch b) {
    constexpr int kRows = kNsTileM / kGramReduceParts;
    const int sv = ns_start_of_lane();
    const int lt = blockIdx.x;  // one block per (worker, tile, 16 rows)
    const int w = lt / b.tiles_per_worker_all;
    const int lw = lt - w * b.tiles_per_worker_all;
    const NsMat M = load_ns_mat(find_ns_mat(sv, lw));
    const int rows0 = (lw - M.tile_begin) % kGramReduceParts * kRows;  // this block's rows
    int t = (lw - M.tile_begin) / kGramReduceParts;
    const int r = M.R <= M.C ? M.R : M.C;
    const int T_ = (r + kNsTileM - 1) / kNsTileM;
    const int tile = t;
    int ti = 0;
    while (t >= T_ - ti) {
        t -= T_ - ti;
        ++ti;
    }
    const int tj = ti + t;
    const int tiles = T_ * (T_ + 1) / 2;
    const float *part = static_cast<const float *>(M.out) +
                        ((int64_t)(w * tiles + tile) * M.split) * (kNsTileM * kNsTileM);
    void *a = static_cast<char *>(M.a) + (int64_t)w * r * r * (int64_t)sizeof(typename Elem<BF16>::T);
    const float scale = b.use_scales ? b.scales[M.unit_begin + w].y : 1.0f;
    const int c4 = (threadIdx.x & 63) * 4;
    for (int row = rows0 + (threadIdx.x >> 6); row < rows0 + kRows; row += 4) {
        const int gi = ti * kNsTileM + row, gj = tj * kNsTileM + c4;
        if (gi >= r || gj >= r) continue;
        float4 sum = *reinterpret_cast<const float4 *>(part + row * kNsTileM + c4);
        for (int s = 1; s < M.split; ++s) {
            const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)s * kNsTileM * kNsTileM +
                                                               row * kNsTileM + c4);
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
        }
        const float v[4] = {sum.x * scale, sum.y * scale, sum.z * scale, sum.w * scale};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (gj + e >= r) break;
            store_val<BF16>(a, (int64_t)gi * r + gj + e, v[e]);
            if (ti < tj) store_val<BF16>(a, (int64_t)(gj + e) * r + gi, v[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// Product tile: X' = gamma (A X - 3 X) or (X A - 3 X), with the epilogue EPI.
// ---------------------------------------------------------------------------
struct ProductArgs {
    void *out;       // this worker's output (U / next iterate) or W
    uint64_t *pk;    // this worker's packed words or nullptr
    float *u_out;    // EPI_WUPD: U (fp32) as well, or nullptr
    int8_t *i8;      // EPI_FINAL_I8: this worker's int8 signs
    int R, C, ti, tj;
    LateScale s;     // -0.5 s is the epilogue's factor gamma
    float eta;
    IdCoef idc;      // coefficient of the identity term
    float s2;        // spectral0: the accumulators' factor before the epilogue
    int spectral0;   // first product under spectral scaling (A unscaled)
};

// First product under spectral scaling: acc *= s^2 (see IdCoef).
__device__ __forceinline__ void scale_acc(f32x16_t (&acc)[kFM][kFN], float s2) {
#pragma unroll
    for (int f = 0; f < kFM; ++f)
#pragma unroll
        for (int g = 0; g < kFN; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] *= s2;
}

// Epilogue of the product, 32 rows of the wave's tile at a time through
// LDS: u = gamma * acc row-major (4 columns per lane), stored as
// EPI asks; int8 signs (u >= 0 -> +1, else -1) go out 4 per lane; for the
// fused sign + pack, u goes back to LDS and each packed word is the ballot of
// 64 consecutive columns of one row (needs C % 64 == 0).
template <bool BF16, int EPI, bool FAST>
__device__ __forceinline__ void product_epilogue(const ProductArgs &pa, f32x16_t (&acc)[kFM][kFN],
                                                 char *smem) {
    const int R = pa.R, C = pa.C;
    const float gamma = -0.5f * pa.s.get();
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int m0 = pa.ti * kNsTileM + ProdLay::m0(wid), n0 = pa.tj * kNsProdTileN + ProdLay::n0(wid);
    float *stage = reinterpret_cast<float *>(smem) + wid * 32 * kStageStride;
    constexpr bool kFinal = EPI == EPI_FINAL || EPI == EPI_FINAL_I8;
    const bool want_out = EPI == EPI_ITER || EPI == EPI_WUPD || (kFinal && pa.out);
    const bool want_pack = EPI == EPI_FINAL && pa.pk;
    constexpr bool want_i8 = EPI == EPI_FINAL_I8;
#pragma unroll
    for (int f = 0; f < kFM; ++f) {
        stage_rows(acc, f, stage, 1.0f);
        wave_lds_fence();
#pragma unroll 4
        for (int it = 0; it < 32 / kRowsPerInstr; ++it) {
            const int row = it * kRowsPerInstr + lane / kLanesPerRow, c4 = (lane % kLanesPerRow) * 4;
            const int gm = m0 + f * 32 + row, gn = n0 + c4;
            const int64_t idx = (int64_t)gm * C + gn;
            float *sp = stage + row * kStageStride + c4;
            const float4 v4 = *reinterpret_cast<const float4 *>(sp);
            const float v[4] = {v4.x, v4.y, v4.z, v4.w};
            float u[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool ok = FAST || (gm < R && gn + t < C);
                u[t] = ok ? gamma * v[t] : 0.f;
            }
            if (want_out) {
                if (EPI == EPI_ITER) {
                    store4<BF16, FAST>(pa.out, idx, u, gm < R, C - gn);
                } else if (kFinal) {
                    store4<false, FAST>(pa.out, idx, u, gm < R, C - gn);
                } else {
                    float w[4];
                    load4<false, FAST>(pa.out, idx, w, gm < R, C - gn);
#pragma unroll
                    for (int t = 0; t < 4; ++t) w[t] = __builtin_fmaf(-pa.eta, u[t], w[t]);
                    store4<false, FAST>(pa.out, idx, w, gm < R, C - gn);
                    if (pa.u_out) store4<false, FAST>(pa.u_out, idx, u, gm < R, C - gn);
                }
            }
            if (want_i8) {
                uint32_t q = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) q |= (u[t] >= 0.f ? 0x01u : 0xffu) << (8 * t);
                if (FAST) {
                    *reinterpret_cast<uint32_t *>(pa.i8 + idx) = q;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (gm < R && gn + t < C) pa.i8[idx + t] = (int8_t)(q >> (8 * t));
                }
            }
            if (want_pack) *reinterpret_cast<float4 *>(sp) = make_float4(u[0], u[1], u[2], u[3]);
        }
        if (want_pack) {
            wave_lds_fence();
            // word q: row q / kWordsPerRow, columns 64 (q % kWordsPerRow) ..
            uint64_t mine = 0;
#pragma unroll 8
            for (int q = 0; q < 32 * kWordsPerRow; ++q) {
                const float v = stage[(q / kWordsPerRow) * kStageStride + 64 * (q % kWordsPerRow) + lane];
                const uint64_t bal = __ballot(v >= 0.f);
                if (lane == q) mine = bal;
            }
            const int gm = m0 + f * 32 + lane / kWordsPerRow, gn0 = n0 + 64 * (lane % kWordsPerRow);
            if (lane < 32 * kWordsPerRow && gm < R && gn0 < C) pa.pk[((int64_t)gm * C + gn0) >> 6] = mine;
        }
        wave_lds_fence();
    }
}

// Sign + pack straight from the accumulators (final iteration, no U output):
// u = gamma * acc, bit = (u >= 0). With the MFMA 32x32 layout, the ballot of
// register rr of block (f, g) holds row R0 (lanes 0-31) and row R0 + 4
// (lanes 32-63) over the block's 32 columns; blocks 2 gp and 2 gp + 1 give
// the 64 columns of one packed word (C % 64 == 0). Word id of the wave goes
// to lane id % 64, slot id / 64; each lane then stores its kSignSlots words.
// dst in lane `lane` <- val (a uniform value); the other lanes keep dst.
__device__ __forceinline__ int write_lane(int dst, uint32_t val, int lane) {
    asm("v_writelane_b32 %0, %1, %2" : "+v"(dst) : "s"(val), "i"(lane));
    return dst;
}

constexpr int kSignSlots = kWaveM * kWordsPerRow / kWave;  // sign words per lane

// Gathers the wave's sign words (u = gamma * acc, bit = (u >= 0)) into
// lo / hi (32-bit halves): word id of the wave sits in lane id % 64, slot
// id / 64.
template <class Tid>
__device__ __forceinline__ void gather_sign_words(const ProductArgs &pa, const f32x16_t (&acc)[kFM][kFN], Tid tid,
                                                  int (&lo)[kSignSlots], int (&hi)[kSignSlots]) {
    const float gamma = -0.5f * pa.s.get();
    (void)tid;
#pragma unroll
    for (int sl = 0; sl < kSignSlots; ++sl) lo[sl] = hi[sl] = 0;
#pragma unroll
    for (int f = 0; f < kFM; ++f) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
#pragma unroll
            for (int gp = 0; gp < kWordsPerRow; ++gp) {
                const uint64_t b0 = __ballot(gamma * acc[f][2 * gp][rr] >= 0.f);
                const uint64_t b1 = __ballot(gamma * acc[f][2 * gp + 1][rr] >= 0.f);
                const int id = ((f * 16 + rr) * kWordsPerRow + gp) * 2;  // even
                // row R0: lanes 0-31 of both blocks; row R0 + 4: lanes 32-63
                lo[id >> 6] = write_lane(lo[id >> 6], (uint32_t)b0, id & 63);
                hi[id >> 6] = write_lane(hi[id >> 6], (uint32_t)b1, id & 63);
                lo[id >> 6] = write_lane(lo[id >> 6], (uint32_t)(b0 >> 32), (id + 1) & 63);
                hi[id >> 6] = write_lane(hi[id >> 6], (uint32_t)(b1 >> 32), (id + 1) & 63);
                // consume each pair of ballots before the next (bounds the
                // live scalar masks)
                __builtin_amdgcn_sched_barrier(0);
            }
    }
}

// Matrix row and first column of word id of wave wid's tile part.
__device__ __forceinline__ void sign_word_origin(const ProductArgs &pa, int wid, int id, int &gm, int &gn0) {
    const int m0 = pa.ti * kNsTileM + ProdLay::m0(wid), n0 = pa.tj * kNsProdTileN + ProdLay::n0(wid);
    const int hrow = id & 1, gp = (id >> 1) % kWordsPerRow, fr = (id >> 1) / kWordsPerRow;
    const int rr = fr & 15, f = fr >> 4;
    gm = m0 + f * 32 + 8 * (rr >> 2) + (rr & 3) + 4 * hrow;
    gn0 = n0 + 64 * gp;
}

template <class Tid = HwTid>
__device__ __forceinline__ void pack_from_registers(const ProductArgs &pa, const f32x16_t (&acc)[kFM][kFN],
                                                    Tid tid = Tid{}) {
    int lo[kSignSlots], hi[kSignSlots];
    gather_sign_words(pa, acc, tid, lo, hi);
    const int lane = tid() & (kWave - 1), wid = tid() / kWave;
#pragma unroll
    for (int sl = 0; sl < kSignSlots; ++sl) {
        int gm, gn0;
        sign_word_origin(pa, wid, sl * 64 + lane, gm, gn0);
        const uint64_t word = (uint64_t)(uint32_t)lo[sl] | ((uint64_t)(uint32_t)hi[sl] << 32);
        if (gm < pa.R && gn0 < pa.C) pa.pk[((int64_t)gm * pa.C + gn0) >> 6] = word;
    }
}

// The same signs as int8 (+1 / -1), straight from the sign words: table entry
// b holds the 8 bytes of the 8 bits of b (LSB first), so a word's 64 columns
// are four 16-byte pieces (C % 64 == 0, 16-byte aligned rows). The four lanes
// of a quad take the quad's four words in turn (a quad_perm broadcast), and
// lane 4k + p writes piece p: each store instruction covers 16 rows with 64
// contiguous bytes each, where one lane per row would scatter 16 bytes into
// each of 64 rows.
template <class Tid>
__device__ __forceinline__ void int8_from_registers(const ProductArgs &pa, const f32x16_t (&acc)[kFM][kFN],
                                                    Tid tid, const uint2 *table) {
    int lo[kSignSlots], hi[kSignSlots];
    gather_sign_words(pa, acc, tid, lo, hi);
    const int lane = tid() & (kWave - 1), wid = tid() / kWave;
    const int p = lane & 3;
#pragma unroll
    for (int sl = 0; sl < kSignSlots; ++sl)
        static_for(std::make_integer_sequence<int, 4>{}, [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int kQuad = j * 0x55;  // quad_perm: every lane of the quad reads its lane j
            const uint32_t wl = (uint32_t)__builtin_amdgcn_update_dpp(0, lo[sl], kQuad, 0xf, 0xf, false);
            const uint32_t wh = (uint32_t)__builtin_amdgcn_update_dpp(0, hi[sl], kQuad, 0xf, 0xf, false);
            int gm, gn0;
            sign_word_origin(pa, wid, sl * 64 + (lane & ~3) + j, gm, gn0);
            const uint32_t bits = ((p < 2 ? wl : wh) >> (16 * (p & 1))) & 0xffffu;
            const uint2 a = table[bits & 0xffu], b = table[bits >> 8];
            if (gm < pa.R && gn0 < pa.C)
                *reinterpret_cast<uint4 *>(pa.i8 + (int64_t)gm * pa.C + gn0 + 16 * p) = make_uint4(a.x, a.y, b.x, b.y);
        });
}

// Epilogue of the walk for the next bf16 iterate (EPI_ITER), staged 8 rows
// at a time through the wave's own 8 x kStageStride floats outside the stage
// buffers, so that the next tile's loads keep landing meanwhile. Register
// 4q + t of block (f, g) holds row 8q + 4h + t (h = lane / 32) of the block;
// the arithmetic is that of product_epilogue (u = gamma * acc, one RNE
// rounding to bf16). (The W update is not walked: its loads of W, waited for
// one pass at a time, would serialise the epilogue.)
template <int EPI, bool FAST, class Tid>
__device__ __forceinline__ void walk_staged_epilogue(const ProductArgs &pa, const f32x16_t (&acc)[kFM][kFN],
                                                     Tid tid, float *estage) {
    const float gamma = -0.5f * pa.s.get();
    const int lane = tid() & (kWave - 1), wid = tid() / kWave;
    const int m0 = pa.ti * kNsTileM + ProdLay::m0(wid), n0 = pa.tj * kNsProdTileN + ProdLay::n0(wid);
    float *st = estage + wid * 8 * kStageStride;
    const int R = pa.R, C = pa.C;
#pragma unroll
    for (int f = 0; f < kFM; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int g = 0; g < kFN; ++g)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    st[(4 * (lane >> 5) + t) * kStageStride + 32 * g + (lane & 31)] = acc[f][g][4 * q + t] * 1.0f;
            wave_lds_fence();
#pragma unroll
            for (int it = 0; it < 8 / kRowsPerInstr; ++it) {
                const int row = it * kRowsPerInstr + lane / kLanesPerRow, c4 = (lane % kLanesPerRow) * 4;
                const int gm = m0 + f * 32 + 8 * q + row, gn = n0 + c4;
                const int64_t idx = (int64_t)gm * C + gn;
                const float4 v4 = *reinterpret_cast<const float4 *>(st + row * kStageStride + c4);
                const float v[4] = {v4.x, v4.y, v4.z, v4.w};
                float u[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) u[e] = (FAST || (gm < R && gn + e < C)) ? gamma * v[e] : 0.f;
                static_assert(EPI == EPI_ITER, "the staged walk epilogue writes the next iterate");
                store4<true, FAST>(pa.out, idx, u, gm < R, C - gn);
            }
            wave_lds_fence();
        }
}

// Entry e of the int8 table: byte j is +1 where bit j of e is set, else -1.
__device__ __forceinline__ uint2 int8_table_entry(int e) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j >> 2] |= (((e >> j) & 1) ? 0x01u : 0xffu) << (8 * (j & 3));
    return make_uint2(w[0], w[1]);
}

template <bool BF16, bool QKC, int EPI>
__device__ __forceinline__ void product_tile(const Operand &P, const Operand &Q, char *smem,
                                             const ProductArgs &pa) {
    f32x16_t acc[kFM][kFN];
    // wide (Q = X, mn-contiguous): -3 X enters on the P side at the output
    // rows; tall (Q = A): on the Q side at the output columns.
    if constexpr (QKC)
        tile_mainloop<ProdLay, BF16, true, QKC, ID_Q>(P, Q, smem, acc, pa.tj * kNsProdTileN, pa.idc);
    else
        tile_mainloop<ProdLay, BF16, true, QKC, ID_P>(P, Q, smem, acc, pa.ti * kNsTileM, pa.idc);
    if (pa.spectral0) scale_acc(acc, pa.s2);
    if (EPI == EPI_FINAL && pa.pk && !pa.out) {
        pack_from_registers(pa, acc);
        return;
    }
    const bool fast = P.vec && (pa.ti + 1) * kNsTileM <= pa.R && (pa.tj + 1) * kNsProdTileN <= pa.C;
    if (fast)
        product_epilogue<BF16, EPI, true>(pa, acc, smem);
    else
        product_epilogue<BF16, EPI, false>(pa, acc, smem);
}

template <bool BF16, int EPI>
__global__ __launch_bounds__(ProdLay::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_product_kernel(NsBatch b) {
    using T = typename Elem<BF16>::T;
    __shared__ __attribute__((aligned(16))) char smem[ProdLay::kLdsBytes];
    const int sv = ns_start_of_lane();
    const int lt = xcd_remap(blockIdx.x, b.total_tiles);  // the grid is one block per tile
    const int w = lt / b.tiles_per_worker_all;
    const int lw = lt - w * b.tiles_per_worker_all;
    const NsMat M = load_ns_mat(find_ns_mat(sv, lw));
    const int t = lw - M.tile_begin;
    const int R = M.R, C = M.C;
    const bool wide = R <= C;
    const int r = wide ? R : C;
    const int tiles_n = (C + kNsProdTileN - 1) / kNsProdTileN;
    const int ti = t / tiles_n, tj = t - ti * tiles_n;
    const int64_t n = (int64_t)R * C;
    const char *x = static_cast<const char *>(M.x) + (int64_t)w * n * (int64_t)sizeof(T);
    const char *a = static_cast<const char *>(M.a) + (int64_t)w * r * r * (int64_t)sizeof(T);
    // Buffer offsets are 32-bit: the 16-byte path needs the matrix under 2 GiB.
    const bool vec = (C % Elem<BF16>::EPC) == 0 && (r % Elem<BF16>::EPC) == 0 &&
                     n * (int64_t)sizeof(T) < ((int64_t)1 << 31);

    ProductArgs pa;
    pa.R = R;
    pa.C = C;
    pa.ti = ti;
    pa.tj = tj;
    const float2 sc = b.scales[M.unit_begin + w];
    pa.s = LateScale{sc.x, b.use_scales};
    pa.eta = b.eta;
    pa.spectral0 = b.id_scaled;
    pa.s2 = sc.y;
    pa.idc = b.id_scaled ? id_coef_spectral(sc.y) : kIdMinus3;
    if (EPI == EPI_ITER)
        pa.out = static_cast<char *>(M.out) + (int64_t)w * n * (int64_t)sizeof(T);
    else if (EPI == EPI_FINAL || EPI == EPI_FINAL_I8)
        pa.out = M.out ? static_cast<void *>(static_cast<float *>(M.out) + (int64_t)w * n) : nullptr;
    else
        pa.out = M.out;
    pa.u_out = EPI == EPI_WUPD ? M.u_out : nullptr;
    pa.pk = M.packed ? M.packed + (int64_t)w * ((n + 63) >> 6) : nullptr;
    pa.i8 = EPI == EPI_FINAL_I8 ? M.i8 + (int64_t)w * n : nullptr;

    if (wide) {
        // out[m][n] = sum_k A[m][k] X[k][n]: P = A (k-contiguous), Q(n, k) = X[k][n]
        Operand P{a + (int64_t)ti * kNsTileM * r * (int64_t)sizeof(T), r, R - ti * kNsTileM, r, vec};
        Operand Q{x + (int64_t)tj * kNsProdTileN * (int64_t)sizeof(T), C, C - tj * kNsProdTileN, r, vec};
        product_tile<BF16, false, EPI>(P, Q, smem, pa);
    } else {
        // out[m][n] = sum_k X[m][k] A[k][n] = sum_k X[m][k] A[n][k] (A symmetric)
        Operand P{x + (int64_t)ti * kNsTileM * C * (int64_t)sizeof(T), C, R - ti * kNsTileM, r, vec};
        Operand Q{a + (int64_t)tj * kNsProdTileN * r * (int64_t)sizeof(T), r, C - tj * kNsProdTileN, r, vec};
        product_tile<BF16, true, EPI>(P, Q, smem, pa);
    }
}

// ---------------------------------------------------------------------------
// Persistent product for a bf16 launch: the final product with the signs
// (packed, or int8) straight from the accumulators (no U output, C % 64 ==
// 0), or an intermediate product whose output (the next iterate) is staged
// through LDS outside the stage buffers; 16-byte operands. One workgroup per CU walks the tiles vb =
// blockIdx.x, vb + gridDim.x, ... in the same XCD-contiguous order as the
// one-tile-per-block kernel. The direct-to-LDS pipeline runs on across tile
// boundaries: the loads that a tile's last iterations would issue past its
// own k range fetch the first slices of the workgroup's next tile instead,
// and the epilogue, which touches no LDS, runs while they are in flight. A
// tile therefore starts with its pipeline full; the next tile's descriptor
// is decoded (scalar loads) at the start of the current one.
// ---------------------------------------------------------------------------
template <bool BF16>
struct PackTile {
    Operand P, Q;   // Q = A (k-contiguous) when tall, else Q = X (mn-contiguous)
    ProductArgs pa;
    int tall;
    int kt_n, rot, iters;

    // Slice read by iteration j (the k loop starts at the tile's own 256 k on
    // the identity side; iterations past kt_n read zeros).
    __device__ __forceinline__ int slice(int j) const {
        const int t = j + rot;
        return j >= kt_n ? kt_n : (t < kt_n ? t : t - kt_n);
    }

    // EPI: what the tile's epilogue writes (packed signs to M.packed, int8
    // signs to M.i8, or the next iterate to M.out). SPEC: the first product
    // under spectral scaling (NsBatch::id_scaled).
    template <int EPI, bool SPEC>
    __device__ __forceinline__ void decode(const NsBatch &b, int sv, int lt) {
        using T = typename Elem<BF16>::T;
        constexpr int BK = Elem<BF16>::BK;
        const int w = lt / b.tiles_per_worker_all;
        const int lw = lt - w * b.tiles_per_worker_all;
        const NsMat M = load_ns_mat_scalar(find_ns_mat(sv, lw));
        const int t = lw - M.tile_begin;
        const int R = M.R, C = M.C;
        tall = R > C;
        const int r = tall ? C : R;
        const int tiles_n = (C + kNsProdTileN - 1) / kNsProdTileN;
        const int ti = t / tiles_n, tj = t - ti * tiles_n;
        const int64_t n = (int64_t)R * C;
        const char *x = static_cast<const char *>(M.x) + (int64_t)w * n * (int64_t)sizeof(T);
        const char *a = static_cast<const char *>(M.a) + (int64_t)w * r * r * (int64_t)sizeof(T);
        pa.out = EPI == EPI_ITER ? static_cast<char *>(M.out) + (int64_t)w * n * (int64_t)sizeof(T) : nullptr;
        pa.u_out = nullptr;
        pa.i8 = EPI == EPI_FINAL_I8 ? M.i8 + (int64_t)w * n : nullptr;
        pa.pk = EPI == EPI_FINAL ? M.packed + (int64_t)w * ((n + 63) >> 6) : nullptr;
        pa.R = R;
        pa.C = C;
        pa.ti = ti;
        pa.tj = tj;
        pa.s = LateScale{load_scale_scalar(b.scales, M.unit_begin + w, 0), b.use_scales};
        pa.eta = 0.f;
        pa.spectral0 = SPEC;
        if constexpr (SPEC) {
            pa.s2 = load_scale_scalar(b.scales, M.unit_begin + w, 1);
            pa.idc = id_coef_spectral(pa.s2);
        }
        if (!tall) {
            // out[m][n] = sum_k A[m][k] X[k][n]; -3 X on the P side at the output rows
            P = Operand{a + (int64_t)ti * kNsTileM * r * (int64_t)sizeof(T), r, R - ti * kNsTileM, r, true};
            Q = Operand{x + (int64_t)tj * kNsProdTileN * (int64_t)sizeof(T), C, C - tj * kNsProdTileN, r, true};
        } else {
            // out[m][n] = sum_k X[m][k] A[n][k]; -3 X on the Q side at the output columns
            P = Operand{x + (int64_t)ti * kNsTileM * C * (int64_t)sizeof(T), C, R - ti * kNsTileM, r, true};
            Q = Operand{a + (int64_t)tj * kNsProdTileN * r * (int64_t)sizeof(T), r, C - tj * kNsProdTileN, r, true};
        }
        constexpr int NID = kNsTileM / BK;  // = kNsProdTileN / BK
        kt_n = (r + BK - 1) / BK;
        rot = ((tall ? tj * kNsProdTileN : ti * kNsTileM) / BK) % kt_n;
        iters = kt_n > NID ? kt_n : NID;
    }

    // No further tile: an empty buffer, so its loads read zeros.
    __device__ __forceinline__ void none() {
        P = Q = Operand{nullptr, 0, 0, 0, true};
        tall = 0;
        kt_n = 1;
        rot = 0;
        iters = 1;
    }
};

// Load i of slice kt of a 256-row operand, its buffer offset computed from
// the operand's scalar description alone (the same chunk that
// DmaSlices::setup assigns to the lane), for the next tile's first slices:
// no per-lane state of that tile is held through the current tile's loop.
template <bool BF16>
__device__ __forceinline__ uint32_t walk_offset(const Operand &op, bool kc, int kt, int i, GivenTid tid) {
    using E = Elem<BF16>;
    constexpr uint32_t sz = sizeof(typename E::T);
    const int lane = tid() & (kWave - 1);
    const int b = i * ProdLay::kWaves + __builtin_amdgcn_readfirstlane(tid() / kWave);
    static_assert(BF16, "the walk's layouts are the bf16 ones");
    int mn, k;
    if (kc) {  // 16 rows of 64 bytes, 16-byte chunks swizzled
        mn = b * 16 + (lane >> 2);
        k = ((lane & 3) ^ ((lane >> 4) & 3)) * E::EPC;
    } else {   // 8 blocks of 4 (k) x 16 (mn)
        k = (b >> 1) * 4 + ((lane & 7) >> 1);
        mn = ((b & 1) * 8 + (lane >> 3)) * 16 + (lane & 1) * 8;
    }
    const int kk = kt * E::BK + k;
    const bool ok = mn < op.rows && kk < op.K;
    const uint32_t ld = (uint32_t)op.ld;
    const uint32_t o = kc ? ((uint32_t)mn * ld + (uint32_t)kk) * sz : ((uint32_t)kk * ld + (uint32_t)mn) * sz;
    return ok ? o : kOOB;
}

template <bool BF16>
__device__ __forceinline__ v4u32 walk_rsrc(const Operand &op, bool kc) {
    const uint64_t base = reinterpret_cast<uint64_t>(op.base);
    const int64_t ext = kc ? operand_extent<BF16, true>(op) : operand_extent<BF16, false>(op);
    return v4u32{(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, (uint32_t)ext, 0x00020000u};
}

// One tile of the walk: the k loop of cur (its loads from lp / lq, set up
// for cur), whose loads past its last iteration fetch nxt's first slices.
// Every tile's iteration count is a multiple of the stage count S and at
// least NID + S (the launcher checks), so iteration j of any tile uses LDS
// stage j % S, nxt's slice s lands in stage s, and the last S iterations
// (the tail, unrolled) are the only ones that load for nxt. The first
// fragments are read at the tile's start (slice 0 has landed and the
// barrier that handed it over has passed).
template <bool BF16, bool QKC, bool SPEC>
__device__ __forceinline__ void pack_tile_kloop(const PackTile<BF16> &cur, const PackTile<BF16> &nxt,
                                                const DmaSlices<BF16, 256, ProdLay::kWaves> &lp,
                                                const DmaSlices<BF16, 256, ProdLay::kWaves> &lq, char *smem,
                                                f32x16_t (&acc)[kFM][kFN], GivenTid tid) {
    using L = ProdLay;
    using E = Elem<BF16>;
    constexpr int TN = L::kTileN, S = L::kStages;
    constexpr int SIDE = QKC ? ID_Q : ID_P;
    const int wid = __builtin_amdgcn_readfirstlane(tid() / kWave);
    const int wm0 = L::m0(wid), wn0 = L::n0(wid);
    const int w0 = SIDE == ID_Q ? wn0 : wm0;
    const IdCoef ic = SPEC ? cur.pa.idc : kIdMinus3;
#pragma unroll
    for (int f = 0; f < kFM; ++f)
#pragma unroll
        for (int gg = 0; gg < kFN; ++gg)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][gg][r] = 0.f;
    constexpr int PL = L::kPLoads, QL = L::kQLoads, NLD = PL + QL;
    const uint32_t lds0 = lds_addr(smem);
    Frags<BF16> fa, fb;
    read_frags<BF16, true, QKC, TN, GivenTid>(fa, smem, smem + L::kPBytes, wm0, wn0, 0, tid);
    constexpr int NID = (SIDE == ID_Q ? TN : L::kTileM) / E::BK;
    const int iters = cur.iters;
    constexpr int kSteps = kFM * kFN, kFrag = kFM + kFN;
    constexpr int eQ = kSteps / QL, eP = kSteps / PL;
    static_assert(kFrag <= kSteps && eQ * QL == kSteps && eP * PL == kSteps, "interleave");
    static_assert(NID % S == 0, "identity iterations fill whole stage rounds");
    // Iteration j: as in tile_mainloop, the first half's MFMAs (fa) run with
    // the reads of the second half (fb) and the Q loads of walk iteration
    // j + S - 1; after the barrier that hands over the next slice, the second
    // half's MFMAs (fb) run with the reads of the next slice's first half and
    // the P loads of walk iteration j + S. Tail iteration TL (j = iters - S +
    // TL) loads nxt's slice TL - 1 (Q part, TL >= 1) and slice TL (P part).
    auto iteration = [&](int j, auto jid, auto tl) {
        constexpr int JID = decltype(jid)::value, TL = decltype(tl)::value;
        const int js = TL >= 0 ? TL : j % S;  // j % S
        const char *cb = smem + js * L::kStageBytes;
        const uint32_t late_dst = lds0 + ((js + S - 1) % S) * L::kStageBytes + L::kPBytes;
        const int late = TL >= 1 ? nxt.slice(TL - 1) : cur.slice(j + S - 1);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            mma_step<BF16>(fa, acc, i);
            if (i < kFrag) read_frag<BF16, true, QKC, TN, GivenTid>(fb, cb, cb + L::kPBytes, wm0, wn0, 1, i, tid);
            if (i % eQ == eQ - 1) {
                if constexpr (TL >= 1)
                    lq.issue_at(late_dst, i / eQ, walk_offset<BF16>(nxt.Q, QKC, late, i / eQ, tid),
                                walk_rsrc<BF16>(nxt.Q, QKC));
                else
                    lq.issue_one(late, late_dst, i / eQ);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (JID >= 0) mma_identity_at<BF16, SIDE, JID, GivenTid>(fa, acc, w0, 0, ic, tid);
        wait_vm_lgkm0<(S - 2) * NLD>();
        lds_barrier();
        const char *nb = smem + ((js + 1) % S) * L::kStageBytes;
        const uint32_t dst = lds0 + js * L::kStageBytes;
        const int refill = TL >= 0 ? nxt.slice(TL) : cur.slice(j + S);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            mma_step<BF16>(fb, acc, i);
            if (i < kFrag) read_frag<BF16, true, QKC, TN, GivenTid>(fa, nb, nb + L::kPBytes, wm0, wn0, 0, i, tid);
            if (i % eP == eP - 1) {
                if constexpr (TL >= 0)
                    lp.issue_at(dst, i / eP, walk_offset<BF16>(nxt.P, true, refill, i / eP, tid),
                                walk_rsrc<BF16>(nxt.P, true));
                else
                    lp.issue_one(refill, dst, i / eP);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (JID >= 0) mma_identity_at<BF16, SIDE, JID, GivenTid>(fb, acc, w0, 1, ic, tid);
    };
    using NoTail = std::integral_constant<int, -1>;
    static_for(std::make_integer_sequence<int, NID>{},
               [&](auto jid) { iteration(decltype(jid)::value, jid, NoTail{}); });
    for (int j = NID; j < iters - S; ++j) iteration(j, std::integral_constant<int, -1>{}, NoTail{});
    static_for(std::make_integer_sequence<int, S>{},
               [&](auto tl) { iteration(iters - S + decltype(tl)::value, NoTail{}, tl); });
}

// QKC: every matrix of the launch is tall (true) or wide (false). EPI:
// EPI_FINAL (packed signs), EPI_FINAL_I8 (int8 signs) or EPI_ITER (the next
// iterate). SPEC: the first product under spectral scaling (b.id_scaled).
template <bool BF16, bool QKC, int EPI, bool SPEC>
__global__ __launch_bounds__(ProdLay::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_product_pack_kernel(NsBatch b) {
    static_assert(BF16, "the walk is built for bf16 operands");
    constexpr bool kI8 = EPI == EPI_FINAL_I8;
    static_assert(EPI == EPI_FINAL || EPI == EPI_FINAL_I8 || EPI == EPI_ITER, "walked epilogues");
    constexpr bool kStaged = EPI == EPI_ITER;
    using L = ProdLay;
    constexpr int S = L::kStages, PL = L::kPLoads, QL = L::kQLoads, NLD = PL + QL;
    __shared__ __attribute__((aligned(16))) char smem[L::kLdsBytes];
    // The matrix start table, one entry per lane, kept in LDS for the whole
    // walk (read back per tile: a register copy would be spilled, and its
    // reload would wait for every load in flight).
    __shared__ int starts[kWave];
    __shared__ uint2 i8_table[kI8 ? 256 : 1];
    __shared__ __attribute__((aligned(16))) float estage[kStaged ? L::kWaves * 8 * kStageStride : 1];
    const int sv = ns_start_of_lane();
    if (threadIdx.x < kWave) starts[threadIdx.x] = sv;
    if (kI8 && threadIdx.x < 256) i8_table[threadIdx.x] = int8_table_entry((int)threadIdx.x);
    const int wid0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int total = b.total_tiles, G = gridDim.x;
    int vb = blockIdx.x;
    PackTile<BF16> cur, nxt;
    DmaSlices<BF16, 256, L::kWaves> lp, lq;
    cur.template decode<EPI, SPEC>(b, sv, xcd_remap(vb, total));
    lp.template setup<true>(cur.P);
    lq.template setup<QKC>(cur.Q);
    // The first tile fills the pipeline itself: slices 0 .. S - 2 and the P
    // part of slice S - 1.
    const uint32_t lds0 = lds_addr(smem);
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
        lp.issue(cur.slice(st), lds0 + st * L::kStageBytes);
        lq.issue(cur.slice(st), lds0 + st * L::kStageBytes + L::kPBytes);
    }
    lp.issue(cur.slice(S - 1), lds0 + (S - 1) * L::kStageBytes);
    wait_vm_lgkm0<(S - 2) * NLD + PL>();  // slice 0 landed
    lds_barrier();
    f32x16_t acc[kFM][kFN];
    for (;;) {
        // The thread index, produced afresh for each tile where the compiler
        // cannot hoist it (the lane from v_mbcnt in an asm statement, the
        // wave from a scalar register), so that lane arithmetic (identity
        // fragments, LDS addresses) is redone per tile instead of held in
        // registers across the whole walk.
        int lane;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
        const GivenTid tid{(unsigned)(wid0 * kWave + lane)};
        const int vn = vb + G;
        const bool more = vn < total;
        if (more)
            nxt.template decode<EPI, SPEC>(b, starts[lane], xcd_remap(vn, total));
        else
            nxt.none();
        pack_tile_kloop<BF16, QKC, SPEC>(cur, nxt, lp, lq, smem, acc, tid);
        if constexpr (SPEC) scale_acc(acc, cur.pa.s2);
        if constexpr (kI8) {
            int8_from_registers(cur.pa, acc, tid, i8_table);
        } else if constexpr (kStaged) {
            if ((cur.pa.ti + 1) * kNsTileM <= cur.pa.R && (cur.pa.tj + 1) * kNsProdTileN <= cur.pa.C)
                walk_staged_epilogue<EPI, true>(cur.pa, acc, tid, estage);
            else
                walk_staged_epilogue<EPI, false>(cur.pa, acc, tid, estage);
        } else {
            pack_from_registers<GivenTid>(cur.pa, acc, tid);
        }
        if (!more) break;
        vb = vn;
        cur = nxt;
        lp.template setup<true, GivenTid>(cur.P, tid);
        lq.template setup<QKC, GivenTid>(cur.Q, tid);
    }
    wait_vm_lgkm0<0>();  // the zero-fill loads past the last tile write LDS too
}

// ---------------------------------------------------------------------------
// Persistent Gram for a bf16 launch: one workgroup per CU walks Gram tiles of
// wide and tall matrices alike (a launch of one orientation would leave its
// last round of tiles mostly empty when a shape has few tiles per CU). The
// launch numbers its tiles matrix-major -- matrix (longest k first), then
// worker, then the tile within the worker's upper triangle -- so that tiles
// that share a panel of Y sit next to each other and tile costs (k slices)
// never increase along the order. Round rho hands positions rho * G ..
// rho * G + G - 1 (G workgroups) out in a snake: XCD-contiguous positions in
// even rounds, reversed in odd ones, which evens out the work per CU when
// the costs fall along the order. As in the product walk, the loads a tile's
// last iterations would issue past its k range fetch the first slices of
// the workgroup's next tile (whatever its orientation: the load offsets come
// from the next tile's scalar description), and the epilogue, staged 8 rows
// at a time through LDS beside the stage buffers, runs while they land.
// A tile loads two 256-row groups of Y (P: group ti, Q: group tj), eight
// 64-row panels ("slots" 0-3 of P, 4-7 of Q), and each wave computes two
// 64 x 64 blocks of A that share their column panel: rows from slots a1 and
// a2, columns from slot b (a 128 x 64 result, as in ns_gram_kernel). The
// upper triangle is covered block by block: a cross tile (ti < tj) takes the
// 16 blocks of groups ti x tj; the ten blocks inside one group (four on the
// diagonal, six above it) take five waves, so a pair tile holds all of one
// group's (waves 0-4, P) and three or two waves of another's (waves 5-7, Q),
// and three groups need two tiles where whole diagonal tiles would need three
// (a fifth fewer MFMAs at r = 768). Every block's entries come out of the same
// MFMA chain over the same k order as in ns_gram_kernel (the products of bf16
// values are exact, and an entry and its mirror add the same products), so A
// is the same bit for bit.
// ---------------------------------------------------------------------------
enum GramWalkKind { GW_CROSS = 0, GW_PAIR3 = 1, GW_PAIR2 = 2, GW_SINGLE = 3 };

// Slots of wave wid in a tile of the given kind: a1 | a2 << 4 | b << 8, and
// bit 12 set when the wave's blocks are part of A (idle waves compute on
// whatever their slots hold and store nothing). One group's ten blocks as
// five waves (a1, a2; b): (0, 2; 0) (1, 3; 1) (2, 3; 2) (3, 0; 3) (0, 2; 1).
__device__ __forceinline__ int gram_wave_slots(int kind, int wid) {
    if (kind == GW_CROSS) return (2 * (wid >> 2)) | ((2 * (wid >> 2) + 1) << 4) | ((4 + (wid & 3)) << 8) | (1 << 12);
    constexpr uint64_t kGroupWaves = 0x120ull << 48 | 0x303ull << 36 | 0x232ull << 24 | 0x131ull << 12 | 0x020ull;
    int w = wid, add = 0, live = 1;
    if (wid >= 5) {
        w = (kind == GW_PAIR3 ? 0 : 3) + wid - 5;
        add = 0x444;
        live = kind == GW_PAIR3 || (kind == GW_PAIR2 && wid < 7);
        if (!live) w = 0;
    }
    return ((int)(kGroupWaves >> (12 * w)) & 0xfff) + add + (live << 12);
}

struct GramWalkTile {
    Operand P, Q;   // row groups ti and tj of Y (X when wide, X^T when tall)
    char *a;        // this worker's Gram matrix [r][r]
    LateScale sc;   // s^2 of the first iteration (applied in the epilogue)
    int tall;       // Y = X^T: both panels mn-contiguous
    int kind;       // GramWalkKind
    int ti, tj, r;
    int kt_n;       // k slices of the tile

    __device__ __forceinline__ int slice(int j) const { return j < kt_n ? j : kt_n; }

    __device__ __forceinline__ void decode(const NsBatch &b, int sv, int L) {
        constexpr int64_t sz = 2;  // bf16
        const NsMat M = load_ns_mat_scalar(find_ns_mat(sv, L));
        const int rem = L - M.tile_begin;
        const int w = rem / M.tiles_per_worker;
        int t = rem - w * M.tiles_per_worker;
        tall = M.R > M.C;
        r = tall ? M.C : M.R;
        const int c = tall ? M.R : M.C;
        // A worker's tiles: the in-group tiles first (pairs of groups 3u, 3u + 1
        // and 3u + 2, 3u + 1, then the groups left over alone), then the
        // cross tiles in row-major order of the upper triangle of groups.
        const int T_ = (r + kNsTileM - 1) / kNsTileM;
        const int trip = T_ / 3, nd = 2 * trip + T_ % 3;
        if (t < 2 * trip) {
            tj = 3 * (t >> 1) + 1;
            ti = tj + ((t & 1) ? 1 : -1);
            kind = (t & 1) ? GW_PAIR2 : GW_PAIR3;
        } else if (t < nd) {
            ti = tj = 3 * trip + t - 2 * trip;
            kind = GW_SINGLE;
        } else {
            t -= nd;
            int i = 0;
            while (t >= T_ - 1 - i) {
                t -= T_ - 1 - i;
                ++i;
            }
            ti = i;
            tj = i + 1 + t;
            kind = GW_CROSS;
        }
        const char *y = static_cast<const char *>(M.x) + (int64_t)w * M.R * M.C * sz;
        a = static_cast<char *>(M.a) + (int64_t)w * r * r * sz;
        sc = LateScale{load_scale_scalar(b.scales, M.unit_begin + w, 1), b.use_scales};
        if (!tall) {  // Y = X: k-contiguous rows
            P = Operand{y + (int64_t)ti * kNsTileM * M.C * sz, M.C, r - ti * kNsTileM, c, true};
            Q = Operand{y + (int64_t)tj * kNsTileM * M.C * sz, M.C, r - tj * kNsTileM, c, true};
        } else {      // Y = X^T: element (i, k) at X[k][i], mn-contiguous
            P = Operand{y + (int64_t)ti * kNsTileM * sz, M.C, r - ti * kNsTileM, c, true};
            Q = Operand{y + (int64_t)tj * kNsTileM * sz, M.C, r - tj * kNsTileM, c, true};
        }
        if (kind == GW_SINGLE) Q = Operand{nullptr, 0, 0, 0, true};  // nothing to load: zeros
        kt_n = (c + Elem<true>::BK - 1) / Elem<true>::BK;
    }

    // No further tile: an empty buffer, so its loads read zeros.
    __device__ __forceinline__ void none() {
        P = Q = Operand{nullptr, 0, 0, 0, true};
        a = nullptr;
        sc = LateScale{1.0f, 0};
        tall = 0;
        kind = GW_SINGLE;
        ti = tj = r = 0;
        kt_n = 1;
    }
};

// LDS byte offset of slot s (a 64-row panel; 0-3 in P, 4-7 in Q) within a
// stage: both layouts are linear in 64-row steps, and Q follows P.
template <bool KC>
__device__ __forceinline__ uint32_t gram_slot_off(int s) {
    return KC ? (uint32_t)s * (64 * kRowBytes) : (uint32_t)(s & 3) * 512u + (uint32_t)(s >> 2) * GramLay::kPBytes;
}

// Fragment j of one half for a wave whose P blocks come from the slots at
// LDS offsets o1 (m-blocks 0, 1) and o2 (2, 3) and its Q blocks from ob.
template <bool KC>
__device__ __forceinline__ void gram_read_frag(Frags<true> &fr, const char *cb, uint32_t o1, uint32_t o2,
                                               uint32_t ob, int half, int j, GivenTid tid) {
    if (j < 2)
        fr.p[j] = frag_bf16<KC, 256, GivenTid>(cb + o1, 32 * j, half, tid);
    else if (j < kFM)
        fr.p[j] = frag_bf16<KC, 256, GivenTid>(cb + o2, 32 * (j - 2), half, tid);
    else
        fr.q[j - kFM] = frag_bf16<KC, 256, GivenTid>(cb + ob, 32 * (j - kFM), half, tid);
}

// The k loop of one Gram tile of the walk (KC: both panels k-contiguous,
// i.e. a wide X), with the same per-iteration schedule as pack_tile_kloop
// (no identity term, no rotation): its last S iterations load nxt's first
// slices. Every tile's slice count is a multiple of S and at least 2 S (the
// launcher checks), so iteration j uses LDS stage j % S and nxt's slice s
// lands in stage s.
template <bool KC>
__device__ __forceinline__ void gram_walk_kloop(const GramWalkTile &cur, const GramWalkTile &nxt,
                                                const DmaSlices<true, 256, GramLay::kWaves> &lp,
                                                const DmaSlices<true, 256, GramLay::kWaves> &lq, char *smem,
                                                f32x16_t (&acc)[kFM][kFN], GivenTid tid) {
    using L = GramLay;
    constexpr int S = L::kStages;
    const int wid = __builtin_amdgcn_readfirstlane(tid() / kWave);
    const int sl = __builtin_amdgcn_readfirstlane(gram_wave_slots(cur.kind, wid));
    const uint32_t o1 = gram_slot_off<KC>(sl & 15), o2 = gram_slot_off<KC>((sl >> 4) & 15),
                   ob = gram_slot_off<KC>((sl >> 8) & 15);
#pragma unroll
    for (int f = 0; f < kFM; ++f)
#pragma unroll
        for (int gg = 0; gg < kFN; ++gg)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][gg][r] = 0.f;
    constexpr int PL = L::kPLoads, QL = L::kQLoads, NLD = PL + QL;
    const uint32_t lds0 = lds_addr(smem);
    Frags<true> fa, fb;
#pragma unroll
    for (int j = 0; j < kFM + kFN; ++j) gram_read_frag<KC>(fa, smem, o1, o2, ob, 0, j, tid);
    const int iters = cur.kt_n;
    const bool nkc = !nxt.tall;
    constexpr int kSteps = kFM * kFN, kFrag = kFM + kFN;
    constexpr int eQ = kSteps / QL, eP = kSteps / PL;
    static_assert(kFrag <= kSteps && eQ * QL == kSteps && eP * PL == kSteps, "interleave");
    auto iteration = [&](int j, auto tl) {
        constexpr int TL = decltype(tl)::value;
        const int js = TL >= 0 ? TL : j % S;
        const char *cb = smem + js * L::kStageBytes;
        const uint32_t late_dst = lds0 + ((js + S - 1) % S) * L::kStageBytes + L::kPBytes;
        const int late = TL >= 1 ? nxt.slice(TL - 1) : cur.slice(j + S - 1);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            mma_step<true>(fa, acc, i);
            if (i < kFrag) gram_read_frag<KC>(fb, cb, o1, o2, ob, 1, i, tid);
            if (i % eQ == eQ - 1) {
                if constexpr (TL >= 1)
                    lq.issue_at(late_dst, i / eQ, walk_offset<true>(nxt.Q, nkc, late, i / eQ, tid),
                                walk_rsrc<true>(nxt.Q, nkc));
                else
                    lq.issue_one(late, late_dst, i / eQ);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vm_lgkm0<(S - 2) * NLD>();
        lds_barrier();
        const char *nb = smem + ((js + 1) % S) * L::kStageBytes;
        const uint32_t dst = lds0 + js * L::kStageBytes;
        const int refill = TL >= 0 ? nxt.slice(TL) : cur.slice(j + S);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            mma_step<true>(fb, acc, i);
            if (i < kFrag) gram_read_frag<KC>(fa, nb, o1, o2, ob, 0, i, tid);
            if (i % eP == eP - 1) {
                if constexpr (TL >= 0)
                    lp.issue_at(dst, i / eP, walk_offset<true>(nxt.P, nkc, refill, i / eP, tid),
                                walk_rsrc<true>(nxt.P, nkc));
                else
                    lp.issue_one(refill, dst, i / eP);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using NoTail = std::integral_constant<int, -1>;
    for (int j = 0; j < iters - S; ++j) iteration(j, NoTail{});
    static_for(std::make_integer_sequence<int, S>{},
               [&](auto tl) { iteration(iters - S + decltype(tl)::value, tl); });
}

// Epilogue of a walked Gram tile: A = scale * acc rounded to bf16, each of
// the wave's two 64 x 64 blocks and (off the diagonal) its mirror, 8 rows of
// the wave's 128 x 64 result at a time through the wave's 8 x kStageStride
// floats outside the stage buffers. Register 4q + t of block (f, g) holds
// row 8q + 4h + t (h = lane / 32) of the block. Direct rows: 8 lanes per
// row, 8 columns (16 bytes) each. Mirror: lane l reads staged column l, i.e.
// 8 consecutive entries of mirrored row n0 + l, and stores them as 16 bytes.
// A diagonal block holds both triangles and is stored once. FAST: the tile's
// groups lie inside the matrix and r % 8 == 0.
// 4 x 4 transpose of 16-byte pieces within each quad of lanes: lane 4k + r
// holds x[c] = T[r][c] before and x[c] = T[c][r] after (two exchanges, with
// the lane at distance 1 and then 2; each lane sends the piece its partner
// needs).
__device__ __forceinline__ uint4 dpp_quad(uint4 v, int ctrl_is_swap2) {
    // quad_perm [1, 0, 3, 2] (swap with lane ^ 1) or [2, 3, 0, 1] (lane ^ 2)
    if (ctrl_is_swap2)
        return make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, 0x4e, 0xf, 0xf, false),
                          (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, 0x4e, 0xf, 0xf, false),
                          (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, 0x4e, 0xf, 0xf, false),
                          (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, 0x4e, 0xf, 0xf, false));
    return make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, 0xb1, 0xf, 0xf, false),
                      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, 0xb1, 0xf, 0xf, false),
                      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, 0xb1, 0xf, 0xf, false),
                      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, 0xb1, 0xf, 0xf, false));
}

__device__ __forceinline__ uint4 sel4(bool c, uint4 a, uint4 b) {  // c ? a : b, per component
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

__device__ __forceinline__ void quad_transpose(uint4 (&x)[4], int lane) {
    const bool odd = lane & 1, high = lane & 2;
#pragma unroll
    for (int c = 0; c < 4; c += 2) {  // pieces c, c + 1 across lane ^ 1
        const uint4 x0 = x[c], x1 = x[c + 1];
        const uint4 got = dpp_quad(sel4(odd, x0, x1), 0);
        x[c] = sel4(odd, got, x0);
        x[c + 1] = sel4(odd, x1, got);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {  // pieces c, c + 2 across lane ^ 2
        const uint4 x0 = x[c], x2 = x[c + 2];
        const uint4 got = dpp_quad(sel4(high, x0, x2), 1);
        x[c] = sel4(high, got, x0);
        x[c + 2] = sel4(high, x2, got);
    }
}

// Epilogue of a walked Gram tile: A = scale * acc rounded to bf16, each of
// the wave's two 64 x 64 blocks and (off the diagonal) its mirror, 8 rows of
// the wave's 128 x 64 result at a time through the wave's 8 x kStageStride
// floats outside the stage buffers. Register 4q + t of block (f, g) holds
// row 8q + 4h + t (h = lane / 32) of the block. Direct rows: 8 lanes per
// row, 8 columns (16 bytes) each. Mirror: lane l reads staged column l, i.e.
// 8 consecutive entries of mirrored row n0 + l (16 bytes); FAST keeps the
// four such pieces of a 32-row block, transposes them within each quad of
// lanes and writes 16 mirrored rows x 64 contiguous bytes per store (one
// lane per row would scatter 16 bytes into each of 64 rows). A diagonal
// block holds both triangles and is stored once. FAST: the tile's groups
// lie inside the matrix and r % 8 == 0.
template <bool FAST>
__device__ __forceinline__ void gram_walk_epilogue(const GramWalkTile &g, const f32x16_t (&acc)[kFM][kFN],
                                                   GivenTid tid, float *estage) {
    const float scale = g.sc.get();
    const int lane = tid() & (kWave - 1), wid = tid() / kWave;
    const int sl = __builtin_amdgcn_readfirstlane(gram_wave_slots(g.kind, wid));
    if (!((sl >> 12) & 1)) return;  // an idle wave of a pair or single tile
    auto row_of = [&](int slot) { return (slot < 4 ? g.ti : g.tj) * kNsTileM + 64 * (slot & 3); };
    const int s1 = sl & 15, s2 = (sl >> 4) & 15, sb = (sl >> 8) & 15;
    const int m1 = row_of(s1), m2 = row_of(s2), n0 = row_of(sb);
    float *st = estage + wid * 8 * kStageStride;
    uint16_t *a = reinterpret_cast<uint16_t *>(g.a);
    const int r = g.r;
#pragma unroll
    for (int f = 0; f < kFM; ++f) {
        const int mb = (f < 2 ? m1 : m2) + 32 * (f & 1);  // first row of 32-row block f
        const bool mirror = (f < 2 ? s1 : s2) != sb;
        uint4 mp[4];  // FAST mirror: this lane's pieces of mirrored row n0 + lane, q = 0..3
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int gg = 0; gg < kFN; ++gg)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    st[(4 * (lane >> 5) + t) * kStageStride + 32 * gg + (lane & 31)] = acc[f][gg][4 * q + t] * scale;
            wave_lds_fence();
            {
                const int row = lane >> 3, c8 = (lane & 7) * 8;
                const int gi = mb + 8 * q + row, gj = n0 + c8;
                const float4 lo = *reinterpret_cast<const float4 *>(st + row * kStageStride + c8);
                const float4 hi = *reinterpret_cast<const float4 *>(st + row * kStageStride + c8 + 4);
                const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                if (FAST) {
                    *reinterpret_cast<uint4 *>(a + (int64_t)gi * r + gj) =
                        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                   pack_bf16x2(v[6], v[7]));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (gi < r && gj + e < r) a[(int64_t)gi * r + gj + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                }
            }
            if (mirror) {
                const int gj = n0 + lane, gi = mb + 8 * q;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = st[e * kStageStride + lane];
                if (FAST) {
                    mp[q] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                       pack_bf16x2(v[6], v[7]));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (gj < r && gi + e < r) a[(int64_t)gj * r + gi + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                }
            }
            wave_lds_fence();
        }
        if (FAST && mirror) {
            // lane 4k + p now takes piece p of mirrored rows n0 + 4k + j, j = 0..3
            quad_transpose(mp, lane);
            const int p = lane & 3, k4 = lane & ~3;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint4 *>(a + (int64_t)(n0 + k4 + j) * r + mb + 8 * p) = mp[j];
        }
    }
}

// Logical tile of workgroup position pos in round rho (snake order).
__device__ __forceinline__ int gram_walk_tile(int rho, int pos, int G) {
    return rho * G + ((rho & 1) ? G - 1 - pos : pos);
}

__global__ __launch_bounds__(GramLay::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ns_gram_walk_kernel(NsBatch b) {
    using L = GramLay;
    constexpr int S = L::kStages, PL = L::kPLoads, QL = L::kQLoads, NLD = PL + QL;
    __shared__ __attribute__((aligned(16))) char smem[L::kLdsBytes];
    __shared__ int starts[kWave];  // the matrix start table (see ns_product_pack_kernel)
    __shared__ __attribute__((aligned(16))) float estage[L::kWaves * 8 * kStageStride];
    const int sv = ns_start_of_lane();
    if (threadIdx.x < kWave) starts[threadIdx.x] = sv;
    const int wid0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int total = b.total_tiles, G = gridDim.x;
    const int pos = xcd_remap(blockIdx.x, G);  // XCD-contiguous positions
    int rho = 0;
    GramWalkTile cur, nxt;
    DmaSlices<true, 256, L::kWaves> lp, lq;
    cur.decode(b, sv, gram_walk_tile(0, pos, G));  // G <= total: round 0 is full
    if (cur.tall) {
        lp.template setup<false>(cur.P);
        lq.template setup<false>(cur.Q);
    } else {
        lp.template setup<true>(cur.P);
        lq.template setup<true>(cur.Q);
    }
    const uint32_t lds0 = lds_addr(smem);
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
        lp.issue(cur.slice(st), lds0 + st * L::kStageBytes);
        lq.issue(cur.slice(st), lds0 + st * L::kStageBytes + L::kPBytes);
    }
    lp.issue(cur.slice(S - 1), lds0 + (S - 1) * L::kStageBytes);
    wait_vm_lgkm0<(S - 2) * NLD + PL>();  // slice 0 landed
    lds_barrier();
    f32x16_t acc[kFM][kFN];
    for (;;) {
        int lane;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
        const GivenTid tid{(unsigned)(wid0 * kWave + lane)};
        const int ln = gram_walk_tile(rho + 1, pos, G);
        const bool more = ln < total;
        if (more)
            nxt.decode(b, starts[lane], ln);
        else
            nxt.none();
        if (cur.tall)
            gram_walk_kloop<false>(cur, nxt, lp, lq, smem, acc, tid);
        else
            gram_walk_kloop<true>(cur, nxt, lp, lq, smem, acc, tid);
        if ((cur.ti + 1) * kNsTileM <= cur.r && (cur.tj + 1) * kNsTileM <= cur.r)
            gram_walk_epilogue<true>(cur, acc, tid, estage);
        else
            gram_walk_epilogue<false>(cur, acc, tid, estage);
        if (!more) break;
        ++rho;
        cur = nxt;
        if (cur.tall) {
            lp.template setup<false, GivenTid>(cur.P, tid);
            lq.template setup<false, GivenTid>(cur.Q, tid);
        } else {
            lp.template setup<true, GivenTid>(cur.P, tid);
            lq.template setup<true, GivenTid>(cur.Q, tid);
        }
    }
    wait_vm_lgkm0<0>();  // the zero-fill loads past the last tile write LDS too
}

}  // namespace

void launch_ns_gram(const NsBatch &b, bool ns_bf16, hipStream_t s) {
    dim3 grid(b.total_tiles), block(GramLay::kThreads);
    if (ns_bf16)
        hipLaunchKernelGGL(ns_gram_kernel<true>, grid, block, 0, s, b);
    else
        hipLaunchKernelGGL(ns_gram_kernel<false>, grid, block, 0, s, b);
}

void launch_ns_gram_split(const NsBatch &b, bool ns_bf16, hipStream_t s) {
    dim3 grid(b.total_tiles), block(GramLay::kThreads);
    if (ns_bf16)
        hipLaunchKernelGGL((ns_gram_kernel<true, true>), grid, block, 0, s, b);
    else
        hipLaunchKernelGGL((ns_gram_kernel<false, true>), grid, block, 0, s, b);
}

void launch_gram_reduce(const NsBatch &b, bool ns_bf16, hipStream_t s) {
    dim3 grid(b.total_tiles), block(256);
    if (ns_bf16)
        hipLaunchKernelGGL(gram_reduce_kernel<true>, grid, block, 0, s, b);
    else
        hipLaunchKernelGGL(gram_reduce_kernel<false>, grid, block, 0, s, b);
}

void launch_ns_product(const NsBatch &b, bool ns_bf16, NsEpilogue epi, hipStream_t s) {
    dim3 grid(b.total_tiles), block(ProdLay::kThreads);
#define SM_PROD(BF, E) hipLaunchKernelGGL((ns_product_kernel<BF, E>), grid, block, 0, s, b)
    if (ns_bf16) {
        if (epi == EPI_ITER) SM_PROD(true, EPI_ITER);
        else if (epi == EPI_FINAL) SM_PROD(true, EPI_FINAL);
        else if (epi == EPI_FINAL_I8) SM_PROD(true, EPI_FINAL_I8);
        else SM_PROD(true, EPI_WUPD);
    } else {
        if (epi == EPI_ITER) SM_PROD(false, EPI_ITER);
        else if (epi == EPI_FINAL) SM_PROD(false, EPI_FINAL);
        else if (epi == EPI_FINAL_I8) SM_PROD(false, EPI_FINAL_I8);
        else SM_PROD(false, EPI_WUPD);
    }
#undef SM_PROD
}

void launch_ns_gram_walk(const NsBatch &b, int grid_blocks, hipStream_t s) {
    dim3 grid(grid_blocks), block(GramLay::kThreads);
    hipLaunchKernelGGL(ns_gram_walk_kernel, grid, block, 0, s, b);
}

void launch_ns_product_pack(const NsBatch &b, bool tall, NsEpilogue epi, int grid_blocks, hipStream_t s) {
    dim3 grid(grid_blocks), block(ProdLay::kThreads);
#define SM_WALK(TALL, E, SP) hipLaunchKernelGGL((ns_product_pack_kernel<true, TALL, E, SP>), grid, block, 0, s, b)
#define SM_WALK2(E)                               \
    do {                                          \
        if (b.id_scaled) {                        \
            if (tall) SM_WALK(true, E, true);     \
            else SM_WALK(false, E, true);         \
        } else {                                  \
            if (tall) SM_WALK(true, E, false);    \
            else SM_WALK(false, E, false);        \
        }                                         \
    } while (0)
    if (epi == EPI_FINAL_I8) SM_WALK2(EPI_FINAL_I8);
    else if (epi == EPI_ITER) SM_WALK2(EPI_ITER);
    else SM_WALK2(EPI_FINAL);
#undef SM_WALK2
#undef SM_WALK
}

}  // namespace sm
