// spectral.hip -- spectral normalisation of the Newton-Schulz input for
// gfx950: power iteration on each worker's Gram matrix and the scale it
// gives.
//
// Method: "SignMuon: Communication-Efficient Distributed Muon Optimization"
// (gist.science, paper 2605.16311, technical summary), §4 "nanoGPT" (the
// results hold with spectral as with Frobenius scaling of the Newton-Schulz
// input). The summary gives no procedure; the one built here: A_raw is the
// stored Gram matrix of the stored momentum (the Newton-Schulz orientation),
// lambda is the last ||A v|| of p power-iteration steps from the all-ones
// vector (w = A v, lambda = ||w||, v = w / lambda), s = 1 / sqrt(lambda), and
// the first iteration uses A_0 = s^2 A_raw with s^2 = fp32(1 / lambda) and
// X_0 = s M. lambda = 0 gives s = 0 (U = 0). A_raw is not rescaled in memory:
// the first product multiplies its fp32 accumulators of (A_raw - 3 / s^2 I) M
// by s^2 (ns_gemm.hip, IdCoef).
#include "sm_internal.h"

namespace sm {
namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;

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

// Fixed butterfly over the wave: the order does not depend on timing.
__device__ __forceinline__ double wave_sum(double v) {
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Sum of squares of the previous step's vector of one worker, from its block
// partial sums in block order (one wave).
__device__ __forceinline__ double prev_norm2(const double *part, int bpw) {
    const int lane = threadIdx.x & (kWave - 1);
    double ss = 0.0;
    for (int i = lane; i < bpw; i += kWave) ss += part[i];
    return wave_sum(ss);
}

// One power-iteration step: w = A v with v the all-ones vector / sqrt(r)
// (step 0) or the previous step's w / ||w||. Each block takes 32 rows of one
// worker's Gram matrix: v goes to LDS (r floats, sized at launch), each wave
// computes 8 rows with the loads of all 8 in flight together and reduces
// each in a fixed order, and the block writes the sum of squares of its rows.
constexpr int kRowsPerWave = kPowRowsPerBlock / (kThreads / kWave);

template <bool BF16>
__global__ __launch_bounds__(kThreads) void power_step_kernel(PowBatch b) {
    extern __shared__ float v[];
    __shared__ double red[kThreads / kWave];
    __shared__ float inv_s;
    const int blk = blockIdx.x;
    const int mi = find_start(b.starts, blk);
    const PowMat &M = b.mat[mi];
    const int local = blk - b.starts.v[mi];
    const int w = local / M.bpw, rb = local - w * M.bpw;
    const int r = M.r;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int cur = b.it & 1, prev = cur ^ 1;
    float *wcur = M.w + ((int64_t)cur * b.workers + w) * r;
    const float *wprev = M.w + ((int64_t)prev * b.workers + w) * r;
    if (b.it == 0) {
        const float v0 = (float)(1.0 / sqrt((double)r));
        for (int l = threadIdx.x; l < r; l += kThreads) v[l] = v0;
    } else {
        if (wave == 0) {
            const double n2 = prev_norm2(M.part + ((int64_t)prev * b.workers + w) * M.bpw, M.bpw);
            if (lane == 0) inv_s = n2 > 0.0 ? (float)(1.0 / sqrt(n2)) : 0.0f;
        }
        __syncthreads();
        const float inv = inv_s;
        for (int l = threadIdx.x; l < r; l += kThreads) v[l] = wprev[l] * inv;
    }
    __syncthreads();
    const char *a = static_cast<const char *>(M.a) + ((int64_t)w * r * r) * (BF16 ? 2 : 4);
    const int i0 = rb * kPowRowsPerBlock + wave * kRowsPerWave;
    const int nrows = r - i0 < kRowsPerWave ? (r - i0 > 0 ? r - i0 : 0) : kRowsPerWave;  // uniform
    float acc[kRowsPerWave];
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) acc[q] = 0.f;
    if (BF16 && (r % 8) == 0) {
        const uint16_t *rows = reinterpret_cast<const uint16_t *>(a) + (int64_t)i0 * r;
        for (int l0 = lane * 8; l0 < r; l0 += kWave * 8) {
            uint4 h[kRowsPerWave];
#pragma unroll
            for (int q = 0; q < kRowsPerWave; ++q)
                h[q] = q < nrows ? *reinterpret_cast<const uint4 *>(rows + (int64_t)q * r + l0) : make_uint4(0, 0, 0, 0);
            float vv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = v[l0 + e];
#pragma unroll
            for (int q = 0; q < kRowsPerWave; ++q) {
                const uint32_t hw[4] = {h[q].x, h[q].y, h[q].z, h[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[q] = __builtin_fmaf(bf16_bits_to_f32(hw[e] & 0xffffu), vv[2 * e], acc[q]);
                    acc[q] = __builtin_fmaf(bf16_bits_to_f32(hw[e] >> 16), vv[2 * e + 1], acc[q]);
                }
            }
        }
    } else if (!BF16 && (r % 4) == 0) {
        const float *rows = reinterpret_cast<const float *>(a) + (int64_t)i0 * r;
        for (int l0 = lane * 4; l0 < r; l0 += kWave * 4) {
            float4 f[kRowsPerWave];
#pragma unroll
            for (int q = 0; q < kRowsPerWave; ++q)
                f[q] = q < nrows ? *reinterpret_cast<const float4 *>(rows + (int64_t)q * r + l0) : make_float4(0, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < kRowsPerWave; ++q) {
                acc[q] = __builtin_fmaf(f[q].x, v[l0], acc[q]);
                acc[q] = __builtin_fmaf(f[q].y, v[l0 + 1], acc[q]);
                acc[q] = __builtin_fmaf(f[q].z, v[l0 + 2], acc[q]);
                acc[q] = __builtin_fmaf(f[q].w, v[l0 + 3], acc[q]);
            }
        }
    } else {
        for (int q = 0; q < nrows; ++q) {
            const int64_t base = (int64_t)(i0 + q) * r;
            for (int l = lane; l < r; l += kWave) {
                const float aij = BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a)[base + l])
                                       : reinterpret_cast<const float *>(a)[base + l];
                acc[q] = __builtin_fmaf(aij, v[l], acc[q]);
            }
        }
    }
    double sq = 0.0;
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
        const float t = wave_sum_f32(acc[q]);
        if (q < nrows) {
            if (lane == 0) wcur[i0 + q] = t;
            sq += (double)t * t;
        }
    }
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int k = 0; k < kThreads / kWave; ++k) t += red[k];
        M.part[((int64_t)cur * b.workers + w) * M.bpw + rb] = t;
    }
}

// lambda = ||A v|| of the last step; s = 1 / sqrt(lambda), s^2 = 1 / lambda
// per (matrix, worker) (0 when lambda = 0). One wave per (matrix, worker).
__global__ __launch_bounds__(kThreads) void power_finalize_kernel(PowBatch b) {
    const int u = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave);
    if (u >= b.nmat * b.workers) return;
    const PowMat &M = b.mat[u / b.workers];
    const int w = u % b.workers;
    const int last = b.it & 1;
    const double n2 = prev_norm2(M.part + ((int64_t)last * b.workers + w) * M.bpw, M.bpw);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        const double lambda = sqrt(n2);
        float s = 0.f, s2 = 0.f;
        if (lambda > 0.0) {
            s = (float)(1.0 / sqrt(lambda));
            s2 = (float)(1.0 / lambda);
        }
        b.scales[M.unit_begin + w] = make_float2(s, s2);
    }
}

// ---------------------------------------------------------------------------
// The whole power iteration of one (matrix, worker) in one workgroup: the p
// steps and the scale, in one launch over every unit. A is stored symmetric (each
// off-diagonal entry with its mirror), so a step reads the upper part only.
// Rows go in groups of 8: group g is rows 8g .. 8g + 7, and it reads the
// 16-byte chunks from its 8 x 8 diagonal block to the row end. For row j of
// group g:
//   row sum:     sum over c >= 8g of A[j][c] v[c]  (the few c < j of the
//                diagonal block are its stored lower entries)
//   column sums: A[j][c] v[j] added to column c for every c >= 8g + 8.
// A pair (j, c) with c < 8g is then covered by row c's column sums, and no
// pair twice: w[c] = row sum of c + the column sums of c.
// Group g's chunk count falls by one diagonal block per group, so groups g
// and G - 1 - g (G = r / 8) together have r / EPC + 8 / EPC chunks whatever
// g is: a wave takes such a pair at a time, its chunk list spread over the
// lanes (position p in slot p / 64 of lane p % 64), and few lanes idle.
// Lane sums go to the 16 row sums by one butterfly and to the column sums
// in LDS, one array per wave for each side of the pair (lanes of one load
// never share a column chunk within a side). Every sum runs in a fixed
// order, so results do not depend on timing. The working set of the units
// in flight is their upper triangles (about 0.6 MB at r = 768), which the
// Infinity Cache holds across the p steps, where one launch per step over
// every unit streams all of A from HBM each time.
// ---------------------------------------------------------------------------
constexpr int kFusedThreads = 512, kFusedWaves = kFusedThreads / kWave;

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every extent: loads read zeros, stores drop

template <bool BF16, int T>  // T: chunk slots per lane, T * 64 >= (r + 8) / EPC
__global__ __launch_bounds__(kFusedThreads) void power_fused_kernel(PowBatch b) {
    constexpr int EPC = BF16 ? 8 : 4;                // entries per 16-byte chunk
    constexpr uint32_t ES = BF16 ? 2 : 4;            // bytes per entry
    constexpr int DQ = 8 / EPC;                      // chunks per row of an 8 x 8 block
    extern __shared__ float lds[];                   // v [r], row sums / w [r], column sums [2][waves][r]
    __shared__ double red[kFusedWaves];
    __shared__ double tot;
    const int mi = blockIdx.x / b.workers, w = blockIdx.x - mi * b.workers;
    const PowMat &M = b.mat[mi];
    const int r = M.r;  // r % 8 == 0, (r + 8) / EPC <= T * 64 (the launcher checks)
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float *v = lds, *rowsum = lds + r;
    float *col_a = lds + (2 + wave) * r, *col_b = lds + (2 + kFusedWaves + wave) * r;
    char *a = static_cast<char *>(const_cast<void *>(M.a)) + (int64_t)w * r * r * ES;
    // A buffer over this unit's A: a position that a pair does not fill, and
    // any pair past the last, takes the offset kOOB and reads zeros. Every
    // pair thus issues the same loads with no branch around them, and the
    // compiler can wait for one pair's loads while the next pair's stay in
    // flight.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(a, 0, (int)((uint32_t)r * r * ES), 0x00020000);
    const int nch = r / EPC, G = r / 8, npairs = (G + 1) / 2;
    const float v0 = (float)(1.0 / sqrt((double)r));
    for (int c = threadIdx.x; c < r; c += kFusedThreads) v[c] = v0;
    __syncthreads();
    // Pair k: groups k and G - 1 - k (the same group once when G is odd).
    // Position p: chunk DQ k + p of group k for p < La, else chunk
    // DQ (G - 1 - k) + p - La of the other group.
    struct Pos {
        int row0, q;
        bool first, ok;
    };
    auto where = [&](int k, int t) {
        const int ga = k, gb = G - 1 - k;
        const int la = nch - DQ * ga, lb = gb > ga ? nch - DQ * gb : 0;
        const int p = lane + kWave * t;
        Pos o;
        o.first = p < la;
        o.ok = k < npairs && p < la + lb;
        o.row0 = 8 * (o.first ? ga : gb);
        o.q = o.first ? DQ * ga + p : DQ * gb + (p - la);
        return o;
    };
    auto issue = [&](int k, v4u32 (&h)[T][8]) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const Pos o = where(k, t);
            const uint32_t off = ((uint32_t)o.row0 * r + (uint32_t)o.q * EPC) * ES;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                h[t][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, o.ok ? off + (uint32_t)i * r * ES : kOOB, 0, 0);
        }
    };
    // Pair k (k < npairs): its 16 row sums to LDS, its column sums added to
    // the wave's arrays.
    auto consume = [&](int k, const v4u32 (&h)[T][8]) {
        const int ga = k, gb = G - 1 - k;
        const bool two = gb > ga;
        const int np = nch - DQ * ga + (two ? nch - DQ * gb : 0);
        float va[8], vb[8], ra[8], rb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            va[i] = v[8 * ga + i];
            vb[i] = two ? v[8 * gb + i] : 0.f;
            ra[i] = rb[i] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (kWave * t >= np) continue;  // uniform: no position in this slot
            const Pos o = where(k, t);
            if (!o.ok) continue;
            float vc[EPC], cs[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                vc[e] = v[o.q * EPC + e];
                cs[e] = 0.f;
            }
            // the group's diagonal chunks add nothing to the column sums:
            // multiplied by 0 (a non-finite A gives s = 0 either way)
            const bool cols = o.q >= o.row0 / EPC + DQ;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float x[EPC];
                if constexpr (BF16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[2 * e] = bf16_bits_to_f32(h[t][i][e] & 0xffffu);
                        x[2 * e + 1] = bf16_bits_to_f32(h[t][i][e] >> 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(h[t][i][e]);
                }
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) d = __builtin_fmaf(x[e], vc[e], d);
                ra[i] += o.first ? d : 0.f;
                rb[i] += o.first ? 0.f : d;
                const float vj = cols ? (o.first ? va[i] : vb[i]) : 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) cs[e] = __builtin_fmaf(x[e], vj, cs[e]);
            }
            float *cp = (o.first ? col_a : col_b) + o.q * EPC;
#pragma unroll
            for (int e = 0; e < EPC; ++e) cp[e] += cs[e];
        }
        // 16 sums over the wave: each exchange halves the values a lane
        // keeps, so lane l ends with the whole sum of value
        // 8 l5 + 4 l4 + 2 l3 + l2 (l5 .. l2: bits of l).
        float s[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = ra[i];
            s[8 + i] = rb[i];
        }
#pragma unroll
        for (int half = 8, bit = 32; half >= 1; half >>= 1, bit >>= 1) {
            const bool hi = (lane & bit) != 0;
#pragma unroll
            for (int m = 0; m < half; ++m) {
                const float keep = hi ? s[half + m] : s[m], send = hi ? s[m] : s[half + m];
                s[m] = keep + __shfl_xor(send, bit, kWave);
            }
        }
        s[0] += __shfl_xor(s[0], 2, kWave);
        s[0] += __shfl_xor(s[0], 1, kWave);
        const int idx = lane >> 2;  // 8 l5 + 4 l4 + 2 l3 + l2
        if ((lane & 3) == 0 && (idx < 8 || two)) rowsum[idx < 8 ? 8 * ga + idx : 8 * gb + idx - 8] = s[0];
    };
    double n2 = 0.0;
    for (int it = 0; it < b.it; ++it) {
        for (int c = lane; c < r; c += kWave) col_a[c] = col_b[c] = 0.f;  // this wave's arrays
        // The wave's pairs k = wave, wave + 8, ... two at a time in two
        // register sets: a pair's loads are issued before the pair ahead of
        // it is summed.
        v4u32 ha[T][8], hb[T][8];
        issue(wave, ha);
        for (int k = wave; k < npairs; k += 2 * kFusedWaves) {
            issue(k + kFusedWaves, hb);
            consume(k, ha);
            issue(k + 2 * kFusedWaves, ha);
            if (k + kFusedWaves < npairs) consume(k + kFusedWaves, hb);
        }
        __syncthreads();  // every read of v done; row and column sums complete
        double sq = 0.0;
        for (int c = threadIdx.x; c < r; c += kFusedThreads) {
            float wc = rowsum[c];
#pragma unroll
            for (int k = 0; k < 2 * kFusedWaves; ++k) wc += lds[(2 + k) * r + c];
            rowsum[c] = wc;
            sq += (double)wc * wc;
        }
        sq = wave_sum(sq);
        if (lane == 0) red[wave] = sq;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t2 = 0.0;
            for (int k = 0; k < kFusedWaves; ++k) t2 += red[k];
            tot = t2;
        }
        __syncthreads();
        n2 = tot;
        const float inv = n2 > 0.0 ? (float)(1.0 / sqrt(n2)) : 0.0f;
        for (int c = threadIdx.x; c < r; c += kFusedThreads) v[c] = rowsum[c] * inv;
        __syncthreads();
    }
    // lambda = ||A v|| of the last step; s = 1 / sqrt(lambda), s^2 = 1 / lambda
    float s = 0.f, s2 = 0.f;
    const double lambda = sqrt(n2);
    if (lambda > 0.0) {
        s = (float)(1.0 / sqrt(lambda));
        s2 = (float)(1.0 / lambda);
    }
    if (threadIdx.x == 0) b.scales[M.unit_begin + w] = make_float2(s, s2);
}

}  // namespace

int32_t power_blocks_per_worker(int64_t r) { return (int32_t)((r + kPowRowsPerBlock - 1) / kPowRowsPerBlock); }

void launch_power_step(const PowBatch &b, bool bf16, hipStream_t s) {
    dim3 grid(b.total_blocks), block(kThreads);
    int rmax = 0;
    for (int i = 0; i < b.nmat; ++i) rmax = b.mat[i].r > rmax ? b.mat[i].r : rmax;
    const size_t lds = (size_t)rmax * sizeof(float);  // v; rmax <= kMaxPowR
    if (bf16)
        hipLaunchKernelGGL(power_step_kernel<true>, grid, block, lds, s, b);
    else
        hipLaunchKernelGGL(power_step_kernel<false>, grid, block, lds, s, b);
}

void launch_power_finalize(const PowBatch &b, hipStream_t s) {
    const int units = b.nmat * b.workers;
    hipLaunchKernelGGL(power_finalize_kernel, dim3((units + 3) / 4), dim3(kThreads), 0, s, b);
}

void launch_power_fused(const PowBatch &b, bool bf16, hipStream_t s) {
    int rmax = 0;
    for (int i = 0; i < b.nmat; ++i) rmax = b.mat[i].r > rmax ? b.mat[i].r : rmax;
    const size_t lds = (size_t)rmax * (2 + 2 * kFusedWaves) * sizeof(float);
    dim3 grid(b.nmat * b.workers), block(kFusedThreads);
    const int epc = bf16 ? 8 : 4;
    const int slots = ((rmax + 8) / epc + kWave - 1) / kWave;  // chunk slots per lane for a pair of row groups
#define SM_FUSED(BF, TS) hipLaunchKernelGGL((power_fused_kernel<BF, TS>), grid, block, lds, s, b)
    if (bf16) {
        if (slots <= 1) SM_FUSED(true, 1);
        else SM_FUSED(true, 2);
    } else {
        if (slots <= 1) SM_FUSED(false, 1);
        else SM_FUSED(false, 2);
    }
#undef SM_FUSED
}

}  // namespace sm
