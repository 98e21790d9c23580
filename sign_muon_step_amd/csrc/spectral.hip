// spectral.hip -- spectral normalisation of the Newton-Schulz input for
// gfx950: power iteration on each worker's Gram matrix, the scale it gives,
// and the rescaling of the stored Gram matrix.
//
// Method: "SignMuon: Communication-Efficient Distributed Muon Optimization"
// (gist.science, paper 2605.16311, technical summary), §4 "nanoGPT" (the
// results hold with spectral as with Frobenius scaling of the Newton-Schulz
// input). The summary gives no procedure; the one built here: A_raw is the
// stored Gram matrix of the stored momentum (the Newton-Schulz orientation),
// lambda is the last ||A v|| of p power-iteration steps from the all-ones
// vector (w = A v, lambda = ||w||, v = w / lambda), s = 1 / sqrt(lambda), and
// the first iteration uses A_0 = round(fp32(1 / lambda) * A_raw) with
// X_0 = s M. lambda = 0 gives s = 0 (U = 0).
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

// A <- round(s^2 * A) in place for every (matrix, worker) Gram matrix; 8
// entries per thread. Blocks: per matrix, workers x rescale_bpw.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void gram_rescale_kernel(PowBatch b) {
    const int blk = blockIdx.x;
    const int mi = find_start(b.starts, blk);
    const PowMat &M = b.mat[mi];
    const int local = blk - b.starts.v[mi];
    const int w = local / M.bpw, cb = local - w * M.bpw;
    const int64_t rr = (int64_t)M.r * M.r;
    const float s2 = b.scales[M.unit_begin + w].y;
    const int64_t e0 = ((int64_t)cb * kThreads + threadIdx.x) * 8;
    char *a = static_cast<char *>(const_cast<void *>(M.a)) + (int64_t)w * rr * (BF16 ? 2 : 4);
    if ((rr & 7) == 0 && e0 + 8 <= rr) {  // 16-byte aligned: one (bf16) or two (fp32) vector accesses
        if (BF16) {
            uint4 *p = reinterpret_cast<uint4 *>(a + e0 * 2);
            const uint4 q = *p;
            uint32_t h[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int t = 0; t < 4; ++t)
                h[t] = pack_bf16x2(s2 * bf16_bits_to_f32(h[t] & 0xffffu), s2 * bf16_bits_to_f32(h[t] >> 16));
            *p = make_uint4(h[0], h[1], h[2], h[3]);
        } else {
            float4 *p = reinterpret_cast<float4 *>(a + e0 * 4);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float4 v = p[t];
                v.x *= s2; v.y *= s2; v.z *= s2; v.w *= s2;
                p[t] = v;
            }
        }
        return;
    }
    for (int64_t e = e0; e < e0 + 8 && e < rr; ++e) {
        if (BF16) {
            uint16_t *p = reinterpret_cast<uint16_t *>(a) + e;
            *p = (uint16_t)f32_to_bf16_bits(s2 * bf16_bits_to_f32(*p));
        } else {
            float *p = reinterpret_cast<float *>(a) + e;
            *p = s2 * *p;
        }
    }
}

// ---------------------------------------------------------------------------
// The whole power iteration of one (matrix, worker) in one workgroup: the p
// steps, the scale and (for the first Newton-Schulz iteration) the rescale
// of A, in one launch over every unit. A is stored symmetric (each
// off-diagonal entry with its mirror), so a step reads the upper part only.
// Rows go in groups of 8 (rows j0 .. j0 + 7), one group per wave at a time.
// For row j of a group:
//   row sum:     sum over c >= j0 of A[j][c] v[c]   (whole 16-byte chunks;
//                the few c < j of the group's own chunk are the stored
//                lower entries of the diagonal block)
//   column sums: A[j][c] v[j] added to column c for every c >= j0 + 8.
// A pair (j, c) with c < j0 is then covered by row c's column sums (c's
// group ends at or before j0), and no pair twice: w[c] = row sum of c + the
// eight waves' column sums of c, in wave order. Lane l owns the 16-byte
// column chunks l, l + 64, ... and keeps their column sums in registers over
// the wave's groups. Every sum runs in a fixed order, so results do not
// depend on timing. The working set of the units in flight is their upper
// triangles (about 0.6 MB at r = 768), which the Infinity Cache holds
// across the p steps, where one launch per step over every unit streams all
// of A from HBM each time.
// ---------------------------------------------------------------------------
constexpr int kFusedThreads = 512, kFusedWaves = kFusedThreads / kWave;

template <bool BF16, int T>  // T: chunk slots per lane, T * 64 * EPC >= r
__global__ __launch_bounds__(kFusedThreads) void power_fused_kernel(PowBatch b, int rescale) {
    constexpr int EPC = BF16 ? 8 : 4;                // entries per 16-byte chunk
    extern __shared__ float lds[];                   // v [r], row sums / w [r], column sums [waves][r]
    __shared__ double red[kFusedWaves];
    __shared__ double tot;
    const int mi = blockIdx.x / b.workers, w = blockIdx.x - mi * b.workers;
    const PowMat &M = b.mat[mi];
    const int r = M.r;  // r % 8 == 0, r <= T * 64 * EPC (the launcher checks)
    float *v = lds, *rowsum = lds + r, *colsum = lds + 2 * r;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    char *a = static_cast<char *>(const_cast<void *>(M.a)) + (int64_t)w * r * r * (BF16 ? 2 : 4);
    const int nch = r / EPC;  // chunks per row
    const float v0 = (float)(1.0 / sqrt((double)r));
    for (int c = threadIdx.x; c < r; c += kFusedThreads) v[c] = v0;
    __syncthreads();
    double n2 = 0.0;
    for (int it = 0; it < b.it; ++it) {
        float col[T][EPC];
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int e = 0; e < EPC; ++e) col[t][e] = 0.f;
        // Row groups j0 = 8 wave, 8 wave + 64, ...: the next group's chunks are
        // loaded while the current one is summed.
        auto load_group = [&](int j0, uint4 (&h)[T][8]) {
            const int qa = j0 / EPC;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int q = lane + kWave * t;
                const bool ok = j0 < r && q >= qa && q < nch;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    h[t][i] = ok ? *reinterpret_cast<const uint4 *>(
                                       a + ((int64_t)(j0 + i) * r + (int64_t)q * EPC) * (BF16 ? 2 : 4))
                                 : make_uint4(0, 0, 0, 0);
            }
        };
        uint4 hc[T][8];
        load_group(8 * wave, hc);
        for (int j0 = 8 * wave; j0 < r; j0 += 8 * kFusedWaves) {
            uint4 hn[T][8];
            load_group(j0 + 8 * kFusedWaves, hn);
            const int qa = j0 / EPC, qb = (j0 + 8) / EPC;  // first chunk read; first with column sums
            float vj[8], row[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                vj[i] = v[j0 + i];
                row[i] = 0.f;
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int q = lane + kWave * t;
                if (kWave * t + kWave <= qa || kWave * t >= nch) continue;  // uniform: no chunk of this slot
                if (q < qa || q >= nch) continue;
                float vc[EPC];
#pragma unroll
                for (int e = 0; e < EPC; ++e) vc[e] = v[q * EPC + e];
                // the group's own chunk (q < qb) adds nothing to the column sums:
                // multiplied by 0 (a non-finite A gives s = 0 either way)
                const bool cols = q >= qb;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float x[EPC];
                    if constexpr (BF16) {
                        const uint32_t hw[4] = {hc[t][i].x, hc[t][i].y, hc[t][i].z, hc[t][i].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[2 * e] = bf16_bits_to_f32(hw[e] & 0xffffu);
                            x[2 * e + 1] = bf16_bits_to_f32(hw[e] >> 16);
                        }
                    } else {
                        x[0] = __uint_as_float(hc[t][i].x);
                        x[1] = __uint_as_float(hc[t][i].y);
                        x[2] = __uint_as_float(hc[t][i].z);
                        x[3] = __uint_as_float(hc[t][i].w);
                    }
                    const float cs = cols ? vj[i] : 0.f;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        row[i] = __builtin_fmaf(x[e], vc[e], row[i]);
                        col[t][e] = __builtin_fmaf(x[e], cs, col[t][e]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float s = wave_sum_f32(row[i]);
                if (lane == 0) rowsum[j0 + i] = s;
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) hc[t][i] = hn[t][i];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int q = lane + kWave * t;
            if (q < nch)
#pragma unroll
                for (int e = 0; e < EPC; ++e) colsum[wave * r + q * EPC + e] = col[t][e];
        }
        __syncthreads();  // every read of v done; row and column sums complete
        double sq = 0.0;
        for (int c = threadIdx.x; c < r; c += kFusedThreads) {
            float wc = rowsum[c];
#pragma unroll
            for (int k = 0; k < kFusedWaves; ++k) wc += colsum[k * r + c];
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
    if (!rescale) return;
    // A <- round(s^2 * A), 16 bytes per access (r % 8 == 0), eight accesses of
    // each thread in flight at a time
    constexpr int kIn = 8;
    const int64_t nq = (int64_t)r * r / EPC;
    uint4 *p = reinterpret_cast<uint4 *>(a);
    for (int64_t i0 = threadIdx.x; i0 < nq; i0 += (int64_t)kIn * kFusedThreads) {
        uint4 h[kIn];
#pragma unroll
        for (int u = 0; u < kIn; ++u) {
            const int64_t i = i0 + (int64_t)u * kFusedThreads;
            h[u] = i < nq ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kIn; ++u) {
            const int64_t i = i0 + (int64_t)u * kFusedThreads;
            if (i >= nq) break;
            if constexpr (BF16) {
                uint32_t hw[4] = {h[u].x, h[u].y, h[u].z, h[u].w};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    hw[t] = pack_bf16x2(s2 * bf16_bits_to_f32(hw[t] & 0xffffu), s2 * bf16_bits_to_f32(hw[t] >> 16));
                p[i] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            } else {
                p[i] = make_uint4(__float_as_uint(s2 * __uint_as_float(h[u].x)),
                                  __float_as_uint(s2 * __uint_as_float(h[u].y)),
                                  __float_as_uint(s2 * __uint_as_float(h[u].z)),
                                  __float_as_uint(s2 * __uint_as_float(h[u].w)));
            }
        }
    }
}

}  // namespace

int32_t power_blocks_per_worker(int64_t r) { return (int32_t)((r + kPowRowsPerBlock - 1) / kPowRowsPerBlock); }
int32_t rescale_blocks_per_worker(int64_t r) { return (int32_t)((r * r + kThreads * 8 - 1) / (kThreads * 8)); }

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

void launch_power_fused(const PowBatch &b, bool bf16, bool rescale, hipStream_t s) {
    int rmax = 0;
    for (int i = 0; i < b.nmat; ++i) rmax = b.mat[i].r > rmax ? b.mat[i].r : rmax;
    const size_t lds = (size_t)rmax * (2 + kFusedWaves) * sizeof(float);
    dim3 grid(b.nmat * b.workers), block(kFusedThreads);
    const int slots = (rmax / (bf16 ? 8 : 4) + kWave - 1) / kWave;  // chunk slots per lane
    const int rs = rescale ? 1 : 0;
#define SM_FUSED(BF, TS) hipLaunchKernelGGL((power_fused_kernel<BF, TS>), grid, block, lds, s, b, rs)
    if (bf16) {
        if (slots <= 1) SM_FUSED(true, 1);
        else SM_FUSED(true, 2);
    } else {
        if (slots <= 1) SM_FUSED(false, 1);
        else SM_FUSED(false, 2);
    }
#undef SM_FUSED
}

void launch_gram_rescale(const PowBatch &b, bool bf16, hipStream_t s) {
    dim3 grid(b.total_blocks), block(kThreads);
    if (bf16)
        hipLaunchKernelGGL(gram_rescale_kernel<true>, grid, block, 0, s, b);
    else
        hipLaunchKernelGGL(gram_rescale_kernel<false>, grid, block, 0, s, b);
}

}  // namespace sm
