// api.hip -- host side of the C ABI declared in include/signmuon.h: argument
// checks, workspace layout and the launch sequence of the Sign-Muon step.
//
// Method: "SignMuon: Communication-Efficient Distributed Muon Optimization"
// (gist.science, paper 2605.16311, technical summary), §2 "Algorithmic flow".
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "signmuon.h"
#include "sm_internal.h"

// Device scratch of signmuon_step_noalloc: the workspace of an allocation-
// free step lives here, one copy per GPU, held until the process ends. Host
// code never passes this name to a kernel or a copy (on the host it only
// stands for the symbol): it uses the device address hipGetSymbolAddress
// returns for the current device (noalloc_scratch below).
static __device__ __align__(256) char scratch[SIGNMUON_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_hip_err[192] = "";

constexpr int64_t kMaxDim = (int64_t)1 << 20;   // rows or cols
constexpr int64_t kMaxN = ((int64_t)1 << 31) - 1;  // entries per matrix
constexpr int32_t kMaxWorkers = 255;             // vote counters are 8 bit-planes
constexpr int32_t kMaxIters = 1000;
constexpr size_t kSectionAlign = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool dtype_ok(int d) { return d == SIGNMUON_F32 || d == SIGNMUON_BF16; }
inline size_t esize(signmuon_dtype d) { return d == SIGNMUON_BF16 ? 2 : 4; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return SIGNMUON_OK;
    std::snprintf(g_hip_err, sizeof g_hip_err, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return SIGNMUON_EHIP;
}

inline int last_launch() { return hip_status(hipGetLastError()); }

// Optional per-launch event recording (signmuon_step_traced).
struct Tracer {
    signmuon_trace *t = nullptr;
    hipStream_t st = nullptr;
    int begin() {
        if (!t) return SIGNMUON_OK;
        t->launches = 0;
        if (t->events && t->capacity > 0)
            return hip_status(hipEventRecord(static_cast<hipEvent_t>(t->events[0]), st));
        return SIGNMUON_OK;
    }
    // Check the launch just made, then record its event.
    int after(int kind) {
        if (int rc = last_launch()) return rc;
        if (!t) return SIGNMUON_OK;
        const int32_t i = t->launches++;
        if (t->events && i + 1 < t->capacity) {
            if (t->kinds) t->kinds[i] = kind;
            return hip_status(hipEventRecord(static_cast<hipEvent_t>(t->events[i + 1]), st));
        }
        return SIGNMUON_OK;
    }
};

struct MatPlan {
    int64_t R, C, n, r, nw;
    int32_t mom_bpw;        // momentum blocks per worker
    int32_t partial_begin;  // first partial of (matrix, worker 0)
    int32_t unit_begin;     // scales index of (matrix, worker 0)
    size_t gram_off;        // bytes from the Gram section: [Mw][r][r]
    size_t iter_off;        // bytes from each iterate section: [Mw][n]
    size_t post_gram_off;   // post-vote step: [r][r]
    size_t post_iter_off;   // post-vote step: [n]
    size_t vns_off;         // vote in NS storage: [n]
    size_t u_off;           // fp32 U scratch [Mw][n] (unfused pack only)
    size_t pw_off;          // spectral: power vectors [2][Mw][r] (floats from the section)
    size_t pwp_off;         // spectral: block sums [2][Mw][pw_bpw] (doubles from the section)
    int32_t pw_bpw;         // spectral: power-step blocks per worker
    int32_t gram_split;     // k chunks per Gram tile (0: the Gram kernel stores A itself)
    size_t gpart_off;       // split Gram: partial tiles [Mw][Gram tiles][split][256][256] fp32
    bool fused_k0;          // k = 0: the momentum kernel packs the signs (bits payload)
    bool fused_pack;        // the last product packs the signs itself (bits payload)
    bool fused_i8;          // the last product writes the int8 signs itself (int8 payload)
    bool u_scratch;         // U goes through workspace scratch
};

struct Plan {
    std::vector<MatPlan> m;
    int32_t units = 0, post_unit_base = 0, partials = 0;
    size_t off_partials = 0, off_scales = 0, off_nnz = 0, off_gram = 0, off_iter[2] = {0, 0};
    size_t off_vns = 0, off_u = 0, off_pw = 0, off_pwp = 0, off_gpart = 0, total = 0;
    size_t off_fix = 0;  // k = 0 packed by the momentum kernel: per-unit flags
    bool any_k0 = false;
    bool spectral = false;
    bool i8 = false;  // int8 payload
};

// Shapes, counts and dtypes (not pointers). Fills the plan.
int make_plan(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p, bool step,
              Plan &pl) {
    if (!mats || !p || n_mats < 1 || n_mats > SIGNMUON_MAX_MATRICES) return SIGNMUON_EINVAL;
    if (p->workers < 1 || p->ns_iters < 0 || p->post_polar_iters < 0) return SIGNMUON_EINVAL;
    if (p->ns_iters > kMaxIters || p->post_polar_iters > kMaxIters) return SIGNMUON_ERANGE;
    if (p->workers > kMaxWorkers) return SIGNMUON_ERANGE;
    if (!std::isfinite(p->beta) || !std::isfinite(p->eta)) return SIGNMUON_EINVAL;
    if (!dtype_ok(p->grad_dtype) || !dtype_ok(p->mom_dtype) || !dtype_ok(p->ns_dtype))
        return SIGNMUON_EDTYPE;
    if (p->mom_dtype != p->ns_dtype) return SIGNMUON_EDTYPE;  // X0 is read in place from M
    if (p->norm != SIGNMUON_NORM_FROBENIUS && p->norm != SIGNMUON_NORM_SPECTRAL) return SIGNMUON_EINVAL;
    pl.spectral = p->norm == SIGNMUON_NORM_SPECTRAL;
    if (p->payload != SIGNMUON_PAYLOAD_BITS && p->payload != SIGNMUON_PAYLOAD_INT8) return SIGNMUON_EINVAL;
    pl.i8 = step && p->payload == SIGNMUON_PAYLOAD_INT8;
    if (pl.i8 && p->post_polar_iters > 0) return SIGNMUON_EINVAL;
    if (pl.spectral && p->power_iters < 1) return SIGNMUON_EINVAL;
    if (pl.spectral && p->power_iters > kMaxIters) return SIGNMUON_ERANGE;
    const int64_t mw = p->workers;
    const size_t ns = esize(p->ns_dtype);
    const bool post = step && p->post_polar_iters > 0;
    size_t pw = 0, pwp = 0;
    pl.m.assign(n_mats, MatPlan{});
    size_t gram = 0, iter = 0, post_gram = 0, post_iter = 0, vns = 0, u = 0, gpart = 0;
    int64_t partials = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const signmuon_matrix &s = mats[i];
        if (s.rows < 1 || s.cols < 1) return SIGNMUON_EINVAL;
        if (s.rows > kMaxDim || s.cols > kMaxDim || s.rows * s.cols > kMaxN) return SIGNMUON_ERANGE;
        MatPlan &q = pl.m[i];
        q.R = s.rows;
        q.C = s.cols;
        q.n = q.R * q.C;
        q.r = q.R < q.C ? q.R : q.C;
        q.nw = (q.n + 63) / 64;
        q.mom_bpw = (int32_t)((q.n + sm::kMomChunk - 1) / sm::kMomChunk);
        q.partial_begin = (int32_t)partials;
        partials += mw * q.mom_bpw;
        q.unit_begin = pl.units;
        pl.units += (int32_t)mw;
        q.gram_off = gram;
        gram += align_up((size_t)(mw * q.r * q.r) * ns, kSectionAlign);
        q.gram_split = sm::ns_gram_split(q.R, q.C, p->ns_dtype == SIGNMUON_BF16);
        q.gpart_off = gpart;
        if (q.gram_split > 0)
            gpart += (size_t)mw * sm::ns_gram_tiles(q.R, q.C) * q.gram_split * sm::kNsTileM * sm::kNsTileM *
                     sizeof(float);
        q.iter_off = iter;
        iter += align_up((size_t)(mw * q.n) * ns, kSectionAlign);
        q.post_gram_off = post_gram;
        post_gram += align_up((size_t)(q.r * q.r) * ns, kSectionAlign);
        q.post_iter_off = post_iter;
        post_iter += align_up((size_t)q.n * ns, kSectionAlign);
        q.vns_off = vns;
        if (post) vns += align_up((size_t)q.n * ns, kSectionAlign);
        // k = 0 (Frobenius scale, no U output): the momentum kernel packs
        // sign(M), the signs of M / ||M||_F unless finalize_scales flags the
        // unit (a NaN or Inf entry; the fix-up kernel then redoes it)
        q.fused_k0 = step && !pl.i8 && p->ns_iters == 0 && !pl.spectral && s.polar_out == nullptr &&
                     (q.n % 64) == 0;
        pl.any_k0 = pl.any_k0 || q.fused_k0;
        q.fused_pack = step && !pl.i8 && p->ns_iters > 0 && (q.C % 64) == 0;
        q.fused_i8 = pl.i8 && p->ns_iters > 0;
        q.u_scratch = step && p->ns_iters > 0 && !q.fused_pack && !q.fused_i8 && s.polar_out == nullptr;
        q.u_off = u;
        if (q.u_scratch) u += align_up((size_t)(mw * q.n) * 4, kSectionAlign);
        q.pw_bpw = sm::power_blocks_per_worker(q.r);
        q.pw_off = pw;
        q.pwp_off = pwp;
        if (pl.spectral) {
            if (q.r > sm::kMaxPowR) return SIGNMUON_ERANGE;
            pw += (size_t)(2 * mw * q.r + 63) / 64 * 64;
            pwp += (size_t)(2 * mw * q.pw_bpw + 31) / 32 * 32;
        }
    }
    if (partials > INT32_MAX / 2) return SIGNMUON_ERANGE;
    pl.partials = (int32_t)partials;
    pl.post_unit_base = pl.units;
    const int32_t scale_count = pl.units + n_mats;

    size_t off = 0;
    pl.off_partials = off;
    off += align_up((size_t)partials * sizeof(double), kSectionAlign);
    pl.off_scales = off;
    off += align_up((size_t)scale_count * sizeof(float2), kSectionAlign);
    pl.off_fix = off;
    off += pl.any_k0 ? align_up((size_t)pl.units * sizeof(int32_t), kSectionAlign) : 0;
    pl.off_nnz = off;
    off += align_up((size_t)n_mats * sizeof(uint32_t), kSectionAlign);
    pl.off_pw = off;
    off += align_up(pw * sizeof(float), kSectionAlign);
    pl.off_pwp = off;
    off += align_up(pwp * sizeof(double), kSectionAlign);
    pl.off_gram = off;
    const bool need_gram = p->ns_iters > 0 || post || pl.spectral;
    off += need_gram ? (gram > post_gram ? gram : post_gram) : 0;
    pl.off_gpart = off;
    off += need_gram ? align_up(gpart, kSectionAlign) : 0;
    size_t iter_need = 0;
    if (p->ns_iters >= 2) iter_need = iter;
    if (post && p->post_polar_iters >= 2 && post_iter > iter_need) iter_need = post_iter;
    pl.off_iter[0] = off;
    off += iter_need;
    pl.off_iter[1] = off;
    off += iter_need;
    pl.off_vns = off;
    off += vns;
    pl.off_u = off;
    off += u;
    pl.total = off;
    return SIGNMUON_OK;
}

int check_step_pointers(const signmuon_matrix *mats, int32_t n_mats, bool step, bool i8) {
    for (int32_t i = 0; i < n_mats; ++i) {
        const signmuon_matrix &s = mats[i];
        if (!s.grad || !s.momentum) return SIGNMUON_EINVAL;
        if (step && (!(i8 ? (const void *)s.signs_i8 : (const void *)s.packed) || !s.weight))
            return SIGNMUON_EINVAL;
        if (!step && !s.polar_out) return SIGNMUON_EINVAL;
        const void *ptrs[7] = {s.grad, s.momentum, s.polar_out, s.packed, s.weight, s.vote_out,
                               i8 ? s.signs_i8 : nullptr};
        for (const void *q : ptrs)
            if (q && !aligned16(q)) return SIGNMUON_EALIGN;
    }
    return SIGNMUON_OK;
}

template <typename T>
T *ws_at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// ---------------------------------------------------------------------------
// Launch sequence shared by signmuon_momentum_ns and signmuon_step.
// ---------------------------------------------------------------------------
int run_momentum(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                 const Plan &pl, void *ws, hipStream_t st, Tracer &tr) {
    for (int32_t c0 = 0; c0 < n_mats; c0 += sm::kMaxMatsPerLaunch) {
        const int32_t cn = n_mats - c0 < sm::kMaxMatsPerLaunch ? n_mats - c0 : sm::kMaxMatsPerLaunch;
        sm::MomBatch b{};
        b.nmat = cn;
        b.workers = p->workers;
        b.beta = p->beta;
        b.g_bf16 = p->grad_dtype == SIGNMUON_BF16;
        b.m_bf16 = p->mom_dtype == SIGNMUON_BF16;
        b.partials = ws_at<double>(ws, pl.off_partials);
        b.scales = ws_at<float2>(ws, pl.off_scales);
        b.pack_fix = pl.any_k0 ? ws_at<int32_t>(ws, pl.off_fix) : nullptr;
        bool packs = false;
        int64_t blocks = 0;
        for (int32_t j = 0; j < cn; ++j) {
            const MatPlan &q = pl.m[c0 + j];
            sm::MomMat &d = b.mat[j];
            d.g = mats[c0 + j].grad;
            d.m = mats[c0 + j].momentum;
            d.packed = q.fused_k0 ? mats[c0 + j].packed : nullptr;
            packs = packs || q.fused_k0;
            d.n = q.n;
            d.block_begin = (int32_t)blocks;
            b.starts.v[j] = d.block_begin;
            d.blocks_per_worker = q.mom_bpw;
            d.partial_begin = q.partial_begin;
            d.unit_begin = q.unit_begin;
            blocks += (int64_t)p->workers * q.mom_bpw;
        }
        if (blocks > INT32_MAX) return SIGNMUON_ERANGE;
        b.total_blocks = (int32_t)blocks;
        sm::launch_momentum(b, st);
        if (int rc = tr.after(SIGNMUON_K_MOMENTUM)) return rc;
        sm::launch_finalize_scales(b, st);
        if (int rc = tr.after(SIGNMUON_K_SCALES)) return rc;
        if (packs) {
            sm::launch_pack_fixup(b, b.m_bf16, st);
            if (int rc = tr.after(SIGNMUON_K_PACK)) return rc;
        }
    }
    return SIGNMUON_OK;
}

// Compute units of the current device (the persistent product's grid), read
// once per device.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Launch groups of one Newton-Schulz pass. Product: LG_DIRECT (one block per
// tile) or the persistent walk, whose wide and tall matrices go in separate
// launches (LG_WALK_WIDE, LG_WALK_TALL). Gram: LG_DIRECT (one block per tile,
// whole k range), LG_GRAM_SPLIT (split k, then the reduce) or LG_GRAM_WALK
// (the persistent walk, wide and tall matrices in one launch).
enum LaunchGroup { LG_DIRECT = 0, LG_WALK_WIDE = 1, LG_WALK_TALL = 2, LG_GRAM_SPLIT = 1, LG_GRAM_WALK = 2 };

// The Gram walk takes bf16 matrices that are not split, with 16-byte rows of
// X and of A, and a k loop of whole stage rounds (the 4 pipeline stages) at
// least two rounds long.
int gram_group(const MatPlan &q, bool bf16) {
    if (q.gram_split > 0) return LG_GRAM_SPLIT;
    if (!bf16) return LG_DIRECT;
    const int64_t c = q.R > q.C ? q.R : q.C;
    const int64_t kt_n = (c + 31) / 32;  // 32-wide bf16 k slices
    if (q.C % 8 || q.r % 8 || q.n * 2 >= ((int64_t)1 << 31)) return LG_DIRECT;
    if (kt_n % 4 || kt_n < 8) return LG_DIRECT;
    return LG_GRAM_WALK;
}

// The walk takes bf16 matrices whose k loop suits it (16-byte operands, k
// slices a multiple of the 4 pipeline stages and at least the 256 identity
// k plus one stage round), for the next iterate or the final signs (packed
// or int8) straight from the accumulators.
int product_group(const MatPlan &q, const sm::NsMat &d, bool bf16, sm::NsEpilogue epi) {
    if (!bf16) return LG_DIRECT;
    if (epi == sm::EPI_FINAL || epi == sm::EPI_FINAL_I8) {
        // signs straight from the accumulators: no U output
        if (d.out || !(d.packed || d.i8) || q.C % 64) return LG_DIRECT;
    } else if (epi != sm::EPI_ITER) {
        return LG_DIRECT;  // the W update stays on the one-tile-per-block kernel
    }
    const int64_t kt_n = (q.r + 31) / 32;  // 32-wide bf16 k slices
    if (q.C % 8 || q.r % 8 || q.n * 2 >= ((int64_t)1 << 31)) return LG_DIRECT;
    if (kt_n % 4 || kt_n < 256 / 32 + 4) return LG_DIRECT;
    return q.R > q.C ? LG_WALK_TALL : LG_WALK_WIDE;
}

// One Newton-Schulz launch pass over every (matrix, worker): iteration j's
// Gram matrix (pass 0) or product (pass 1). use_scales folds s^2 (Gram) or s
// (product) of iteration 0 in. The last product's epilogue writes U
// (polar_out or scratch) and, for step, the signs (packed or int8).
int ns_pass(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p, const Plan &pl,
            void *ws, bool step, int j, int pass, bool use_scales, hipStream_t st, Tracer &tr,
            bool muon = false) {
    const int k = p->ns_iters;
    const bool last = j == k - 1;
    const bool bf16 = p->ns_dtype == SIGNMUON_BF16;
    const float2 *scales = ws_at<float2>(ws, pl.off_scales);
    // Descriptor of matrix i for this pass.
    auto describe = [&](int32_t i, sm::NsMat &d) {
        const MatPlan &q = pl.m[i];
        const signmuon_matrix &s = mats[i];
        d = sm::NsMat{};
        d.R = (int32_t)q.R;
        d.C = (int32_t)q.C;
        d.unit_begin = q.unit_begin;
        d.x = j == 0 ? s.momentum : ws_at<const char>(ws, pl.off_iter[(j - 1) & 1] + q.iter_off);
        d.a = ws_at<char>(ws, pl.off_gram + q.gram_off);
        if (!last) {
            d.out = ws_at<char>(ws, pl.off_iter[j & 1] + q.iter_off);
        } else if (muon) {
            d.out = s.weight;
            d.u_out = s.polar_out;
        } else if (s.polar_out) {
            d.out = s.polar_out;
        } else if (q.u_scratch) {
            d.out = ws_at<char>(ws, pl.off_u + q.u_off);
        } else {
            d.out = nullptr;
        }
        d.packed = (last && step && q.fused_pack) ? s.packed : nullptr;
        d.i8 = (last && step && q.fused_i8) ? s.signs_i8 : nullptr;
        d.tiles_per_worker = pass == 0 ? sm::ns_gram_tiles(q.R, q.C) : sm::ns_product_tiles(q.R, q.C);
    };
    const sm::NsEpilogue epi = !last ? sm::EPI_ITER
                                     : (muon ? sm::EPI_WUPD : (step && pl.i8 ? sm::EPI_FINAL_I8 : sm::EPI_FINAL));
    // The matrices of each launch group, in order.
    std::vector<int32_t> groups[3];
    for (int32_t i = 0; i < n_mats; ++i) {
        int g = LG_DIRECT;
        if (pass == 1) {
            sm::NsMat d;
            describe(i, d);
            g = product_group(pl.m[i], d, bf16, epi);
        } else {
            g = gram_group(pl.m[i], bf16);
        }
        groups[g].push_back(i);
    }
    // The Gram's tiles take time in proportion to their k range and blocks
    // are handed out in order: longest k first (stable), so that the short
    // tiles fill the end of the launch. Each tile is computed on its own, so
    // the order changes no result.
    if (pass == 0)
        for (auto &idx : groups)
            std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
                const int64_t cx = pl.m[x].R > pl.m[x].C ? pl.m[x].R : pl.m[x].C;
                const int64_t cy = pl.m[y].R > pl.m[y].C ? pl.m[y].R : pl.m[y].C;
                return cx > cy;
            });
    for (int g = 0; g < 3; ++g) {
        const std::vector<int32_t> &idx = groups[g];
        for (size_t c0 = 0; c0 < idx.size(); c0 += sm::kMaxMatsPerLaunch) {
            const int32_t cn = (int32_t)std::min(idx.size() - c0, (size_t)sm::kMaxMatsPerLaunch);
            sm::NsBatch b{};
            b.nmat = cn;
            b.workers = p->workers;
            b.use_scales = use_scales;
            b.scales = scales;
            b.eta = p->eta;  // the W-update epilogue
            b.id_scaled = pass == 1 && use_scales && pl.spectral ? 1 : 0;
            const bool split = pass == 0 && g == LG_GRAM_SPLIT;
            const bool gram_walk = pass == 0 && g == LG_GRAM_WALK;
            // split Gram: Gram tiles x split blocks per worker; the reduce
            // then runs 16 blocks per Gram tile. The Gram walk numbers its
            // tiles matrix-major (all workers of a matrix, then the next).
            auto number_tiles = [&](int per_tile) {
                int64_t tiles = 0;
                const int64_t per_mat = gram_walk ? p->workers : 1;
                for (int32_t i = 0; i < cn; ++i) {
                    sm::NsMat &d = b.mat[i];
                    d.tile_begin = (int32_t)tiles;
                    b.starts.v[i] = d.tile_begin;
                    tiles += (int64_t)d.tiles_per_worker * (per_tile ? per_tile : d.split) * per_mat;
                }
                b.tiles_per_worker_all = (int32_t)(tiles / per_mat);
                b.total_tiles = (int32_t)(gram_walk ? tiles : tiles * p->workers);
                return tiles * (gram_walk ? 1 : p->workers) <= INT32_MAX;
            };
            for (int32_t i = 0; i < cn; ++i) {
                sm::NsMat &d = b.mat[i];
                describe(idx[c0 + i], d);
                if (gram_walk) d.tiles_per_worker = sm::ns_gram_walk_tiles(pl.m[idx[c0 + i]].R, pl.m[idx[c0 + i]].C);
                if (split) {
                    const MatPlan &q = pl.m[idx[c0 + i]];
                    d.split = q.gram_split;
                    d.out = ws_at<char>(ws, pl.off_gpart + q.gpart_off);
                }
            }
            if (!number_tiles(split ? 0 : 1)) return SIGNMUON_ERANGE;
            if (split) {
                sm::launch_ns_gram_split(b, bf16, st);
                if (int rc = tr.after(SIGNMUON_K_GRAM)) return rc;
                if (!number_tiles(sm::kGramReduceParts)) return SIGNMUON_ERANGE;
                sm::launch_gram_reduce(b, bf16, st);
            } else if (gram_walk)
                sm::launch_ns_gram_walk(b, std::min(b.total_tiles, device_cus()), st);
            else if (pass == 0)
                sm::launch_ns_gram(b, bf16, st);
            else if (g == LG_DIRECT)
                sm::launch_ns_product(b, bf16, epi, st);
            else
                sm::launch_ns_product_pack(b, g == LG_WALK_TALL, epi, std::min(b.total_tiles, device_cus()), st);
            if (int rc = tr.after(pass == 0 ? SIGNMUON_K_GRAM : SIGNMUON_K_PRODUCT)) return rc;
        }
    }
    return SIGNMUON_OK;
}

// Spectral normalisation (see signmuon_params.power_iters): the unscaled Gram
// matrix of the stored momentum, power_iters power steps on it and the
// scales {s, s^2}. A stays unscaled: the first product applies s^2 itself
// (NsBatch::id_scaled).
int run_spectral(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                 const Plan &pl, void *ws, hipStream_t st, Tracer &tr) {
    if (int rc = ns_pass(mats, n_mats, p, pl, ws, false, 0, 0, false, st, tr)) return rc;
    const bool bf16 = p->ns_dtype == SIGNMUON_BF16;
    for (int32_t c0 = 0; c0 < n_mats; c0 += sm::kMaxMatsPerLaunch) {
        const int32_t cn = n_mats - c0 < sm::kMaxMatsPerLaunch ? n_mats - c0 : sm::kMaxMatsPerLaunch;
        sm::PowBatch b{};
        b.nmat = cn;
        b.workers = p->workers;
        b.scales = ws_at<float2>(ws, pl.off_scales);
        int64_t blocks = 0;
        for (int32_t i = 0; i < cn; ++i) {
            const MatPlan &q = pl.m[c0 + i];
            sm::PowMat &d = b.mat[i];
            d.a = ws_at<char>(ws, pl.off_gram + q.gram_off);
            d.w = ws_at<float>(ws, pl.off_pw) + q.pw_off;
            d.part = ws_at<double>(ws, pl.off_pwp) + q.pwp_off;
            d.r = (int32_t)q.r;
            d.bpw = q.pw_bpw;
            d.unit_begin = q.unit_begin;
            b.starts.v[i] = (int32_t)blocks;
            blocks += (int64_t)p->workers * q.pw_bpw;
        }
        if (blocks > INT32_MAX) return SIGNMUON_ERANGE;
        b.total_blocks = (int32_t)blocks;
        // One workgroup per (matrix, worker) runs every step and the scale
        // when each Gram matrix suits it and there are enough units to fill
        // the device; otherwise one launch per step.
        bool fused = (int64_t)cn * p->workers >= device_cus() / 2;
        for (int32_t i = 0; i < cn; ++i)
            fused = fused && pl.m[c0 + i].r % 8 == 0 && pl.m[c0 + i].r <= sm::max_fused_pow_r(bf16);
        if (fused) {
            b.it = p->power_iters;
            sm::launch_power_fused(b, bf16, st);
            if (int rc = tr.after(SIGNMUON_K_POWER)) return rc;
            continue;
        }
        for (int it = 0; it < p->power_iters; ++it) {
            b.it = it;
            sm::launch_power_step(b, bf16, st);
            if (int rc = tr.after(SIGNMUON_K_POWER)) return rc;
        }
        b.it = p->power_iters - 1;
        sm::launch_power_finalize(b, st);
        if (int rc = tr.after(SIGNMUON_K_POWER)) return rc;
    }
    return SIGNMUON_OK;
}

// Newton-Schulz iterations of every (matrix, worker); with spectral
// normalisation the first Gram matrix comes from run_spectral.
int run_newton_schulz(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                      const Plan &pl, void *ws, bool step, hipStream_t st, Tracer &tr,
                      bool muon = false) {
    for (int j = 0; j < p->ns_iters; ++j) {
        if (j == 0 && pl.spectral) {
            if (int rc = run_spectral(mats, n_mats, p, pl, ws, st, tr)) return rc;
        } else {
            if (int rc = ns_pass(mats, n_mats, p, pl, ws, step, j, 0, j == 0, st, tr)) return rc;
        }
        if (int rc = ns_pass(mats, n_mats, p, pl, ws, step, j, 1, j == 0, st, tr, muon)) return rc;
    }
    return SIGNMUON_OK;
}

// Sign + pack from a stored value: the scaled momentum (k = 0) or a U that the
// last product could not pack itself.
int run_pack(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p, const Plan &pl,
             void *ws, bool step, hipStream_t st, Tracer &tr) {
    const bool k0 = p->ns_iters == 0;
    std::vector<int32_t> sel;
    for (int32_t i = 0; i < n_mats; ++i)
        if ((k0 && !pl.m[i].fused_k0) || (!k0 && step && !pl.m[i].fused_pack && !pl.m[i].fused_i8))
            sel.push_back(i);
    for (size_t c0 = 0; c0 < sel.size(); c0 += sm::kMaxMatsPerLaunch) {
        const size_t cn = sel.size() - c0 < (size_t)sm::kMaxMatsPerLaunch ? sel.size() - c0
                                                                          : (size_t)sm::kMaxMatsPerLaunch;
        sm::PackBatch b{};
        b.nmat = (int32_t)cn;
        b.workers = p->workers;
        b.u_bf16 = k0 ? p->mom_dtype == SIGNMUON_BF16 : 0;
        b.scales = k0 ? ws_at<float2>(ws, pl.off_scales) : nullptr;
        int64_t blocks = 0;
        for (size_t i = 0; i < cn; ++i) {
            const int32_t mi = sel[c0 + i];
            const MatPlan &q = pl.m[mi];
            const signmuon_matrix &s = mats[mi];
            sm::PackMat &d = b.mat[i];
            if (k0) {
                d.u = s.momentum;
                d.u_out = s.polar_out;
            } else {
                d.u = s.polar_out ? (const void *)s.polar_out : ws_at<const char>(ws, pl.off_u + q.u_off);
                d.u_out = nullptr;
            }
            d.packed = step && !pl.i8 ? s.packed : nullptr;
            d.i8 = step && pl.i8 ? s.signs_i8 : nullptr;
            d.n = q.n;
            d.unit_begin = q.unit_begin;
            const int64_t wpb = sm::pack_words_per_block(b.u_bf16 != 0);
            d.blocks_per_worker = (int32_t)((q.nw + wpb - 1) / wpb);
            d.block_begin = (int32_t)blocks;
            b.starts.v[i] = d.block_begin;
            blocks += (int64_t)p->workers * d.blocks_per_worker;
        }
        if (blocks > INT32_MAX) return SIGNMUON_ERANGE;
        b.total_blocks = (int32_t)blocks;
        sm::launch_sign_pack(b, st);
        if (int rc = tr.after(SIGNMUON_K_PACK)) return rc;
    }
    return SIGNMUON_OK;
}

// The vote from the int8 payload: one batched launch per kMaxMatsPerLaunch
// matrices (the standalone entry point is a batch of one).
int run_vote_int8(const int8_t *const *signs, float *const *weights, int8_t *const *votes,
                  const int64_t *ns, int32_t n_mats, int32_t workers, float eta, hipStream_t st,
                  Tracer &tr) {
    for (int32_t c0 = 0; c0 < n_mats; c0 += sm::kMaxMatsPerLaunch) {
        const int32_t cn = n_mats - c0 < sm::kMaxMatsPerLaunch ? n_mats - c0 : sm::kMaxMatsPerLaunch;
        sm::VoteI8Batch b{};
        b.nmat = cn;
        b.workers = workers;
        b.eta = eta;
        int64_t blocks = 0;
        for (int32_t i = 0; i < cn; ++i) {
            sm::VoteI8Mat &d = b.mat[i];
            d.signs = signs[c0 + i];
            d.w = weights[c0 + i];
            d.vote = votes[c0 + i];
            d.n = ns[c0 + i];
            d.vec = (d.n % 16) == 0;
            d.block_begin = (int32_t)blocks;
            b.starts.v[i] = d.block_begin;
            blocks += sm::vote_int8_blocks(d.n);
        }
        if (blocks > INT32_MAX) return SIGNMUON_ERANGE;
        b.total_blocks = (int32_t)blocks;
        sm::launch_vote_update_int8(b, st);
        if (int rc = tr.after(SIGNMUON_K_VOTE_I8)) return rc;
    }
    return SIGNMUON_OK;
}

int run_vote(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p, const Plan &pl,
             void *ws, hipStream_t st, Tracer &tr) {
    if (pl.i8) {
        std::vector<const int8_t *> sg(n_mats);
        std::vector<float *> wt(n_mats);
        std::vector<int8_t *> vt(n_mats);
        std::vector<int64_t> ns(n_mats);
        for (int32_t i = 0; i < n_mats; ++i) {
            sg[i] = mats[i].signs_i8;
            wt[i] = mats[i].weight;
            vt[i] = mats[i].vote_out;
            ns[i] = pl.m[i].n;
        }
        return run_vote_int8(sg.data(), wt.data(), vt.data(), ns.data(), n_mats, p->workers, p->eta,
                             st, tr);
    }
    const bool post = p->post_polar_iters > 0;
    uint32_t *nnz = ws_at<uint32_t>(ws, pl.off_nnz);
    if (post) {
        sm::launch_zero_u32(nnz, n_mats, st);
        if (int rc = tr.after(SIGNMUON_K_AUX)) return rc;
    }
    for (int32_t c0 = 0; c0 < n_mats; c0 += sm::kMaxMatsPerLaunch) {
        const int32_t cn = n_mats - c0 < sm::kMaxMatsPerLaunch ? n_mats - c0 : sm::kMaxMatsPerLaunch;
        sm::VoteBatch b{};
        b.nmat = cn;
        b.workers = p->workers;
        b.eta = p->eta;
        b.v_ns_bf16 = p->ns_dtype == SIGNMUON_BF16;
        int64_t blocks = 0;
        for (int32_t i = 0; i < cn; ++i) {
            const MatPlan &q = pl.m[c0 + i];
            const signmuon_matrix &s = mats[c0 + i];
            sm::VoteMat &d = b.mat[i];
            d.packed = s.packed;
            d.w = post ? nullptr : s.weight;
            d.vote = s.vote_out;
            d.v_ns = post ? ws_at<char>(ws, pl.off_vns + q.vns_off) : nullptr;
            d.nnz = post ? nnz + c0 + i : nullptr;
            d.n = q.n;
            d.block_begin = (int32_t)blocks;
            b.starts.v[i] = d.block_begin;
            blocks += (q.nw + sm::kVoteWordsPerBlock - 1) / sm::kVoteWordsPerBlock;
        }
        if (blocks > INT32_MAX) return SIGNMUON_ERANGE;
        b.total_blocks = (int32_t)blocks;
        sm::launch_vote_update(b, st);
        if (int rc = tr.after(SIGNMUON_K_VOTE)) return rc;
    }
    return SIGNMUON_OK;
}

// Optional local polar step on the vote (summary §2 "Algorithmic flow", step
// 5): Frobenius-scaled Newton-Schulz on S-bar, then W <- fmaf(-eta, Y, W).
int run_post_polar(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                   const Plan &pl, void *ws, hipStream_t st, Tracer &tr) {
    const int k = p->post_polar_iters;
    const bool bf16 = p->ns_dtype == SIGNMUON_BF16;
    float2 *scales = ws_at<float2>(ws, pl.off_scales);
    sm::launch_nnz_scales(ws_at<uint32_t>(ws, pl.off_nnz), n_mats, scales + pl.post_unit_base, st);
    if (int rc = tr.after(SIGNMUON_K_AUX)) return rc;
    for (int j = 0; j < k; ++j) {
        const bool last = j == k - 1;
        for (int pass = 0; pass < 2; ++pass) {
            for (int32_t c0 = 0; c0 < n_mats; c0 += sm::kMaxMatsPerLaunch) {
                const int32_t cn =
                    n_mats - c0 < sm::kMaxMatsPerLaunch ? n_mats - c0 : sm::kMaxMatsPerLaunch;
                sm::NsBatch b{};
                b.nmat = cn;
                b.workers = 1;
                b.use_scales = j == 0;
                b.scales = scales;
                b.eta = p->eta;
                int64_t tiles = 0;
                for (int32_t i = 0; i < cn; ++i) {
                    const MatPlan &q = pl.m[c0 + i];
                    sm::NsMat &d = b.mat[i];
                    d.R = (int32_t)q.R;
                    d.C = (int32_t)q.C;
                    d.unit_begin = pl.post_unit_base + c0 + i;
                    d.x = j == 0 ? ws_at<const char>(ws, pl.off_vns + q.vns_off)
                                 : ws_at<const char>(ws, pl.off_iter[(j - 1) & 1] + q.post_iter_off);
                    d.a = ws_at<char>(ws, pl.off_gram + q.post_gram_off);
                    d.out = last ? (void *)mats[c0 + i].weight
                                 : ws_at<char>(ws, pl.off_iter[j & 1] + q.post_iter_off);
                    d.packed = nullptr;
                    d.tiles_per_worker = pass == 0 ? sm::ns_gram_tiles(q.R, q.C) : sm::ns_product_tiles(q.R, q.C);
                    d.tile_begin = (int32_t)tiles;
                    b.starts.v[i] = d.tile_begin;
                    tiles += d.tiles_per_worker;
                }
                if (tiles > INT32_MAX) return SIGNMUON_ERANGE;
                b.tiles_per_worker_all = (int32_t)tiles;
                b.total_tiles = (int32_t)tiles;
                if (pass == 0)
                    sm::launch_ns_gram(b, bf16, st);
                else
                    sm::launch_ns_product(b, bf16, last ? sm::EPI_WUPD : sm::EPI_ITER, st);
                if (int rc = tr.after(pass == 0 ? SIGNMUON_K_GRAM : SIGNMUON_K_PRODUCT)) return rc;
            }
        }
    }
    return SIGNMUON_OK;
}

int check_workspace(const Plan &pl, void *ws, size_t ws_bytes) {
    if (pl.total == 0) return SIGNMUON_OK;
    if (!ws || ws_bytes < pl.total) return SIGNMUON_EWORKSPACE;
    if (!aligned16(ws)) return SIGNMUON_EALIGN;
    return SIGNMUON_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

int noalloc_scratch(void **out) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return SIGNMUON_ERANGE;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
                return hip_status(e);
            if (!p) return hip_status(hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SIGNMUON_OK;
}

}  // namespace

extern "C" {

size_t signmuon_packed_words(int64_t n) { return n <= 0 ? 0 : (size_t)((n + 63) / 64); }

int signmuon_abi_version(void) { return SIGNMUON_ABI_VERSION; }

const char *signmuon_strerror(int status) {
    switch (status) {
    case SIGNMUON_OK: return "ok";
    case SIGNMUON_EINVAL: return "invalid argument (null pointer, size or count out of range)";
    case SIGNMUON_EDTYPE: return "dtype not accepted (momentum and Newton-Schulz storage must match)";
    case SIGNMUON_EALIGN: return "device pointer not 16-byte aligned";
    case SIGNMUON_EWORKSPACE: return "workspace missing or too small";
    case SIGNMUON_EHIP: return g_hip_err[0] ? g_hip_err : "HIP error";
    case SIGNMUON_ERANGE: return "size beyond the kernels' limits";
    case SIGNMUON_ESCRATCH:
        return "the step needs more workspace than the static scratch of signmuon_step_noalloc holds "
               "(SIGNMUON_STATIC_SCRATCH_BYTES); call signmuon_step with a workspace instead";
    default: return "unknown status";
    }
}

size_t signmuon_workspace_bytes(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p) {
    Plan pl;
    if (make_plan(mats, n_mats, p, true, pl) != SIGNMUON_OK) return 0;
    return pl.total;
}

int signmuon_momentum_ns(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                         void *workspace, size_t workspace_bytes, signmuon_stream stream) {
    Plan pl;
    if (int rc = make_plan(mats, n_mats, p, false, pl)) return rc;
    if (int rc = check_step_pointers(mats, n_mats, false, false)) return rc;
    if (int rc = check_workspace(pl, workspace, workspace_bytes)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr;
    if (int rc = run_momentum(mats, n_mats, p, pl, workspace, st, tr)) return rc;
    if (p->ns_iters == 0) {
        if (pl.spectral)
            if (int rc = run_spectral(mats, n_mats, p, pl, workspace, st, tr)) return rc;
        return run_pack(mats, n_mats, p, pl, workspace, false, st, tr);
    }
    return run_newton_schulz(mats, n_mats, p, pl, workspace, false, st, tr);
}

int signmuon_step_traced(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                         void *workspace, size_t workspace_bytes, signmuon_stream stream,
                         signmuon_trace *trace) {
    Plan pl;
    if (int rc = make_plan(mats, n_mats, p, true, pl)) return rc;
    if (int rc = check_step_pointers(mats, n_mats, true, pl.i8)) return rc;
    if (int rc = check_workspace(pl, workspace, workspace_bytes)) return rc;
    if (trace && trace->capacity > 0 && !trace->events) return SIGNMUON_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr;
    tr.t = trace;
    tr.st = st;
    if (int rc = tr.begin()) return rc;
    if (int rc = run_momentum(mats, n_mats, p, pl, workspace, st, tr)) return rc;
    if (p->ns_iters > 0) {
        if (int rc = run_newton_schulz(mats, n_mats, p, pl, workspace, true, st, tr)) return rc;
    } else if (pl.spectral) {
        if (int rc = run_spectral(mats, n_mats, p, pl, workspace, st, tr)) return rc;
    }
    if (int rc = run_pack(mats, n_mats, p, pl, workspace, true, st, tr)) return rc;
    if (int rc = run_vote(mats, n_mats, p, pl, workspace, st, tr)) return rc;
    if (p->post_polar_iters > 0)
        if (int rc = run_post_polar(mats, n_mats, p, pl, workspace, st, tr)) return rc;
    return SIGNMUON_OK;
}

int signmuon_muon_step(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                       void *workspace, size_t workspace_bytes, signmuon_stream stream) {
    Plan pl;
    if (int rc = make_plan(mats, n_mats, p, false, pl)) return rc;
    if (p->workers != 1 || p->ns_iters < 1 || p->post_polar_iters != 0) return SIGNMUON_EINVAL;
    for (int32_t i = 0; i < n_mats; ++i) {
        const signmuon_matrix &s = mats[i];
        if (!s.grad || !s.momentum || !s.weight) return SIGNMUON_EINVAL;
        const void *ptrs[4] = {s.grad, s.momentum, s.weight, s.polar_out};
        for (const void *q : ptrs)
            if (q && !aligned16(q)) return SIGNMUON_EALIGN;
    }
    if (int rc = check_workspace(pl, workspace, workspace_bytes)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Tracer tr;
    if (int rc = run_momentum(mats, n_mats, p, pl, workspace, st, tr)) return rc;
    return run_newton_schulz(mats, n_mats, p, pl, workspace, false, st, tr, true);
}

int signmuon_step(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                  void *workspace, size_t workspace_bytes, signmuon_stream stream) {
    return signmuon_step_traced(mats, n_mats, p, workspace, workspace_bytes, stream, nullptr);
}

int signmuon_step_noalloc(const signmuon_matrix *mats, int32_t n_mats, const signmuon_params *p,
                          signmuon_stream stream) {
    // The sizes are checked before any HIP call, so an oversized step is
    // refused with nothing enqueued and no device touched.
    Plan pl;
    if (int rc = make_plan(mats, n_mats, p, true, pl)) return rc;
    if (int rc = check_step_pointers(mats, n_mats, true, pl.i8)) return rc;
    if (pl.total > (size_t)SIGNMUON_STATIC_SCRATCH_BYTES) return SIGNMUON_ESCRATCH;
    void *ws = nullptr;
    if (int rc = noalloc_scratch(&ws)) return rc;
    return signmuon_step_traced(mats, n_mats, p, ws, SIGNMUON_STATIC_SCRATCH_BYTES, stream, nullptr);
}

int signmuon_sign_pack(const void *u, signmuon_dtype u_dtype, int64_t n, int32_t workers,
                       uint64_t *packed, signmuon_stream stream) {
    if (!u || !packed || n < 1 || workers < 1) return SIGNMUON_EINVAL;
    if (!dtype_ok(u_dtype)) return SIGNMUON_EDTYPE;
    if (!aligned16(u) || !aligned16(packed)) return SIGNMUON_EALIGN;
    if (n > kMaxN) return SIGNMUON_ERANGE;
    const int64_t nw = (n + 63) / 64;
    const int64_t wpb = sm::pack_words_per_block(u_dtype == SIGNMUON_BF16);
    const int64_t bpw = (nw + wpb - 1) / wpb;
    if (bpw * workers > INT32_MAX) return SIGNMUON_ERANGE;
    sm::PackBatch b{};
    b.nmat = 1;
    b.workers = workers;
    b.u_bf16 = u_dtype == SIGNMUON_BF16;
    b.scales = nullptr;
    b.mat[0].u = u;
    b.mat[0].packed = packed;
    b.mat[0].u_out = nullptr;
    b.mat[0].n = n;
    b.mat[0].block_begin = 0;
    b.starts.v[0] = 0;
    b.mat[0].blocks_per_worker = (int32_t)bpw;
    b.mat[0].unit_begin = 0;
    b.total_blocks = (int32_t)(bpw * workers);
    sm::launch_sign_pack(b, static_cast<hipStream_t>(stream));
    return last_launch();
}

int signmuon_vote_update(const uint64_t *packed, int32_t workers, int64_t n, float *weight, float eta,
                         int8_t *vote_out, signmuon_stream stream) {
    if (!packed || n < 1 || workers < 1 || (!weight && !vote_out)) return SIGNMUON_EINVAL;
    if (!std::isfinite(eta)) return SIGNMUON_EINVAL;
    if (workers > kMaxWorkers || n > kMaxN) return SIGNMUON_ERANGE;
    if (!aligned16(packed) || (weight && !aligned16(weight)) || (vote_out && !aligned16(vote_out)))
        return SIGNMUON_EALIGN;
    const int64_t nw = (n + 63) / 64;
    sm::VoteBatch b{};
    b.nmat = 1;
    b.workers = workers;
    b.eta = eta;
    b.mat[0].packed = packed;
    b.mat[0].w = weight;
    b.mat[0].vote = vote_out;
    b.mat[0].v_ns = nullptr;
    b.mat[0].nnz = nullptr;
    b.mat[0].n = n;
    b.mat[0].block_begin = 0;
    b.starts.v[0] = 0;
    b.total_blocks = (int32_t)((nw + sm::kVoteWordsPerBlock - 1) / sm::kVoteWordsPerBlock);
    sm::launch_vote_update(b, static_cast<hipStream_t>(stream));
    return last_launch();
}

int signmuon_sign_int8(const void *u, signmuon_dtype u_dtype, int64_t n, int32_t workers, int8_t *signs,
                       signmuon_stream stream) {
    if (!u || !signs || n < 1 || workers < 1) return SIGNMUON_EINVAL;
    if (!dtype_ok(u_dtype)) return SIGNMUON_EDTYPE;
    if (!aligned16(u) || !aligned16(signs)) return SIGNMUON_EALIGN;
    if (n > kMaxN || workers > kMaxWorkers) return SIGNMUON_ERANGE;
    const int64_t total = n * workers;
    if (sm::sign_int8_blocks(total) > INT32_MAX) return SIGNMUON_ERANGE;
    sm::launch_sign_int8(u, u_dtype == SIGNMUON_BF16, total, signs, static_cast<hipStream_t>(stream));
    return last_launch();
}

int signmuon_vote_update_int8(const int8_t *signs, int32_t workers, int64_t n, float *weight, float eta,
                              int8_t *vote_out, signmuon_stream stream) {
    if (!signs || n < 1 || workers < 1 || (!weight && !vote_out)) return SIGNMUON_EINVAL;
    if (!std::isfinite(eta)) return SIGNMUON_EINVAL;
    if (workers > kMaxWorkers || n > kMaxN) return SIGNMUON_ERANGE;
    if (!aligned16(signs) || (weight && !aligned16(weight)) || (vote_out && !aligned16(vote_out)))
        return SIGNMUON_EALIGN;
    Tracer tr;
    if (int rc = run_vote_int8(&signs, &weight, &vote_out, &n, 1, workers, eta,
                               static_cast<hipStream_t>(stream), tr))
        return rc;
    return last_launch();
}

}  // extern "C"
