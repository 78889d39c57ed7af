// q4k_api.hip -- the C ABI of libq4k.so (declared in include/q4k.h):
// argument validation, variant selection and launch.
//
// Every argument is checked before the first HIP call, so a bad call returns
// its status without touching the device (realizar 0.8.5,
// q4k_gemv_cached.rs: `q4k_gemv_indexed_async` validates the weight pointer
// because a launch with a null pointer poisons the context).  Size arithmetic
// is overflow-checked (turbospark-runtime 0.1.0, real_forward_dispatch.rs:
// `validate_block_quant_embedding`).  Unsupported batch widths are refused by
// name, never looped (real_forward_dispatch.rs: doc of `encode_gemm_any`).

#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "../../include/q4k.h"
#include "q4k_kernels.h"

namespace {

using q4k::GemvPlan;

constexpr int64_t kInt32Max = 2147483647;
// Single-stage x budget: 48 KiB, the pages' 12288-float shared-memory limit
// (realizar 0.8.5, q4k_gemv_cached.rs: MAX_TILED_K in `q4k_gemv_cached`),
// i.e. three 4096-element spans of one vector.
constexpr int64_t kSingleStageBytes = 48 * 1024;
constexpr int64_t kSpanBytes = (int64_t)q4k::kSpan * 4;          // 16 KiB per vector
constexpr int64_t kSpanSumBytes = 64 * 8;                        // per vector
constexpr int kMaxDevices = 64;

std::atomic<int> g_lds_max[kMaxDevices];  // 0 = not queried yet

inline bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline int hip_status(hipError_t e)
{
    return e == hipSuccess ? Q4K_OK : Q4K_ERR_HIP + (int)e;
}

// Shape rules shared by every entry point: 1 <= n <= 2^31-1,
// 256 <= k <= 2^31-1, k % 256 == 0.
inline int check_nk(int64_t n, int64_t k)
{
    if (n < 1 || n > kInt32Max || k < q4k::kQK || k > kInt32Max || k % q4k::kQK != 0) {
        return Q4K_ERR_SHAPE;
    }
    return Q4K_OK;
}

int device_lds_max(size_t* out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        return hip_status(e);
    }
    if (dev < 0 || dev >= kMaxDevices) {
        return Q4K_ERR_UNSUPPORTED;
    }
    int v = g_lds_max[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) {
            return hip_status(e);
        }
        g_lds_max[dev].store(v, std::memory_order_relaxed);
    }
    *out = (size_t)v;
    return Q4K_OK;
}

// Plan of the line-streamed kernels (weights 128-byte aligned; m <= 8, kernels
// 5 and 6 m <= 16):
// kernel 3 (m = 1, integer dot products on the vector ALU, any k), kernel 4
// (one MFMA group per vector; k a multiple of 2048), kernel 5 (one MFMA per
// sub-block and quad of vectors) and kernel 6 (kernel 5 with x converted per
// column by each wave).  A task is a 16-row tile times a group of slabs of
// eight superblock columns (the last slab of a row may be partial); x
// (every vector) is staged whole, except for kernel 6.
int make_plan_lines(int64_t n, int64_t k, int64_t m, const q4k_launch* o, size_t lds_max,
                    GemvPlan* p, int kernel)
{
    const int S = (int)(k / q4k::kQK);
    if (S % 8 != 0 && kernel == 4) {
        return Q4K_ERR_UNSUPPORTED;    // rows of whole slabs (kernels 3, 5, 6: any rows)
    }
    if (m > q4k::kMaxM && kernel < 5) {
        return Q4K_ERR_UNSUPPORTED;    // 9-16 vectors: the sub-block kernels only
    }
    const int nslabs = (S + 7) / 8;
    const int nw = (o && o->waves_per_block) ? o->waves_per_block : 8;
    if (nw != 4 && nw != 8 && nw != 16) {
        return Q4K_ERR_UNSUPPORTED;
    }
    if (o && (o->cols_per_task < 0 || o->rows_per_block < 0 || o->variant != 0 ||
              o->spans_per_chunk != 0 || o->rows_per_wave != 0 || o->x_in_registers != 0 ||
              o->rows_per_task != 0 ||
              (o->ring_depth != 0 && o->ring_depth != 3 && o->ring_depth != 9))) {
        return Q4K_ERR_UNSUPPORTED;
    }
    const int ring = (o && o->ring_depth) ? o->ring_depth : 3;
    if (nw == 16 && ring == 9) {
        return Q4K_ERR_UNSUPPORTED;    // 1024-lane workgroups cap a lane at 128 VGPRs
    }
    if ((m > 1 || kernel >= 5) && (nw != 8 || ring != 3)) {
        return Q4K_ERR_UNSUPPORTED;    // several vectors: eight waves, three lines in flight
    }
    if (kernel == 3 && (m != 1 || S * 16 > 4 * 64 * nw || (S % 8 != 0 && ring != 3))) {
        return Q4K_ERR_UNSUPPORTED;    // one vector; x in at most four groups per lane;
                                       // rows of any length: three lines in flight
    }
    const int64_t ntiles = (n + 15) / 16;
    int64_t spt = 1;
    if (o && o->cols_per_task) {
        if (o->cols_per_task % 8 != 0 || nslabs % (o->cols_per_task / 8) != 0) {
            return Q4K_ERR_UNSUPPORTED;
        }
        spt = o->cols_per_task / 8;
    }
    int64_t rpb;
    if (o && o->rows_per_block > 0) {
        rpb = o->rows_per_block;
    } else {
        // at most about one workgroup per CU of a 256-CU part: each stages
        // all of x, which costs as much as decoding a few tiles
        rpb = 16 * ((ntiles + 255) / 256);
    }
    const size_t lds_x = kernel == 6   ? q4k::jit_lds_bytes(S, (int)m)
                         : kernel == 5 ? q4k::sub_lds_bytes(S, (int)m)
                         : kernel == 3 ? q4k::dot4_lds_bytes(S, nw)
                                       : q4k::lines_lds_bytes(S, (int)m, nw);
    if (!(o && o->cols_per_task)) {
        // whole rows per task when the workgroup has a tile for every wave
        // (no row sums to combine), else one slab per task, so that every
        // wave streams; whole rows too when the per-slab row sums do not fit
        // the LDS (choices measured on MI355X: with fewer tiles than waves,
        // whole rows leave waves idle, 0.3-0.8 us on 16384-28672-row shapes)
        const bool fits = lds_x + (size_t)nslabs * rpb * 4 * m <= lds_max;
        spt = (rpb / 16 >= nw || !fits) ? nslabs : 1;
    }
    const int64_t ncg = nslabs / spt;
    if (rpb > kInt32Max / (ncg * m)) {
        return Q4K_ERR_SHAPE;
    }
    const int64_t grid = (n + rpb - 1) / rpb;
    const size_t lds = lds_x + (ncg > 1 ? (size_t)ncg * rpb * 4 * m : 0);

    p->n = (int)n;
    p->k = (int)k;
    p->S = S;
    p->m = (int)m;
    p->nspans = (S + q4k::kSpanSB - 1) / q4k::kSpanSB;
    p->spans_per_chunk = 0;
    p->nchunks = 1;
    p->rows_per_block = (int)rpb;
    p->rows_per_wave = 0;
    p->waves_per_block = nw;
    p->x_in_registers = 0;
    p->grid = (int)grid;
    p->lds_bytes = lds;
    p->kernel = kernel;
    p->ring_depth = ring;
    p->rows_per_task = 0;
    p->cols_per_task = (int)(spt * 8);
    return Q4K_OK;
}

// Resolve launch options into a plan.  Pure host arithmetic, no HIP calls.
// Plans needing more LDS than lds_max are returned as they are; the caller
// refuses them.
// The automatic kernel (choices measured on MI355X).  The line-streamed
// kernels apply when the weights are 128-byte aligned and their LDS (staged
// x, the line rings) fits; kernel 4 also needs k a multiple of 2048.  m > 1:
// the sub-block kernel (5, m >= 3) or the per-vector line-streamed kernel
// (4, m = 2), the other one if only it fits, then the sub-block kernel with
// per-wave x (6), else the x-stager kernel (1, m <= 8; 9-16 vectors are
// refused there).
// m = 1: the line-streamed vector-ALU kernel (3) where it applies and the
// weights take at least 16 MiB, else the streaming kernel, whose shorter
// start wins on smaller matrices; m = 1 takes the matrix cores only when
// asked to.
// Options other than `kernel` keep the earlier families: streaming for
// m = 1, x-stager otherwise.
bool any_option(const q4k_launch* o)
{
    return o && (o->variant || o->spans_per_chunk || o->rows_per_block || o->rows_per_wave ||
                 o->waves_per_block || o->x_in_registers || o->ring_depth || o->rows_per_task ||
                 o->cols_per_task);
}

int auto_kernel(int64_t n, int64_t k, int64_t m, const q4k_launch* o, bool w_aligned128,
                size_t lds_max)
{
    GemvPlan lp;
    if (m != 1) {
        // several vectors: a line-streamed kernel whenever one applies; the
        // sub-block kernel from three vectors on; per-wave x conversion when
        // no whole x stage fits the LDS
        if (!any_option(o) && w_aligned128) {
            const int first = m >= 3 ? 5 : 4;
            for (int kern : {first, 9 - first, 6}) {
                if (make_plan_lines(n, k, m, nullptr, lds_max, &lp, kern) == Q4K_OK &&
                    lp.lds_bytes <= lds_max) {
                    return kern;
                }
            }
        }
        return 1;
    }
    if (any_option(o)) {
        return 2;
    }
    const int64_t bytes = n * (k / q4k::kQK) * q4k::kBlockBytes;
    if (w_aligned128 && bytes >= ((int64_t)16 << 20) &&
        make_plan_lines(n, k, 1, nullptr, lds_max, &lp, 3) == Q4K_OK && lp.lds_bytes <= lds_max) {
        return 3;
    }
    return 2;
}

int make_plan(int64_t n, int64_t k, int64_t m, const q4k_launch* o, size_t lds_max, GemvPlan* p,
              bool w_aligned128 = true)
{
    const int S = (int)(k / q4k::kQK);
    const int nspans = (S + q4k::kSpanSB - 1) / q4k::kSpanSB;
    const int variant = o ? o->variant : 0;
    if (variant < 0 || variant > 2) {
        return Q4K_ERR_UNSUPPORTED;
    }
    const bool fits_single = m * nspans * kSpanBytes <= kSingleStageBytes;
    const int auto_chunk = (int)(kSingleStageBytes / (m * kSpanBytes)) > 0
                               ? (int)(kSingleStageBytes / (m * kSpanBytes)) : 1;
    int spc;
    if (variant == 1) {
        spc = nspans;
    } else if (variant == 2) {
        spc = (o->spans_per_chunk > 0) ? o->spans_per_chunk : auto_chunk;
    } else {
        spc = fits_single ? nspans : auto_chunk;
    }
    if (spc > nspans) {
        spc = nspans;
    }
    const int nchunks = (nspans + spc - 1) / spc;

    const int kernel = (o && o->kernel) ? o->kernel : auto_kernel(n, k, m, o, w_aligned128, lds_max);
    if (kernel < 1 || kernel > 6 || ((kernel == 2 || kernel == 3) && m != 1) ||
        (kernel == 1 && m > q4k::kMaxM)) {
        return Q4K_ERR_UNSUPPORTED;
    }
    if (kernel >= 3) {
        return make_plan_lines(n, k, m, o, lds_max, p, kernel);
    }
    if (o && o->cols_per_task) {
        return Q4K_ERR_UNSUPPORTED;   // line-streamed kernels only
    }
    int nw = (o && o->waves_per_block) ? o->waves_per_block
                                       : (kernel == 2 ? (nspans > 8 ? 16 : 8) : 8);
    if (nw != 4 && nw != 8 && !(nw == 16 && kernel == 2)) {
        return Q4K_ERR_UNSUPPORTED;
    }
    // streaming kernel: about 2048 wave tasks (8 per CU of a 256-CU part),
    // measured best on MI355X for the 4096- to 32000-row shapes; then, within
    // a factor of two of that, the rows per task whose workgroups fill the
    // 256 CUs in the fewest rounds for the least work per workgroup (342
    // workgroups of 12 rows take two rounds where 256 of 16 take one:
    // 4096 x 11008 14.7 -> 11.2 us)
    int64_t auto_rpt = ((int64_t)nspans * n + 2047) / 2048;
    auto_rpt = auto_rpt < 1 ? 1 : auto_rpt > 64 ? 64 : auto_rpt;
    if (kernel == 2 && !(o && (o->rows_per_task || o->rows_per_block))) {
        const int64_t groups = nw > nspans ? nw / nspans : 1;
        // from the largest down, so ties keep the fewer workgroups
        int64_t best = auto_rpt, best_cost = 0;
        for (int64_t r = 2 * auto_rpt < 64 ? 2 * auto_rpt : 64; r >= (auto_rpt + 1) / 2; --r) {
            const int64_t rpb_r = groups * r;
            const int64_t cost = ((n + rpb_r - 1) / rpb_r + 255) / 256 * rpb_r;
            if (best_cost == 0 || cost < best_cost) {
                best = r;
                best_cost = cost;
            }
        }
        auto_rpt = best;
    }
    const int64_t rows_per_task = (o && o->rows_per_task) ? o->rows_per_task : auto_rpt;
    const int ring_cap = nw == 16 ? 2 : 3;
    const int ring_depth = (o && o->ring_depth) ? o->ring_depth
                                                : (rows_per_task >= 8 ? ring_cap : 1);
    // 16-wave workgroups cap a lane at 128 VGPRs: at most 2 rows in flight there
    if (kernel == 2 && (ring_depth < 1 || ring_depth > 4 || rows_per_task < 1 ||
                        rows_per_task > kInt32Max || (nw == 16 && ring_depth > 2))) {
        return Q4K_ERR_UNSUPPORTED;
    }
    int R = (o && o->rows_per_wave) ? o->rows_per_wave : 2;
    if (!(R == 1 || R == 2 || (R == 4 && m == 1))) {
        return Q4K_ERR_UNSUPPORTED;
    }
    const int xo = o ? o->x_in_registers : 0;
    if (xo < 0 || xo > 2) {
        return Q4K_ERR_UNSUPPORTED;
    }
    int xreg = (m == 1 && nspans == 1) ? 1 : 0;
    if (xo == 1) {
        if (!xreg) {
            return Q4K_ERR_UNSUPPORTED;
        }
    } else if (xo == 2) {
        xreg = 0;
    }

    int64_t rpb;
    if (o && o->rows_per_block > 0) {
        rpb = o->rows_per_block;
    } else if (kernel == 2) {
        // as many row groups as give every wave one task
        const int64_t groups = nw > nspans ? nw / nspans : 1;
        rpb = groups * rows_per_task;
    } else {
        // about two workgroups per CU of a 256-CU part (one for several
        // vectors, whose x stage fills most of the LDS), whole row groups
        const int64_t unit = (int64_t)R * nw;
        rpb = m == 1 ? (n + 511) / 512 : (n + 255) / 256;
        rpb = ((rpb + unit - 1) / unit) * unit;
        if (rpb < unit) {
            rpb = unit;
        }
    }
    if (rpb > kInt32Max) {
        rpb = kInt32Max;
    }
    const size_t lds_x = (size_t)m * spc * (kSpanBytes + kSpanSumBytes);
    const size_t lds_row = kernel == 2 ? 0 : nchunks > 1 ? (size_t)m * 64 * 4 : 0;   // parked lane partials
    if (lds_row && !(o && o->rows_per_block > 0) && lds_x + (size_t)rpb * lds_row > lds_max) {
        // automatic row blocks shrink to whole row groups that fit the LDS;
        // an automatic row count per wave, then wave count, shrinks first
        // when not even one group fits
        const int64_t fit = lds_x < lds_max ? (int64_t)((lds_max - lds_x) / lds_row) : 0;
        if (!(o && o->rows_per_wave) && fit < (int64_t)R * nw) {
            R = 1;
        }
        if (!(o && o->waves_per_block) && fit < (int64_t)R * nw) {
            nw = 4;
        }
        const int64_t unit = (int64_t)R * nw;
        if (fit >= unit) {
            rpb = (fit / unit) * unit;
        }
    }
    const int64_t grid = (n + rpb - 1) / rpb;
    if (grid > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    size_t lds;
    if (kernel == 2) {
        // x chunk (no LDS sums: each wave sums its own x) + per-span row sums
        lds = (size_t)spc * kSpanBytes + (nspans > 1 ? (size_t)nspans * rpb * 4 : 0);
    } else {
        // partial sums are parked per row group, so round the rows up to whole groups
        lds = lds_x + (size_t)((rpb + R - 1) / R) * R * lds_row;
    }

    p->n = (int)n;
    p->k = (int)k;
    p->S = S;
    p->m = (int)m;
    p->nspans = nspans;
    p->spans_per_chunk = spc;
    p->nchunks = nchunks;
    p->rows_per_block = (int)rpb;
    p->rows_per_wave = R;
    p->waves_per_block = nw;
    p->x_in_registers = xreg;
    p->grid = (int)grid;
    p->lds_bytes = lds;
    p->kernel = kernel;
    p->ring_depth = ring_depth;
    p->rows_per_task = (int)rows_per_task;
    p->cols_per_task = 0;
    return Q4K_OK;
}

// 9-16 vectors, automatic plan: one pass of the sub-block kernels over the
// weights where their whole x stage fits or where eight vectors would take
// kernel 6 anyway; else two launches (vectors 0-7, then the rest).  Measured
// on MI355X, two launches of eight against one pass of sixteen: 4096 x 14336
// 2 x 21.0 against 34.0 us; 14336 x 4096 28.7 against 33.8 and 32000 x 4096
// 43.9 against 61.1 us (with four vector quads kernel 6 holds only one x
// column in registers ahead of its step, where kernel 5 of eight vectors
// stages x whole).  Two launches also serve weights that are not 128-byte
// aligned and rows whose sixteen-vector plan does not fit the LDS.
bool split_wide(int64_t n, int64_t k, int64_t m, const q4k_launch* o, bool w128, size_t lds_max)
{
    if (m <= q4k::kMaxM || (o && (o->kernel || any_option(o)))) {
        return false;
    }
    GemvPlan pw, p8;
    if (make_plan(n, k, m, nullptr, lds_max, &pw, w128) != Q4K_OK || pw.kernel < 5 ||
        pw.lds_bytes > lds_max) {
        return true;
    }
    if (pw.kernel == 5) {
        return false;
    }
    return make_plan(n, k, q4k::kMaxM, nullptr, lds_max, &p8, w128) != Q4K_OK || p8.kernel != 6;
}

// The plan gemv_checked would launch, for a given LDS budget; shape and
// option checks in the same order.  *split (may be NULL: then never): the
// automatic plan of 9-16 vectors is two launches, `plan` the first (vectors
// 0-7), plan_checked(m - 8) the second.
int plan_checked(int64_t n, int64_t k, int64_t m, const q4k_launch* opts, bool w128,
                 size_t lds_max, GemvPlan* plan, bool* split = nullptr)
{
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (m < 1) {
        return Q4K_ERR_SHAPE;
    }
    if (m > q4k::kMaxMWide) {
        return Q4K_ERR_UNSUPPORTED;
    }
    if (split) {
        *split = false;
        if (m > q4k::kMaxM && !(opts && (opts->kernel || any_option(opts)))) {
            if (lds_max == 0) {
                rc = device_lds_max(&lds_max);
                if (rc != Q4K_OK) {
                    return rc;
                }
            }
            if (split_wide(n, k, m, opts, w128, lds_max)) {
                *split = true;
                return plan_checked(n, k, q4k::kMaxM, opts, w128, lds_max, plan);
            }
        }
    }
    // options are validated before the first HIP call (unbounded LDS), then
    // planned for the LDS size
    rc = make_plan(n, k, m, opts, SIZE_MAX, plan, w128);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (lds_max == 0) {
        rc = device_lds_max(&lds_max);
        if (rc != Q4K_OK) {
            return rc;
        }
    }
    rc = make_plan(n, k, m, opts, lds_max, plan, w128);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (plan->lds_bytes > lds_max) {
        return Q4K_ERR_UNSUPPORTED;
    }
    if (plan->kernel >= 3 && !w128) {
        return Q4K_ERR_UNSUPPORTED;    // whole-line reads need 128-byte aligned rows
    }
    return Q4K_OK;
}

int gemv_checked(const void* w, const float* x, float* y, int64_t n, int64_t k, int64_t m,
                 const q4k_launch* opts, void* stream)
{
    if (!w || !x || !y) {
        return Q4K_ERR_NULL;
    }
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (m < 1) {
        return Q4K_ERR_SHAPE;
    }
    if (m > q4k::kMaxMWide) {
        return Q4K_ERR_UNSUPPORTED;
    }
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) {
        return Q4K_ERR_ALIGN;
    }
    const bool w128 = (reinterpret_cast<uintptr_t>(w) & 127u) == 0;
    GemvPlan plan;
    bool split = false;
    rc = plan_checked(n, k, m, opts, w128, 0, &plan, &split);
    if (rc != Q4K_OK) {
        return rc;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (split) {
        // both launches planned before the first goes out
        GemvPlan rest;
        rc = plan_checked(n, k, m - q4k::kMaxM, opts, w128, 0, &rest);
        if (rc != Q4K_OK) {
            return rc;
        }
        rc = hip_status(q4k::launch_gemv(plan, w, x, y, s));
        if (rc != Q4K_OK) {
            return rc;
        }
        return hip_status(q4k::launch_gemv(rest, w, x + (size_t)q4k::kMaxM * (size_t)k,
                                           y + (size_t)q4k::kMaxM * (size_t)n, s));
    }
    return hip_status(q4k::launch_gemv(plan, w, x, y, s));
}

}  // namespace

extern "C" {

size_t q4k_row_bytes(int64_t k)
{
    if (k < q4k::kQK || k % q4k::kQK != 0) {
        return 0;
    }
    return (size_t)(k / q4k::kQK) * q4k::kBlockBytes;
}

int q4k_load(void* w_dev, const void* src_host, size_t src_bytes, int64_t n, int64_t k,
             void* stream)
{
    if (!w_dev || !src_host) {
        return Q4K_ERR_NULL;
    }
    const int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    const size_t row = q4k_row_bytes(k);
    if ((size_t)n > SIZE_MAX / row || (size_t)n * row != src_bytes) {
        return Q4K_ERR_SIZE;
    }
    if (!aligned16(w_dev)) {
        return Q4K_ERR_ALIGN;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(w_dev, src_host, src_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) {
        e = hipStreamSynchronize(s);
    }
    return hip_status(e);
}

int q4k_gemv(const void* w, const float* x, float* y, int64_t n, int64_t k, int64_t m,
             void* stream)
{
    return gemv_checked(w, x, y, n, k, m, nullptr, stream);
}

int q4k_gemv_ex(const void* w, const float* x, float* y, int64_t n, int64_t k, int64_t m,
                const q4k_launch* opts, void* stream)
{
    return gemv_checked(w, x, y, n, k, m, opts, stream);
}

int q4k_plan(int64_t n, int64_t k, int64_t m, const q4k_launch* opts, int w_aligned128,
             size_t lds_max, q4k_plan_info* out)
{
    if (!out) {
        return Q4K_ERR_NULL;
    }
    GemvPlan plan, rest;
    bool split = false;
    int rc = plan_checked(n, k, m, opts, w_aligned128 != 0, lds_max, &plan, &split);
    if (rc == Q4K_OK && split) {
        rc = plan_checked(n, k, m - q4k::kMaxM, opts, w_aligned128 != 0, lds_max, &rest);
    }
    if (rc != Q4K_OK) {
        return rc;
    }
    out->launches = split ? 2 : 1;
    out->kernel = plan.kernel;
    out->grid = plan.grid;
    out->threads = plan.waves_per_block * 64;
    out->lds_bytes = (int32_t)plan.lds_bytes;
    out->rows_per_block = plan.rows_per_block;
    out->cols_per_task = plan.kernel >= 3 ? plan.cols_per_task : 0;
    out->ring_depth = plan.ring_depth;
    out->spans_per_chunk = plan.kernel <= 2 ? plan.spans_per_chunk : 0;
    return Q4K_OK;
}

int q4k_dequantize(const void* w, float* out, int64_t n, int64_t k, void* stream)
{
    if (!w || !out) {
        return Q4K_ERR_NULL;
    }
    const int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (!aligned16(w) || !aligned16(out)) {
        return Q4K_ERR_ALIGN;
    }
    const int64_t nsb = n * (k / q4k::kQK);
    if ((nsb * 32 + 255) / 256 > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    return hip_status(q4k::launch_dequant(w, out, nsb, static_cast<hipStream_t>(stream)));
}

const char* q4k_status_string(int rc)
{
    switch (rc) {
    case Q4K_OK: return "ok";
    case Q4K_ERR_NULL: return "a required pointer is NULL";
    case Q4K_ERR_SHAPE: return "bad shape: need 1 <= n, 256 <= k, k % 256 == 0, 1 <= m, n and k below 2^31";
    case Q4K_ERR_SIZE: return "byte count does not match n*(k/256)*144";
    case Q4K_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case Q4K_ERR_UNSUPPORTED:
        return "unsupported: m > 16, or launch options that do not fit the shape, m or the "
               "device";
    default: break;
    }
    if (rc >= Q4K_ERR_HIP) {
        return "HIP runtime error (status - 1000 is the hipError_t)";
    }
    return "unknown status";
}

int q4k_read_calibrate_blocks(void)
{
    return q4k::kReadBlocks;
}

int q4k_read_calibrate(const void* buf, size_t bytes, float* out, void* stream)
{
    if (!buf || !out) {
        return Q4K_ERR_NULL;
    }
    if (bytes == 0 || bytes % 16 != 0) {
        return Q4K_ERR_SIZE;
    }
    if (!aligned16(buf)) {
        return Q4K_ERR_ALIGN;
    }
    return hip_status(q4k::launch_read(buf, bytes / 16, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
