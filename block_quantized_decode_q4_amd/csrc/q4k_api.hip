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
// 5 and 7 m <= 16, kernel 6 m <= 32):
// kernel 3 (m = 1, integer dot products on the vector ALU, any k), kernel 4
// (one MFMA group per vector; k a multiple of 2048), kernel 5 (one MFMA per
// sub-block and quad of vectors), kernel 6 (kernel 5 with x converted per
// column by each wave) and kernel 7 (kernel 5 with x converted by the
// workgroup one column ahead into a two-column window of every slab; at most
// one task of one slab per wave).  A task is a 16-row tile times a group of
// slabs of eight superblock columns (the last slab of a row may be partial);
// x (every vector) is staged whole, except for kernels 6 and 7.
int make_plan_lines(int64_t n, int64_t k, int64_t m, const q4k_launch* o, size_t lds_max,
                    GemvPlan* p, int kernel)
{
    const int S = (int)(k / q4k::kQK);
    if (S % 8 != 0 && (kernel == 4 || kernel == 7)) {
        return Q4K_ERR_UNSUPPORTED;    // rows of whole slabs (kernels 3, 5, 6: any rows)
    }
    if (m > q4k::kMaxM && kernel < 5) {
        return Q4K_ERR_UNSUPPORTED;    // 9-32 vectors: the sub-block kernels only
    }
    if (m > q4k::kMaxMStaged && kernel != 6) {
        return Q4K_ERR_UNSUPPORTED;    // 17-32 vectors: eight quads, x per wave (kernel 6)
    }
    if (kernel == 4 && m > 2) {
        return Q4K_ERR_UNSUPPORTED;    // one MFMA group per vector: one or two vectors
    }
    const int nslabs = (S + 7) / 8;
    // kernel 6 with more than eight vectors: four waves (see jit_waves)
    const int nw_multi = kernel == 6 ? q4k::jit_waves((int)m) : 8;
    const int nw = (o && o->waves_per_block) ? o->waves_per_block : (m > 1 || kernel >= 5 ? nw_multi : 8);
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
    if ((m > 1 || kernel >= 5) && (nw != nw_multi || ring != 3)) {
        return Q4K_ERR_UNSUPPORTED;    // several vectors: eight waves (kernel 6 with more
                                       // than eight: four), three lines in flight
    }
    if (nw == 16) {
        return Q4K_ERR_UNSUPPORTED;    // 1024-lane workgroups cap a lane at 128 VGPRs,
                                       // below what the exact x terms need
    }
    if ((kernel == 3 || kernel == 8) &&
        (m != 1 || S * 16 > 4 * 64 * nw || (S % 8 != 0 && ring != 3))) {
        return Q4K_ERR_UNSUPPORTED;    // one vector; x in at most four groups per lane;
                                       // rows of any length: three lines in flight
    }
    // kernel 7: at most one window pair (slab, vector quad) per wave; one
    // slab per task and a task for at most every wave
    const int quads = m > 8 ? 4 : m > 4 ? 2 : 1;
    if (kernel == 7 && (nslabs * quads > nw || nslabs > nw ||
                        (o && o->cols_per_task && o->cols_per_task != 8))) {
        return Q4K_ERR_UNSUPPORTED;
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
        if (kernel == 7 && (rpb + 15) / 16 * nslabs > nw) {
            return Q4K_ERR_UNSUPPORTED;
        }
    } else if (kernel == 7) {
        rpb = 16 * (nw / nslabs);            // a task for every wave
    } else if (kernel == 6 && m > q4k::kMaxMStaged) {
        // eight quads: each wave converts its own x, so workgroups cost no
        // extra conversions; about two four-wave workgroups per CU (two
        // waves a SIMD; measured on MI355X, 14336 x 4096 x 32: 148 us
        // against 233 us with one)
        rpb = 16 * ((ntiles + 511) / 512);
    } else {
        // at most about one workgroup per CU of a 256-CU part: each stages
        // all of x, which costs as much as decoding a few tiles
        rpb = 16 * ((ntiles + 255) / 256);
    }
    const size_t lds_x = kernel == 8   ? q4k::q8_lds_bytes(S, nw)
                         : kernel == 7 ? q4k::win_lds_bytes(S, (int)m)
                         : kernel == 6 ? q4k::jit_lds_bytes(S, (int)m)
                         : kernel == 5 ? q4k::sub_lds_bytes(S, (int)m)
                         : kernel == 3 ? q4k::dot4_lds_bytes(S, nw)
                                       : q4k::lines_lds_bytes(S, (int)m, nw);
    if (kernel == 7) {
        spt = 1;
    } else if (!(o && o->cols_per_task)) {
        // whole rows per task when the workgroup has a tile for every wave
        // (no row sums to combine), else one slab per task, so that every
        // wave streams; whole rows too when the per-slab row sums do not fit
        // the LDS (choices measured on MI355X: with fewer tiles than waves,
        // whole rows leave waves idle, 0.3-0.8 us on 16384-28672-row shapes)
        const bool fits = lds_x + (size_t)nslabs * rpb * 8 * m <= lds_max;
        const bool wide = kernel == 6 && m > q4k::kMaxMStaged;   // slab tasks measured faster
        spt = ((rpb / 16 >= nw && !wide) || !fits) ? nslabs : 1;
    }
    const int64_t ncg = nslabs / spt;
    if (rpb > kInt32Max / (ncg * m)) {
        return Q4K_ERR_SHAPE;
    }
    const int64_t grid = (n + rpb - 1) / rpb;
    // row sums of the slab groups: f64
    const size_t lds = lds_x + (ncg > 1 ? (size_t)ncg * rpb * 8 * m : 0);

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
// a column window (7), then with per-wave x (6), else the x-stager kernel
// (1, m <= 8; 9-32 vectors are refused there).  17-32 vectors: kernel 6
// only.
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
        // sub-block kernel from three vectors on; when no whole x stage fits
        // the LDS, the workgroup's column window, else per-wave x conversion
        if (!any_option(o) && w_aligned128) {
            const int first = m >= 3 ? 5 : 4;
            for (int kern : {first, 9 - first, 7, 6}) {
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
    if (kernel < 1 || kernel > 7 || ((kernel == 2 || kernel == 3) && m != 1) ||
        (kernel == 1 && m > q4k::kMaxM)) {
        return Q4K_ERR_UNSUPPORTED;
    }
    if (kernel >= 3) {
        return make_plan_lines(n, k, m, o, lds_max, p, kernel);
    }
    if (o && o->cols_per_task) {
        return Q4K_ERR_UNSUPPORTED;   // line-streamed kernels only
    }
    // four or eight waves: the f64 x of the streaming kernel (128 VGPRs a
    // lane) leaves no room in 1024-lane workgroups
    int nw = (o && o->waves_per_block) ? o->waves_per_block : 8;
    if (nw != 4 && nw != 8) {
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
    const int ring_depth = (o && o->ring_depth) ? o->ring_depth : (rows_per_task >= 8 ? 3 : 1);
    if (kernel == 2 && (ring_depth < 1 || ring_depth > 4 || rows_per_task < 1 ||
                        rows_per_task > kInt32Max)) {
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
    const size_t lds_x = (size_t)m * spc * kSpanBytes;
    const size_t lds_row = kernel == 2 ? 0 : nchunks > 1 ? (size_t)m * 64 * 8 : 0;   // parked lane partials (f64)
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
        // x chunk + per-span row sums (f64)
        lds = (size_t)spc * kSpanBytes + (nspans > 1 ? (size_t)nspans * rpb * 8 : 0);
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

// The plan gemv_checked would launch, for a given LDS budget; shape and
// option checks in the same order.  9-32 vectors run in one pass over the
// weights on the sub-block kernels (5-7; 6 beyond 16) or are refused: a batch is never
// split into several launches (turbospark-runtime 0.1.0,
// real_forward_dispatch.rs: doc of `encode_gemm_any`).
int plan_checked(int64_t n, int64_t k, int64_t m, const q4k_launch* opts, bool w128,
                 size_t lds_max, GemvPlan* plan)
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
    if (m > q4k::kMaxM && plan->kernel < 5) {
        return Q4K_ERR_UNSUPPORTED;    // 9-32 vectors: the sub-block kernels only
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
    rc = plan_checked(n, k, m, opts, w128, 0, &plan);
    if (rc != Q4K_OK) {
        return rc;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(q4k::launch_gemv(plan, w, x, y, s));
}

// ------------------------------------------------------------------ Q6_K
constexpr int64_t kQ6Bytes = 210;

// The row stride in bytes (0: dense), checked against the row and the
// 16-byte rule.
int q6k_stride(int64_t k, int64_t row_stride, int64_t* out)
{
    const int64_t dense = (k / q4k::kQK) * kQ6Bytes;
    const int64_t stride = row_stride == 0 ? dense : row_stride;
    if (stride < dense || stride > ((int64_t)1 << 40)) {
        return Q4K_ERR_SHAPE;
    }
    if (stride % 16 != 0) {
        return Q4K_ERR_ALIGN;
    }
    *out = stride;
    return Q4K_OK;
}

// Tiles of 16 rows; about one workgroup of NW waves per CU: a workgroup
// takes ceil(tiles / 256) tiles and, when that leaves waves idle, splits each
// tile's columns into up to eight groups (powers of two, at most S).
int make_q6k_plan(int64_t n, int64_t k, int64_t stride, bool w128, const q6k_launch* o,
                  size_t lds_max, q4k::Q6kPlan* p)
{
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    const int S = (int)(k / q4k::kQK);
    const int64_t tiles = (n + 15) / 16;
    p->n = (int)n;
    p->k = (int)k;
    p->S = S;
    p->row_stride = stride;
    const bool lines = w128;       // whole lines: any 16-byte row stride, w 128-byte aligned
    const int unit = o ? o->unit_bytes : 0;
    if (unit == 0) {
        p->unit = lines ? 128 : 64;
    } else if (unit == 64 || (unit == 128 && lines)) {
        p->unit = unit;
    } else {
        return Q4K_ERR_UNSUPPORTED;
    }
    const bool no_phase = p->unit == 64 || stride % 128 == 0;
    const int batch = o ? o->batch_bytes : 0;
    if (batch == 0) {
        p->batch = no_phase ? 256 : 128;
    } else if ((batch == 128 && p->unit == 128) || (batch == 256 && no_phase)) {
        p->batch = batch;
    } else {
        return Q4K_ERR_UNSUPPORTED;
    }
    const int nw = o ? o->waves_per_block : 0;
    if (nw != 0 && nw != 4 && nw != 8) {
        return Q4K_ERR_UNSUPPORTED;
    }
    p->waves_per_block = nw == 0 ? 8 : nw;
    if (S * 16 > 4 * p->waves_per_block * 64) {
        return Q4K_ERR_UNSUPPORTED;      // at most four groups of 16 x values per thread
    }
    int64_t tpb = o && o->tiles_per_block ? o->tiles_per_block : (tiles + 255) / 256;
    if (tpb < 1 || tpb * 16 > kInt32Max / 64) {
        return Q4K_ERR_UNSUPPORTED;
    }
    tpb = tpb > tiles ? tiles : tpb;
    int ncg = o ? o->column_groups : 0;
    if (ncg == 0) {
        ncg = 1;
        while (ncg * 2 <= 8 && ncg * 2 <= S && tpb * ncg < p->waves_per_block) {
            ncg *= 2;
        }
    } else if (ncg < 1 || ncg > 16 || ncg > S) {
        return Q4K_ERR_UNSUPPORTED;
    }
    p->ncg = ncg;
    p->rows_per_block = (int)(16 * tpb);
    const int64_t grid = (tiles + tpb - 1) / tpb;
    if (grid > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    p->grid = (int)grid;
    p->lds_bytes = q4k::q6k_lds_bytes(S, p->waves_per_block, p->rows_per_block, ncg);
    if (p->lds_bytes > lds_max) {
        return Q4K_ERR_UNSUPPORTED;
    }
    return Q4K_OK;
}

int q6k_gemv_checked(const void* w, const float* x, float* y, int64_t n, int64_t k,
                     int64_t row_stride, const q6k_launch* opts, void* stream)
{
    if (!w || !x || !y) {
        return Q4K_ERR_NULL;
    }
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    int64_t stride = 0;
    rc = q6k_stride(k, row_stride, &stride);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (n > INT64_MAX / stride) {
        return Q4K_ERR_SHAPE;
    }
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) {
        return Q4K_ERR_ALIGN;
    }
    // options and shape first (no HIP call), then the device's LDS limit
    const bool w128 = (reinterpret_cast<uintptr_t>(w) & 127u) == 0;
    q4k::Q6kPlan plan;
    rc = make_q6k_plan(n, k, stride, w128, opts, SIZE_MAX, &plan);
    if (rc != Q4K_OK) {
        return rc;
    }
    size_t lds_max = 0;
    rc = device_lds_max(&lds_max);
    if (rc != Q4K_OK) {
        return rc;
    }
    rc = make_q6k_plan(n, k, stride, w128, opts, lds_max, &plan);
    if (rc != Q4K_OK) {
        return rc;
    }
    return hip_status(q4k::launch_q6k_gemv(plan, w, x, y, static_cast<hipStream_t>(stream)));
}

// Arguments of the prefill GEMM (before any HIP call).
int f16_gemm_checks(const void* w16, const void* x16, const float* y, int64_t m, int64_t n,
                    int64_t k)
{
    if (!w16 || !x16 || !y) {
        return Q4K_ERR_NULL;
    }
    if (m < 1 || n < 1 || k < 1 || m > kInt32Max || n > kInt32Max || k > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    if (k % 64 != 0) {
        return Q4K_ERR_UNSUPPORTED;      // the k step of the tile
    }
    if (!aligned16(w16) || !aligned16(x16) || !aligned16(y)) {
        return Q4K_ERR_ALIGN;
    }
    if (q4k::f16_gemm_grid(m, n) > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    return Q4K_OK;
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
    GemvPlan plan;
    const int rc = plan_checked(n, k, m, opts, w_aligned128 != 0, lds_max, &plan);
    if (rc != Q4K_OK) {
        return rc;
    }
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

int q4k_gemv_q8(const void* w, const float* x, float* y, int64_t n, int64_t k, int64_t m,
                void* stream)
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
    if (m != 1) {
        return Q4K_ERR_UNSUPPORTED;    // one vector (the pages' decode GEMV)
    }
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) {
        return Q4K_ERR_ALIGN;
    }
    if ((reinterpret_cast<uintptr_t>(w) & 127u) != 0) {
        return Q4K_ERR_UNSUPPORTED;    // whole-line reads need 128-byte aligned rows
    }
    GemvPlan plan;
    rc = make_plan_lines(n, k, 1, nullptr, SIZE_MAX, &plan, 8);
    if (rc != Q4K_OK) {
        return rc;
    }
    size_t lds_max = 0;
    rc = device_lds_max(&lds_max);
    if (rc != Q4K_OK) {
        return rc;
    }
    rc = make_plan_lines(n, k, 1, nullptr, lds_max, &plan, 8);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (plan.lds_bytes > lds_max) {
        return Q4K_ERR_UNSUPPORTED;
    }
    return hip_status(q4k::launch_gemv_q8(plan, w, x, y, static_cast<hipStream_t>(stream)));
}

int q4k_quantize_q8(const float* x, int8_t* q, float* d, int64_t k, int64_t m, void* stream)
{
    if (!x || !q || !d) {
        return Q4K_ERR_NULL;
    }
    if (k < 32 || k % 32 != 0 || m < 1 || k > kInt32Max || m > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    if (!aligned16(x) || !aligned16(q) || !aligned16(d)) {
        return Q4K_ERR_ALIGN;
    }
    const int64_t nblocks = m * (k / 32);
    if ((nblocks + 255) / 256 > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    return hip_status(q4k::launch_quantize_q8(x, q, d, nblocks, static_cast<hipStream_t>(stream)));
}

size_t q6k_row_bytes(int64_t k)
{
    if (k < q4k::kQK || k % q4k::kQK != 0) {
        return 0;
    }
    return (size_t)(k / q4k::kQK) * (size_t)kQ6Bytes;
}

int q6k_load(void* w_dev, const void* src_host, size_t src_bytes, int64_t n, int64_t k,
             int64_t row_stride, void* stream)
{
    if (!w_dev || !src_host) {
        return Q4K_ERR_NULL;
    }
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    int64_t stride = 0;
    rc = q6k_stride(k, row_stride, &stride);
    if (rc != Q4K_OK) {
        return rc;
    }
    const size_t row = q6k_row_bytes(k);
    if ((size_t)n > SIZE_MAX / row || (size_t)n * row != src_bytes ||
        (size_t)n > SIZE_MAX / (size_t)stride) {
        return Q4K_ERR_SIZE;
    }
    if (!aligned16(w_dev)) {
        return Q4K_ERR_ALIGN;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpy2DAsync(w_dev, (size_t)stride, src_host, row, row, (size_t)n,
                                    hipMemcpyHostToDevice, s);
    if (e == hipSuccess) {
        e = hipStreamSynchronize(s);
    }
    return hip_status(e);
}

int q6k_gemv(const void* w, const float* x, float* y, int64_t n, int64_t k, int64_t row_stride,
             void* stream)
{
    return q6k_gemv_checked(w, x, y, n, k, row_stride, nullptr, stream);
}

int q6k_gemv_ex(const void* w, const float* x, float* y, int64_t n, int64_t k,
                int64_t row_stride, const q6k_launch* opts, void* stream)
{
    return q6k_gemv_checked(w, x, y, n, k, row_stride, opts, stream);
}

int q6k_plan(int64_t n, int64_t k, int64_t row_stride, int w_aligned128, const q6k_launch* opts,
             size_t lds_max, q6k_plan_info* out)
{
    if (!out) {
        return Q4K_ERR_NULL;
    }
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    int64_t stride = 0;
    rc = q6k_stride(k, row_stride, &stride);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (lds_max == 0) {
        rc = device_lds_max(&lds_max);
        if (rc != Q4K_OK) {
            return rc;
        }
    }
    q4k::Q6kPlan plan;
    rc = make_q6k_plan(n, k, stride, w_aligned128 != 0, opts, lds_max, &plan);
    if (rc != Q4K_OK) {
        return rc;
    }
    out->unit_bytes = plan.unit;
    out->batch_bytes = plan.batch;
    out->waves_per_block = plan.waves_per_block;
    out->column_groups = plan.ncg;
    out->rows_per_block = plan.rows_per_block;
    out->grid = plan.grid;
    out->lds_bytes = (int32_t)plan.lds_bytes;
    return Q4K_OK;
}

int q6k_dequantize(const void* w, float* out, int64_t n, int64_t k, int64_t row_stride,
                   void* stream)
{
    if (!w || !out) {
        return Q4K_ERR_NULL;
    }
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    int64_t stride = 0;
    rc = q6k_stride(k, row_stride, &stride);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (!aligned16(out)) {
        return Q4K_ERR_ALIGN;
    }
    const int64_t groups = n * (k / q4k::kQK) * 16;
    if ((groups + 255) / 256 > kInt32Max || n > INT64_MAX / stride) {
        return Q4K_ERR_SHAPE;
    }
    return hip_status(q4k::launch_q6k_dequant(w, out, n, (int)(k / q4k::kQK), stride,
                                              static_cast<hipStream_t>(stream)));
}

int q4k_mirror_f16(const void* w, void* w16, int64_t n, int64_t k, void* stream)
{
    if (!w || !w16) {
        return Q4K_ERR_NULL;
    }
    const int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (!aligned16(w) || !aligned16(w16)) {
        return Q4K_ERR_ALIGN;
    }
    const int64_t nsb = n * (k / q4k::kQK);
    if ((nsb * 32 + 255) / 256 > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    return hip_status(q4k::launch_dequant_f16(w, w16, nsb, static_cast<hipStream_t>(stream)));
}

int q6k_mirror_f16(const void* w, void* w16, int64_t n, int64_t k, int64_t row_stride,
                   void* stream)
{
    if (!w || !w16) {
        return Q4K_ERR_NULL;
    }
    int rc = check_nk(n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    int64_t stride = 0;
    rc = q6k_stride(k, row_stride, &stride);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (!aligned16(w16)) {
        return Q4K_ERR_ALIGN;
    }
    const int64_t groups = n * (k / q4k::kQK) * 16;
    if ((groups + 255) / 256 > kInt32Max || n > INT64_MAX / stride) {
        return Q4K_ERR_SHAPE;
    }
    return hip_status(q4k::launch_q6k_dequant_f16(w, w16, n, (int)(k / q4k::kQK), stride,
                                                  static_cast<hipStream_t>(stream)));
}

int q4k_f16_cvt(const float* x, void* x16, int64_t count, void* stream)
{
    if (!x || !x16) {
        return Q4K_ERR_NULL;
    }
    if (count < 1 || (count + 1023) / 1024 > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    if (!aligned16(x) || !aligned16(x16)) {
        return Q4K_ERR_ALIGN;
    }
    return hip_status(q4k::launch_f16_cvt(x, x16, count, static_cast<hipStream_t>(stream)));
}


int q4k_f16_gemm(const void* w16, const void* x16, float* y, int64_t m, int64_t n, int64_t k,
                 void* stream)
{
    const int rc = f16_gemm_checks(w16, x16, y, m, n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    return hip_status(q4k::launch_f16_gemm(w16, x16, y, (int)m, (int)n, (int)k,
                                           static_cast<hipStream_t>(stream)));
}

int q4k_f16_gemm_f32x(const void* w16, const float* x, void* xh, float* y, int64_t m,
                      int64_t n, int64_t k, void* stream)
{
    if (!x || !xh) {
        return Q4K_ERR_NULL;
    }
    int rc = f16_gemm_checks(w16, xh, y, m, n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (!aligned16(x)) {
        return Q4K_ERR_ALIGN;
    }
    if ((m * k + 1023) / 1024 > kInt32Max) {
        return Q4K_ERR_SHAPE;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    rc = hip_status(q4k::launch_f16_cvt(x, xh, m * k, s));
    if (rc != Q4K_OK) {
        return rc;
    }
    return hip_status(q4k::launch_f16_gemm(w16, xh, y, (int)m, (int)n, (int)k, s));
}

int q4k_f16_gemm_f32x_noalloc(const void* w16, const float* x, float* y, int64_t m, int64_t n,
                              int64_t k, void* stream)
{
    if (!x) {
        return Q4K_ERR_NULL;
    }
    // the checks of q4k_f16_gemm with the scratch standing in for xh (any
    // non-null, aligned value: the array is 256-byte aligned)
    int rc = f16_gemm_checks(w16, reinterpret_cast<const void*>(uintptr_t{256}), y, m, n, k);
    if (rc != Q4K_OK) {
        return rc;
    }
    if (!aligned16(x)) {
        return Q4K_ERR_ALIGN;
    }
    if (m * k > q4k::kScratchHalves) {
        return Q4K_ERR_UNSUPPORTED;      // beyond the static scratch (4 Mi halves)
    }
    void* xh = nullptr;
    rc = hip_status(q4k::f16_scratch(&xh));
    if (rc != Q4K_OK) {
        return rc;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    rc = hip_status(q4k::launch_f16_cvt(x, xh, m * k, s));
    if (rc != Q4K_OK) {
        return rc;
    }
    return hip_status(q4k::launch_f16_gemm(w16, xh, y, (int)m, (int)n, (int)k, s));
}

const char* q4k_status_string(int rc)
{
    switch (rc) {
    case Q4K_OK: return "ok";
    case Q4K_ERR_NULL: return "a required pointer is NULL";
    case Q4K_ERR_SHAPE: return "bad shape: need 1 <= n, 256 <= k, k % 256 == 0, 1 <= m, n and k below 2^31";
    case Q4K_ERR_SIZE: return "byte count does not match n rows of the format (144 or 210 bytes per 256 weights)";
    case Q4K_ERR_ALIGN: return "a pointer, or a Q6_K row stride, is not 16-byte aligned";
    case Q4K_ERR_UNSUPPORTED:
        return "unsupported: m > 32, or launch options that do not fit the shape, m or the "
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
