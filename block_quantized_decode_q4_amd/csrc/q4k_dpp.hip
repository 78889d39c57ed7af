// q4k_dpp.hip -- Q4_K GEMV for one vector on the vector ALU: the line stream
// of q4k_lines.h feeding integer dot products (v_dot4c_i32_i8), with x
// shared across the 16 rows of a tile by DPP broadcast instead of LDS reads.
//
// Arithmetic (Q4_K superblock format; per sub-block j of 32 weights,
// w = d * sc_j * q - dmin * m_j, so
//   sum_i w_i x_i = d * sc_j * sum_i q_i x_i - dmin * m_j * sum_i x_i):
//  * x is held as integers on a per-sub-block grid, xi = rint(x * 2^s),
//    |xi| < 2^30, in four signed base-256 digits, each element certified to
//    a relative error of 2^-17 (q4k_xrep.h); elements that cannot be
//    certified are left out of the digits and added exactly below.
//  * The 4-bit codes stay packed: for a dword of four code bytes, the low
//    nibbles (byte & 0x0F) and 16 q - 128 for the high nibbles
//    ((byte & 0xF0) ^ 0x80) are signed int8 operands; four v_dot4c_i32_i8
//    per nibble half and dword (one per digit) accumulate exact int32 sums
//    T_l = sum q * D_l.  sum q xi = T_0 + 256 T_1 + 65536 T_2 + 2^24 T_3 for
//    the low sub-block, exactly in f64; the high one adds 128 * XI (XI =
//    sum xi) and is 16 times sum q xi.
//  * Superblock scales: fp16 d and dmin and the 6-bit (sc, m) pairs of the
//    lane's two sub-blocks (two byte permutes, gather_scales); each
//    sub-block's 2^-s (d sc T - dmin m XI) joins an f64 sum per lane with an
//    error-free product (subblock_term), so neither the grid nor cancelling
//    weights (d sc q close to dmin m) cost accuracy beyond 2^-17 sum |w||x|.
//  * An element the grid cannot carry (a value far below its sub-block's
//    largest, or inf/NaN) is listed per column (up to kCorr of them; a
//    column with more is scanned again from x in global memory); a column
//    with such elements takes a branch in which the lanes of each element's
//    chunk add fl32(d sc q - dmin m) * x in f64, the oracle's own
//    arithmetic.
//
// Lane layout of a 16-row tile step (one superblock column): lane l = 16 g +
// j takes row j, chunk g (bytes 16 + 32 g .. of the superblock: elements
// 64 g + i as low nibbles, 64 g + 32 + i as high nibbles).  All 16 lanes of a
// DPP row (the same g) need the same 64 x values.  Each of them reads one 16
// byte slot of the staged x -- lane j holds the four digit dwords of code
// dword u = j / 2, low half (j even) or high half (j odd) -- and the dot
// products take their x operand from lane 2u or 2u + 1 of the row through
// DPP row_newbcast, folded into the dot instruction itself.  So a lane reads
// 16 bytes of x per superblock from LDS, not 256.
//
// Staged x per superblock column (kDotCol bytes): four chunks of sixteen
// 16-byte slots (D0, D1, D2, D3) in the lane order above, eight {2^-s, XI}
// f64 pairs in sub-block order, the number of uncertified elements of the
// column and the first kCorr of them {element, x}.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_device.h"
#include "q4k_kernels.h"
#include "q4k_lines.h"
#include "q4k_xrep.h"

namespace q4k {

constexpr int kDotConst = 4 * 16 * 16;                 // {2^-s, XI} of the eight sub-blocks
constexpr int kDotWord = kDotConst + 8 * 16;           // uncertified elements of the column
constexpr int kDotList = kDotWord + 16;                // the first kCorr of them
constexpr int kDotCol = kDotList + kCorr * 8;

// One v_dot4c_i32_i8 whose first operand is lane N of the DPP row.
#define Q4K_DOTB(ACC, X, C, N) \
    "v_dot4c_i32_i8_dpp %" #ACC ", %" #X ", %" #C " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n"
// The eight dot products of code dword u: low codes (operand CL) against the
// four digits of lane NL = 2u, high codes (CH) against lane NH = 2u + 1.
#define Q4K_DOTU(CL, CH, NL, NH)                                              \
    Q4K_DOTB(0, 8, CL, NL) Q4K_DOTB(1, 9, CL, NL) Q4K_DOTB(2, 10, CL, NL)     \
    Q4K_DOTB(3, 11, CL, NL) Q4K_DOTB(4, 8, CH, NH) Q4K_DOTB(5, 9, CH, NH)     \
    Q4K_DOTB(6, 10, CH, NH) Q4K_DOTB(7, 11, CH, NH)

// Digit sums of one superblock step: t[0..3] (low sub-block) and t[4..7]
// (high) += the 64 dot products of the lane's eight code dwords.  The
// compiler does not see the dot instructions inside the block, so the block
// keeps their hazards itself: a DPP operand needs two wait states after a
// VALU write of it and five after a VALU write of EXEC (the leading s_nop),
// and another VALU instruction may read a dot result three wait states
// after the dot at the earliest (the trailing s_nop; without it, waves
// running alone on a SIMD read stale sums).  Within the block each
// accumulator is rewritten eight instructions after its last write.
__device__ __forceinline__ void dot_step(const uint4& xd, const int (&cl)[8], const int (&ch)[8],
                                         int (&t)[8])
{
    asm("s_nop 4\n"
        Q4K_DOTU(12, 20, 0, 1) Q4K_DOTU(13, 21, 2, 3) Q4K_DOTU(14, 22, 4, 5)
        Q4K_DOTU(15, 23, 6, 7) Q4K_DOTU(16, 24, 8, 9) Q4K_DOTU(17, 25, 10, 11)
        Q4K_DOTU(18, 26, 12, 13) Q4K_DOTU(19, 27, 14, 15)
        "s_nop 2\n"
        : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]),
          "+v"(t[7])
        : "v"(xd.x), "v"(xd.y), "v"(xd.z), "v"(xd.w),
          "v"(cl[0]), "v"(cl[1]), "v"(cl[2]), "v"(cl[3]), "v"(cl[4]), "v"(cl[5]), "v"(cl[6]),
          "v"(cl[7]),
          "v"(ch[0]), "v"(ch[1]), "v"(ch[2]), "v"(ch[3]), "v"(ch[4]), "v"(ch[5]), "v"(ch[6]),
          "v"(ch[7]));
}

#undef Q4K_DOTU
#undef Q4K_DOTB

// Convert 16 consecutive x values (group G of 16: column G / 16, elements
// 16 (G % 16) ..) into digit slots; lanes G and G ^ 1 hold one sub-block and
// meet through DPP (its largest |x| and its integer sum), the 16 lanes of a
// column through a row scan (its uncertified elements, listed in element
// order).  Every lane of the wave calls this; `store` is false for groups
// past the last column.
__device__ __forceinline__ void convert_group_dot(const float4 (&v)[4], int G, bool store,
                                                  unsigned char* xs)
{
    const float e[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                         v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    const Conv16 cv = convert16(e);
    if (store) {
        unsigned char* col = xs + (size_t)(G >> 4) * kDotCol;
        const int e0 = (G & 15) * 16;               // first element within the column
        const int chunk = e0 >> 6;
        const int high = (e0 & 63) >= 32 ? 1 : 0;
        const int u0 = (e0 & 31) >> 2;              // first code dword
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            *reinterpret_cast<uint4*>(col + chunk * 256 + (2 * (u0 + t) + high) * 16) =
                make_uint4(cv.plane[0][t], cv.plane[1][t], cv.plane[2][t], cv.plane[3][t]);
        }
        if ((G & 1) == 0) {
            *reinterpret_cast<double2*>(col + kDotConst + ((G & 15) >> 1) * 16) =
                make_double2(grid_scale(cv.sigma), cv.xsum);
        }
        if ((G & 15) == 0) {
            *reinterpret_cast<uint32_t*>(col + kDotWord) = (uint32_t)cv.total;
        }
        store_corrections(col + kDotList, cv, e, e0);
    }
}

// ANY: rows of any whole number of superblocks (line_stream_any, four-line
// rings, per-row start offsets); else S % 8 == 0 (line_stream).
template <int NW, int P, int XC, bool ANY, bool ONEBODY = false>
__global__ void __launch_bounds__(NW * 64)
gemv_dot4_lines_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                       float* __restrict__ y, int n, int S, int rows_per_block, int slabs_per_task)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ncg = ((S + 7) >> 3) / slabs_per_task;
    constexpr int kWaveRing = ANY ? kRing4Wave : kRingWave;

    // LDS: staged x (S columns), the line rings, row sums of slab groups
    const size_t xbytes = (size_t)S * kDotCol;
    unsigned char* ring = smem + xbytes + wave * kWaveRing;
    double* ypart = reinterpret_cast<double*>(smem + xbytes + NW * kWaveRing);

    // XC groups of 16 x values per thread: all of x when S * 16 <= XC * 64 NW;
    // loads past the end are clamped, their results not stored
    const int ngroups = S * 16;
    float4 xv[XC][4];
    auto issue_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int G = min(tid + i * NW * 64, ngroups - 1);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                xv[i][t] = reinterpret_cast<const float4*>(x)[4 * G + t];
            }
        }
    };
    auto convert_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int G = tid + i * NW * 64;
            convert_group_dot(xv[i], G, G < ngroups, smem);
        }
    };

    // the lane's (row, chunk) sum over its tasks' superblocks, in f64
    double acc = 0.0;
    const ScaleGather sg = scale_gather(g);
    auto dot_math = [&](const uint4& h, const uint4& q0, const uint4& q1, int c, auto corr) __attribute__((always_inline)) {
        const unsigned char* col = smem + (size_t)c * kDotCol;
        const uint4 xd = *reinterpret_cast<const uint4*>(col + g * 256 + j * 16);
        const double2 klo = *reinterpret_cast<const double2*>(col + kDotConst + g * 32);
        const double2 khi = *reinterpret_cast<const double2*>(col + kDotConst + g * 32 + 16);
        const uint32_t cnt = *reinterpret_cast<const uint32_t*>(col + kDotWord);
        const uint32_t D[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        int cl[8], ch[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            cl[u] = (int)(D[u] & 0x0F0F0F0Fu);
            ch[u] = (int)((D[u] & 0xF0F0F0F0u) ^ 0x80808080u);
        }
        int t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        dot_step(xd, cl, ch, t);
        const uint32_t sm = gather_scales(h, sg);
        const half2_t dd = __builtin_bit_cast(half2_t, h.x);
        const float d = (float)dd.x;
        const float dmin = (float)dd.y;
        // d sc and dmin m are exact in f32 (at most 17 significant bits), and
        // so is d sc / 16 for the high sub-block, whose digit sums carry 16 q
        const float Dlo = d * (float)(sm & 0xFFu);
        const float Dhi = d * (float)((sm >> 8) & 0xFFu);
        const float Mlo = dmin * (float)((sm >> 16) & 0xFFu);
        const float Mhi = dmin * (float)(sm >> 24);
        const double Tlo = digits_exact(t[0], t[1], t[2], t[3]);
        const double Thi16 = __builtin_fma(khi.y, 128.0, digits_exact(t[4], t[5], t[6], t[7]));
        acc = subblock_term(acc, Dlo, Tlo, Mlo, klo.y, klo.x);
        acc = subblock_term(acc, Dhi * 0.0625f, Thi16, Mhi, khi.y, khi.x);
        if constexpr (decltype(corr)::value) {
            // a slab with elements the digits leave out: their exact terms
            const uint32_t ncorr = __builtin_amdgcn_readfirstlane(cnt);
            if (ncorr != 0u) {
                acc = column_corrections(acc, ncorr, col + kDotList, D, g, Dlo, Dhi, Mlo, Mhi,
                                         klo.x, khi.x, x + (size_t)c * 256);
            }
        } else {
            (void)cnt;
        }
    };
    // whether slab sl (eight columns) has a column with uncertified elements:
    // one bit per column in scalar registers, gathered by ballots on the
    // first call (after the x stage; at most 128 columns, four groups of 16
    // elements per lane)
    uint64_t cmask[2] = {0, 0};
    bool have_mask = false;
    auto slab_flag = [&](int sl) __attribute__((always_inline)) {
        if (!have_mask) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 64 * h + lane;
                const uint32_t cnt =
                    c < S ? *reinterpret_cast<const uint32_t*>(smem + (size_t)c * kDotCol + kDotWord)
                          : 0u;
                cmask[h] = __ballot(cnt != 0u);
            }
            have_mask = true;
        }
        const int c0 = 8 * sl;
        const uint64_t bits = c0 < 64 ? cmask[0] >> c0 : cmask[1] >> (c0 - 64);
        return (bits & 0xFFu) != 0u;
    };
    auto task_end = [&](int task) __attribute__((always_inline)) {
        const int r = (task / ncg) * 16 + j;
        double v = acc;
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (g == 0 && r < rows_here) {
            if (ncg == 1) {
                y[row0 + r] = (float)v;
            } else {
                ypart[(task % ncg) * rows_per_block + r] = v;
            }
        }
        acc = 0.0;
    };
    if constexpr (ANY) {
        // row j starts loff bytes into its first line (tiles start on a
        // line); pieces wrap in the row's four-line window individually
        constexpr uint32_t kWindow = 511u;
        const uint32_t loff = (uint32_t)(j * 144 * S) & 127u;
        auto step = [&](int c, const unsigned char* rr, uint32_t b0, auto corr) __attribute__((always_inline)) {
            const uint32_t b = b0 + loff;
            const uint4 h = *reinterpret_cast<const uint4*>(rr + (b & kWindow));
            const uint4 q0 =
                *reinterpret_cast<const uint4*>(rr + ((b + 16u + 32u * (uint32_t)g) & kWindow));
            const uint4 q1 =
                *reinterpret_cast<const uint4*>(rr + ((b + 32u + 32u * (uint32_t)g) & kWindow));
            dot_math(h, q0, q1, c, corr);
        };
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step, task_end, slab_flag);
    } else {
        // superblock c' of a slab starts at 144 c' mod 256 in the two-line
        // window of its ring row: the header at that compile-time offset, the
        // lane's 32 code bytes 16 + 32 g further, mod 256 (both 16-byte
        // halves on the same side of the wrap), so their eight addresses are
        // lane constants
        const unsigned char* qa[8];
#pragma unroll
        for (int cp = 0; cp < 8; ++cp) {
            qa[cp] = ring + j * kRingRow + ((144u * (uint32_t)cp + 16u + 32u * (uint32_t)g) & 255u);
        }
        auto step = [&](int c, const unsigned char* rr, uint32_t b0, auto corr) __attribute__((always_inline)) {
            const int cp = (int)(b0 / 144u);         // b0 = 144 cp
            const uint4 h = *reinterpret_cast<const uint4*>(rr + (b0 & 255u));
            const uint4 q0 = *reinterpret_cast<const uint4*>(qa[cp]);
            const uint4 q1 = *reinterpret_cast<const uint4*>(qa[cp] + 16);
            dot_math(h, q0, q1, c, corr);
        };
        line_stream<NW, P, decltype(issue_x), decltype(convert_x), decltype(step),
                    decltype(task_end), decltype(slab_flag), true, ONEBODY>(
            w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x, step, task_end,
            slab_flag);
    }

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here; i += NW * 64) {
            double a = 0.0;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[cg * rows_per_block + i];
            }
            y[row0 + i] = (float)a;
        }
    }
}

template <int NW, int P, int XC>
static hipError_t launch_dot4_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                hipStream_t stream)
{
    if constexpr (P == 3) {
        if (p.S % 8 != 0) {
            hipLaunchKernelGGL((gemv_dot4_lines_kernel<NW, 3, XC, true>), dim3(p.grid),
                               dim3(NW * 64), p.lds_bytes, stream, w, x, y, p.n, p.S,
                               p.rows_per_block, p.cols_per_task / 8);
            return hipGetLastError();
        }
    }
    if constexpr (P == 3) {
        // one slab per task: the slab body without the per-slab choice of a
        // correction-free copy (FFN-down 11.20 -> 11.01 us; whole-row tasks,
        // as on the LM head, keep the two copies: 14.55 against 14.74 us)
        if (p.cols_per_task == 8) {
            hipLaunchKernelGGL((gemv_dot4_lines_kernel<NW, 3, XC, false, true>), dim3(p.grid),
                               dim3(NW * 64), p.lds_bytes, stream, w, x, y, p.n, p.S,
                               p.rows_per_block, 1);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemv_dot4_lines_kernel<NW, P, XC, false>), dim3(p.grid), dim3(NW * 64),
                       p.lds_bytes, stream, w, x, y, p.n, p.S, p.rows_per_block,
                       p.cols_per_task / 8);
    return hipGetLastError();
}

// XC: groups of 16 x values each thread converts, the power of two covering
// S * 16 / (64 NW), at most 4 (k <= 16384 per 64 NW lanes)
template <int NW, int P>
static hipError_t launch_dot4_p(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                hipStream_t stream)
{
    const int per = (p.S * 16 + NW * 64 - 1) / (NW * 64);
    if (per <= 1) return launch_dot4_x<NW, P, 1>(p, w, x, y, stream);
    if (per <= 2) return launch_dot4_x<NW, P, 2>(p, w, x, y, stream);
    if (per <= 4) return launch_dot4_x<NW, P, 4>(p, w, x, y, stream);
    return hipErrorInvalidValue;
}

template <int NW>
static hipError_t launch_dot4_w(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                hipStream_t stream)
{
    if (p.ring_depth == 9) return launch_dot4_p<NW, 9>(p, w, x, y, stream);
    return launch_dot4_p<NW, 3>(p, w, x, y, stream);
}

hipError_t launch_gemv_dot4(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    switch (p.waves_per_block) {
    case 4: return launch_dot4_w<4>(p, wb, x, y, stream);
    case 8: return launch_dot4_w<8>(p, wb, x, y, stream);
    default: return hipErrorInvalidValue;
    }
}

size_t dot4_lds_bytes(int S, int waves)
{
    return (size_t)S * kDotCol + (size_t)waves * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

}  // namespace q4k
