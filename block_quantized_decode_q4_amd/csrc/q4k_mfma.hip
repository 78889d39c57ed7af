// q4k_mfma.hip -- Q4_K GEMV for a small batch of vectors (m <= 8; kernels 5
// and 6 up to 16) on the CDNA4 int8 matrix cores, fed by the line stream of
// q4k_lines.h.
//
// With several vectors the same decoded weights meet m different x, which
// makes the multiply a real (small) contraction: the matrix cores take it,
// and the vector ALU keeps the nibble unpack, the header decode and the
// per-superblock scaling.  Two kernels:
//  * gemv_i8_lines_kernel<NW, P, XC, M>: four v_mfma_i32_16x16x64_i8 per
//    superblock and vector (one 16-row tile, one vector per MFMA group);
//    automatic for m = 2.  With m = 1 it runs only when asked for, as the
//    measured matrix-core counterpart of the vector-ALU kernel (q4k_dpp.hip).
//  * gemv_i8_sub_kernel<NW, XC, NQ, false> (kernel 5): one
//    v_mfma_i32_16x16x32_i8 per 32-element sub-block and quad of vectors
//    (up to four quads: one pass over the weights for 16 vectors);
//    automatic for m >= 3.
//  * gemv_i8_sub_kernel<NW, XC, NQ, true> (kernel 6): the same decode with
//    x converted per column by each wave for itself, for batches whose x
//    does not fit the LDS as one stage (m k large).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_device.h"
#include "q4k_kernels.h"
#include "q4k_lines.h"
#include "q4k_xrep.h"

namespace q4k {


// ---------------------------------------------------------------------------
// Line-streamed int8 matrix-core kernel, one MFMA group per vector
// (v_mfma_i32_16x16x64_i8).
//
// Operands of one MFMA (16 x 16 x 64): lane l = 16 g + j holds
//   A[i = j][k = 16g .. 16g+15] (16 bytes), B[k = 16g .. 16g+15][j], D[4g + r][j].
//
//  * B = codes of 16 weight rows (j = row).  Lane group g reads chunk g of its
//    row (32 code bytes: sub-block 2g in the low nibbles, 2g+1 in the high
//    ones).  Low codes: byte & 0x0F (one AND per four codes).  High codes:
//    (byte & 0xF0) ^ 0x80 = 16 q - 128 as a signed byte (one three-input
//    bit operation per four codes).  Four MFMAs per superblock and vector:
//    bytes 0-15 and 16-31 of the chunk (mu = 0, 1: low codes; 2, 3: high).
//  * A = x on the grid of q4k_xrep.h, four signed digits per element.  Row
//    i = 4g' + l of A holds digit l of the 16 elements of chunk g' that
//    operand mu covers, in k-group g', and zero elsewhere, so D rows
//    4g .. 4g+3 of lane (g, j) are the four digit sums of exactly the
//    sub-block whose scales lane (g, j) decodes.  Inactive lanes read a zero
//    slot of the stage.
//  * Per step, vector and lane: the same exact sums and f64 scaling as the
//    vector-ALU kernel (q4k_dpp.hip), and the same exact terms for the
//    column's uncertified elements (the lane holds chunk g of row j, as
//    there).
//
// Staged x per (column, vector) pair (kK4Pair bytes): four operand blocks of
// sixteen 16-byte digit slots (slot 4 g + l: digit l of chunk g's sixteen
// elements) and a zero slot, eight {2^-s, XI} f64 pairs, the count of the
// pair's uncertified elements and the first kCorr of them.
// ---------------------------------------------------------------------------

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kK4Mu = 17 * 16;                  // 16 digit slots + a zero slot
constexpr int kK4Zero = 16 * 16;
constexpr int kK4Const = 4 * kK4Mu;
constexpr int kK4Word = kK4Const + 8 * 16;
constexpr int kK4List = kK4Word + 16;
constexpr int kK4Pair = kK4List + kCorr * 8;

__device__ __forceinline__ i32x4_t lo_codes(const uint4& q)
{
    return i32x4_t{(int)(q.x & 0x0F0F0F0Fu), (int)(q.y & 0x0F0F0F0Fu), (int)(q.z & 0x0F0F0F0Fu),
                   (int)(q.w & 0x0F0F0F0Fu)};
}

__device__ __forceinline__ i32x4_t hi_codes(const uint4& q)
{
    return i32x4_t{(int)((q.x & 0xF0F0F0F0u) ^ 0x80808080u), (int)((q.y & 0xF0F0F0F0u) ^ 0x80808080u),
                   (int)((q.z & 0xF0F0F0F0u) ^ 0x80808080u), (int)((q.w & 0xF0F0F0F0u) ^ 0x80808080u)};
}

// Convert the 16 elements lane l holds of a (column, vector) pair: elements
// 16 (l % 16) .. of the column, which operand mu = (l % 16) % 4 of chunk
// (l % 16) / 4 covers.  The 16 lanes of a DPP row hold one pair.
__device__ __forceinline__ void convert_pair_k4(const float4 (&v)[4], unsigned char* pair, int lane,
                                                bool store)
{
    const float e[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                         v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    const Conv16 cv = convert16(e);
    if (!store) {
        return;
    }
    const int t = lane & 15;
    const int mu = t & 3;
    const int g = t >> 2;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        *reinterpret_cast<uint4*>(pair + mu * kK4Mu + (4 * g + l) * 16) =
            make_uint4(cv.plane[l][0], cv.plane[l][1], cv.plane[l][2], cv.plane[l][3]);
    }
    if (t < 4) {
        *reinterpret_cast<uint4*>(pair + t * kK4Mu + kK4Zero) = make_uint4(0u, 0u, 0u, 0u);
    }
    if ((t & 1) == 0) {
        *reinterpret_cast<double2*>(pair + kK4Const + (t >> 1) * 16) =
            make_double2(grid_scale(cv.sigma), cv.xsum);
    }
    if (t == 0) {
        *reinterpret_cast<uint32_t*>(pair + kK4Word) = (uint32_t)cv.total;
    }
    store_corrections(pair + kK4List, cv, e, 16 * t);
}

// The 16 x elements lane l converts, of pair p (column p / m of vector p % m).
__device__ __forceinline__ void load_x_quarter(const float* __restrict__ x, int k, int m, int p,
                                               int lane, float4 (&v)[4])
{
    const float* src = x + (size_t)(p % m) * k + (size_t)(p / m) * 256 + 16 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = reinterpret_cast<const float4*>(src)[i];
    }
}

template <int NW, int P, int XC, int M>
__global__ void __launch_bounds__(NW * 64)
gemv_i8_lines_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                     float* __restrict__ y, int n, int S, int rows_per_block, int slabs_per_task)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    const uint32_t a_off =
        (j >> 2) == g ? (uint32_t)((g * 4 + (j & 3)) * 16) : (uint32_t)kK4Zero;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ncg = (S >> 3) / slabs_per_task;

    // LDS: staged x (S columns of M vectors, column-major, and a spare
    // pair), the line rings, row sums (f64)
    const int npairs = S * M;
    const size_t xbytes = (size_t)(npairs + 1) * kK4Pair;
    unsigned char* ring = smem + xbytes + wave * kRingWave;
    double* ypart = reinterpret_cast<double*>(smem + xbytes + NW * kRingWave);
    const int k = S * 256;

    // XC groups of four (column, vector) pairs of x per wave, one pair per
    // 16-lane group: all of them when S * M <= 4 * XC * NW; pair p is column
    // p / M of vector p % M
    float4 xv[XC][4];
    auto issue_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int pr = min(4 * (wave + i * NW) + (lane >> 4), npairs - 1);
            load_x_quarter(x, k, M, pr, lane, xv[i]);
        }
    };
    // every lane converts (the conversion exchanges values between lanes);
    // pairs past the last are not stored
    auto convert_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int pr = 4 * (wave + i * NW) + (lane >> 4);
            convert_pair_k4(xv[i], smem + (size_t)min(pr, npairs) * kK4Pair, lane, pr < npairs);
        }
        for (int q = XC * NW + wave; 4 * q < npairs; q += NW) {
            const int pr = 4 * q + (lane >> 4);
            float4 v[4];
            load_x_quarter(x, k, M, min(pr, npairs - 1), lane, v);
            convert_pair_k4(v, smem + (size_t)min(pr, npairs) * kK4Pair, lane, pr < npairs);
        }
    };

    double acc[M];
#pragma unroll
    for (int b = 0; b < M; ++b) {
        acc[b] = 0.0;
    }
    const ScaleGather sg = scale_gather(g);
    auto step = [&](int c, const unsigned char* rr, uint32_t b0, auto corr) __attribute__((always_inline)) {
        const uint4 h = *reinterpret_cast<const uint4*>(rr + (b0 & 255u));
        const uint4 q0 = *reinterpret_cast<const uint4*>(rr + ((b0 + 16u + 32u * (uint32_t)g) & 255u));
        const uint4 q1 = *reinterpret_cast<const uint4*>(rr + ((b0 + 32u + 32u * (uint32_t)g) & 255u));
        const uint32_t D[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        const i32x4_t lo0 = lo_codes(q0), lo1 = lo_codes(q1);
        const i32x4_t hi0 = hi_codes(q0), hi1 = hi_codes(q1);
        const uint32_t sm = gather_scales(h, sg);
        const half2_t dd = __builtin_bit_cast(half2_t, h.x);
        const float d = (float)dd.x;
        const float dmin = (float)dd.y;
        const float Dlo = d * (float)(sm & 0xFFu);
        const float Dhi = d * (float)((sm >> 8) & 0xFFu);
        const float Mlo = dmin * (float)((sm >> 16) & 0xFFu);
        const float Mhi = dmin * (float)(sm >> 24);
#pragma unroll
        for (int b = 0; b < M; ++b) {
            const unsigned char* pair = smem + (size_t)(c * M + b) * kK4Pair;
            const i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(pair + a_off);
            const i32x4_t a1 = *reinterpret_cast<const i32x4_t*>(pair + kK4Mu + a_off);
            const i32x4_t a2 = *reinterpret_cast<const i32x4_t*>(pair + 2 * kK4Mu + a_off);
            const i32x4_t a3 = *reinterpret_cast<const i32x4_t*>(pair + 3 * kK4Mu + a_off);
            const double2 klo = *reinterpret_cast<const double2*>(pair + kK4Const + g * 32);
            const double2 khi = *reinterpret_cast<const double2*>(pair + kK4Const + g * 32 + 16);
            const uint32_t cnt = *reinterpret_cast<const uint32_t*>(pair + kK4Word);
            const i32x4_t zero = {0, 0, 0, 0};
            i32x4_t Dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, lo0, zero, 0, 0, 0);
            Dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, lo1, Dl, 0, 0, 0);
            i32x4_t Dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, hi0, zero, 0, 0, 0);
            Dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, hi1, Dh, 0, 0, 0);
            const double Tlo = digits_exact(Dl[0], Dl[1], Dl[2], Dl[3]);
            const double Thi16 = __builtin_fma(khi.y, 128.0, digits_exact(Dh[0], Dh[1], Dh[2], Dh[3]));
            acc[b] = subblock_term(acc[b], Dlo, Tlo, Mlo, klo.y, klo.x);
            acc[b] = subblock_term(acc[b], Dhi * 0.0625f, Thi16, Mhi, khi.y, khi.x);
            if constexpr (decltype(corr)::value) {
                const uint32_t ncorr = __builtin_amdgcn_readfirstlane(cnt);
                if (ncorr != 0u) {
                    acc[b] = column_corrections(acc[b], ncorr, pair + kK4List, D, g, Dlo, Dhi, Mlo,
                                                Mhi, klo.x, khi.x, x + (size_t)b * k + (size_t)c * 256);
                }
            } else {
                (void)cnt;
            }
        }
    };
    // whether slab sl has a (column, vector) pair with uncertified elements
    auto slab_flag = [&](int sl) __attribute__((always_inline)) {
        uint32_t f = 0;
        for (int pr = 8 * sl * M; pr < 8 * (sl + 1) * M; ++pr) {
            f |= *reinterpret_cast<const uint32_t*>(smem + (size_t)pr * kK4Pair + kK4Word);
        }
        return __builtin_amdgcn_readfirstlane(f) != 0u;
    };
    auto task_end = [&](int task) __attribute__((always_inline)) {
        const int r = (task / ncg) * 16 + j;
#pragma unroll
        for (int b = 0; b < M; ++b) {
            double v = acc[b];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (g == 0 && r < rows_here) {
                if (ncg == 1) {
                    y[(size_t)b * n + row0 + r] = (float)v;
                } else {
                    ypart[(b * ncg + task % ncg) * rows_per_block + r] = v;
                }
            }
            acc[b] = 0.0;
        }
    };
    line_stream<NW, P>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x, step,
                       task_end, slab_flag);

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here * M; i += NW * 64) {
            const int b = i / rows_here;
            const int r = i - b * rows_here;
            double a = 0.0;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[(b * ncg + cg) * rows_per_block + r];
            }
            y[(size_t)b * n + row0 + r] = (float)a;
        }
    }
}

// ---------------------------------------------------------------------------
// Sub-block int8 matrix-core kernel for several vectors
// (v_mfma_i32_16x16x32_i8, line-streamed weights).
//
// Operands of one MFMA (16 x 16 x 32): lane l = 16 g + j holds
//   A[i = j][k = 8g .. 8g+7] (8 bytes), B[k = 8g .. 8g+7][j], D[4g + r][j].
//
// One MFMA covers one 32-element sub-block s for four vectors: B = the codes
// of sub-block s of the 16 rows of the tile (lane group g: elements 8g ..
// 8g+7, taken from bytes 8g .. 8g+7 of the chunk, low or high nibbles as in
// the kernels above), A row 4 b' + l = digit l of vector b' of the quad (x
// on the grid of q4k_xrep.h).  A is dense, so a superblock costs eight
// small MFMAs per quad of vectors instead of four large ones per vector, and
// lane (g, j) ends with the four digit sums of vector g of the quad for row
// j: it needs no other lane, but it scales all eight sub-blocks of its row,
// each with the exact sums and the one-rounding f64 term of subblock_term.
// A vector's uncertified elements are added exactly, per element, as in
// the kernels above (their codes read again from the row's ring).
// ---------------------------------------------------------------------------

constexpr int kSbBlock = 4 * 4 * 4 * 8;       // k-group x vector x digit, 8 bytes each
constexpr int kSbConst = 8 * kSbBlock;        // {2^-s, XI} per (vector, sub-block)
constexpr int kSbWord = kSbConst + 4 * 8 * 16;   // uncertified elements per vector
constexpr int kSbList = kSbWord + 16;         // the first kCorr of each vector
constexpr int kSbGroup = kSbList + 4 * kCorr * 8;   // one column, one quad
constexpr int kSbLists = kSbGroup - kSbWord;  // the counts and lists of a group
constexpr int kSigmaFromX = 1 << 20;          // rescan_subblock: no exponent given

// Convert one (column, vector quad): lane l takes vector l / 16 of the quad
// and elements 16 (l % 16) .. +15 of the column (half of sub-block (l % 16) /
// 2); digit l of elements 8 gk .. 8 gk + 7 of sub-block s of vector b' goes
// to slot (gk, b', l) of block s.  Every lane calls this (the conversion
// exchanges values between lanes).  The count of each vector's uncertified
// elements and the first kCorr of them go to lists (kSbLists bytes: four
// counts, then four lists).  Returns the lane's vector's count (the same in
// its 16 lanes).
__device__ __forceinline__ int convert_quad(const float4 (&v)[4], unsigned char* grp,
                                            unsigned char* lists, int lane)
{
    const float e[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                         v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    const Conv16 cv = convert16(e);
    const int t = lane & 15;
    const int bq = lane >> 4;                 // vector within the quad
    const int s = t >> 1;                     // sub-block
    const int half = t & 1;
    unsigned char* blk = grp + s * kSbBlock;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int gk = 2 * half + h;          // k-group of these eight elements
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            *reinterpret_cast<uint2*>(blk + ((gk * 4 + bq) * 4 + l) * 8) =
                make_uint2(cv.plane[l][2 * h], cv.plane[l][2 * h + 1]);
        }
    }
    if (half == 0) {
        *reinterpret_cast<double2*>(grp + kSbConst + (bq * 8 + s) * 16) =
            make_double2(grid_scale(cv.sigma), cv.xsum);
    }
    if (t == 0) {
        *reinterpret_cast<uint32_t*>(lists + bq * 4) = (uint32_t)cv.total;
    }
    store_corrections(lists + 16 + bq * (kCorr * 8), cv, e, 16 * t);
    return cv.total;
}

// The eight sub-block scales and mins of a header as floats.
struct RowScales {
    float d, dmin;
    float sc[8], m[8];
};

__device__ __forceinline__ RowScales decode_row(const uint4& h)
{
    RowScales r;
    const half2_t dd = __builtin_bit_cast(half2_t, h.x);
    r.d = (float)dd.x;
    r.dmin = (float)dd.y;
    const uint32_t sc03 = h.y & 0x3F3F3F3Fu;
    const uint32_t m03 = h.z & 0x3F3F3F3Fu;
    const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        r.sc[b] = (float)((sc03 >> (8 * b)) & 0xFFu);
        r.m[b] = (float)((m03 >> (8 * b)) & 0xFFu);
        r.sc[4 + b] = (float)((sc47 >> (8 * b)) & 0xFFu);
        r.m[4 + b] = (float)((m47 >> (8 * b)) & 0xFFu);
    }
    return r;
}

// v[s] for a per-lane s in 0..7, by masks (an indexed read would go through
// scratch memory)
__device__ __forceinline__ float pick8(const float (&v)[8], int s)
{
    uint32_t r = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        r |= __builtin_bit_cast(uint32_t, v[t]) & (0u - (uint32_t)(s == t));
    }
    return __builtin_bit_cast(float, r);
}

// The exact terms of sub-block se's uncertified elements for the lane's row
// (xs: the sub-block's 32 values of x, sigma: its grid exponent), each
// element tested as the conversion tested it: fl32(d sc q - dmin m) * x in
// f64, the oracle's own arithmetic.  Ds, Ms: d sc_j (/ 16 for odd j) and
// dmin m_j of the row; its codes are read again from its ring (rr, b: the
// superblock's first byte, window: the ring's size minus one).
__device__ __forceinline__ double rescan_subblock(double acc, const float* __restrict__ xs, int se,
                                                  int sigma, const float (&Ds)[8],
                                                  const float (&Ms)[8], const unsigned char* rr,
                                                  uint32_t b, uint32_t window)
{
    const float4* src = reinterpret_cast<const float4*>(xs);
    float4 xv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        xv[t] = src[t];
    }
    const uint32_t cb = b + 16u + 32u * (uint32_t)(se >> 1);
    const uint4 c0 = *reinterpret_cast<const uint4*>(rr + (cb & window));
    const uint4 c1 = *reinterpret_cast<const uint4*>(rr + ((cb + 16u) & window));
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    if (sigma == kSigmaFromX) {           // the conversion's own exponent, from x
        float mx = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            mx = fmaxf(mx, fabsf(xv[t].x));
            mx = fmaxf(mx, fabsf(xv[t].y));
            mx = fmaxf(mx, fabsf(xv[t].z));
            mx = fmaxf(mx, fabsf(xv[t].w));
        }
        sigma = grid_sigma(mx);
    }
    const float Dw = pick8(Ds, se) * ((se & 1) ? 16.0f : 1.0f);
    const float Mw = pick8(Ms, se);
    const uint32_t sh = 4u * (uint32_t)(se & 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float xe[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t u;
            int cert;
            grid_element(xe[i], sigma, u, cert);
            const uint32_t q = (cw[t] >> (8 * i + sh)) & 15u;
            const float wv = __builtin_fmaf(Dw, (float)q, -Mw);
            const double tv = (double)wv * (double)xe[i];
            acc = cert ? acc : acc + tv;
        }
    }
    return acc;
}

// The exact terms of one vector's uncertified elements in one column for
// the lane's row: cnt of them, listed in `list` when cnt <= kCorr, else
// found again by rescan_subblock (xg: the vector's 256 values of the column;
// cst: its {2^-s, XI} per sub-block, or null: the exponents are found again
// from x).  Arguments otherwise as there.
__device__ __forceinline__ double vector_corrections(double acc, uint32_t cnt, const unsigned char* list,
                                                     const double2* cst, const float* __restrict__ xg,
                                                     const float (&Ds)[8], const float (&Ms)[8],
                                                     const unsigned char* rr, uint32_t b,
                                                     uint32_t window)
{
    if (cnt <= (uint32_t)kCorr) {
        for (uint32_t k = 0; k < cnt; ++k) {
            const Corr c = *reinterpret_cast<const Corr*>(list + k * 8);
            const int se = (int)(c.e >> 5);              // sub-block 2 chunk + half
            const uint32_t byte = rr[(b + 16u + 32u * (uint32_t)(se >> 1) + (c.e & 31u)) & window];
            const uint32_t q = (se & 1) ? byte >> 4 : byte & 15u;
            const float Dw = pick8(Ds, se) * ((se & 1) ? 16.0f : 1.0f);
            const float Mw = pick8(Ms, se);
            const float wv = __builtin_fmaf(Dw, (float)q, -Mw);
            acc += (double)wv * (double)c.x;             // exact product
        }
        return acc;
    }
#pragma nounroll
    for (int se = 0; se < 8; ++se) {
        acc = rescan_subblock(acc, xg + 32 * se, se, cst ? grid_sigma_of(cst[se].x) : kSigmaFromX,
                              Ds, Ms, rr, b, window);
    }
    return acc;
}

// The row sums of up to eight vector quads as named values: the correction
// loops pick a quad at run time, and an array indexed so would be kept in
// scratch memory (the compiler turns a chain of selects over an array's
// elements back into an indexed load).
struct QuadAcc {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0, a4 = 0.0, a5 = 0.0, a6 = 0.0, a7 = 0.0;

    template <int Q>
    __device__ __forceinline__ double& at()
    {
        static_assert(Q >= 0 && Q < 8, "eight quads at most");
        if constexpr (Q == 0) {
            return a0;
        } else if constexpr (Q == 1) {
            return a1;
        } else if constexpr (Q == 2) {
            return a2;
        } else if constexpr (Q == 3) {
            return a3;
        } else if constexpr (Q == 4) {
            return a4;
        } else if constexpr (Q == 5) {
            return a5;
        } else if constexpr (Q == 6) {
            return a6;
        } else {
            return a7;
        }
    }
    __device__ __forceinline__ double get(int q) const
    {
        return q == 0   ? a0
               : q == 1 ? a1
               : q == 2 ? a2
               : q == 3 ? a3
               : q == 4 ? a4
               : q == 5 ? a5
               : q == 6 ? a6
                        : a7;
    }
    __device__ __forceinline__ void set(int q, double v)
    {
        a0 = q == 0 ? v : a0;
        a1 = q == 1 ? v : a1;
        a2 = q == 2 ? v : a2;
        a3 = q == 3 ? v : a3;
        a4 = q == 4 ? v : a4;
        a5 = q == 5 ? v : a5;
        a6 = q == 6 ? v : a6;
        a7 = q == 7 ? v : a7;
    }
};

// Columns of x a wave of kernel 6 holds in registers ahead of its step: with
// four, waiting for a column's x (loads complete in order) never waits for
// a weight line before the line stream itself would (the lines are three
// ahead); two vector quads take two, as 4 x 32 registers do not fit, four
// quads one (64 registers), eight quads one (128).
template <int NQ>
constexpr int jit_ahead()
{
    return NQ == 1 ? 4 : NQ == 2 ? 2 : 1;
}

// The three ways the sub-block kernel gets x into LDS (the kernel numbers
// of the launch options).
constexpr int kModeStaged = 5;   // x staged whole before the stream
constexpr int kModeJit = 6;      // each wave converts the column of each step for itself
constexpr int kModeWindow = 7;   // the workgroup converts each column once, just ahead

// Columns of x an owner of a window pair holds in registers ahead of its
// conversion.
constexpr int kWinAhead = 2;

// MODE kModeStaged (kernel 5): x staged whole in LDS before the stream.
// kModeJit (kernel 6): each wave converts the x column of each of its steps
// for itself into its own LDS group, from registers loaded jit_ahead columns
// earlier -- for batches whose whole x stage does not fit the LDS.
// kModeWindow (kernel 7): every wave has at most one task of one slab, so
// step s of every wave is superblock column 8 cg + s of its slab cg; the
// LDS holds two columns of every slab (a double-buffered window), and at step
// s the waves convert column s + 1 of every slab (pair (cg, q) of slab and
// vector quad by wave (cg NQ + q) mod NW) while they decode column s: one
// conversion per column and workgroup, with one LDS barrier per step.  Waves
// without a task go through the same conversions and barriers.
// ANY: rows of any whole number of superblocks (line_stream_any: four-line
// rings, per-row start offsets); else S % 8 == 0 (line_stream; always so
// for kModeWindow).
template <int NW, int XC, int NQ, int MODE, bool ANY>
__global__ void __launch_bounds__(NW * 64)
gemv_i8_sub_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                   float* __restrict__ y, int n, int S, int m, int rows_per_block,
                   int slabs_per_task)
{
    static_assert(MODE != kModeWindow || !ANY, "the window needs whole slabs");
    constexpr bool JIT = MODE == kModeJit;
    constexpr bool WIN = MODE == kModeWindow;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    // A row of this lane: vector j / 4 of the quad, digit j % 4
    const uint32_t a_off = (uint32_t)(((g * 4 + (j >> 2)) * 4 + (j & 3)) * 8);
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ncg = ((S + 7) >> 3) / slabs_per_task;
    const int k = S * 256;
    constexpr int kWaveRing = ANY ? kRing4Wave : kRingWave;
    constexpr uint32_t kWindow = ANY ? 511u : 255u;        // ring window of a row, minus one
    // byte offset of the lane's row within its first line (tiles start on a line)
    const uint32_t loff = ANY ? (uint32_t)(j * 144 * S) & 127u : 0u;

    // LDS: staged x (S columns x NQ quads and a spare group; JIT: per wave
    // the digits and constants of one group and the lists of NQ; window: two
    // columns of every slab), the line rings, row sums (f64)
    const int ngroups = S * NQ;
    constexpr int kJitWave = kSbWord + NQ * kSbLists;
    const size_t xbytes = JIT   ? (size_t)NW * kJitWave
                          : WIN ? (size_t)ncg * 2 * NQ * kSbGroup
                                : (size_t)(ngroups + 1) * kSbGroup;
    unsigned char* xw = smem + (JIT ? (size_t)wave * kJitWave : 0);
    unsigned char* xl = xw + kSbWord;            // JIT: the lists of quad q at xl + q kSbLists
    unsigned char* ring = smem + xbytes + wave * kWaveRing;
    double* ypart = reinterpret_cast<double*>(smem + xbytes + NW * kWaveRing);

    // group q0 = column q0 / NQ, quad q0 % NQ; 16-lane group l / 16 takes
    // vector 4 (q0 % NQ) + l / 16 (past the last vector the last vector
    // again: its sums reach only lanes whose results are never stored)
    float4 xv[XC][4];
    auto load_group = [&](int q0, float4 (&v)[4]) __attribute__((always_inline)) {
        int qc = min(q0, ngroups - 1);
        if constexpr (NQ > 4) {
            // eight quads: each address from the group index at its use (the
            // compiler would otherwise keep all eight quads' pointers, and
            // more, live across the stream and spill them)
            asm volatile("" : "+s"(qc));
        }
        const int b = 4 * (qc % NQ) + (lane >> 4);
        const float* src = x + (size_t)min(b, m - 1) * k + (size_t)(qc / NQ) * 256 + 16 * (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = reinterpret_cast<const float4*>(src)[i];
        }
    };
    // JIT: slot a holds the x of a column with c mod kA = a (first column
    // of the wave's first slab: c_first); with eight quads a slot holds
    // four of them (kXQ), and each quad's registers are refilled with the
    // quad four on as soon as it is converted
    constexpr int kA = JIT ? jit_ahead<NQ>() : 1;
    constexpr int kXQ = NQ > 4 ? 4 : NQ;
    float4 xa[kA][kXQ][4];
    const int ntasks = ((rows_here + 15) >> 4) * ncg;
    const int c_first = 8 * ((min(wave, ntasks - 1) % ncg) * slabs_per_task);
    // window: group of quad q of the column in slot sl (column parity) of slab cg
    auto win = [&](int cg, int sl, int q) __attribute__((always_inline)) {
        return smem + (size_t)((cg * 2 + sl) * NQ + q) * kSbGroup;
    };
    // window: the wave's pairs (cg, q) = p / NQ, p % NQ for p = wave + i NW,
    // and the x of columns s, s + 1 of its slab in slot s mod 2
    const int npairs = ncg * NQ;
    float4 xp[WIN ? XC : 1][kWinAhead][4];
    auto pair_load = [&](int i, int s) __attribute__((always_inline)) {
        const int pr = min(wave + i * NW, npairs - 1);
        load_group((8 * (pr / NQ) + min(s, 7)) * NQ + pr % NQ, xp[i][s % kWinAhead]);
    };
    auto pair_convert = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int pr = wave + i * NW;
            if (pr < npairs) {                    // wave-uniform
                unsigned char* grp = win(pr / NQ, s & 1, pr % NQ);
                convert_quad(xp[i][s % kWinAhead], grp, grp + kSbWord, lane);
                pair_load(i, s + kWinAhead);
            }
        }
    };
    auto issue_x = [&]() __attribute__((always_inline)) {
        if constexpr (WIN) {
#pragma unroll
            for (int i = 0; i < XC; ++i) {
#pragma unroll
                for (int a = 0; a < kWinAhead; ++a) {
                    pair_load(i, a);
                }
            }
            return;
        }
        if constexpr (JIT) {
#pragma unroll
            for (int a = 0; a < kA; ++a) {
#pragma unroll
                for (int q = 0; q < kXQ; ++q) {
                    load_group((c_first + a) * NQ + q, xa[a][q]);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            load_group(wave + i * NW, xv[i]);
        }
    };
    auto convert_x = [&]() __attribute__((always_inline)) {
        if constexpr (JIT) {
            return;
        }
        if constexpr (WIN) {
            pair_convert(0);
            return;
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int q0 = wave + i * NW;
            unsigned char* grp = smem + (size_t)min(q0, ngroups) * kSbGroup;
            convert_quad(xv[i], grp, grp + kSbWord, lane);
        }
        for (int q0 = XC * NW + wave; q0 < ngroups; q0 += NW) {
            float4 v[4];
            load_group(q0, v);
            convert_quad(v, smem + (size_t)q0 * kSbGroup, smem + (size_t)q0 * kSbGroup + kSbWord, lane);
        }
    };

    QuadAcc acc;
    // The lane's part of one superblock (column c) of its tile row (ring row
    // rr, offset b0): its codes of the eight sub-blocks as MFMA B operands,
    // and d sc_j (/ 16 for the high sub-blocks, whose digit sums carry 16 q)
    // and dmin m_j, exact in f32.
    struct Tile {
        long codes[8];
        float Ds[8], Ms[8];
        uint32_t b;
    };
    auto prep = [&](const unsigned char* rr, uint32_t b0) __attribute__((always_inline)) {
        Tile t;
        t.b = b0 + loff;
        const uint4 hdr = *reinterpret_cast<const uint4*>(rr + (t.b & kWindow));
        uint2 raw[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            raw[cc] = *reinterpret_cast<const uint2*>(rr + ((t.b + 16u + 32u * cc + 8u * g) & kWindow));
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            t.codes[2 * cc] = __builtin_bit_cast(long, make_uint2(raw[cc].x & 0x0F0F0F0Fu,
                                                                   raw[cc].y & 0x0F0F0F0Fu));
            t.codes[2 * cc + 1] = __builtin_bit_cast(
                long, make_uint2((raw[cc].x & 0xF0F0F0F0u) ^ 0x80808080u,
                                 (raw[cc].y & 0xF0F0F0F0u) ^ 0x80808080u));
        }
        const RowScales rs = decode_row(hdr);
#pragma unroll
        for (int sb = 0; sb < 8; ++sb) {
            t.Ds[sb] = rs.d * rs.sc[sb] * ((sb & 1) ? 0.0625f : 1.0f);
            t.Ms[sb] = rs.dmin * rs.m[sb];
        }
        return t;
    };
    // quad q of the tile against the x group grp: eight MFMAs, the exact
    // sums scaled once per sub-block
    auto quad = [&](const Tile& t, auto qc, const unsigned char* grp) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        const double2* cst = reinterpret_cast<const double2*>(grp + kSbConst + g * 128);
#pragma unroll
        for (int sb = 0; sb < 8; ++sb) {
            const long a = *reinterpret_cast<const long*>(grp + sb * kSbBlock + a_off);
            const double2 k2 = cst[sb];                   // {2^-s, XI}
            const i32x4_t zero = {0, 0, 0, 0};
            const i32x4_t D = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, t.codes[sb], zero, 0, 0, 0);
            double T = digits_exact(D[0], D[1], D[2], D[3]);
            if (sb & 1) {
                T = __builtin_fma(k2.y, 128.0, T);
            }
            acc.at<q>() = subblock_term(acc.at<q>(), t.Ds[sb], T, t.Ms[sb], k2.y, k2.x);
            if constexpr (NQ > 4) {
                // eight quads: the sum is formed here, not sunk towards its
                // use at the task's end (which keeps every quad's MFMA
                // results live and spills)
                asm volatile("" : "+v"(acc.at<q>()));
            }
        }
    };
    // kernel 5: the column's groups of the stage, one quad after the other
    // (a quad's operands are dead before the next one's are read); in a
    // flagged slab then the exact terms of the column's uncertified
    // elements, quad by quad in a loop (one copy of that code per step)
    auto step = [&](int c, const unsigned char* rr, uint32_t b0, auto corr) __attribute__((always_inline)) {
        const Tile t = prep(rr, b0);
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            quad(t, qc, smem + (size_t)(c * NQ + decltype(qc)::value) * kSbGroup);
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (decltype(corr)::value) {
#pragma nounroll
            for (int q = 0; q < NQ; ++q) {
                const unsigned char* grp = smem + (size_t)(c * NQ + q) * kSbGroup;
                const uint4 cnts = *reinterpret_cast<const uint4*>(grp + kSbWord);
                const uint32_t any = __builtin_amdgcn_readfirstlane(cnts.x | cnts.y | cnts.z | cnts.w);
                if (any != 0u) {
                    const uint32_t cnt = g == 0 ? cnts.x : g == 1 ? cnts.y : g == 2 ? cnts.z : cnts.w;
                    const int bv = min(4 * q + g, m - 1);
                    const double a = vector_corrections(
                        acc.get(q), cnt, grp + kSbList + g * (kCorr * 8),
                        reinterpret_cast<const double2*>(grp + kSbConst + g * 128),
                        x + (size_t)bv * k + (size_t)c * 256, t.Ds, t.Ms, rr, t.b, kWindow);
                    acc.set(q, a);
                }
            }
        }
    };
    // kernel 6: convert quad q of column c (registers of slot cp mod kA)
    // into the wave's one group and decode it, quad after quad (the wave's
    // LDS accesses complete in order, so a conversion overwrites the group
    // only after the previous quad's reads); a quad of which some vector has
    // uncertified elements in the column sets its bit in `dirty`, and those
    // quads' exact terms follow, found again from x.  Then the slot is
    // refilled with the column kA positions on (ca: past cend, the next
    // slab's or task's, from cn); with eight quads each quad's registers are
    // refilled right after its conversion, with the quad four on (of this
    // column, then of ca).  Positions past a partial slab's end (invalid)
    // keep the slots cycling.
    auto step_jit = [&](int c, int cend, int cn, const unsigned char* rr, uint32_t b0, int cp,
                        bool valid) __attribute__((always_inline)) {
        float4 (&v)[kXQ][4] = xa[JIT ? cp % kA : 0];
        const int ca = c + kA < cend ? c + kA : cn + (c + kA - cend);
        __builtin_amdgcn_sched_barrier(0);
        if (valid) {
            const Tile t = prep(rr, b0);
            uint32_t dirty = 0;
            static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                int lo = q * kSbLists;
                if constexpr (NQ > 4) {
                    asm volatile("" : "+s"(lo));
                }
                const int total = convert_quad(v[q % kXQ], xw, xl + lo, lane);
                if constexpr (NQ > kXQ) {
                    load_group(q + kXQ < NQ ? c * NQ + q + kXQ : ca * NQ + q + kXQ - NQ,
                               v[q % kXQ]);
                }
                dirty |= (total != 0 ? 1u : 0u) << q;
                quad(t, qc, xw);
                __builtin_amdgcn_sched_barrier(0);
            });
            if (__builtin_amdgcn_readfirstlane(__ballot(dirty != 0u) != 0 ? 1 : 0) != 0) {
#pragma nounroll
                for (int q = 0; q < NQ; ++q) {
                    if ((dirty >> q) & 1u) {
                        const unsigned char* lq = xl + q * kSbLists;
                        const uint32_t cnt = *reinterpret_cast<const uint32_t*>(lq + g * 4);
                        const int bv = min(4 * q + g, m - 1);
                        const double a = vector_corrections(
                            acc.get(q), cnt, lq + 16 + g * (kCorr * 8), nullptr,
                            x + (size_t)bv * k + (size_t)c * 256, t.Ds, t.Ms, rr, t.b, kWindow);
                        acc.set(q, a);
                    }
                }
            }
        }
        if (NQ <= kXQ || !valid) {
#pragma unroll
            for (int q = 0; q < kXQ; ++q) {
                load_group(ca * NQ + q, v[q]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // window: all LDS accesses of this wave done, then every wave at the
    // same point (LDS only: the line loads in flight are not waited for)
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    // window step s = c mod 8: after the barrier, column s is in slot s mod 2
    // of every slab and column s - 1's slot is free: convert column s + 1
    // into it, then decode column c (quads one after the other, the exact
    // terms of a quad with uncertified elements in a loop after them)
    auto step_win = [&](int c, const unsigned char* rr, uint32_t b0) __attribute__((always_inline)) {
        const int sidx = (int)(b0 / 144u);         // c mod 8, a compile-time constant
        if (sidx > 0) {
            lds_barrier();
        }
        if (sidx < 7) {
            pair_convert(sidx + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        const Tile t = prep(rr, b0);
        const int cg = c >> 3;
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            quad(t, qc, win(cg, sidx & 1, decltype(qc)::value));
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma nounroll
        for (int q = 0; q < NQ; ++q) {
            const unsigned char* grp = win(cg, sidx & 1, q);
            const uint4 cnts = *reinterpret_cast<const uint4*>(grp + kSbWord);
            const uint32_t any = __builtin_amdgcn_readfirstlane(cnts.x | cnts.y | cnts.z | cnts.w);
            if (any != 0u) {
                const uint32_t cnt = g == 0 ? cnts.x : g == 1 ? cnts.y : g == 2 ? cnts.z : cnts.w;
                const int bv = min(4 * q + g, m - 1);
                const double a = vector_corrections(
                    acc.get(q), cnt, grp + kSbList + g * (kCorr * 8),
                    reinterpret_cast<const double2*>(grp + kSbConst + g * 128),
                    x + (size_t)bv * k + (size_t)c * 256, t.Ds, t.Ms, rr, t.b, kWindow);
                acc.set(q, a);
            }
        }
    };
    // whether slab sl has a column with uncertified elements in any vector:
    // one bit per column in scalar registers, gathered by a ballot on the
    // first call (after the x stage)
    uint64_t cmask[2] = {0, 0};
    bool have_mask = false;
    auto slab_flag = [&](int sl) __attribute__((always_inline)) {
        if (!have_mask) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 64 * h + lane;
                uint32_t f = 0;
                if (c < S) {
                    for (int q = 0; q < NQ; ++q) {
                        const uint4 cn = *reinterpret_cast<const uint4*>(
                            smem + (size_t)(c * NQ + q) * kSbGroup + kSbWord);
                        f |= cn.x | cn.y | cn.z | cn.w;
                    }
                }
                cmask[h] = __ballot(f != 0u);
            }
            have_mask = true;
        }
        const int c0 = 8 * sl;
        if (c0 >= 128) {
            return true;
        }
        const uint64_t bits = c0 < 64 ? cmask[0] >> c0 : cmask[1] >> (c0 - 64);
        return (bits & 0xFFu) != 0u;
    };
    auto task_end = [&](int task) __attribute__((always_inline)) {
        const int r = (task / ncg) * 16 + j;
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            int b4 = 4 * q;
            if constexpr (NQ > 4) {
                asm volatile("" : "+s"(b4));     // the row's address at its use, as above
            }
            const int b = b4 + g;
            if (b < m && r < rows_here) {
                if (ncg == 1) {
                    y[(size_t)b * n + row0 + r] = (float)acc.at<q>();
                } else {
                    ypart[(b * ncg + task % ncg) * rows_per_block + r] = acc.at<q>();
                }
            }
            acc.at<q>() = 0.0;
        });
    };
    if constexpr (WIN) {
        line_stream<NW, 3>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                           step_win, task_end);
        // a wave without a task: the same conversions and barriers as the
        // eight steps of a slab
        if (wave >= ntasks) {
            static_for<8>([&](auto sc) __attribute__((always_inline)) {
                constexpr int sidx = decltype(sc)::value;
                if constexpr (sidx > 0) {
                    lds_barrier();
                }
                if constexpr (sidx < 7) {
                    pair_convert(sidx + 1);
                }
            });
        }
    } else if constexpr (JIT && ANY) {
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step_jit, task_end);
    } else if constexpr (JIT) {
        line_stream<NW, 3>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                           step_jit, task_end);
    } else if constexpr (ANY) {
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step, task_end, slab_flag);
    } else {
        line_stream<NW, 3>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                           step, task_end, slab_flag);
    }

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here * m; i += NW * 64) {
            const int b = i / rows_here;
            const int r = i - b * rows_here;
            double a = 0.0;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[(b * ncg + cg) * rows_per_block + r];
            }
            y[(size_t)b * n + row0 + r] = (float)a;
        }
    }
}

template <int XC, int NQ, int MODE = kModeStaged, int NW = 8>
static hipError_t launch_sub_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    if (p.waves_per_block != NW) {
        return hipErrorInvalidValue;
    }
    if constexpr (MODE == kModeWindow) {
        // one slab per task, a task for at most every wave, pairs within XC
        // per wave: the plan ensures it; refused here too, as a wave with two
        // tasks would not meet the others at the barriers
        const int ncg = p.S / 8;
        if (p.S % 8 != 0 || p.cols_per_task != 8 || ((p.rows_per_block + 15) / 16) * ncg > NW ||
            ncg * NQ > XC * NW) {
            return hipErrorInvalidValue;
        }
        hipLaunchKernelGGL((gemv_i8_sub_kernel<NW, XC, NQ, MODE, false>), dim3(p.grid),
                           dim3(NW * 64), p.lds_bytes, stream, w, x, y, p.n, p.S, p.m,
                           p.rows_per_block, 1);
    } else if (p.S % 8 != 0) {
        hipLaunchKernelGGL((gemv_i8_sub_kernel<NW, XC, NQ, MODE, true>), dim3(p.grid), dim3(NW * 64),
                           p.lds_bytes, stream, w, x, y, p.n, p.S, p.m, p.rows_per_block,
                           p.cols_per_task / 8);
    } else {
        hipLaunchKernelGGL((gemv_i8_sub_kernel<NW, XC, NQ, MODE, false>), dim3(p.grid), dim3(NW * 64),
                           p.lds_bytes, stream, w, x, y, p.n, p.S, p.m, p.rows_per_block,
                           p.cols_per_task / 8);
    }
    return hipGetLastError();
}

// (column, quad) groups each of the eight waves converts before the first
// barrier: the power of two covering S * NQ / 8, at most 4
template <int NQ>
static hipError_t launch_sub(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                             hipStream_t stream)
{
    const int per = (p.S * NQ + 7) / 8;
    if (per <= 1) return launch_sub_x<1, NQ>(p, w, x, y, stream);
    if (per <= 2) return launch_sub_x<2, NQ>(p, w, x, y, stream);
    return launch_sub_x<4, NQ>(p, w, x, y, stream);
}

template <int NW, int P, int XC, int M>
static hipError_t launch_lines_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                 hipStream_t stream)
{
    hipLaunchKernelGGL((gemv_i8_lines_kernel<NW, P, XC, M>), dim3(p.grid), dim3(NW * 64),
                       p.lds_bytes, stream, w, x, y, p.n, p.S, p.rows_per_block,
                       p.cols_per_task / 8);
    return hipGetLastError();
}

// groups of four (column, vector) pairs of x each wave converts before the
// first barrier: the power of two covering S * m / (4 NW), at most 4 (the
// rest follow in a loop)
template <int NW, int P>
static hipError_t launch_lines_p(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                 hipStream_t stream)
{
    const int per = (p.S + 4 * NW - 1) / (4 * NW);
    if (per <= 1) return launch_lines_x<NW, P, 1, 1>(p, w, x, y, stream);
    if (per <= 2) return launch_lines_x<NW, P, 2, 1>(p, w, x, y, stream);
    return launch_lines_x<NW, P, 4, 1>(p, w, x, y, stream);
}

template <int NW>
static hipError_t launch_lines(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    if (p.ring_depth == 9) return launch_lines_p<NW, 9>(p, w, x, y, stream);
    return launch_lines_p<NW, 3>(p, w, x, y, stream);
}

// several vectors: eight waves, three lines in flight
template <int M>
static hipError_t launch_lines_m(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                 hipStream_t stream)
{
    const int per = (p.S * M + 31) / 32;
    if (per <= 1) return launch_lines_x<8, 3, 1, M>(p, w, x, y, stream);
    if (per <= 2) return launch_lines_x<8, 3, 2, M>(p, w, x, y, stream);
    return launch_lines_x<8, 3, 4, M>(p, w, x, y, stream);
}

// vector quads of the sub-block kernels' launch for m vectors (1, 2, 4 or 8)
static int sub_quads(int m)
{
    return m > kMaxMStaged ? 8 : m > 8 ? 4 : m > 4 ? 2 : 1;
}

hipError_t launch_gemv_mfma(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    if (p.kernel >= 5) {
        const int nq = sub_quads(p.m);         // the quads the LDS sizes count
        if (nq == 8 && p.kernel != 6) {
            return hipErrorInvalidValue;   // eight quads: per-wave x only
        }
        if (p.kernel == 5) {
            if (nq == 4) return launch_sub<4>(p, wb, x, y, stream);
            if (nq == 2) return launch_sub<2>(p, wb, x, y, stream);
            return launch_sub<1>(p, wb, x, y, stream);
        }
        if (p.kernel == 7) {
            // one pair of the window per wave
            if (nq == 4) return launch_sub_x<1, 4, kModeWindow>(p, wb, x, y, stream);
            if (nq == 2) return launch_sub_x<1, 2, kModeWindow>(p, wb, x, y, stream);
            return launch_sub_x<1, 1, kModeWindow>(p, wb, x, y, stream);
        }
        // four or eight quads: four waves, whose lanes may hold 512
        // registers (the x of the next column takes 64 or 128 of them)
        if (nq == 8) return launch_sub_x<1, 8, kModeJit, 4>(p, wb, x, y, stream);
        if (nq == 4) return launch_sub_x<1, 4, kModeJit, 4>(p, wb, x, y, stream);
        if (nq == 2) return launch_sub_x<1, 2, kModeJit>(p, wb, x, y, stream);
        return launch_sub_x<1, 1, kModeJit>(p, wb, x, y, stream);
    }
    if (p.m == 2) {
        return launch_lines_m<2>(p, wb, x, y, stream);
    }
    if (p.m != 1) {
        return hipErrorInvalidValue;   // one MFMA group per vector: one or two vectors
    }
    if (p.waves_per_block == 8) return launch_lines<8>(p, wb, x, y, stream);
    return launch_lines<4>(p, wb, x, y, stream);
}

size_t sub_lds_bytes(int S, int m)
{
    const int nq = sub_quads(m);
    return (size_t)(S * nq + 1) * kSbGroup + (size_t)8 * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

int jit_waves(int m)
{
    return sub_quads(m) >= 4 ? 4 : 8;
}

size_t jit_lds_bytes(int S, int m)
{
    const int nw = jit_waves(m);
    return (size_t)nw * (kSbWord + sub_quads(m) * kSbLists) +
           (size_t)nw * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

// the window kernel: two columns of every slab (S % 8 == 0), eight rings
size_t win_lds_bytes(int S, int m)
{
    return (size_t)(S / 8) * 2 * sub_quads(m) * kSbGroup + (size_t)8 * kRingWave;
}

size_t lines_lds_bytes(int S, int m, int waves)
{
    return (size_t)(S * m + 1) * kK4Pair + (size_t)waves * kRingWave;
}

}  // namespace q4k
